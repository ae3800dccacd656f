"""Seeded synthetic inputs shared by the HIP path's tests, the bench and the oracle.

Holds none of the method's arithmetic: it draws numbers, L2-normalizes the
query and key vectors (the caller's job, since phi is the identity) and rounds
to bfloat16.  The rounded bfloat16 tensor is the single source of truth; both
sides read exactly those values (bf16 -> fp64 is exact).

Shapes follow the pages' ~125M-parameter models (12 heads x 64 dims, arXiv
2608.27763 as summarised by the 163.com article, section 03) and the
workloads below; no dataset item is used.
"""
from __future__ import annotations

import numpy as np

# name -> recipe.  seq: (batch, heads, L, dk, dv); decode: (nseq, heads, dk, dv)
WORKLOADS = {
    "recurrent_f32_1x1x64x16": dict(kind="seq", shape=(1, 1, 64, 16, 16), dtype="f32",
                                    seed=1001, beta=0.5, lam=0.01, eps=1e-6),
    "chunk_8x12x2048x64": dict(kind="seq", shape=(8, 12, 2048, 64, 64), dtype="bf16",
                               seed=1002, beta=0.5, lam=0.01, eps=1e-6, chunk=64),
    "chunk_percol_8x12x4096x64": dict(kind="seq", shape=(8, 12, 4096, 64, 64), dtype="bf16",
                                      seed=1003, beta=None, lam=0.02, eps=1e-6, chunk=64,
                                      beta_per_channel=True),
    "chunk_window4_4x16x8192x128": dict(kind="seq", shape=(4, 16, 8192, 128, 128),
                                        dtype="bf16", seed=1004, beta=0.5, lam=0.01,
                                        eps=1e-6, chunk=64, window=4),
    "masked_256x12x64x64": dict(kind="seq", shape=(256, 12, 64, 64, 64), dtype="bf16",
                                seed=1006, beta=0.5, lam=0.01, eps=1e-6, chunk=64),
    "decode_512x12x64": dict(kind="decode", shape=(512, 12, 64, 64), dtype="bf16",
                             seed=1005, beta=0.5, lam=0.01, eps=1e-6, s_std=0.02),
}


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array of the bfloat16-rounded values of ``a``."""
    return bf16_bits_to_f32(bf16_round_bits(a))


def _l2n(a: np.ndarray) -> np.ndarray:
    return (a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True))).astype(np.float32)


def seq_inputs(batch, heads, L, dk, dv, *, seed, dtype="bf16", beta_per_token=False,
               beta_per_channel=False, with_k_prev=False, with_S0=False, s_std=0.02,
               history=0, key_norms=None):
    """q, k [B,H,L,dk], v [B,H,L,dv] ~ N(0,1) with q, k L2-normalized per token.

    Returns a dict of float32 arrays holding exactly the values of the chosen
    dtype (bf16-rounded when dtype == "bf16"); optional beta_t
    (sigmoid(N(0,1)) per token, or per token and value channel), k_prev
    (one normalized key per (batch, head)), S0 (N(0, s_std^2)) and, with
    history = n > 0, a carried window history x_hist [B,H,n,dk] (normalized
    keys) and y_hist [B,H,n,dv] (N(0,1)), drawn after everything else.
    key_norms = (lo, hi) rescales every key (and k_prev, x_hist) to a norm drawn
    log-uniformly from [lo, hi], after all other draws (unnormalized keys: the
    step size beta / (eps + ||x||^2) then varies from token to token).
    """
    rng = np.random.default_rng(seed)
    q = _l2n(rng.standard_normal((batch, heads, L, dk), dtype=np.float32))
    k = _l2n(rng.standard_normal((batch, heads, L, dk), dtype=np.float32))
    v = rng.standard_normal((batch, heads, L, dv), dtype=np.float32)
    out = dict(q=q, k=k, v=v)
    if beta_per_channel:
        z = rng.standard_normal((batch, heads, L, dv), dtype=np.float32)
        out["beta_t"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    elif beta_per_token:
        z = rng.standard_normal((batch, heads, L), dtype=np.float32)
        out["beta_t"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if with_k_prev:
        out["k_prev"] = _l2n(rng.standard_normal((batch, heads, dk), dtype=np.float32))
    if with_S0:
        out["S0"] = (s_std * rng.standard_normal((batch, heads, dv, dk),
                                                 dtype=np.float32)).astype(np.float32)
    if history > 0:
        out["x_hist"] = _l2n(rng.standard_normal((batch, heads, history, dk), dtype=np.float32))
        out["y_hist"] = rng.standard_normal((batch, heads, history, dv), dtype=np.float32)
    if key_norms is not None:
        lo, hi = np.log(key_norms[0]), np.log(key_norms[1])
        for name in ("k", "k_prev", "x_hist"):
            if name in out:
                r = np.exp(rng.uniform(lo, hi, size=out[name].shape[:-1] + (1,)))
                out[name] = (out[name] * r).astype(np.float32)
    if dtype == "bf16":
        for name in ("q", "k", "v", "beta_t", "k_prev", "x_hist", "y_hist"):
            if name in out:
                out[name] = to_bf16_values(out[name])
    return out


def decode_inputs(nseq, heads, dk, dv, *, seed, steps=1, s_std=0.02, dtype="bf16",
                  beta_per_channel=False, history=0):
    """Decode workload: S [N,H,dv,dk] ~ N(0, s_std^2) fp32, k_prev [N,H,dk], and a
    pool of ``steps`` per-step (q, k, v) with q, k normalized; bf16-rounded.  With
    history = n > 0 also a window history x_hist [N,H,n,dk], y_hist [N,H,n,dv]."""
    rng = np.random.default_rng(seed)
    S = (s_std * rng.standard_normal((nseq, heads, dv, dk), dtype=np.float32)).astype(np.float32)
    k_prev = _l2n(rng.standard_normal((nseq, heads, dk), dtype=np.float32))
    q = _l2n(rng.standard_normal((steps, nseq, heads, dk), dtype=np.float32))
    k = _l2n(rng.standard_normal((steps, nseq, heads, dk), dtype=np.float32))
    v = rng.standard_normal((steps, nseq, heads, dv), dtype=np.float32)
    out = dict(S=S, k_prev=k_prev, q=q, k=k, v=v)
    if beta_per_channel:
        z = rng.standard_normal((steps, nseq, heads, dv), dtype=np.float32)
        out["beta_t"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if history > 0:
        out["x_hist"] = _l2n(rng.standard_normal((nseq, heads, history, dk), dtype=np.float32))
        out["y_hist"] = rng.standard_normal((nseq, heads, history, dv), dtype=np.float32)
    if dtype == "bf16":
        for name in ("q", "k", "v", "k_prev", "beta_t", "x_hist", "y_hist"):
            if name in out:
                out[name] = to_bf16_values(out[name])
    return out

"""Runs the fp64 oracle over groups of independent (batch, head) chains in worker
processes, for the parity tests at the full workload sizes.

Every chain of the recurrence is independent of every other (the update and the
readout act per (batch, head)), so evaluating the oracle on a group of chains
gives exactly the rows of one call over the whole batch.  The workers are
started (spawned, numpy only) before any test touches the GPU, by
``start()`` from conftest; without a pool the same functions run in-process.
"""
from __future__ import annotations

import os

import numpy as np

_POOL = None


def start(n=None):
    """Spawn the worker pool (call before the GPU is initialised)."""
    global _POOL
    if _POOL is not None:
        return
    import multiprocessing as mp
    if n is None:
        n = min(16, len(os.sched_getaffinity(0)))
    if n < 2:
        return
    _POOL = mp.get_context("spawn").Pool(n)


def stop():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def workers():
    return _POOL._processes if _POOL is not None else 1


def _flat(a):
    return None if a is None else a.reshape((-1,) + a.shape[2:])


def _recurrence_group(args):
    from oracle import falcon_oracle as fo
    variant, arrs, kw = args
    o, S, _ = fo.falcon_recurrence(variant, arrs["q"], arrs["k"], arrs["v"],
                                   beta_t=arrs.get("beta_t"), k_prev=arrs.get("k_prev"),
                                   S0=arrs.get("S0"), **kw)
    return o[:, 0], S[:, 0]


def recurrence_all_chains(variant, inp, **kw):
    """The oracle's (o, S_L) for every chain of ``inp`` (dict of [B, H, ...]
    arrays), as [B*H, L, dv] and [B*H, dv, dk]."""
    names = [n for n in ("q", "k", "v", "beta_t", "k_prev", "S0") if inp.get(n) is not None]
    nchain = inp["q"].shape[0] * inp["q"].shape[1]
    groups = np.array_split(np.arange(nchain), min(workers() * 2, nchain))
    jobs = [(variant, {n: _flat(inp[n])[g][:, None] for n in names}, kw) for g in groups]
    res = _POOL.map(_recurrence_group, jobs) if _POOL is not None else list(map(_recurrence_group, jobs))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def _decode_group(args):
    from oracle import falcon_oracle as fo
    variant, S, kp, q, k, v, bt, steps, check, kw = args
    pool = q.shape[0]
    outs = {}
    for s in range(1, steps + 1):
        p = (s - 1) % pool
        o, S, kp = fo.falcon_decode_step(variant, S, kp, q[p], k[p], v[p],
                                         beta_t=None if bt is None else bt[p], **kw)
        if s in check:
            outs[s] = o[:, 0]
    return outs, S[:, 0], kp[:, 0]


def decode_all_pairs(variant, inp, steps, check, **kw):
    """The oracle's decode run over every (sequence, head) pair: o at the steps in
    ``check`` ([N*H, dv] each), S and k_prev after ``steps`` steps.  ``inp`` is a
    decode_inputs dict (S [N,H,dv,dk], k_prev [N,H,dk], pools q, k, v [P,N,H,.])."""
    N, H = inp["S"].shape[:2]
    groups = np.array_split(np.arange(N * H), min(workers() * 2, N * H))
    pf = lambda a: a.reshape((a.shape[0], N * H) + a.shape[3:])
    q, k, v = pf(inp["q"]), pf(inp["k"]), pf(inp["v"])
    bt = pf(inp["beta_t"]) if inp.get("beta_t") is not None else None
    S, kp = _flat(inp["S"]), _flat(inp["k_prev"])
    jobs = [(variant, S[g][:, None].astype(np.float64), kp[g][:, None].astype(np.float64),
             q[:, g][:, :, None], k[:, g][:, :, None], v[:, g][:, :, None],
             None if bt is None else bt[:, g][:, :, None], steps, set(check), kw)
            for g in groups]
    res = _POOL.map(_decode_group, jobs) if _POOL is not None else list(map(_decode_group, jobs))
    o = {s: np.concatenate([r[0][s] for r in res]) for s in check}
    return o, np.concatenate([r[1] for r in res]), np.concatenate([r[2] for r in res])


def _backward_group(args):
    from oracle import falcon_oracle as fo
    variant, arrs, kw = args
    g = fo.falcon_backward(variant, arrs["q"], arrs["k"], arrs["v"], arrs["dO"], **kw)
    return {n: a[:, 0] for n, a in g.items()}


def backward_all_chains(variant, inp, dO, **kw):
    """The oracle's gradients for every chain, each as [B*H, ...]; ``inp`` holds
    q, k, v [B, H, L, .] (no optional inputs), dO [B, H, L, dv]."""
    nchain = inp["q"].shape[0] * inp["q"].shape[1]
    groups = np.array_split(np.arange(nchain), min(workers() * 2, nchain))
    src = dict(q=inp["q"], k=inp["k"], v=inp["v"], dO=dO)
    jobs = [(variant, {n: _flat(a)[g][:, None] for n, a in src.items()}, kw) for g in groups]
    res = _POOL.map(_backward_group, jobs) if _POOL is not None else list(map(_backward_group, jobs))
    return {n: np.concatenate([r[n] for r in res]) for n in res[0]}

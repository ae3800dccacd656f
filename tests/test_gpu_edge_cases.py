"""GPU parity on the method's own edge cases, for every chunk kernel family and
for the recurrent and decode kernels (the oracle decides).

* strong decay: lambda * beta in {0.5, 0.9, 0.99}, so the per-step decay
  a_t = 1 - eta_t lambda falls to about 0.01 and its products over a chunk
  leave the float32 range (the decayed NLMS write of the 163.com article,
  section 02 (1));
* unnormalized keys, norms 0.1 .. 3: the step eta_t = beta / (eps + n_t) varies
  by a factor of about 900 from token to token;
* lambda = eps = 0 with a carried key: textbook NLMS (163.com 02 (1));
* beta = 1, lambda = eps = 0 in fp32: every write interpolates its sample,
  S_t x_t = y_t (explainer 核心方法 §1: one normalized step on the squared
  error with unit gain).
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import decode_inputs, seq_inputs, to_bf16_values
from parity_util import TOL_BF16, TOL_FP32_MATH, state_err, to_dev, token_normwise_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


# (label, variant, dk, dv, window, gains, chunk): one entry per chunk kernel
# family and shape class the dispatcher distinguishes
FAMILIES = [
    ("wy", fw.FALCON_1, 64, 64, 1, "scalar", 64),
    ("wy_1a", fw.FALCON_1A, 64, 64, 1, "token", 64),
    ("wy_dk32", fw.FALCON_1, 32, 32, 1, "token", 64),
    ("w1_percol", fw.FALCON_2, 64, 64, 1, "channel", 64),
    ("w1_percol_2a", fw.FALCON_2A, 32, 16, 1, "channel", 64),
    ("w1_percol_c16", fw.FALCON_2, 64, 32, 1, "channel", 16),
    ("w1_dk128", fw.FALCON_1, 128, 32, 1, "scalar", 64),
    ("w1_dk16", fw.FALCON_1, 16, 32, 1, "token", 64),
    ("wyb_w4", fw.FALCON_3, 128, 32, 4, "scalar", 64),        # two kernels (pre-pass + state)
    ("wyb_w2", fw.FALCON_3, 64, 64, 2, "token", 64),
    ("wyb_w4_fused", fw.FALCON_3, 128, 32, 4, "token", 64),   # one kernel (no workspace)
    ("wyb_w2_fused", fw.FALCON_3, 64, 64, 2, "scalar", 64),
    ("ip_w4", fw.FALCON_3A, 128, 64, 4, "scalar", 64),
    ("ip_1a_dk128", fw.FALCON_1A, 128, 32, 1, "token", 64),
    ("ip_w8", fw.FALCON_3A, 64, 32, 8, "token", 64),
    ("generic_w3", fw.FALCON_3, 64, 32, 3, "token", 64),
    ("generic_w2_dk32", fw.FALCON_3A, 32, 32, 2, "scalar", 32),
]


def _inputs(label, variant, dk, dv, gains, L, seed, **extra):
    return seq_inputs(2, 2, L, dk, dv, seed=seed, dtype="bf16",
                      beta_per_channel=gains == "channel", beta_per_token=gains == "token",
                      **extra)


def _chunk_vs_oracle(label, variant, dk, dv, window, gains, chunk, inp, *, beta, lam, eps,
                     carried=False):
    dt = torch.bfloat16
    q, k, v = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    bt = to_dev(torch, inp["beta_t"], dt) if "beta_t" in inp else None
    kp = to_dev(torch, inp["k_prev"], dt) if carried else None
    S0 = to_dev(torch, inp["S0"], torch.float32) if carried and "S0" in inp else None
    b = beta if gains == "scalar" else None
    print("%s: launching" % label, flush=True)
    ws = None if label.endswith("_fused") else "auto"
    o, S = fw.fwd_chunk(q, k, v, variant=variant, beta=b, lam=lam, eps=eps, window=window,
                        chunk=chunk, beta_t=bt, k_prev=kp, S0=S0, return_state=True, workspace=ws)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta=b,
                                           lam=lam, eps=eps, window=window,
                                           beta_t=inp.get("beta_t"),
                                           k_prev=inp["k_prev"] if carried else None,
                                           S0=inp["S0"] if carried and "S0" in inp else None)
    o = o.cpu().numpy()
    S = S.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)), "non-finite output"
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("%s: o err %.3e S err %.3e" % (label, err, serr))
    assert zok and err <= TOL_BF16 and serr <= TOL_BF16


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("lam_beta", [0.5, 0.9, 0.99])
def test_chunk_strong_decay(fam, lam_beta):
    """eta_t lambda close to lam_beta at every step: gains near 1 (scalar 1, or
    per-token / per-channel gains in [0.95, 1]) and lambda = lam_beta * window,
    so with unit keys (n_t = window) the decay a_t = 1 - eta_t lambda sits
    between 1 - lam_beta and about 1.05 (1 - lam_beta); at 0.99 the product of
    the decays over 32 steps is far below the float32 range."""
    label, variant, dk, dv, window, gains, chunk = fam
    L = 3 * 64 + 11
    inp = _inputs(label, variant, dk, dv, gains, L, seed=900 + int(100 * lam_beta) + dk + window)
    if "beta_t" in inp:
        inp["beta_t"] = to_bf16_values(0.95 + 0.05 * inp["beta_t"])
    _chunk_vs_oracle("%s lam*beta %.2f" % (label, lam_beta), variant, dk, dv, window, gains,
                     chunk, inp, beta=1.0, lam=lam_beta * window, eps=1e-6)


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_chunk_unnormalized_keys(fam):
    label, variant, dk, dv, window, gains, chunk = fam
    L = 2 * 64 + 37
    inp = _inputs(label, variant, dk, dv, gains, L, seed=950 + dk + window,
                  key_norms=(0.1, 3.0), with_k_prev=True)
    _chunk_vs_oracle(label + " key norms 0.1..3", variant, dk, dv, window, gains, chunk, inp,
                     beta=0.5, lam=0.01, eps=1e-6, carried=True)


REGRESSION_FAMILIES = [f for f in FAMILIES if fo.is_regression(f[1])]


@pytest.mark.parametrize("fam", REGRESSION_FAMILIES, ids=[f[0] for f in REGRESSION_FAMILIES])
def test_chunk_exact_nlms_carried_key(fam):
    """lambda = eps = 0: no decay, eta_t = beta / ||x_t||^2 (textbook NLMS); the
    carried key makes x_1 non-zero, so no step has a zero normalizer."""
    label, variant, dk, dv, window, gains, chunk = fam
    L = 2 * 64 + 9
    inp = _inputs(label, variant, dk, dv, gains, L, seed=970 + dk + window, with_k_prev=True)
    _chunk_vs_oracle(label + " NLMS", variant, dk, dv, window, gains, chunk, inp, beta=0.7,
                     lam=0.0, eps=0.0, carried=True)


@pytest.mark.parametrize("variant,window", [(fw.FALCON_1, 1), (fw.FALCON_2, 1), (fw.FALCON_3, 3)])
@pytest.mark.parametrize("dk,dv", [(64, 64), (16, 32), (128, 16)])
def test_recurrent_interpolation_fp32(variant, window, dk, dv):
    """beta = 1, lambda = eps = 0, fp32 inputs: after the call the state maps the
    last window's newest sample onto its value, and o matches the oracle."""
    per_ch = variant == fw.FALCON_2
    L = 40
    inp = seq_inputs(1, 2, L, dk, dv, seed=990 + variant + dk, dtype="f32", with_k_prev=True,
                     beta_per_channel=per_ch)
    if per_ch:
        inp["beta_t"] = np.ones_like(inp["beta_t"])
    dt = torch.float32
    q, k, v, kp = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "k_prev"))
    bt = to_dev(torch, inp["beta_t"], dt) if per_ch else None
    o, S = fw.fwd_recurrent(q, k, v, variant=variant, beta=None if per_ch else 1.0, lam=0.0,
                            eps=0.0, window=window, beta_t=bt, k_prev=kp, return_state=True)
    torch.cuda.synchronize()
    S = S.cpu().numpy().astype(np.float64)
    x_last = inp["k"][:, :, L - 2].astype(np.float64)          # x_L = k_{L-1}
    y_last = inp["v"][:, :, L - 1].astype(np.float64)
    Sx = np.einsum("bhik,bhk->bhi", S, x_last)
    interp = float(np.max(np.abs(Sx - y_last)) / np.max(np.abs(y_last)))
    o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"],
                                           beta=None if per_ch else 1.0, lam=0.0, eps=0.0,
                                           window=window, beta_t=inp.get("beta_t"),
                                           k_prev=inp["k_prev"])
    err, zok = token_normwise_err(o.cpu().numpy(), o_ref)
    print("recurrent interpolation v%d w%d dk %d: |S x - y| %.2e, o err %.2e"
          % (variant, window, dk, interp, err))
    if window == 1:
        assert interp <= TOL_FP32_MATH
    assert zok and err <= TOL_FP32_MATH and state_err(S, S_ref) <= TOL_FP32_MATH


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_2])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 32)])
def test_decode_interpolation_fp32(variant, dk, dv):
    """One decode step with beta = 1, lambda = eps = 0: S_new k_prev = v."""
    per_ch = variant == fw.FALCON_2
    inp = decode_inputs(4, 3, dk, dv, seed=995 + variant + dk, steps=3, s_std=0.3, dtype="f32",
                        beta_per_channel=per_ch)
    dt = torch.float32
    S = to_dev(torch, inp["S"], torch.float32)
    kp = to_dev(torch, inp["k_prev"], dt)
    S_r, kp_r = inp["S"].astype(np.float64), inp["k_prev"].astype(np.float64)
    for s in range(3):
        x = kp.cpu().numpy().astype(np.float64)
        bt = torch.ones((4, 3, dv), device="cuda", dtype=dt) if per_ch else None
        o = fw.decode_step(S, kp, to_dev(torch, inp["q"][s], dt), to_dev(torch, inp["k"][s], dt),
                           to_dev(torch, inp["v"][s], dt), variant=variant,
                           beta=None if per_ch else 1.0, lam=0.0, eps=0.0, beta_t=bt)
        o_r, S_r, kp_r = fo.falcon_decode_step(variant, S_r, kp_r, inp["q"][s], inp["k"][s],
                                               inp["v"][s], beta=None if per_ch else 1.0,
                                               lam=0.0, eps=0.0,
                                               beta_t=np.ones((4, 3, dv)) if per_ch else None)
        torch.cuda.synchronize()
        Sn = S.cpu().numpy().astype(np.float64)
        Sx = np.einsum("nhik,nhk->nhi", Sn, x)
        y = inp["v"][s].astype(np.float64)
        interp = float(np.max(np.abs(Sx - y)) / np.max(np.abs(y)))
        err, zok = token_normwise_err(o.cpu().numpy(), o_r)
        print("decode interpolation v%d dk %d step %d: |S x - y| %.2e, o err %.2e"
              % (variant, dk, s, interp, err))
        assert interp <= TOL_FP32_MATH
        assert zok and err <= TOL_FP32_MATH
    assert state_err(S.cpu().numpy(), S_r) <= TOL_FP32_MATH


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_chunk_zero_decay(fam):
    """a_t = 0 exactly: one-hot keys (unit norm in bfloat16), eps = 0, gains 1 and
    lambda = window, so eta_t lambda = 1 at every step whose window is full; the
    state forgets everything but the current write (inner-product family) or
    its projection (regression family)."""
    label, variant, dk, dv, window, gains, chunk = fam
    L = 2 * 64 + 21
    inp = _inputs(label, variant, dk, dv, gains, L, seed=980 + dk + window, with_k_prev=True)
    rng = np.random.default_rng(981 + dk + window)
    onehot = lambda shape: np.eye(dk, dtype=np.float32)[rng.integers(0, dk, size=shape)]
    inp["k"] = onehot(inp["k"].shape[:-1])
    inp["k_prev"] = onehot(inp["k_prev"].shape[:-1])
    if "beta_t" in inp:
        inp["beta_t"] = np.ones_like(inp["beta_t"])
    _chunk_vs_oracle(label + " zero decay", variant, dk, dv, window, gains, chunk, inp,
                     beta=1.0, lam=float(window), eps=0.0, carried=True)


@pytest.mark.parametrize("variant,window", [(fw.FALCON_1, 1), (fw.FALCON_2, 1), (fw.FALCON_3, 4),
                                            (fw.FALCON_1A, 1), (fw.FALCON_3A, 3)])
@pytest.mark.parametrize("lam_beta", [0.5, 0.9])
def test_backward_strong_decay(variant, window, lam_beta):
    """The backward's 16-step chunks keep their decay products in range up to
    eta_t lambda of about 0.95: gradients match the oracle's at 0.5 and 0.9."""
    per_ch = variant == fw.FALCON_2
    L, dk, dv = 53, 32, 16
    inp = seq_inputs(2, 2, L, dk, dv, seed=1300 + variant + window + int(10 * lam_beta),
                     dtype="bf16", beta_per_channel=per_ch, beta_per_token=not per_ch,
                     with_k_prev=True)
    inp["beta_t"] = to_bf16_values(0.95 + 0.05 * inp["beta_t"])
    rng = np.random.default_rng(1301 + variant)
    dO = rng.standard_normal((2, 2, L, dv)).astype(np.float32)
    dev = lambda n: to_dev(torch, inp[n], torch.bfloat16)
    got = fw.bwd_chunk(dev("q"), dev("k"), dev("v"), to_dev(torch, dO, torch.float32),
                       variant=variant, beta=None, lam=lam_beta * window, eps=1e-6,
                       window=window, beta_t=dev("beta_t"), k_prev=dev("k_prev"))
    torch.cuda.synchronize()
    ref = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta=None,
                             lam=lam_beta * window, eps=1e-6, window=window,
                             beta_t=inp["beta_t"], k_prev=inp["k_prev"])
    errs = {}
    for n in ref:
        g = got[n].cpu().numpy().astype(np.float64)
        errs[n] = float(np.max(np.abs(g - ref[n])) / max(np.max(np.abs(ref[n])), 1e-30))
    print("backward strong decay v%d w%d lam*beta %.1f: %s"
          % (variant, window, lam_beta, {n: "%.2e" % e for n, e in errs.items()}))
    assert max(errs.values()) <= TOL_FP32_MATH, errs


@pytest.mark.parametrize("variant,window", [(fw.FALCON_1, 1), (fw.FALCON_3, 4), (fw.FALCON_1A, 1)])
@pytest.mark.parametrize("dv", [16, 64])
def test_backward_out_of_range_is_nan(variant, window, dv):
    """a_t = 0 exactly (one-hot keys, eps = 0, lambda = window): the backward has
    no exact path for such chains and marks every gradient of the chain NaN;
    a chain whose decays stay in range (keys of norm 2: eta_t lambda near 1/4)
    keeps finite, oracle-exact gradients."""
    L, dk = 41, 32
    inp = seq_inputs(1, 2, L, dk, dv, seed=1310 + variant + window + dv, dtype="bf16",
                     with_k_prev=True)
    rng = np.random.default_rng(1311 + dv)
    onehot = lambda shape: np.eye(dk, dtype=np.float32)[rng.integers(0, dk, size=shape)]
    inp["k"][:, 0] = onehot((1, L))             # head 0: zero decay
    inp["k_prev"][:, 0] = onehot((1,))
    inp["k"][:, 1] *= 2.0                       # head 1: keys of norm 2, a_t near 3/4
    inp["k_prev"][:, 1] *= 2.0
    dO = rng.standard_normal((1, 2, L, dv)).astype(np.float32)
    dev = lambda n: to_dev(torch, inp[n], torch.bfloat16)
    got = fw.bwd_chunk(dev("q"), dev("k"), dev("v"), to_dev(torch, dO, torch.float32),
                       variant=variant, beta=1.0, lam=float(window), eps=0.0, window=window,
                       k_prev=dev("k_prev"))
    torch.cuda.synchronize()
    ref = fo.falcon_backward(variant, inp["q"][:, 1:], inp["k"][:, 1:], inp["v"][:, 1:],
                             dO[:, 1:], beta=1.0, lam=float(window), eps=0.0, window=window,
                             k_prev=inp["k_prev"][:, 1:])
    for n, g in got.items():
        g = g.cpu().numpy()
        if n == "dk":
            # k_{L-1} is the next call's carried key, not an input of this call's
            # update: its gradient is dk_last (zero here) whatever the chain
            assert np.all(g[:, 0, L - 1] == 0.0)
            assert np.all(np.isnan(g[:, 0, :L - 1])), n
        else:
            assert np.all(np.isnan(g[:, 0])), n
        assert np.all(np.isfinite(g[:, 1])), n
        err = float(np.max(np.abs(g[:, 1:] - ref[n])) / max(np.max(np.abs(ref[n])), 1e-30))
        assert err <= TOL_FP32_MATH, (n, err)

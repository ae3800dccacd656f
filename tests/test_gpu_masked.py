"""GPU parity of the masked-parallel form (falcon_fwd_masked: a call of L <= 64
steps solved as one masked system) against the fp64 oracle.

The kernel works in fp32 on the exact input values (bf16 inputs are exact in
fp32; the Gram products run on the fp32 matrix cores), so every case is held to
the fp32 gate, bf16 inputs included.  Outputs are compared element by element
(o per token, S_out per chain, the window history bit for bit).
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs
from parity_util import TOL_BF16, TOL_FP32_MATH, state_err, to_dev, token_normwise_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402

ALL = [fw.FALCON_1, fw.FALCON_2, fw.FALCON_3, fw.FALCON_1A, fw.FALCON_2A, fw.FALCON_3A]
PER_CH = (fw.FALCON_2, fw.FALCON_2A)
WINDOWED = (fw.FALCON_3, fw.FALCON_3A)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _run(inp, variant, dtype, *, window, beta, lam, eps, same_step=False, history=False,
         return_history=False):
    dt = _dt(dtype)
    q, k, v = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    bt = to_dev(torch, inp["beta_t"], dt) if "beta_t" in inp else None
    kp = to_dev(torch, inp["k_prev"], dt) if "k_prev" in inp else None
    S0 = to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None
    xh = to_dev(torch, inp["x_hist"], dt) if history else None
    yh = to_dev(torch, inp["y_hist"], dt) if history else None
    res = fw.fwd_masked(q, k, v, variant=variant, beta=beta, lam=lam, eps=eps, window=window,
                        beta_t=bt, k_prev=kp, S0=S0, x_hist=xh, y_hist=yh, return_state=True,
                        return_history=return_history, same_step=same_step)
    torch.cuda.synchronize()
    return [r.float().cpu().numpy() for r in res]


def _ref(inp, variant, *, window, beta, lam, eps, same_step=False, history=False):
    o, S, _ = fo.falcon_recurrence(
        variant, inp["q"], inp["k"], inp["v"], beta=beta, lam=lam, eps=eps, window=window,
        beta_t=inp.get("beta_t"), k_prev=inp.get("k_prev"), S0=inp.get("S0"),
        x_hist=inp.get("x_hist") if history else None,
        y_hist=inp.get("y_hist") if history else None, same_step=same_step)
    return o, S


def _check(o, S, o_ref, S_ref, tol=TOL_FP32_MATH, label=""):
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("%s: o err %.3e S err %.3e" % (label, err, serr))
    assert zok and err <= tol and serr <= tol


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 16, 37, 64])
@pytest.mark.parametrize("dk,dv", [(64, 64), (16, 128), (128, 32)])
def test_masked_fresh(variant, dtype, L, dk, dv):
    """Fresh sequences (x_1 = 0, S_0 = 0), every variant, ragged lengths."""
    win = 4 if variant in WINDOWED else 1
    per_ch = variant in PER_CH
    inp = seq_inputs(2, 3, L, dk, dv, seed=900 + 11 * variant + L + dk, dtype=dtype,
                     beta_per_channel=per_ch, beta_per_token=not per_ch)
    o, S = _run(inp, variant, dtype, window=win, beta=None, lam=0.02, eps=1e-6)
    o_ref, S_ref = _ref(inp, variant, window=win, beta=None, lam=0.02, eps=1e-6)
    _check(o, S, o_ref, S_ref, label="v%d %s L %d dk %d dv %d" % (variant, dtype, L, dk, dv))


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("same_step", [False, True])
@pytest.mark.parametrize("dk,dv", [(32, 16), (64, 64)])
def test_masked_carried_state(variant, same_step, dk, dv):
    """A live start state (and the carried key with prefix pairing); scalar gains;
    windowed variants with their window history in and out."""
    win = 3 if variant in WINDOWED else 1
    inp = seq_inputs(2, 2, 50, dk, dv, seed=960 + 5 * variant + dk, dtype="bf16",
                     with_k_prev=not same_step, with_S0=True, s_std=0.2, history=win - 1)
    hist = win > 1
    res = _run(inp, variant, "bf16", window=win, beta=0.7, lam=0.01, eps=1e-6,
               same_step=same_step, history=hist, return_history=hist)
    o_ref, S_ref = _ref(inp, variant, window=win, beta=0.7, lam=0.01, eps=1e-6,
                        same_step=same_step, history=hist)
    _check(res[0], res[1], o_ref, S_ref, label="v%d same_step %d" % (variant, same_step))
    if hist:
        xr, yr = fo.falcon_history(inp["k"], inp["v"], win, k_prev=inp.get("k_prev"),
                                   x_hist=inp["x_hist"], y_hist=inp["y_hist"],
                                   same_step=same_step)
        np.testing.assert_array_equal(res[2], xr)
        np.testing.assert_array_equal(res[3], yr)


@pytest.mark.parametrize("variant", WINDOWED)
@pytest.mark.parametrize("window", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("L", [5, 64])
def test_masked_windows(variant, window, L):
    """Windows 1..8 with the carried history, per-token gains."""
    inp = seq_inputs(1, 3, L, 64, 32, seed=1000 + 13 * window + L + variant, dtype="bf16",
                     with_k_prev=True, with_S0=True, beta_per_token=True, s_std=0.2,
                     history=window - 1)
    o, S = _run(inp, variant, "bf16", window=window, beta=None, lam=0.02, eps=1e-6,
                history=True)
    o_ref, S_ref = _ref(inp, variant, window=window, beta=None, lam=0.02, eps=1e-6,
                        history=True)
    _check(o, S, o_ref, S_ref, label="v%d window %d L %d" % (variant, window, L))


@pytest.mark.parametrize("variant", ALL)
def test_masked_matches_masked_parallel_oracle(variant):
    """Against the oracle's own masked-parallel evaluation (transition products,
    no residuals) as well as the recurrence."""
    win = 2 if variant in WINDOWED else 1
    per_ch = variant in PER_CH
    inp = seq_inputs(1, 2, 24, 16, 16, seed=740 + variant, dtype="bf16", with_S0=True,
                     with_k_prev=True, beta_per_channel=per_ch, beta_per_token=not per_ch,
                     s_std=0.2, history=win - 1)
    if win > 1:   # a windowed state travels with its history: zero samples here
        inp["x_hist"][:] = 0.0
        inp["y_hist"][:] = 0.0
    o, _ = _run(inp, variant, "bf16", window=win, beta=None, lam=0.02, eps=1e-6,
                history=win > 1)
    o_ref = fo.falcon_masked_parallel(variant, inp["q"], inp["k"], inp["v"], beta=None,
                                      lam=0.02, eps=1e-6, window=win, beta_t=inp["beta_t"],
                                      k_prev=inp["k_prev"], S0=inp["S0"])
    err, zok = token_normwise_err(o, o_ref)
    print("v%d: o err %.3e against the masked-parallel oracle" % (variant, err))
    assert zok and err <= TOL_FP32_MATH


@pytest.mark.parametrize("variant,window", [(fw.FALCON_1, 1), (fw.FALCON_2, 1), (fw.FALCON_3, 4),
                                            (fw.FALCON_1A, 1), (fw.FALCON_3A, 4)])
@pytest.mark.parametrize("lam_beta", [0.5, 0.9, 0.99, 0.999])
def test_masked_strong_decay(variant, window, lam_beta):
    """Strong forgetting (eta lambda near 1 on unit keys): the decay products fall
    far below any float range of a scaled chunk form; the masked form multiplies
    them out in order and stays exact."""
    per_ch = variant == fw.FALCON_2
    inp = seq_inputs(2, 2, 64, 64, 64, seed=1100 + variant + int(1000 * lam_beta),
                     dtype="bf16", with_k_prev=True, beta_per_channel=per_ch)
    if per_ch:
        inp["beta_t"] = (0.95 + 0.05 * inp["beta_t"]).astype(np.float32)
        inp["beta_t"] = fo_bf16(inp["beta_t"])
    beta = None if per_ch else 1.0
    lam = lam_beta * window       # window norms sum to about `window` for unit keys
    o, S = _run(inp, variant, "bf16", window=window, beta=beta, lam=lam, eps=1e-6)
    o_ref, S_ref = _ref(inp, variant, window=window, beta=beta, lam=lam, eps=1e-6)
    _check(o, S, o_ref, S_ref, label="v%d lam*beta %.3f" % (variant, lam_beta))


def fo_bf16(a):
    """Round fp32 values to bf16 (nearest even), as the input generator does."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.float().numpy()


def test_masked_interpolation():
    """beta = 1, lambda = eps = 0: every write makes S_t x_t = y_t exactly, so a
    read with q_t = x_t returns o_t = y_t."""
    inp = seq_inputs(1, 2, 40, 32, 16, seed=1200, dtype="f32", with_k_prev=True)
    # query each step with the key it wrote: x_t = k_{t-1} (k_prev at t = 1)
    x = np.concatenate([inp["k_prev"][:, :, None], inp["k"][:, :, :-1]], axis=2)
    inp["q"] = x.copy()
    o, _ = _run(inp, fw.FALCON_1, "f32", window=1, beta=1.0, lam=0.0, eps=0.0)
    np.testing.assert_allclose(o, inp["v"], rtol=0, atol=2e-4)


def test_masked_exact_nlms_unnormalized_keys():
    """lambda = eps = 0 with unnormalized keys (norms 0.1..3): textbook NLMS."""
    inp = seq_inputs(2, 2, 64, 64, 32, seed=1210, dtype="bf16", with_k_prev=True,
                     with_S0=True, s_std=0.3, key_norms=(0.1, 3.0))
    o, S = _run(inp, fw.FALCON_1, "bf16", window=1, beta=0.8, lam=0.0, eps=0.0)
    o_ref, S_ref = _ref(inp, fw.FALCON_1, window=1, beta=0.8, lam=0.0, eps=0.0)
    _check(o, S, o_ref, S_ref, label="NLMS")


def test_masked_in_place_state_and_recurrent_agreement():
    """S_out == S0 (in-place carry) gives the same result; and the masked and
    recurrent kernels agree to fp32 rounding."""
    inp = seq_inputs(3, 4, 33, 64, 64, seed=1220, dtype="bf16", with_k_prev=True,
                     with_S0=True, s_std=0.2, beta_per_token=True)
    dt = torch.bfloat16
    q, k, v, bt, kp = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "beta_t", "k_prev"))
    S0 = to_dev(torch, inp["S0"], torch.float32)
    kw = dict(variant=fw.FALCON_1, beta=None, lam=0.01, eps=1e-6, beta_t=bt, k_prev=kp)
    o1, S1 = fw.fwd_masked(q, k, v, S0=S0, return_state=True, **kw)
    S_inp = S0.clone()
    o2 = fw.fwd_masked(q, k, v, S0=S_inp, S_out=S_inp, **kw)
    o3, S3 = fw.fwd_recurrent(q, k, v, S0=S0, return_state=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S_inp)
    err, _ = token_normwise_err(o1.cpu().numpy(), o3.cpu().numpy())
    assert err <= TOL_FP32_MATH and state_err(S1.cpu().numpy(), S3.cpu().numpy()) <= TOL_FP32_MATH


def test_masked_many_chains():
    """The bench workload's shape (256 sequences x 12 heads, L = 64, d = 64),
    every chain against the oracle."""
    inp = seq_inputs(256, 12, 64, 64, 64, seed=1230, dtype="bf16")
    o, S = _run(inp, fw.FALCON_1, "bf16", window=1, beta=0.5, lam=0.01, eps=1e-6)
    o_ref, S_ref = _ref(inp, fw.FALCON_1, window=1, beta=0.5, lam=0.01, eps=1e-6)
    _check(o, S, o_ref, S_ref, label="256x12x64x64")


def test_masked_deterministic():
    inp = seq_inputs(2, 3, 64, 128, 128, seed=1240, dtype="bf16", with_k_prev=True,
                     with_S0=True, beta_per_token=True, history=3)
    a = _run(inp, fw.FALCON_3, "bf16", window=4, beta=None, lam=0.01, eps=1e-6, history=True)
    b = _run(inp, fw.FALCON_3, "bf16", window=4, beta=None, lam=0.01, eps=1e-6, history=True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_1A, fw.FALCON_3, fw.FALCON_3A])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(16, 32), (64, 64), (128, 128)])
@pytest.mark.parametrize("L,same_step", [(23, False), (64, False), (64, True)])
def test_masked_shared_gains_start_state(variant, dtype, dk, dv, L, same_step):
    """Window 1 with gains shared by the value rows (the one-system matrix-core
    path) and a live start state: both input types (fp32 inputs take their dot
    products on the fp32 matrix cores), per-token gains, wide heads split over
    two row blocks, both pairings, and the windowed variants called with window 1."""
    inp = seq_inputs(2, 2, L, dk, dv, seed=1300 + 7 * variant + dk + L + same_step,
                     dtype=dtype, with_k_prev=not same_step, with_S0=True, s_std=0.3,
                     beta_per_token=True)
    o, S = _run(inp, variant, dtype, window=1, beta=None, lam=0.02, eps=1e-6,
                same_step=same_step)
    o_ref, S_ref = _ref(inp, variant, window=1, beta=None, lam=0.02, eps=1e-6,
                        same_step=same_step)
    _check(o, S, o_ref, S_ref, label="v%d %s dk %d dv %d L %d same %d" % (
        variant, dtype, dk, dv, L, same_step))


def test_masked_shared_gains_deterministic():
    """The one-system path twice on the same inputs: bit-identical outputs."""
    inp = seq_inputs(4, 3, 64, 64, 128, seed=1400, dtype="bf16", with_k_prev=True,
                     with_S0=True, beta_per_token=True)
    a = _run(inp, fw.FALCON_1, "bf16", window=1, beta=None, lam=0.01, eps=1e-6)
    b = _run(inp, fw.FALCON_1, "bf16", window=1, beta=None, lam=0.01, eps=1e-6)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_1A])
@pytest.mark.parametrize("L,carried", [(1, False), (33, True), (64, False), (64, True)])
def test_chunk_call_of_one_chunk_runs_the_masked_kernel(variant, L, carried):
    """falcon_fwd_chunk with at most 64 steps, window 1 and shared gains is one chunk:
    it runs the masked form's one-system kernel, so both entry points return the
    same bits; a 65-step call still takes the chunk kernel and meets the bf16 gate."""
    inp = seq_inputs(3, 2, L, 64, 64, seed=1500 + 3 * variant + L, dtype="bf16",
                     with_k_prev=carried, with_S0=carried, s_std=0.2, beta_per_token=True)
    dt = torch.bfloat16
    q, k, v, bt = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "beta_t"))
    kp = to_dev(torch, inp["k_prev"], dt) if carried else None
    S0 = to_dev(torch, inp["S0"], torch.float32) if carried else None
    kw = dict(variant=variant, beta=None, lam=0.01, eps=1e-6, beta_t=bt, k_prev=kp, S0=S0,
              return_state=True)
    o_c, S_c = fw.fwd_chunk(q, k, v, chunk=64, **kw)
    o_m, S_m = fw.fwd_masked(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_m) and torch.equal(S_c, S_m)


def test_chunk_call_past_one_chunk():
    inp = seq_inputs(3, 2, 65, 64, 64, seed=1520, dtype="bf16", with_k_prev=True,
                     with_S0=True, s_std=0.2)
    dt = torch.bfloat16
    q, k, v, kp = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "k_prev"))
    S0 = to_dev(torch, inp["S0"], torch.float32)
    o, S = fw.fwd_chunk(q, k, v, variant=fw.FALCON_1, beta=0.5, lam=0.01, eps=1e-6, chunk=64,
                        k_prev=kp, S0=S0, return_state=True)
    torch.cuda.synchronize()
    o_ref, S_ref = _ref(inp, fw.FALCON_1, window=1, beta=0.5, lam=0.01, eps=1e-6)
    _check(o.cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, tol=TOL_BF16, label="L 65 chunk")

"""GPU parity of the two-kernel sliding-window form (falcon_fwd_chunk_ws: a
pre-pass writes every sub-chunk's folds to a workspace, a state kernel runs the
sequential part) against the fp64 oracle and against the single-kernel form.

Sequences are long enough that the pre-pass splits each chain into several
runs of sub-chunks (runs of at least 16 sub-chunks = 256 steps), with ragged
tails, carried keys, states and window histories, both pairings.
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs
from parity_util import TOL_BF16, state_err, to_dev, token_normwise_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


def _call(inp, window, *, workspace, beta, lam, eps, carried, same_step=False):
    dt = torch.bfloat16
    q, k, v = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    bt = to_dev(torch, inp["beta_t"], dt) if "beta_t" in inp else None
    kw = dict(variant=fw.FALCON_3, beta=beta, lam=lam, eps=eps, window=window, beta_t=bt,
              return_state=True, workspace=workspace, same_step=same_step)
    if carried:
        if not same_step:
            kw["k_prev"] = to_dev(torch, inp["k_prev"], dt)
        kw["S0"] = to_dev(torch, inp["S0"], torch.float32)
        kw["x_hist"] = to_dev(torch, inp["x_hist"], dt)
        kw["y_hist"] = to_dev(torch, inp["y_hist"], dt)
    o, S = fw.fwd_chunk(q, k, v, chunk=64, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _ref(inp, window, *, beta, lam, eps, carried, same_step=False):
    o, S, _ = fo.falcon_recurrence(
        fw.FALCON_3, inp["q"], inp["k"], inp["v"], beta=beta, lam=lam, eps=eps, window=window,
        beta_t=inp.get("beta_t"),
        k_prev=inp["k_prev"] if carried and not same_step else None,
        S0=inp["S0"] if carried else None,
        x_hist=inp["x_hist"] if carried else None, y_hist=inp["y_hist"] if carried else None,
        same_step=same_step)
    return o, S


@pytest.mark.parametrize("window", [2, 4])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 32), (128, 128), (64, 16)])
@pytest.mark.parametrize("L", [300, 1000])
@pytest.mark.parametrize("carried", [False, True])
def test_two_kernel_vs_oracle(window, dk, dv, L, carried):
    inp = seq_inputs(2, 3, L, dk, dv, seed=1300 + 7 * window + dk + dv + L + carried,
                     dtype="bf16", beta_per_token=True, with_k_prev=carried, with_S0=carried,
                     s_std=0.2, history=window - 1 if carried else 0)
    o, S = _call(inp, window, workspace="auto", beta=None, lam=0.02, eps=1e-6, carried=carried)
    o_ref, S_ref = _ref(inp, window, beta=None, lam=0.02, eps=1e-6, carried=carried)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("window %d dk %d dv %d L %d carried %d: o err %.3e S err %.3e"
          % (window, dk, dv, L, carried, err, serr))
    assert zok and err <= TOL_BF16 and serr <= TOL_BF16


@pytest.mark.parametrize("window", [2, 4])
def test_two_kernel_same_step(window):
    inp = seq_inputs(1, 4, 517, 128, 64, seed=1340 + window, dtype="bf16",
                     beta_per_token=True, with_S0=True, s_std=0.2, history=window - 1)
    o, S = _call(inp, window, workspace="auto", beta=None, lam=0.01, eps=1e-6, carried=True,
                 same_step=True)
    o_ref, S_ref = _ref(inp, window, beta=None, lam=0.01, eps=1e-6, carried=True, same_step=True)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("same-step window %d: o err %.3e S err %.3e" % (window, err, serr))
    assert zok and err <= TOL_BF16 and serr <= TOL_BF16


@pytest.mark.parametrize("window", [2, 4])
def test_two_kernel_matches_single_kernel(window):
    """The two forms compute the same equations; they differ only by rounding."""
    inp = seq_inputs(4, 4, 2048, 128, 128, seed=1350 + window, dtype="bf16")
    o1, S1 = _call(inp, window, workspace="auto", beta=0.5, lam=0.01, eps=1e-6, carried=False)
    o2, S2 = _call(inp, window, workspace=None, beta=0.5, lam=0.01, eps=1e-6, carried=False)
    err, zok = token_normwise_err(o1, o2)
    print("window %d: two-kernel vs one-kernel o diff %.3e S diff %.3e"
          % (window, err, state_err(S1, S2)))
    assert zok and err <= 1e-4 and state_err(S1, S2) <= 1e-4


@pytest.mark.parametrize("lam_beta", [0.9, 0.99])
def test_two_kernel_strong_decay_falls_back(lam_beta):
    """Decay products outside the range of the chunk algebra: the pre-pass flags
    the sub-chunk, the state kernel recomputes the chain exactly."""
    inp = seq_inputs(2, 2, 600, 64, 32, seed=1360 + int(100 * lam_beta), dtype="bf16")
    lam = 4 * lam_beta              # unit keys, window 4: n_t is about 4
    o, S = _call(inp, 4, workspace="auto", beta=1.0, lam=lam, eps=1e-6, carried=False)
    o_ref, S_ref = _ref(inp, 4, beta=1.0, lam=lam, eps=1e-6, carried=False)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("lambda beta %.2f: o err %.3e S err %.3e" % (lam_beta, err, serr))
    assert np.all(np.isfinite(o)) and zok and err <= TOL_BF16 and serr <= TOL_BF16


def test_two_kernel_explicit_workspace_and_reuse():
    """A caller-owned workspace, reused by two calls in a row with different
    inputs; a workspace one byte short runs the single-kernel form."""
    lib = fw.load_library()
    B, H, L, dk, dv = 2, 2, 700, 64, 64
    need = lib.falcon_fwd_workspace_bytes(fw.FALCON_3, 4, 0, B, H, L, dk, dv, 0)
    assert need == B * H * ((L + 15) // 16) * 12416
    ws = torch.empty(int(need), device="cuda", dtype=torch.uint8)
    for seed in (1370, 1371):
        inp = seq_inputs(B, H, L, dk, dv, seed=seed, dtype="bf16")
        o, S = _call(inp, 4, workspace=ws, beta=0.5, lam=0.01, eps=1e-6, carried=False)
        o_ref, S_ref = _ref(inp, 4, beta=0.5, lam=0.01, eps=1e-6, carried=False)
        err, zok = token_normwise_err(o, o_ref)
        assert zok and err <= TOL_BF16 and state_err(S, S_ref) <= TOL_BF16
    short = ws[: int(need) - 1]
    o2, _ = _call(inp, 4, workspace=short, beta=0.5, lam=0.01, eps=1e-6, carried=False)
    o3, _ = _call(inp, 4, workspace=None, beta=0.5, lam=0.01, eps=1e-6, carried=False)
    np.testing.assert_array_equal(o2, o3)


@pytest.mark.parametrize("window", [2, 4])
@pytest.mark.parametrize("L", [1, 7, 16, 17, 33, 48])
@pytest.mark.parametrize("carried", [False, True])
def test_two_kernel_short_sequences(window, L, carried):
    """One to three sub-chunks: the outputs of the last two sub-chunks are
    stored after the state loop, earlier ones inside it."""
    inp = seq_inputs(2, 2, L, 64, 64, seed=1380 + 3 * window + L + carried, dtype="bf16",
                     beta_per_token=True, with_k_prev=carried, with_S0=carried, s_std=0.2,
                     history=window - 1 if carried else 0)
    o, S = _call(inp, window, workspace="auto", beta=None, lam=0.02, eps=1e-6, carried=carried)
    o_ref, S_ref = _ref(inp, window, beta=None, lam=0.02, eps=1e-6, carried=carried)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("window %d L %d carried %d: o err %.3e S err %.3e" % (window, L, carried, err, serr))
    assert zok and err <= TOL_BF16 and serr <= TOL_BF16

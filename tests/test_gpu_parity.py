"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Small cases span several tiles and a ragged tail and are compared element by
element on every output; the full workloads are compared on every (batch, head)
chain, the oracle running over groups of chains in worker processes.
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import WORKLOADS, decode_inputs, seq_inputs
import oracle_pool
from parity_util import (TOL_BF16, TOL_F32, TOL_FP32_MATH, state_err, to_dev,
                         token_normwise_err)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402

ALL = [fw.FALCON_1, fw.FALCON_2, fw.FALCON_3, fw.FALCON_1A, fw.FALCON_2A, fw.FALCON_3A]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


def _win(variant, w=3):
    return w if variant in (fw.FALCON_3, fw.FALCON_3A) else 1


def _run_seq(form, variant, inp, dt, *, beta, lam, eps, window, chunk=64, carried=False):
    q = to_dev(torch, inp["q"], dt)
    k = to_dev(torch, inp["k"], dt)
    v = to_dev(torch, inp["v"], dt)
    bt = to_dev(torch, inp["beta_t"], dt) if "beta_t" in inp else None
    kp = to_dev(torch, inp["k_prev"], dt) if carried else None
    S0 = to_dev(torch, inp["S0"], torch.float32) if carried and "S0" in inp else None
    kw = dict(variant=variant, beta=beta, lam=lam, eps=eps, window=window, beta_t=bt,
              k_prev=kp, S0=S0, return_state=True)
    if form == "chunk":
        o, S = fw.fwd_chunk(q, k, v, chunk=chunk, **kw)
    else:
        o, S = fw.fwd_recurrent(q, k, v, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _oracle(variant, inp, *, beta, lam, eps, window, carried=False, chains=None):
    sel = (lambda a: a) if chains is None else (lambda a: a.reshape((-1,) + a.shape[2:])[chains][:, None])
    return fo.falcon_recurrence(
        variant, sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), beta=beta, lam=lam, eps=eps,
        window=window, beta_t=sel(inp["beta_t"]) if "beta_t" in inp else None,
        k_prev=sel(inp["k_prev"]) if carried else None,
        S0=sel(inp["S0"]) if carried and "S0" in inp else None)


# ---------------------------------------------------------------------------
# recurrent form

def test_recurrent_fp32_1x1x64x16():
    cfg = WORKLOADS["recurrent_f32_1x1x64x16"]
    B, H, L, dk, dv = cfg["shape"]
    inp = seq_inputs(B, H, L, dk, dv, seed=cfg["seed"], dtype="f32")
    o, S = _run_seq("rec", fw.FALCON_1, inp, torch.float32, beta=cfg["beta"], lam=cfg["lam"],
                    eps=cfg["eps"], window=1)
    o_ref, S_ref, _ = _oracle(fw.FALCON_1, inp, beta=cfg["beta"], lam=cfg["lam"], eps=cfg["eps"],
                              window=1)
    err, zok = token_normwise_err(o, o_ref)
    print("recurrent fp32 1x1x64x16: o err %.3e  S err %.3e" % (err, state_err(S, S_ref)))
    assert zok and err <= TOL_F32
    assert state_err(S, S_ref) <= TOL_F32


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("carried", [False, True])
def test_recurrent_small(variant, dtype, carried):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    win = _win(variant)
    if carried and win > 1:
        carried_S0 = False
    else:
        carried_S0 = carried
    inp = seq_inputs(2, 3, 45, 32, 16, seed=200 + variant, dtype=dtype, with_k_prev=carried,
                     with_S0=carried_S0, beta_per_channel=per_ch, beta_per_token=not per_ch,
                     s_std=0.3)
    if carried and not carried_S0:
        inp.pop("S0", None)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o, S = _run_seq("rec", variant, inp, dt, beta=None, lam=0.02, eps=1e-6, window=win,
                    carried=carried)
    o_ref, S_ref, _ = _oracle(variant, inp, beta=None, lam=0.02, eps=1e-6, window=win,
                              carried=carried)
    err, zok = token_normwise_err(o, o_ref)
    assert zok and err <= TOL_FP32_MATH, err
    assert state_err(S, S_ref) <= TOL_FP32_MATH


# ---------------------------------------------------------------------------
# chunk form, small shapes: several tiles, ragged tails, every variant

@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 16), (128, 32), (16, 128)])
def test_chunk_small(variant, chunk, dk, dv):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    windows = [2, 4] if variant in (fw.FALCON_3, fw.FALCON_3A) else [1]
    for win in windows:
        if win > chunk:
            continue
        L = 3 * chunk + 11                                  # ragged tail
        inp = seq_inputs(2, 2, L, dk, dv, seed=300 + variant * 7 + win, dtype="bf16",
                         beta_per_channel=per_ch, beta_per_token=not per_ch)
        o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=None, lam=0.02, eps=1e-6,
                        window=win, chunk=chunk)
        o_ref, S_ref, _ = _oracle(variant, inp, beta=None, lam=0.02, eps=1e-6, window=win)
        err, zok = token_normwise_err(o, o_ref)
        serr = state_err(S, S_ref)
        print("chunk v%d C%d dk%d dv%d B%d: o err %.3e S err %.3e" % (variant, chunk, dk, dv, win,
                                                                    err, serr))
        assert zok, "tokens with o_ref == 0 must be exactly 0"
        assert err <= TOL_BF16 and serr <= TOL_BF16


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_2, fw.FALCON_1A, fw.FALCON_2A])
def test_chunk_carried_state(variant):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    inp = seq_inputs(2, 3, 150, 64, 64, seed=400 + variant, dtype="bf16", with_k_prev=True,
                     with_S0=True, beta_per_channel=per_ch, beta_per_token=not per_ch, s_std=0.2)
    o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=None, lam=0.01, eps=1e-6,
                    window=1, chunk=64, carried=True)
    o_ref, S_ref, _ = _oracle(variant, inp, beta=None, lam=0.01, eps=1e-6, window=1, carried=True)
    err, zok = token_normwise_err(o, o_ref)
    assert zok and err <= TOL_BF16, err
    assert state_err(S, S_ref) <= TOL_BF16


def test_chunk_resume_matches_single_call():
    inp = seq_inputs(1, 4, 256, 64, 64, seed=410, dtype="bf16")
    dt = torch.bfloat16
    q, k, v = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    o_full, S_full = fw.fwd_chunk(q, k, v, variant=fw.FALCON_1, beta=0.5, lam=0.01, eps=1e-6,
                                  return_state=True)
    m = 128
    o1, S1 = fw.fwd_chunk(q[:, :, :m].contiguous(), k[:, :, :m].contiguous(),
                          v[:, :, :m].contiguous(), variant=fw.FALCON_1, beta=0.5, lam=0.01,
                          eps=1e-6, return_state=True)
    kp = k[:, :, m - 1].contiguous()
    o2, S2 = fw.fwd_chunk(q[:, :, m:].contiguous(), k[:, :, m:].contiguous(),
                          v[:, :, m:].contiguous(), variant=fw.FALCON_1, beta=0.5, lam=0.01,
                          eps=1e-6, k_prev=kp, S0=S1, return_state=True)
    torch.cuda.synchronize()
    o_split = torch.cat([o1, o2], dim=2).cpu().numpy()
    err, _ = token_normwise_err(o_split, o_full.cpu().numpy())
    assert err <= 1e-4
    assert state_err(S2.cpu().numpy(), S_full.cpu().numpy()) <= 1e-4


def test_chunk_deterministic():
    inp = seq_inputs(2, 4, 512, 64, 64, seed=420, dtype="bf16")
    outs = []
    for _ in range(2):
        o, S = _run_seq("chunk", fw.FALCON_1, inp, torch.bfloat16, beta=0.5, lam=0.01, eps=1e-6,
                        window=1, chunk=64)
        outs.append((o, S))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("L", [1, 5, 64, 65])
def test_chunk_short_sequences(L):
    inp = seq_inputs(1, 2, L, 64, 32, seed=430 + L, dtype="bf16")
    for variant in (fw.FALCON_1, fw.FALCON_3, fw.FALCON_3A):
        win = _win(variant, 4)
        o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=0.5, lam=0.01, eps=1e-6,
                        window=win, chunk=64)
        o_ref, S_ref, _ = _oracle(variant, inp, beta=0.5, lam=0.01, eps=1e-6, window=win)
        err, zok = token_normwise_err(o, o_ref)
        assert zok and err <= TOL_BF16
        assert state_err(S, S_ref) <= TOL_BF16


@pytest.mark.parametrize("variant", [fw.FALCON_3, fw.FALCON_3A])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 32)])
def test_chunk_window_carried_key(variant, dk, dv):
    """Sliding window with the previous key carried in (x_1 = k_prev), per-token gains."""
    for win in (2, 4):
        inp = seq_inputs(2, 2, 83, dk, dv, seed=470 + variant + win + dk, dtype="bf16",
                         with_k_prev=True, beta_per_token=True)
        o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=None, lam=0.02, eps=1e-6,
                        window=win, chunk=64, carried=True)
        o_ref, S_ref, _ = _oracle(variant, inp, beta=None, lam=0.02, eps=1e-6, window=win,
                                  carried=True)
        err, zok = token_normwise_err(o, o_ref)
        print("window %d dk %d: o err %.3e S err %.3e" % (win, dk, err, state_err(S, S_ref)))
        assert zok and err <= TOL_BF16
        assert state_err(S, S_ref) <= TOL_BF16


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 32)])
@pytest.mark.parametrize("window", [1, 3, 8, 16])
@pytest.mark.parametrize("carried", [False, True])
def test_chunk_inner_product_windows(dk, dv, window, carried):
    """Inner-product family over windows 1..16, several 64-step chunks and a ragged
    tail; carried: previous key and start state in, per-token gains."""
    variant = fw.FALCON_1A if window == 1 else fw.FALCON_3A
    L = 3 * 64 + 29
    inp = seq_inputs(2, 2, L, dk, dv, seed=480 + window + dk + dv, dtype="bf16",
                     with_k_prev=carried, with_S0=carried and window == 1, beta_per_token=carried,
                     s_std=0.2)
    o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=None if carried else 0.5,
                    lam=0.03, eps=1e-6, window=window, chunk=64, carried=carried)
    o_ref, S_ref, _ = _oracle(variant, inp, beta=None if carried else 0.5, lam=0.03, eps=1e-6,
                              window=window, carried=carried)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("inner product dk %d dv %d window %d: o err %.3e S err %.3e" % (dk, dv, window, err, serr))
    assert zok and err <= TOL_BF16
    assert serr <= TOL_BF16


# ---------------------------------------------------------------------------
# chunk form at the full workload sizes: every chain against the oracle

def _full_chunk_case(name, variant, window=1):
    cfg = WORKLOADS[name]
    B, H, L, dk, dv = cfg["shape"]
    per_ch = bool(cfg.get("beta_per_channel"))
    inp = seq_inputs(B, H, L, dk, dv, seed=cfg["seed"], dtype="bf16", beta_per_channel=per_ch)
    beta = cfg["beta"] if cfg["beta"] is not None else None
    print("case %s variant %d: launching" % (name, variant), flush=True)
    o, S = _run_seq("chunk", variant, inp, torch.bfloat16, beta=beta, lam=cfg["lam"],
                    eps=cfg["eps"], window=window, chunk=cfg["chunk"])
    print("case %s variant %d: oracle over %d chains (%d workers)"
          % (name, variant, B * H, oracle_pool.workers()), flush=True)
    o_ref, S_ref = oracle_pool.recurrence_all_chains(variant, inp, beta=beta, lam=cfg["lam"],
                                                     eps=cfg["eps"], window=window)
    err, zok = token_normwise_err(o.reshape(o_ref.shape), o_ref)
    serr = state_err(S.reshape(S_ref.shape), S_ref)
    print("%s variant %d, all %d chains: o err %.3e  S err %.3e" % (name, variant, B * H, err, serr))
    assert zok and err <= TOL_BF16
    assert serr <= TOL_BF16


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_1A])
def test_chunk_8x12x2048x64(variant):
    _full_chunk_case("chunk_8x12x2048x64", variant)


def test_chunk_percol_8x12x4096x64():
    _full_chunk_case("chunk_percol_8x12x4096x64", fw.FALCON_2)


@pytest.mark.parametrize("variant", [fw.FALCON_3, fw.FALCON_3A])
def test_chunk_window4_4x16x8192x128(variant):
    _full_chunk_case("chunk_window4_4x16x8192x128", variant, window=4)


# ---------------------------------------------------------------------------
# decode

def _decode_run(variant, nseq, heads, dk, dv, steps, pool, seed, check_steps,
                beta=0.5, lam=0.01, eps=1e-6, per_ch=False):
    """Every (sequence, head) pair against the oracle's decode run: o at the
    steps in check_steps, S and k_prev at the end."""
    inp = decode_inputs(nseq, heads, dk, dv, seed=seed, steps=pool, beta_per_channel=per_ch)
    dt = torch.bfloat16
    S = to_dev(torch, inp["S"], torch.float32)
    kp = to_dev(torch, inp["k_prev"], dt)
    qs = to_dev(torch, inp["q"], dt)
    ks = to_dev(torch, inp["k"], dt)
    vs = to_dev(torch, inp["v"], dt)
    bs = to_dev(torch, inp["beta_t"], dt) if per_ch else None
    got = {}
    for s in range(1, steps + 1):
        p = (s - 1) % pool
        o = fw.decode_step(S, kp, qs[p], ks[p], vs[p], variant=variant, beta=beta, lam=lam,
                           eps=eps, beta_t=bs[p] if per_ch else None)
        if s in check_steps:
            torch.cuda.synchronize()
            got[s] = o.cpu().numpy().reshape(nseq * heads, dv)
    torch.cuda.synchronize()
    o_ref, S_ref, kp_ref = oracle_pool.decode_all_pairs(variant, inp, steps, check_steps,
                                                        beta=beta, lam=lam, eps=eps)
    worst = 0.0
    for s in sorted(check_steps):
        err, zok = token_normwise_err(got[s], o_ref[s])
        worst = max(worst, err)
        print("decode v%d step %d, all %d pairs: o err %.3e" % (variant, s, nseq * heads, err))
        assert zok and err <= TOL_FP32_MATH
    serr = state_err(S.cpu().numpy().reshape(S_ref.shape), S_ref)
    print("decode v%d after %d steps: S err %.3e" % (variant, steps, serr))
    assert serr <= TOL_FP32_MATH
    np.testing.assert_array_equal(kp.cpu().float().numpy().reshape(kp_ref.shape), kp_ref)
    return worst


def test_decode_512x12x64_1000_steps():
    cfg = WORKLOADS["decode_512x12x64"]
    N, H, dk, dv = cfg["shape"]
    print("decode 512x12x64: 1000 steps on the GPU, then the oracle over all pairs", flush=True)
    _decode_run(fw.FALCON_1, N, H, dk, dv, 1000, 8, cfg["seed"], {1, 10, 100, 1000},
                beta=cfg["beta"], lam=cfg["lam"], eps=cfg["eps"])


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_2, fw.FALCON_1A, fw.FALCON_2A])
@pytest.mark.parametrize("dk,dv", [(64, 64), (16, 128), (128, 32)])
def test_decode_small(variant, dk, dv):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    _decode_run(variant, 3, 2, dk, dv, 20, 4, 500 + variant, {1, 20}, per_ch=per_ch)


# ---------------------------------------------------------------------------
# carried window history (resumed Falcon-3/3A sequences and their decode)

@pytest.mark.parametrize("form", ["rec", "chunk"])
@pytest.mark.parametrize("variant", [fw.FALCON_3, fw.FALCON_3A])
@pytest.mark.parametrize("dk,dv,window", [(64, 64, 2), (64, 64, 4), (128, 32, 4), (32, 32, 3),
                                          (64, 16, 3)])
@pytest.mark.parametrize("same_step", [False, True])
def test_window_history_resume(form, variant, dk, dv, window, same_step):
    """Resumed call: S0, k_prev and the window history in; o, S and the history out."""
    inp = seq_inputs(2, 2, 77, dk, dv, seed=600 + 7 * variant + 3 * window + dk, dtype="bf16",
                     with_k_prev=True, with_S0=True, beta_per_token=True, s_std=0.2,
                     history=window - 1)
    if same_step:
        inp.pop("k_prev")
    dt = torch.bfloat16
    q, k, v, bt, xh, yh = (to_dev(torch, inp[n], dt)
                           for n in ("q", "k", "v", "beta_t", "x_hist", "y_hist"))
    kp = None if same_step else to_dev(torch, inp["k_prev"], dt)
    S0 = to_dev(torch, inp["S0"], torch.float32)
    kw = dict(variant=variant, beta=None, lam=0.02, eps=1e-6, window=window, beta_t=bt,
              k_prev=kp, S0=S0, x_hist=xh, y_hist=yh, return_state=True, return_history=True,
              same_step=same_step)
    if form == "chunk":
        o, S, xo, yo = fw.fwd_chunk(q, k, v, chunk=64, **kw)
    else:
        o, S, xo, yo = fw.fwd_recurrent(q, k, v, **kw)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = fo.falcon_recurrence(
        variant, inp["q"], inp["k"], inp["v"], beta=None, lam=0.02, eps=1e-6, window=window,
        beta_t=inp["beta_t"], k_prev=inp.get("k_prev"), S0=inp["S0"], x_hist=inp["x_hist"],
        y_hist=inp["y_hist"], same_step=same_step)
    xr, yr = fo.falcon_history(inp["k"], inp["v"], window, k_prev=inp.get("k_prev"),
                               x_hist=inp["x_hist"], y_hist=inp["y_hist"], same_step=same_step)
    err, zok = token_normwise_err(o.cpu().numpy(), o_ref)
    serr = state_err(S.cpu().numpy(), S_ref)
    tol = TOL_BF16 if form == "chunk" else TOL_FP32_MATH
    print("%s v%d dk %d window %d: o err %.3e S err %.3e" % (form, variant, dk, window, err, serr))
    assert zok and err <= tol and serr <= tol
    np.testing.assert_array_equal(xo.float().cpu().numpy(), xr)
    np.testing.assert_array_equal(yo.float().cpu().numpy(), yr)


@pytest.mark.parametrize("form", ["rec", "chunk"])
@pytest.mark.parametrize("window", [2, 4])
def test_window_history_split_in_place(form, window):
    """Pieces of 1, 2 and the rest tokens chained with an in-place history carry
    equal one call over the whole sequence (the oracle's)."""
    L, dk, dv = 70, 64, 32
    inp = seq_inputs(1, 3, L, dk, dv, seed=640 + window, dtype="bf16", beta_per_token=True)
    dt = torch.bfloat16
    q, k, v, bt = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "beta_t"))
    xh = torch.zeros((1, 3, window - 1, dk), device="cuda", dtype=dt)
    yh = torch.zeros((1, 3, window - 1, dv), device="cuda", dtype=dt)
    S = torch.zeros((1, 3, dv, dk), device="cuda", dtype=torch.float32)
    kp = None
    outs = []
    for lo, hi in ((0, 1), (1, 3), (3, L)):
        sl = lambda t: t[:, :, lo:hi].contiguous()
        kw = dict(variant=fw.FALCON_3, beta=None, lam=0.02, eps=1e-6, window=window,
                  beta_t=sl(bt), k_prev=kp, S0=S if kp is not None else None,
                  x_hist=xh if kp is not None else None, y_hist=yh if kp is not None else None,
                  S_out=S, return_state=True, x_hist_out=xh, y_hist_out=yh, return_history=True)
        fn = fw.fwd_chunk if form == "chunk" else fw.fwd_recurrent
        o, _, _, _ = fn(sl(q), sl(k), sl(v), **kw)
        kp = k[:, :, hi - 1].contiguous()
        outs.append(o)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = fo.falcon_recurrence(fw.FALCON_3, inp["q"], inp["k"], inp["v"], beta=None,
                                           lam=0.02, eps=1e-6, window=window,
                                           beta_t=inp["beta_t"])
    err, zok = token_normwise_err(torch.cat(outs, dim=2).cpu().numpy(), o_ref)
    serr = state_err(S.cpu().numpy(), S_ref)
    tol = TOL_BF16 if form == "chunk" else TOL_FP32_MATH
    print("%s window %d split: o err %.3e S err %.3e" % (form, window, err, serr))
    assert zok and err <= tol and serr <= tol
    xr, yr = fo.falcon_history(inp["k"], inp["v"], window)
    np.testing.assert_array_equal(xh.float().cpu().numpy(), xr)
    np.testing.assert_array_equal(yh.float().cpu().numpy(), yr)


@pytest.mark.parametrize("variant", [fw.FALCON_3, fw.FALCON_3A])
@pytest.mark.parametrize("dk,dv,window", [(64, 64, 4), (16, 128, 2), (128, 32, 3), (32, 16, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("same_step", [False, True])
def test_decode_window(variant, dk, dv, window, dtype, same_step):
    """Decode steps with the window history updated in place, against the oracle's
    windowed decode step by step."""
    steps, pool = 12, 4
    inp = decode_inputs(3, 2, dk, dv, seed=660 + variant + window + dk, steps=pool, s_std=0.2,
                        dtype=dtype, history=window - 1)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    S = to_dev(torch, inp["S"], torch.float32)
    kp, xh, yh = (to_dev(torch, inp[n], dt) for n in ("k_prev", "x_hist", "y_hist"))
    qs, ks, vs = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    S_r, kp_r, xh_r, yh_r = (inp[n].astype(np.float64) for n in ("S", "k_prev", "x_hist", "y_hist"))
    kp_dev = None if same_step else kp
    for s in range(steps):
        p = s % pool
        o = fw.decode_step(S, kp_dev, qs[p], ks[p], vs[p], variant=variant, beta=0.6, lam=0.02,
                           eps=1e-6, window=window, x_hist=xh, y_hist=yh, same_step=same_step)
        o_r, S_r, kp_r, xh_r, yh_r = fo.falcon_decode_step_window(
            variant, window, S_r, kp_r, xh_r, yh_r, inp["q"][p], inp["k"][p], inp["v"][p],
            beta=0.6, lam=0.02, eps=1e-6, same_step=same_step)
        torch.cuda.synchronize()
        err, zok = token_normwise_err(o.cpu().numpy(), o_r)
        assert zok and err <= TOL_FP32_MATH, (s, err)
    serr = state_err(S.cpu().numpy(), S_r)
    print("decode window %d v%d dk %d dv %d %s: S err %.3e" % (window, variant, dk, dv, dtype, serr))
    assert serr <= TOL_FP32_MATH
    np.testing.assert_array_equal(kp.float().cpu().numpy(), kp_r)
    np.testing.assert_array_equal(xh.float().cpu().numpy(), xh_r)
    np.testing.assert_array_equal(yh.float().cpu().numpy(), yh_r)


# ---------------------------------------------------------------------------
# same-step pairing (x_t = k_t): every kernel family

@pytest.mark.parametrize("form", ["rec", "chunk"])
@pytest.mark.parametrize("variant,dk,dv,window", [
    (fw.FALCON_1, 64, 64, 1), (fw.FALCON_1A, 32, 32, 1), (fw.FALCON_2, 64, 64, 1),
    (fw.FALCON_2A, 32, 16, 1), (fw.FALCON_1, 128, 32, 1), (fw.FALCON_3, 64, 64, 4),
    (fw.FALCON_3A, 128, 32, 2), (fw.FALCON_3, 32, 32, 3), (fw.FALCON_3A, 64, 16, 3)])
@pytest.mark.parametrize("with_S0", [False, True])
def test_same_step_pairing(form, variant, dk, dv, window, with_S0):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    inp = seq_inputs(2, 2, 83, dk, dv, seed=700 + 11 * variant + dk + window, dtype="bf16",
                     with_S0=with_S0, beta_per_channel=per_ch, beta_per_token=not per_ch,
                     s_std=0.2)
    dt = torch.bfloat16
    q, k, v, bt = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "beta_t"))
    S0 = to_dev(torch, inp["S0"], torch.float32) if with_S0 else None
    hist = {}
    if with_S0 and window > 1:   # a windowed state travels with its history (zero: none)
        hist = dict(x_hist=torch.zeros((2, 2, window - 1, dk), device="cuda", dtype=dt),
                    y_hist=torch.zeros((2, 2, window - 1, dv), device="cuda", dtype=dt))
    kw = dict(variant=variant, beta=None, lam=0.02, eps=1e-6, window=window, beta_t=bt, S0=S0,
              same_step=True, return_state=True, **hist)
    if form == "chunk":
        o, S = fw.fwd_chunk(q, k, v, chunk=64, **kw)
    else:
        o, S = fw.fwd_recurrent(q, k, v, **kw)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta=None,
                                           lam=0.02, eps=1e-6, window=window,
                                           beta_t=inp["beta_t"], S0=inp.get("S0"),
                                           same_step=True)
    err, zok = token_normwise_err(o.cpu().numpy(), o_ref)
    serr = state_err(S.cpu().numpy(), S_ref)
    tol = TOL_BF16 if form == "chunk" else TOL_FP32_MATH
    print("same-step %s v%d dk %d dv %d window %d: o err %.3e S err %.3e"
          % (form, variant, dk, dv, window, err, serr))
    assert zok and err <= tol and serr <= tol


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_2, fw.FALCON_1A])
def test_decode_same_step(variant):
    per_ch = variant == fw.FALCON_2
    inp = decode_inputs(3, 2, 64, 32, seed=720 + variant, steps=4, s_std=0.2,
                        beta_per_channel=per_ch)
    dt = torch.bfloat16
    S = to_dev(torch, inp["S"], torch.float32)
    qs, ks, vs = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    bs = to_dev(torch, inp["beta_t"], dt) if per_ch else None
    S_r = inp["S"].astype(np.float64)
    for s in range(8):
        p = s % 4
        o = fw.decode_step(S, None, qs[p], ks[p], vs[p], variant=variant, beta=0.6, lam=0.02,
                           eps=1e-6, beta_t=bs[p] if per_ch else None, same_step=True)
        o_r, S_r, _ = fo.falcon_decode_step(variant, S_r, None, inp["q"][p], inp["k"][p],
                                            inp["v"][p], beta=0.6, lam=0.02, eps=1e-6,
                                            beta_t=inp["beta_t"][p] if per_ch else None,
                                            same_step=True)
        torch.cuda.synchronize()
        err, zok = token_normwise_err(o.cpu().numpy(), o_r)
        assert zok and err <= TOL_FP32_MATH, (s, err)
    assert state_err(S.cpu().numpy(), S_r) <= TOL_FP32_MATH


@pytest.mark.parametrize("variant,base", [(fw.FALCON_3, fw.FALCON_1), (fw.FALCON_3A, fw.FALCON_1A)])
@pytest.mark.parametrize("same_step", [False, True])
def test_decode_windowed_variant_at_window_1(variant, base, same_step):
    """A window of one sample: the windowed variant's decode step is its un-windowed
    base (same bits), and meets the oracle's windowed decode; the binding takes the
    extended entry point for it (the plain one refuses the windowed variants)."""
    inp = decode_inputs(3, 2, 64, 32, seed=730 + variant, steps=4, s_std=0.2)
    dt = torch.bfloat16
    qs, ks, vs = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v"))
    runs = {}
    for var in (variant, base):
        S = to_dev(torch, inp["S"], torch.float32)
        kp = None if same_step else to_dev(torch, inp["k_prev"], dt)
        os_ = [fw.decode_step(S, kp, qs[p], ks[p], vs[p], variant=var, beta=0.6, lam=0.02,
                              eps=1e-6, same_step=same_step).cpu().numpy() for p in range(4)]
        torch.cuda.synchronize()
        runs[var] = (os_, S.cpu().numpy(), None if kp is None else kp.float().cpu().numpy())
    for a, b in zip(runs[variant][0], runs[base][0]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(runs[variant][1], runs[base][1])
    S_r, kp_r = inp["S"].astype(np.float64), inp["k_prev"].astype(np.float64)
    for p in range(4):
        o_r, S_r, kp_r, _, _ = fo.falcon_decode_step_window(
            variant, 1, S_r, kp_r, None, None, inp["q"][p], inp["k"][p], inp["v"][p], beta=0.6,
            lam=0.02, eps=1e-6, same_step=same_step)
        err, zok = token_normwise_err(runs[variant][0][p], o_r)
        assert zok and err <= TOL_FP32_MATH, (p, err)
    assert state_err(runs[variant][1], S_r) <= TOL_FP32_MATH
    if not same_step:
        np.testing.assert_array_equal(runs[variant][2], kp_r)


# ---------------------------------------------------------------------------
# backward of the window-1 chunk form

def _grad_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("variant", [fw.FALCON_1, fw.FALCON_2, fw.FALCON_1A, fw.FALCON_2A])
@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 16), (16, 64)])
@pytest.mark.parametrize("carried,same_step", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_small(variant, dk, dv, carried, same_step, dtype):
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    L = 75
    inp = seq_inputs(2, 2, L, dk, dv, seed=800 + 5 * variant + dk + dv, dtype=dtype,
                     beta_per_channel=per_ch, beta_per_token=not per_ch,
                     with_k_prev=carried and not same_step, with_S0=carried, s_std=0.2)
    rng = np.random.default_rng(801 + variant)
    dO = rng.standard_normal((2, 2, L, dv)).astype(np.float32)
    dS_L = rng.standard_normal((2, 2, dv, dk)).astype(np.float32)
    dk_last = rng.standard_normal((2, 2, dk)).astype(np.float32)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda n: to_dev(torch, inp[n], dt) if n in inp else None
    f32 = lambda a: to_dev(torch, a, torch.float32)
    got = fw.bwd_chunk(dev("q"), dev("k"), dev("v"), f32(dO), variant=variant, beta=None,
                       lam=0.02, eps=1e-6, beta_t=dev("beta_t"), k_prev=dev("k_prev"),
                       S0=to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None,
                       dS_L=f32(dS_L), dk_last=f32(dk_last), same_step=same_step)
    torch.cuda.synchronize()
    ref = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta=None, lam=0.02,
                             eps=1e-6, beta_t=inp["beta_t"], k_prev=inp.get("k_prev"),
                             S0=inp.get("S0"), same_step=same_step, dS_L=dS_L, dk_last=dk_last)
    assert set(got) == set(ref)
    errs = {n: _grad_err(got[n].cpu().numpy(), ref[n]) for n in ref}
    print("backward v%d dk %d dv %d %s: %s" % (variant, dk, dv, dtype,
                                               {n: "%.2e" % e for n, e in errs.items()}))
    assert max(errs.values()) <= TOL_FP32_MATH, errs


@pytest.mark.parametrize("variant", [fw.FALCON_3, fw.FALCON_3A])
@pytest.mark.parametrize("window", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 16)])
@pytest.mark.parametrize("carried,same_step,per_token", [(False, False, False), (True, False, True),
                                                         (False, True, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_window(variant, window, dk, dv, carried, same_step, per_token, dtype):
    """Sliding window: the chunk's unknowns are (step, window slot) pairs; several
    chunks, a ragged tail, halo samples crossing chunk boundaries (from window 5
    on, more than one boundary; windows 3, 5, 6, 7 leave lanes idle)."""
    L = 37
    inp = seq_inputs(2, 2, L, dk, dv, seed=820 + 5 * variant + window + dk + dv, dtype=dtype,
                     beta_per_token=per_token, with_k_prev=carried and not same_step)
    rng = np.random.default_rng(821 + variant + window)
    dO = rng.standard_normal((2, 2, L, dv)).astype(np.float32)
    dS_L = rng.standard_normal((2, 2, dv, dk)).astype(np.float32)
    dk_last = rng.standard_normal((2, 2, dk)).astype(np.float32)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda n: to_dev(torch, inp[n], dt) if n in inp else None
    f32 = lambda a: to_dev(torch, a, torch.float32)
    beta = None if per_token else 0.5
    got = fw.bwd_chunk(dev("q"), dev("k"), dev("v"), f32(dO), variant=variant, beta=beta,
                       lam=0.02, eps=1e-6, window=window, beta_t=dev("beta_t"),
                       k_prev=dev("k_prev"), dS_L=f32(dS_L), dk_last=f32(dk_last),
                       same_step=same_step)
    torch.cuda.synchronize()
    ref = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta=beta, lam=0.02,
                             eps=1e-6, window=window, beta_t=inp.get("beta_t"),
                             k_prev=inp.get("k_prev"), same_step=same_step, dS_L=dS_L,
                             dk_last=dk_last)
    assert set(got) == set(ref)
    errs = {n: _grad_err(got[n].cpu().numpy(), ref[n]) for n in ref}
    print("backward window %d v%d dk %d dv %d %s: %s" % (window, variant, dk, dv, dtype,
                                                         {n: "%.2e" % e for n, e in errs.items()}))
    assert max(errs.values()) <= TOL_FP32_MATH, errs


@pytest.mark.parametrize("variant,window", [(fw.FALCON_1, 1), (fw.FALCON_2, 1), (fw.FALCON_3, 4),
                                            (fw.FALCON_3A, 3), (fw.FALCON_3, 8), (fw.FALCON_3A, 6)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 16), (16, 128)])
def test_backward_wide(variant, window, dk, dv):
    """dk or dv = 128: the value rows of a head are split over several workgroups
    whose partial key and query gradients are summed by a second kernel; the
    carried key lands in a tile row that another wave's commit also covers."""
    per_ch = variant == fw.FALCON_2
    L = 29
    inp = seq_inputs(2, 1, L, dk, dv, seed=840 + variant + dk + dv, dtype="bf16",
                     beta_per_channel=per_ch, beta_per_token=not per_ch, with_k_prev=True,
                     with_S0=window == 1, s_std=0.2)
    rng = np.random.default_rng(841 + variant)
    dO = rng.standard_normal((2, 1, L, dv)).astype(np.float32)
    dS_L = rng.standard_normal((2, 1, dv, dk)).astype(np.float32)
    dk_last = rng.standard_normal((2, 1, dk)).astype(np.float32)
    dev = lambda n: to_dev(torch, inp[n], torch.bfloat16) if n in inp else None
    f32 = lambda a: to_dev(torch, a, torch.float32)
    got = fw.bwd_chunk(dev("q"), dev("k"), dev("v"), f32(dO), variant=variant, beta=None,
                       lam=0.02, eps=1e-6, window=window, beta_t=dev("beta_t"),
                       k_prev=dev("k_prev"),
                       S0=to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None,
                       dS_L=f32(dS_L), dk_last=f32(dk_last))
    torch.cuda.synchronize()
    ref = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta=None, lam=0.02,
                             eps=1e-6, window=window, beta_t=inp["beta_t"],
                             k_prev=inp["k_prev"], S0=inp.get("S0"), dS_L=dS_L, dk_last=dk_last)
    assert set(got) == set(ref)
    errs = {n: _grad_err(got[n].cpu().numpy(), ref[n]) for n in ref}
    print("backward wide v%d w%d dk %d dv %d: %s" % (variant, window, dk, dv,
                                                    {n: "%.2e" % e for n, e in errs.items()}))
    assert max(errs.values()) <= TOL_FP32_MATH, errs


def test_backward_8x12x2048x64():
    """Headline workload: every chain's gradients against the oracle's."""
    cfg = WORKLOADS["chunk_8x12x2048x64"]
    B, H, L, dk, dv = cfg["shape"]
    inp = seq_inputs(B, H, L, dk, dv, seed=cfg["seed"], dtype="bf16")
    rng = np.random.default_rng(809)
    dO = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    dt = torch.bfloat16
    print("backward 8x12x2048x64: launching", flush=True)
    got = fw.bwd_chunk(*(to_dev(torch, inp[n], dt) for n in ("q", "k", "v")),
                       to_dev(torch, dO, torch.float32), variant=fw.FALCON_1, beta=cfg["beta"],
                       lam=cfg["lam"], eps=cfg["eps"])
    torch.cuda.synchronize()
    print("backward 8x12x2048x64: oracle over %d chains" % (B * H), flush=True)
    ref = oracle_pool.backward_all_chains(fw.FALCON_1, inp, dO, beta=cfg["beta"],
                                          lam=cfg["lam"], eps=cfg["eps"])
    errs = {n: _grad_err(got[n].cpu().numpy().reshape(ref[n].shape), ref[n]) for n in ref}
    print("backward 8x12x2048x64, all chains: %s" % {n: "%.2e" % e for n, e in errs.items()})
    assert max(errs.values()) <= TOL_FP32_MATH, errs


# ---------------------------------------------------------------------------
# short sequences: chunk form against the masked-parallel evaluation (explainer §3)

@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("same_step", [False, True])
def test_short_sequence_chunk_matches_masked_parallel(variant, same_step):
    """The chunk form on a short sequence against the oracle's masked-parallel
    evaluation (transition products, no residuals).  The masked-parallel form's
    own kernel (falcon_fwd_masked) has its tests in test_gpu_masked.py."""
    per_ch = variant in (fw.FALCON_2, fw.FALCON_2A)
    win = _win(variant, 2)
    L, dk, dv = 24, 16, 16
    inp = seq_inputs(1, 2, L, dk, dv, seed=740 + variant, dtype="bf16", with_S0=True,
                     beta_per_channel=per_ch, beta_per_token=not per_ch, s_std=0.2)
    dt = torch.bfloat16
    q, k, v, bt = (to_dev(torch, inp[n], dt) for n in ("q", "k", "v", "beta_t"))
    S0 = to_dev(torch, inp["S0"], torch.float32)
    extra = {}
    if win > 1:   # a windowed state travels with its history (zero: none)
        extra = dict(x_hist=torch.zeros((1, 2, win - 1, dk), device="cuda", dtype=dt),
                     y_hist=torch.zeros((1, 2, win - 1, dv), device="cuda", dtype=dt))
    kp = None
    if not same_step:   # a live state needs the key it pairs with the first value
        kp = to_dev(torch, inp["k"][:, :, -1], dt)
    o = fw.fwd_chunk(q, k, v, variant=variant, beta=None, lam=0.02, eps=1e-6, chunk=64,
                     window=win, beta_t=bt, S0=S0, k_prev=kp, same_step=same_step, **extra)
    torch.cuda.synchronize()
    kp_ref = None if same_step else inp["k"][:, :, -1]
    o_ref = fo.falcon_masked_parallel(variant, inp["q"], inp["k"], inp["v"], beta=None, lam=0.02,
                                      eps=1e-6, window=win, beta_t=inp["beta_t"], k_prev=kp_ref,
                                      S0=inp["S0"], same_step=same_step)
    err, zok = token_normwise_err(o.cpu().numpy(), o_ref)
    print("masked-parallel v%d same_step %d: o err %.3e" % (variant, same_step, err))
    assert zok and err <= TOL_BF16


# ---------------------------------------------------------------------------
# error paths through the binding

def test_binding_rejects_unsupported():
    q = torch.zeros((1, 1, 16, 48), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(fw.FalconError) as ei:
        fw.fwd_chunk(q, q, q, variant=fw.FALCON_1)
    assert ei.value.status == 2

"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's update formula: each checks it against an
independent statement (textbook NLMS, a finite-difference gradient, the
interpolation property, causal linear attention, the masked-parallel
expansion, hand-worked values, invariances of the method).
"""
import json
import os

import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs, to_bf16_values

pytestmark = pytest.mark.cpu

ALL = [fo.FALCON_1, fo.FALCON_2, fo.FALCON_3, fo.FALCON_1A, fo.FALCON_2A, fo.FALCON_3A]
NAMES = {"falcon1": fo.FALCON_1, "falcon2": fo.FALCON_2, "falcon3": fo.FALCON_3,
         "falcon1a": fo.FALCON_1A, "falcon2a": fo.FALCON_2A, "falcon3a": fo.FALCON_3A}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed, B=1, H=2, L=6, dk=3, dv=2, **kw):
    return seq_inputs(B, H, L, dk, dv, seed=seed, dtype="f32", **kw)


def _window(variant):
    return 3 if variant in (fo.FALCON_3, fo.FALCON_3A) else 1


# --- NLMS (163.com section 02 (1): lambda = 0, eps = 0 gives classic NLMS) ----------

def _textbook_nlms(x_seq, d_seq, mu):
    """Normalized LMS, one adaptive filter w per output channel (Haykin's form):
    e = d - w.x ; w <- w + mu * e * x / (x.x).  Plain Python loops."""
    dk = len(x_seq[0])
    dv = len(d_seq[0])
    W = [[0.0] * dk for _ in range(dv)]
    hist = []
    for x, d in zip(x_seq, d_seq):
        xx = sum(xi * xi for xi in x)
        for i in range(dv):
            e = d[i] - sum(W[i][c] * x[c] for c in range(dk))
            for c in range(dk):
                W[i][c] += mu * e * x[c] / xx
        hist.append([row[:] for row in W])
    return hist


def test_nlms_reduction():
    inp = _tiny(11, B=1, H=1, L=9, dk=4, dv=3, with_k_prev=True)
    mu = 0.7
    o, S, _, states = fo.falcon_recurrence(fo.FALCON_1, inp["q"], inp["k"], inp["v"],
                                           beta=mu, lam=0.0, eps=0.0,
                                           k_prev=inp["k_prev"], return_states=True)
    k = inp["k"][0, 0].astype(np.float64)
    xs = [inp["k_prev"][0, 0].astype(np.float64)] + [k[t] for t in range(8)]
    ds = [inp["v"][0, 0, t].astype(np.float64) for t in range(9)]
    hist = _textbook_nlms([list(x) for x in xs], [list(d) for d in ds], mu)
    for t in range(9):
        np.testing.assert_allclose(states[0, 0, t], np.array(hist[t]), rtol=1e-12, atol=1e-13)
        qt = inp["q"][0, 0, t].astype(np.float64)
        np.testing.assert_allclose(o[0, 0, t], np.array(hist[t]) @ qt, rtol=1e-12, atol=1e-13)


# --- one normalized gradient step (explainer §1; 163.com 02 (1)) --------------------

def _loss(S, X, Y, lam, regression):
    if regression:
        r = X @ S.T - Y
        data = 0.5 * np.sum(r * r, axis=0)          # per value row
    else:
        data = -np.sum(Y * (X @ S.T), axis=0)
    return data + 0.5 * lam * np.sum(S * S, axis=1)  # per value row


def _fd_grad(S, X, Y, lam, regression, h=1e-5):
    g = np.zeros_like(S)
    for i in range(S.shape[0]):
        for c in range(S.shape[1]):
            Sp = S.copy(); Sp[i, c] += h
            Sm = S.copy(); Sm[i, c] -= h
            g[i, c] = (_loss(Sp, X, Y, lam, regression)[i]
                       - _loss(Sm, X, Y, lam, regression)[i]) / (2 * h)
    return g


@pytest.mark.parametrize("variant", ALL)
def test_gradient_step(variant):
    win = _window(variant)
    per_ch = variant in (fo.FALCON_2, fo.FALCON_2A)
    inp = _tiny(20 + variant, B=1, H=1, L=6, dk=4, dv=3, with_k_prev=True,
                beta_per_channel=per_ch, beta_per_token=not per_ch)
    lam, eps = 0.3, 0.05
    o, S, _, states = fo.falcon_recurrence(
        variant, inp["q"], inp["k"], inp["v"], beta=None, lam=lam, eps=eps, window=win,
        beta_t=inp["beta_t"], k_prev=inp["k_prev"], return_states=True)
    k = inp["k"][0, 0].astype(np.float64)
    x = np.concatenate([inp["k_prev"][0, 0][None].astype(np.float64), k[:-1]])
    y = inp["v"][0, 0].astype(np.float64)
    for t in range(1, 6):
        lo = max(0, t - win + 1)
        X, Y = x[lo:t + 1], y[lo:t + 1]
        Sprev = states[0, 0, t - 1]
        g = _fd_grad(Sprev, X, Y, lam, fo.is_regression(variant))
        bt = inp["beta_t"][0, 0, t]
        b = np.asarray(bt, dtype=np.float64) * np.ones(3)
        eta = b / (eps + np.sum(X * X))
        expect = Sprev - eta[:, None] * g
        np.testing.assert_allclose(states[0, 0, t], expect, rtol=1e-7, atol=1e-9)


# --- interpolation: beta = 1, lambda = eps = 0 writes S x_t = y_t exactly ----------

@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_2])
def test_interpolation(variant):
    inp = _tiny(31, B=2, H=2, L=10, dk=5, dv=4, with_k_prev=True, with_S0=True)
    o, S, _, states = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta=1.0,
                                           lam=0.0, eps=0.0, k_prev=inp["k_prev"],
                                           S0=inp["S0"], return_states=True)
    x = np.concatenate([inp["k_prev"][:, :, None], inp["k"][:, :, :-1]], axis=2)
    Sx = np.einsum("bhtij,bhtj->bhti", states, x.astype(np.float64))
    np.testing.assert_allclose(Sx, inp["v"], rtol=1e-11, atol=1e-12)


def test_interpolation_scalar_closed_form():
    # dk = dv = 1: S_t = y_t / x_t, hence o_t = y_t q_t / x_t
    q = np.array([[[[0.5], [-2.0], [3.0], [1.5]]]])
    k = np.array([[[[2.0], [-0.25], [4.0], [1.0]]]])
    v = np.array([[[[1.0], [3.0], [-5.0], [0.5]]]])
    kp = np.array([[[0.5]]])
    o, _, _ = fo.falcon_recurrence(fo.FALCON_1, q, k, v, beta=1.0, lam=0.0, eps=0.0, k_prev=kp)
    xs = [0.5, 2.0, -0.25, 4.0]
    expect = [v[0, 0, t, 0] * q[0, 0, t, 0] / xs[t] for t in range(4)]
    np.testing.assert_allclose(o[0, 0, :, 0], expect, rtol=1e-15)


# --- A family: causal (decayed) linear attention ----------------------------------

def _decay_matrix(a):
    L = len(a)
    D = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            p = 1.0
            for r in range(s + 1, t + 1):
                p *= a[r]
            D[t, s] = p
    return D


@pytest.mark.parametrize("same_step", [True, False])
@pytest.mark.parametrize("lam", [0.0, 0.2])
def test_inner_product_is_linear_attention(same_step, lam):
    inp = _tiny(41, B=1, H=1, L=8, dk=4, dv=3, with_k_prev=True)
    eps, beta = 1e-3, 0.6
    Q = inp["q"][0, 0].astype(np.float64)
    K = inp["k"][0, 0].astype(np.float64)
    V = inp["v"][0, 0].astype(np.float64)
    Xk = K if same_step else np.concatenate([inp["k_prev"][0, 0][None], K[:-1]])
    eta = beta / (eps + np.sum(Xk * Xk, axis=1))
    D = _decay_matrix(1.0 - eta * lam)
    A = np.tril(Q @ Xk.T) * D * eta[None, :]
    expect = A @ V
    o, _, _ = fo.falcon_recurrence(fo.FALCON_1A, inp["q"], inp["k"], inp["v"], beta=beta,
                                   lam=lam, eps=eps, k_prev=inp["k_prev"], same_step=same_step)
    np.testing.assert_allclose(o[0, 0], expect, rtol=1e-12, atol=1e-13)


# --- masked-parallel expansion == recurrence (explainer §3, ai-feeds 计算形式) ------

@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("start", ["fresh", "carried"])
@pytest.mark.parametrize("same_step", [False, True])
def test_masked_parallel_equals_recurrence(variant, start, same_step):
    per_ch = variant in (fo.FALCON_2, fo.FALCON_2A)
    carried = start == "carried"
    inp = _tiny(50 + variant, B=1, H=2, L=6, dk=3, dv=2, with_k_prev=carried,
                with_S0=carried, beta_per_channel=per_ch, beta_per_token=not per_ch, s_std=0.5)
    kw = dict(beta=None, lam=0.05, eps=1e-3, window=_window(variant), beta_t=inp["beta_t"],
              k_prev=inp.get("k_prev"), S0=inp.get("S0"), same_step=same_step)
    o1, _, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
    o2 = fo.falcon_masked_parallel(variant, inp["q"], inp["k"], inp["v"], **kw)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)


# --- hand-worked values (tests/golden/repeated_key.json) --------------------------

def test_golden_repeated_key():
    with open(os.path.join(GOLDEN, "repeated_key.json")) as f:
        g = json.load(f)
    y = np.array(g["y"])
    key = np.array(g["key"])
    L = len(y)
    k = np.tile(key, (1, 1, L, 1))
    v = y.reshape(1, 1, L, 1)
    for case in g["cases"]:
        variant = NAMES[case["variant"]]
        for q_vec, expect in ((key, np.array(case["o"])), (np.array([0.0, 1.0]), np.zeros(L))):
            q = np.tile(q_vec, (1, 1, L, 1))
            o, _, _ = fo.falcon_recurrence(variant, q, k, v, beta=case["beta"], lam=case["lam"],
                                           eps=0.0, window=case["window"],
                                           k_prev=key.reshape(1, 1, 2))
            np.testing.assert_allclose(o[0, 0, :, 0], expect, rtol=0, atol=1e-15)


# --- invariances of the method ------------------------------------------------------

@pytest.mark.parametrize("pair", [(fo.FALCON_3, fo.FALCON_1), (fo.FALCON_3A, fo.FALCON_1A)])
def test_window_one_is_scalar_variant(pair):
    inp = _tiny(61, B=2, H=1, L=9, dk=4, dv=3, beta_per_token=True)
    kw = dict(beta=None, lam=0.05, eps=1e-6, beta_t=inp["beta_t"], window=1)
    a = fo.falcon_recurrence(pair[0], inp["q"], inp["k"], inp["v"], **kw)
    b = fo.falcon_recurrence(pair[1], inp["q"], inp["k"], inp["v"], **kw)
    np.testing.assert_array_equal(a[0], b[0])


@pytest.mark.parametrize("pair", [(fo.FALCON_2, fo.FALCON_1), (fo.FALCON_2A, fo.FALCON_1A)])
def test_channel_constant_beta_is_scalar_variant(pair):
    inp = _tiny(71, B=2, H=1, L=9, dk=4, dv=3, beta_per_token=True)
    bt4 = np.repeat(inp["beta_t"][..., None], 3, axis=-1)
    a = fo.falcon_recurrence(pair[0], inp["q"], inp["k"], inp["v"], beta=None, lam=0.05,
                             eps=1e-6, beta_t=bt4)
    b = fo.falcon_recurrence(pair[1], inp["q"], inp["k"], inp["v"], beta=None, lam=0.05,
                             eps=1e-6, beta_t=inp["beta_t"])
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_2, fo.FALCON_1A, fo.FALCON_2A])
def test_resume_split(variant):
    # only the fixed-size state (and the carried key) crosses a split (163.com 02 (2))
    per_ch = variant in (fo.FALCON_2, fo.FALCON_2A)
    inp = _tiny(81, B=2, H=2, L=11, dk=4, dv=3, beta_per_channel=per_ch,
                beta_per_token=not per_ch)
    kw = dict(beta=None, lam=0.05, eps=1e-6)
    o, S, kl = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta_t=inp["beta_t"], **kw)
    m = 5
    sl = lambda a, lo, hi: a[:, :, lo:hi]
    o1, S1, k1 = fo.falcon_recurrence(variant, sl(inp["q"], 0, m), sl(inp["k"], 0, m),
                                      sl(inp["v"], 0, m), beta_t=sl(inp["beta_t"], 0, m), **kw)
    o2, S2, k2 = fo.falcon_recurrence(variant, sl(inp["q"], m, 11), sl(inp["k"], m, 11),
                                      sl(inp["v"], m, 11), beta_t=sl(inp["beta_t"], m, 11),
                                      k_prev=k1, S0=S1, **kw)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(k2, kl)


def test_fresh_start_is_zero():
    inp = _tiny(91, B=1, H=3, L=4, dk=4, dv=3)
    for eps in (1e-6, 0.0):
        for variant in ALL:
            o, _, _, st = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta=0.5,
                                               lam=0.01, eps=eps, window=_window(variant),
                                               return_states=True)
            assert np.all(o[:, :, 0] == 0.0) and np.all(st[:, :, 0] == 0.0)


def test_zero_denominator_on_live_state_raises():
    inp = _tiny(92, B=1, H=1, L=3, dk=2, dv=2, with_S0=True)
    with pytest.raises(ZeroDivisionError):
        fo.falcon_recurrence(fo.FALCON_1, inp["q"], inp["k"], inp["v"], beta=0.5, lam=0.0,
                             eps=0.0, S0=inp["S0"])


def test_decode_step_read_after_write():
    # o = S_new q (163.com section 01); equals a S q + eta e (x.q) for the delta write
    rng = np.random.default_rng(5)
    N, H, dk, dv = 3, 2, 4, 3
    S = rng.standard_normal((N, H, dv, dk))
    kp = rng.standard_normal((N, H, dk))
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv))
    o, Sn, kn = fo.falcon_decode_step(fo.FALCON_1, S, kp, q, k, v, beta=0.5, lam=0.1, eps=1e-6)
    np.testing.assert_allclose(o, np.einsum("nhij,nhj->nhi", Sn, q), rtol=1e-13)
    eta = 0.5 / (1e-6 + np.sum(kp * kp, -1))
    e = v - np.einsum("nhij,nhj->nhi", S, kp)
    alt = (1 - 0.1 * eta)[..., None] * np.einsum("nhij,nhj->nhi", S, q) \
        + eta[..., None] * e * np.sum(kp * q, -1)[..., None]
    np.testing.assert_allclose(o, alt, rtol=1e-12)
    np.testing.assert_array_equal(kn, k)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = to_bf16_values(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def _seg(inp, lo, hi):
    return {n: (None if inp.get(n) is None else inp[n][:, :, lo:hi])
            for n in ("q", "k", "v", "beta_t")}


@pytest.mark.parametrize("variant", [fo.FALCON_3, fo.FALCON_3A])
@pytest.mark.parametrize("window", [2, 3, 4])
@pytest.mark.parametrize("cuts", [(5,), (1, 2), (2, 3, 9)])
def test_window_resume_split(variant, window, cuts):
    # a resumed Falcon-3/3A call carries S, the key and the window-1 latest
    # samples; pieces of any length (also shorter than the window) chained this
    # way give the one-call result over the whole sequence
    L = 13
    inp = _tiny(83 + window, B=2, H=2, L=L, dk=4, dv=3, beta_per_token=True)
    kw = dict(beta=None, lam=0.05, eps=1e-6, window=window)
    o, S, kl = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta_t=inp["beta_t"], **kw)
    bounds = [0] + list(cuts) + [L]
    outs, state, kp, xh, yh = [], None, None, None, None
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        sg = _seg(inp, lo, hi)
        oo, state, k_last = fo.falcon_recurrence(variant, sg["q"], sg["k"], sg["v"], beta_t=sg["beta_t"],
                                                 k_prev=kp, S0=state, x_hist=xh, y_hist=yh, **kw)
        xh, yh = fo.falcon_history(sg["k"], sg["v"], window, k_prev=kp, x_hist=xh, y_hist=yh)
        kp = k_last
        outs.append(oo)
    np.testing.assert_allclose(np.concatenate(outs, axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(state, S, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(kp, kl)


def test_window_history_is_the_latest_samples():
    # the carried samples are (x_j, y_j) = (k_{j-1}, v_j) for the last window-1
    # steps, read off a plain list of the samples of every call so far
    rng = np.random.default_rng(12)
    B, H, dk, dv, window = 1, 2, 3, 2, 4
    kp0 = rng.standard_normal((B, H, dk))
    ks = [rng.standard_normal((B, H, n, dk)) for n in (2, 1, 5)]
    vs = [rng.standard_normal((B, H, n, dv)) for n in (2, 1, 5)]
    xs, ys = [], []          # every sample of the sequence, in order
    kp, xh, yh = kp0, None, None
    for k, v in zip(ks, vs):
        for t in range(k.shape[2]):
            xs.append(kp if t == 0 else k[:, :, t - 1])
            ys.append(v[:, :, t])
        xh, yh = fo.falcon_history(k, v, window, k_prev=kp, x_hist=xh, y_hist=yh)
        kp = k[:, :, -1]
        n = window - 1
        pad = max(0, n - len(xs))
        want_x = [np.zeros((B, H, dk))] * pad + xs[len(xs) - (n - pad):]
        want_y = [np.zeros((B, H, dv))] * pad + ys[len(ys) - (n - pad):]
        np.testing.assert_array_equal(xh, np.stack(want_x, axis=2))
        np.testing.assert_array_equal(yh, np.stack(want_y, axis=2))


@pytest.mark.parametrize("variant", [fo.FALCON_3, fo.FALCON_3A])
def test_zero_history_is_no_history(variant):
    # zero samples add nothing to the normalizer or to the write
    inp = _tiny(86, B=1, H=2, L=7, dk=4, dv=3, with_k_prev=True, with_S0=True)
    kw = dict(beta=0.7, lam=0.05, eps=1e-6, window=3, k_prev=inp["k_prev"], S0=inp["S0"])
    a = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
    b = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"],
                             x_hist=np.zeros((1, 2, 2, 4)), y_hist=np.zeros((1, 2, 2, 3)), **kw)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("variant", [fo.FALCON_3, fo.FALCON_3A])
@pytest.mark.parametrize("window", [2, 4])
@pytest.mark.parametrize("same_step", [False, True])
def test_window_decode_equals_recurrence(variant, window, same_step):
    # prefill, then one decode step per token with the carried history, equals
    # the recurrence over the whole sequence (either pairing)
    L, L1 = 9, 3
    inp = _tiny(87, B=2, H=2, L=L, dk=4, dv=3)
    kw = dict(beta=0.6, lam=0.05, eps=1e-6, same_step=same_step)
    o, S, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], window=window, **kw)
    sg = _seg(inp, 0, L1)
    o1, St, kp = fo.falcon_recurrence(variant, sg["q"], sg["k"], sg["v"], window=window, **kw)
    xh, yh = fo.falcon_history(sg["k"], sg["v"], window, same_step=same_step)
    if same_step:
        kp = None
    got = [o1]
    for t in range(L1, L):
        ot, St, kp, xh, yh = fo.falcon_decode_step_window(
            variant, window, St, kp, xh, yh, inp["q"][:, :, t], inp["k"][:, :, t],
            inp["v"][:, :, t], **kw)
        got.append(ot[:, :, None])
    np.testing.assert_allclose(np.concatenate(got, axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(St, S, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_2A])
def test_same_step_decode_equals_recurrence(variant):
    # with same-step pairing a decode step writes (k_t, v_t) and reads with q_t
    inp = _tiny(88, B=2, H=2, L=6, dk=4, dv=3, with_S0=True,
                beta_per_channel=variant == fo.FALCON_2A)
    kw = dict(beta=0.6, lam=0.05, eps=1e-6)
    bt = inp.get("beta_t")
    o, S, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], S0=inp["S0"],
                                   beta_t=bt, same_step=True, **kw)
    St = inp["S0"]
    for t in range(6):
        ot, St, kp = fo.falcon_decode_step(variant, St, None, inp["q"][:, :, t], inp["k"][:, :, t],
                                           inp["v"][:, :, t], same_step=True,
                                           beta_t=None if bt is None else bt[:, :, t], **kw)
        assert kp is None
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(St, S, rtol=1e-13, atol=1e-14)


def _fd_loss(variant, inp, dO, dS_L, dk_last, kw):
    o, S, kl = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], beta_t=inp.get("beta_t"),
                                    k_prev=inp.get("k_prev"), S0=inp.get("S0"), **kw)
    return float(np.sum(dO * o) + np.sum(dS_L * S) + np.sum(dk_last * kl))


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("same_step", [False, True])
@pytest.mark.parametrize("carried", [False, True])
def test_backward_matches_finite_differences(variant, same_step, carried):
    # the backward is the chain rule through the recurrence; central differences
    # of the (pinned) forward along random directions check every input's gradient
    per_ch = variant in (fo.FALCON_2, fo.FALCON_2A)
    window = _window(variant)
    inp = _tiny(95 + variant, B=1, H=2, L=7, dk=4, dv=3, beta_per_channel=per_ch,
                beta_per_token=not per_ch, with_k_prev=carried and not same_step,
                with_S0=carried)
    inp = {n: a.astype(np.float64) for n, a in inp.items()}
    rng = np.random.default_rng(7 + variant)
    dO = rng.standard_normal(inp["v"].shape)
    dS_L = rng.standard_normal((1, 2, 3, 4))
    dk_last = rng.standard_normal((1, 2, 4))
    kw = dict(beta=None, lam=0.05, eps=1e-3, window=window, same_step=same_step)
    g = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta_t=inp["beta_t"],
                           k_prev=inp.get("k_prev"), S0=inp.get("S0"), dS_L=dS_L,
                           dk_last=dk_last, **kw)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta_t": "dbeta_t", "k_prev": "dk_prev",
             "S0": "dS0"}
    h = 1e-6
    for name, gname in names.items():
        if name not in inp:
            assert gname not in g
            continue
        for _ in range(2):
            u = rng.standard_normal(inp[name].shape)
            plus = dict(inp); plus[name] = inp[name] + h * u
            minus = dict(inp); minus[name] = inp[name] - h * u
            fd = (_fd_loss(variant, plus, dO, dS_L, dk_last, kw)
                  - _fd_loss(variant, minus, dO, dS_L, dk_last, kw)) / (2 * h)
            an = float(np.sum(g[gname] * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_backward_of_one_step_by_hand():
    # one Falcon-1 step from S0 with x = k_prev, scalar beta, loss = <dO, o> only:
    # o = S1 q, S1 = a S0 + eta (y - S0 x) x^T; d/dq = S1^T dO and d/dv = eta (x.(S1-adjoint))
    rng = np.random.default_rng(11)
    dk, dv = 3, 2
    S0 = rng.standard_normal((1, 1, dv, dk))
    kp = rng.standard_normal((1, 1, dk))
    q = rng.standard_normal((1, 1, 1, dk))
    k = rng.standard_normal((1, 1, 1, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    dO = rng.standard_normal((1, 1, 1, dv))
    beta, lam, eps = 0.7, 0.1, 0.01
    g = fo.falcon_backward(fo.FALCON_1, q, k, v, dO, beta=beta, lam=lam, eps=eps, k_prev=kp, S0=S0)
    x, s0, qq, y, do = kp[0, 0], S0[0, 0], q[0, 0, 0], v[0, 0, 0], dO[0, 0, 0]
    eta = beta / (eps + x @ x)
    a = 1 - eta * lam
    S1 = a * s0 + eta * np.outer(y - s0 @ x, x)
    G = np.outer(do, qq)                       # adjoint of S1
    np.testing.assert_allclose(g["dq"][0, 0, 0], S1.T @ do, rtol=1e-12)
    np.testing.assert_allclose(g["dv"][0, 0, 0], eta * (G @ x), rtol=1e-12)
    # S0 enters through a S0 and -eta (S0 x) x^T
    np.testing.assert_allclose(g["dS0"][0, 0], a * G - eta * np.outer(G @ x, x), rtol=1e-12)
    # k is not used by this step (it only becomes k_last)
    np.testing.assert_array_equal(g["dk"], np.zeros_like(k))

"""The chunk-parallel algebra (tests/chunk_form_model.py) equals the recurrence.

CPU only.  Checks every variant, window 1..4, chunk sizes that do and do not
divide L, carried key/state, per-token and per-channel gains.
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs
from chunk_form_model import (chunk_backward, chunk_forward, chunk_forward_folded, chunk_forward_wy,
                              masked_blocked)

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_2, fo.FALCON_3,
                                     fo.FALCON_1A, fo.FALCON_2A, fo.FALCON_3A])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("carried", [False, True])
def test_chunk_form_equals_recurrence(variant, chunk, carried):
    per_row = variant in (fo.FALCON_2, fo.FALCON_2A)
    windowed = variant in (fo.FALCON_3, fo.FALCON_3A)
    windows = [2, 3, 4] if windowed else [1]
    for window in windows:
        if carried and window > 1:
            continue
        inp = seq_inputs(1, 1, 96, 8, 5, seed=100 + variant + window, dtype="bf16",
                         beta_per_channel=per_row, beta_per_token=not per_row,
                         with_k_prev=carried, with_S0=carried, s_std=0.3)
        kw = dict(beta=None, lam=0.02, eps=1e-6, window=window, beta_t=inp["beta_t"],
                  k_prev=inp.get("k_prev"), S0=inp.get("S0"))
        o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
        o, S = chunk_forward(fo.is_regression(variant), per_row, inp["q"][0, 0], inp["k"][0, 0],
                             inp["v"][0, 0], beta=None, lam=0.02, eps=1e-6, window=window,
                             chunk=chunk, beta_t=inp["beta_t"][0, 0],
                             k_prev=None if not carried else inp["k_prev"][0, 0],
                             S0=None if not carried else inp["S0"][0, 0])
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_1A])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("carried", [False, True])
def test_precomputed_inverse_form_equals_recurrence(variant, chunk, carried):
    inp = seq_inputs(1, 1, 150, 8, 5, seed=300 + variant + chunk, dtype="bf16",
                     beta_per_token=True, with_k_prev=carried, with_S0=carried, s_std=0.3)
    kw = dict(beta=None, lam=0.02, eps=1e-6, window=1, beta_t=inp["beta_t"],
              k_prev=inp.get("k_prev"), S0=inp.get("S0"))
    o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
    o, S = chunk_forward_wy(fo.is_regression(variant), inp["q"][0, 0], inp["k"][0, 0],
                            inp["v"][0, 0], beta=None, lam=0.02, eps=1e-6, chunk=chunk,
                            beta_t=inp["beta_t"][0, 0],
                            k_prev=None if not carried else inp["k_prev"][0, 0],
                            S0=None if not carried else inp["S0"][0, 0])
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_3, fo.FALCON_1A, fo.FALCON_3A])
@pytest.mark.parametrize("carried_key", [False, True])
def test_key_folded_form_equals_recurrence(variant, carried_key):
    windowed = variant in (fo.FALCON_3, fo.FALCON_3A)
    for window in ([2, 3, 4] if windowed else [1]):
        inp = seq_inputs(1, 1, 75, 8, 5, seed=500 + variant + window, dtype="bf16",
                         beta_per_token=True, with_k_prev=carried_key, s_std=0.3)
        kw = dict(beta=None, lam=0.02, eps=1e-6, window=window, beta_t=inp["beta_t"],
                  k_prev=inp.get("k_prev"))
        o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
        o, S = chunk_forward_folded(fo.is_regression(variant), inp["q"][0, 0], inp["k"][0, 0],
                                    inp["v"][0, 0], beta=None, lam=0.02, eps=1e-6,
                                    window=window, beta_t=inp["beta_t"][0, 0],
                                    k_prev=inp["k_prev"][0, 0] if carried_key else None)
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_2, fo.FALCON_1A, fo.FALCON_2A])
@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("carried,same_step", [(False, False), (True, False), (False, True),
                                               (True, True)])
def test_chunk_backward_equals_oracle_backward(variant, chunk, carried, same_step):
    per_row = variant in (fo.FALCON_2, fo.FALCON_2A)
    inp = seq_inputs(1, 1, 75, 8, 5, seed=900 + variant + chunk, dtype="bf16",
                     beta_per_channel=per_row, beta_per_token=not per_row,
                     with_k_prev=carried and not same_step, with_S0=carried, s_std=0.3)
    rng = np.random.default_rng(3 + variant)
    dO = rng.standard_normal((1, 1, 75, 5))
    dS_L = rng.standard_normal((1, 1, 5, 8))
    dk_last = rng.standard_normal((1, 1, 8))
    kw = dict(beta=None, lam=0.02, eps=1e-6)
    ref = fo.falcon_backward(variant, inp["q"], inp["k"], inp["v"], dO, beta_t=inp["beta_t"],
                             k_prev=inp.get("k_prev"), S0=inp.get("S0"), same_step=same_step,
                             dS_L=dS_L, dk_last=dk_last, **kw)
    sq = lambda a: None if a is None else a[0, 0]
    got = chunk_backward(fo.is_regression(variant), sq(inp["q"]), sq(inp["k"]), sq(inp["v"]),
                         dO[0, 0], chunk=chunk, beta_t=sq(inp["beta_t"]),
                         k_prev=sq(inp.get("k_prev")), S0=sq(inp.get("S0")),
                         same_step=same_step, dS_L=dS_L[0, 0], dk_last=dk_last[0, 0], **kw)
    assert set(got) == set(ref)
    for name in ref:
        np.testing.assert_allclose(got[name], ref[name][0, 0], rtol=1e-8, atol=1e-9,
                                   err_msg=name)


@pytest.mark.parametrize("variant", [fo.FALCON_1, fo.FALCON_1A])
@pytest.mark.parametrize("L", [1, 16, 37, 64])
@pytest.mark.parametrize("case", ["plain", "carried", "same_step", "nlms", "strong", "negative"])
def test_masked_blocked_form_equals_recurrence(variant, L, case):
    """The blocked masked system of the matrix-core masked kernel (window 1, shared
    gains): decay factors as products only, 16-step blocks, T_bb = (I + A_bb)^-1 and
    the block forward substitution; fresh and carried calls, both pairings, exact
    NLMS (lambda = eps = 0, beta = 1), forgetting far past the chunk algebra's range
    and decays below zero."""
    carried = case in ("carried", "nlms", "strong", "negative")
    same_step = case == "same_step"
    beta, lam, eps = {"nlms": (1.0, 0.0, 0.0), "strong": (0.99, 1.0, 1e-6),
                      "negative": (0.5, 3.0, 1e-6)}.get(case, (None, 0.02, 1e-6))
    inp = seq_inputs(1, 1, L, 8, 5, seed=1200 + 7 * variant + L, dtype="bf16",
                     beta_per_token=beta is None, with_k_prev=carried and not same_step,
                     with_S0=carried, s_std=0.3)
    bt = inp["beta_t"] if beta is None else None
    kw = dict(beta=beta, lam=lam, eps=eps, window=1, beta_t=bt,
              k_prev=inp.get("k_prev") if carried else None,
              S0=inp.get("S0") if carried else None, same_step=same_step)
    o_ref, S_ref, _ = fo.falcon_recurrence(variant, inp["q"], inp["k"], inp["v"], **kw)
    o, S = masked_blocked(fo.is_regression(variant), inp["q"][0, 0], inp["k"][0, 0],
                          inp["v"][0, 0], beta=beta, lam=lam, eps=eps,
                          beta_t=None if bt is None else bt[0, 0],
                          k_prev=inp["k_prev"][0, 0] if carried else None,
                          S0=inp["S0"][0, 0] if carried else None, same_step=same_step)
    scale_o = max(np.max(np.abs(o_ref)), 1e-300)
    scale_s = max(np.max(np.abs(S_ref)), 1e-300)
    np.testing.assert_allclose(o / scale_o, o_ref[0, 0] / scale_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S / scale_s, S_ref[0, 0] / scale_s, rtol=0, atol=1e-12)

"""The chunk-parallel algebra (tests/chunk_form_model.py) equals the recurrence.

CPU only.  Checks every variant, window 1..4, chunk sizes that do and do not
divide L, carried key/state, per-token and per-channel gains.
"""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs
from chunk_form_model import chunk_forward, chunk_forward_folded, chunk_forward_wy

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

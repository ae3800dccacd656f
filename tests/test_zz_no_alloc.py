"""The allocation-free backward entry point (falcon_bwd_chunk_noalloc) against
the one that takes a caller workspace (falcon_bwd_chunk): same kernels, so the
gradients must agree bit for bit; two calls in a row, the second smaller, share
the library's per-GPU array."""
import numpy as np
import pytest

from weight_recurrent_memory_amd.inputs import seq_inputs
from parity_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


def _case(B, H, L, dk, dv, variant, window, seed, per_token, carried):
    inp = seq_inputs(B, H, L, dk, dv, seed=seed, dtype="bf16", beta_per_token=per_token,
                     with_k_prev=carried, with_S0=carried and window == 1, s_std=0.2)
    rng = np.random.default_rng(seed + 1)
    dO = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    dS_L = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
    dt = torch.bfloat16
    dev = lambda n: to_dev(torch, inp[n], dt) if n in inp else None
    kw = dict(variant=variant, beta=None if per_token else 0.5, lam=0.02, eps=1e-6, window=window,
              beta_t=dev("beta_t"), k_prev=dev("k_prev"),
              S0=to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None,
              dS_L=to_dev(torch, dS_L, torch.float32))
    return (dev("q"), dev("k"), dev("v"), to_dev(torch, dO, torch.float32)), kw


def test_noalloc_backward_equals_workspace_backward_twice():
    cases = [
        # (B, H, L, dk, dv, variant, window, seed, per-token gains, carried key/state)
        (2, 3, 300, 64, 64, fw.FALCON_1, 1, 1400, True, True),     # ~5 MB of workspace
        (1, 2, 77, 32, 16, fw.FALCON_3, 4, 1410, False, True),     # smaller, windowed
    ]
    for B, H, L, dk, dv, variant, window, seed, per_token, carried in cases:
        args, kw = _case(B, H, L, dk, dv, variant, window, seed, per_token, carried)
        print("no-alloc backward B%d H%d L%d dk %d dv %d variant %d window %d"
              % (B, H, L, dk, dv, variant, window), flush=True)
        got = fw.bwd_chunk_noalloc(*args, **kw)
        ref = fw.bwd_chunk(*args, **kw)
        torch.cuda.synchronize()
        assert set(got) == set(ref)
        for n in ref:
            a, b = got[n].cpu().numpy(), ref[n].cpu().numpy()
            diff = ~((a == b) | (np.isnan(a) & np.isnan(b)))
            if diff.any():
                idx = np.argwhere(diff)
                print("%s: %d of %d differ, NaN in no-alloc %d, NaN in reference %d, first %s"
                      % (n, diff.sum(), diff.size, np.isnan(a).sum(), np.isnan(b).sum(),
                         idx[:4].tolist()))
            np.testing.assert_array_equal(a, b, err_msg=n)


def test_noalloc_backward_rejects_oversize():
    """The headline backward needs more workspace than the library's array."""
    B, H, L, d = 8, 12, 2048, 64
    q = torch.zeros((B, H, L, d), device="cuda", dtype=torch.bfloat16)
    dO = torch.zeros((B, H, L, d), device="cuda", dtype=torch.float32)
    with pytest.raises(fw.FalconError) as ei:
        fw.bwd_chunk_noalloc(q, q, q, dO, variant=fw.FALCON_1)
    assert ei.value.status == 2

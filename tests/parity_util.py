"""Shared helpers of the parity tests: device upload, normwise error, sampling."""
import numpy as np

# Per-token normwise gate on o: max over (b, h, t) of ||o - o_ref||_inf / ||o_ref||_inf,
# over tokens with o_ref != 0; tokens with o_ref == 0 must be exactly 0.
TOL_BF16 = 2e-3      # bf16 inputs, matrix-core chunk path
TOL_F32 = 1e-4       # fp32 inputs
TOL_FP32_MATH = 1e-4  # recurrent and decode kernels compute in fp32 on exact inputs


def to_dev(torch, arr, dtype):
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device="cuda").to(dtype).contiguous()


def token_normwise_err(o, o_ref):
    """o, o_ref [..., dv] arrays.  Returns (max normwise error, zero rows ok)."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    ref_inf = np.max(np.abs(o_ref), axis=-1)
    diff_inf = np.max(np.abs(o - o_ref), axis=-1)
    zero = ref_inf == 0
    zero_ok = bool(np.all(diff_inf[zero] == 0)) if np.any(zero) else True
    nz = ~zero
    err = float(np.max(diff_inf[nz] / ref_inf[nz])) if np.any(nz) else 0.0
    return err, zero_ok


def state_err(S, S_ref):
    S = np.asarray(S, dtype=np.float64)
    S_ref = np.asarray(S_ref, dtype=np.float64)
    return float(np.max(np.abs(S - S_ref)) / max(np.max(np.abs(S_ref)), 1e-30))

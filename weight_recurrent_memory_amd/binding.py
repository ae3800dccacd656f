"""ctypes binding of libfalcon's C entry points (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI; this
module checks torch tensors (device, dtype, contiguity, shape), allocates the
outputs with torch, and passes raw pointers plus the current HIP stream.  When
the library is missing it raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

FALCON_1, FALCON_2, FALCON_3, FALCON_1A, FALCON_2A, FALCON_3A = range(6)
VARIANT_NAMES = {"falcon1": FALCON_1, "falcon2": FALCON_2, "falcon3": FALCON_3,
                 "falcon1a": FALCON_1A, "falcon2a": FALCON_2A, "falcon3a": FALCON_3A}
_BF16, _F32 = 0, 1
_BETA_SCALAR, _BETA_TOKEN, _BETA_CHANNEL = 0, 1, 2
SAME_STEP = 1        # flag: pair v_t with k_t instead of k_{t-1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FalconError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libfalcon.so")


def load_library():
    """Load libfalcon.so from the package directory (built in-tree)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError("libfalcon.so not built at %s; run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.falcon_abi_version.restype = i
    lib.falcon_abi_version.argtypes = []
    lib.falcon_status_string.restype = ctypes.c_char_p
    lib.falcon_status_string.argtypes = [i]
    seq_args = [i, i, f, vp, i, f, f, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.falcon_fwd_recurrent.restype = i
    lib.falcon_fwd_recurrent.argtypes = seq_args + [vp]
    lib.falcon_fwd_chunk.restype = i
    lib.falcon_fwd_chunk.argtypes = seq_args + [i, vp]
    lib.falcon_decode_step.restype = i
    lib.falcon_decode_step.argtypes = [i, f, vp, i, f, f, i, i, i, i, i, vp, vp, vp, vp, vp,
                                       vp, vp]
    ex_args = [i, i, i, f, vp, i, f, f, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
               vp]
    lib.falcon_fwd_recurrent_ex.restype = i
    lib.falcon_fwd_recurrent_ex.argtypes = ex_args + [vp]
    lib.falcon_fwd_chunk_ex.restype = i
    lib.falcon_fwd_chunk_ex.argtypes = ex_args + [i, vp]
    lib.falcon_fwd_masked.restype = i
    lib.falcon_fwd_masked.argtypes = ex_args + [vp]
    lib.falcon_fwd_workspace_bytes.restype = ctypes.c_ulonglong
    lib.falcon_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.falcon_fwd_chunk_ws.restype = i
    lib.falcon_fwd_chunk_ws.argtypes = ex_args + [vp, ctypes.c_ulonglong, i, vp]
    lib.falcon_decode_step_ex.restype = i
    lib.falcon_decode_step_ex.argtypes = [i, i, i, f, vp, i, f, f, i, i, i, i, i, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp]
    lib.falcon_bwd_workspace_bytes.restype = ctypes.c_ulonglong
    lib.falcon_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.falcon_bwd_chunk.restype = i
    lib.falcon_bwd_chunk.argtypes = [i, i, i, f, vp, i, f, f, i, i, i, i, i, i, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_ulonglong,
                                     vp]
    lib.falcon_bwd_chunk_noalloc.restype = i
    lib.falcon_bwd_chunk_noalloc.argtypes = [i, i, i, f, vp, i, f, f, i, i, i, i, i, i, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    _LIB = lib
    return lib


def _variant(v):
    if isinstance(v, str):
        return VARIANT_NAMES[v.lower().replace("-", "")]
    return int(v)


def kind_of(beta_t):
    """Gain kind of a beta_t argument: scalar, per token ([B,H,L]) or per channel."""
    if beta_t is None:
        return _BETA_SCALAR
    return _BETA_TOKEN if beta_t.dim() == 3 else _BETA_CHANNEL


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(torch, t):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError("inputs must be bfloat16 or float32, got %s" % t.dtype)


def _check(torch, name, t, shape, dtype, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must live on %s" % (name, device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s shape %s != %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(torch, device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raise(lib, fn, status):
    if status != 0:
        raise FalconError(fn, status, lib.falcon_status_string(status).decode())


def _seq_call(fn_name, q, k, v, variant, beta, lam, eps, window, beta_t, k_prev, S0,
              out, S_out, return_state, chunk, stream, x_hist=None, y_hist=None,
              return_history=False, x_hist_out=None, y_hist_out=None, same_step=False,
              workspace=None):
    import torch
    lib = load_library()
    variant = _variant(variant)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, L, d]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    dcode = _dtype_code(torch, q)
    _check(torch, "q", q, (B, H, L, dk), dt, dev)
    _check(torch, "k", k, (B, H, L, dk), dt, dev)
    _check(torch, "v", v, (B, H, L, dv), dt, dev)
    _check(torch, "k_prev", k_prev, (B, H, dk), dt, dev)
    _check(torch, "S0", S0, (B, H, dv, dk), torch.float32, dev)
    kind = _BETA_SCALAR
    if beta_t is not None:
        if beta_t.dim() == 3:
            kind = _BETA_TOKEN
            _check(torch, "beta_t", beta_t, (B, H, L), dt, dev)
        else:
            kind = _BETA_CHANNEL
            _check(torch, "beta_t", beta_t, (B, H, L, dv), dt, dev)
    if out is None:
        out = torch.empty((B, H, L, dv), device=dev, dtype=torch.float32)
    _check(torch, "out", out, (B, H, L, dv), torch.float32, dev)
    if S_out is None and return_state:
        S_out = torch.empty((B, H, dv, dk), device=dev, dtype=torch.float32)
    _check(torch, "S_out", S_out, (B, H, dv, dk), torch.float32, dev)
    masked = fn_name == "falcon_fwd_masked"     # one signature, the _ex form
    ws_ptr, ws_bytes = None, 0
    if fn_name == "falcon_fwd_chunk" and workspace is not None:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace: None, 'auto' or a device tensor")
            need = lib.falcon_fwd_workspace_bytes(variant, int(window), kind_of(beta_t), B, H, L,
                                                  dk, dv, dcode)
            workspace = (torch.empty(int(need), device=dev, dtype=torch.uint8) if need > 0
                         else None)
        if workspace is not None:
            if workspace.device != dev or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on the inputs' device")
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    ws = ws_ptr is not None
    ext = (masked or ws or x_hist is not None or y_hist is not None or return_history
           or x_hist_out is not None or y_hist_out is not None or same_step)
    nh = int(window) - 1
    _check(torch, "x_hist", x_hist, (B, H, nh, dk), dt, dev)
    _check(torch, "y_hist", y_hist, (B, H, nh, dv), dt, dev)
    if return_history:
        if x_hist_out is None:
            x_hist_out = torch.empty((B, H, nh, dk), device=dev, dtype=dt)
        if y_hist_out is None:
            y_hist_out = torch.empty((B, H, nh, dv), device=dev, dtype=dt)
    _check(torch, "x_hist_out", x_hist_out, (B, H, nh, dk), dt, dev)
    _check(torch, "y_hist_out", y_hist_out, (B, H, nh, dv), dt, dev)
    args = [float(beta if beta is not None else 0.0), _ptr(beta_t), kind,
            float(lam), float(eps), B, H, L, dk, dv, dcode, _ptr(q), _ptr(k), _ptr(v),
            _ptr(k_prev), _ptr(S0)]
    if ext:
        if ws:
            fn_name += "_ws"
        elif not masked:
            fn_name += "_ex"
        args = [variant, int(window), SAME_STEP if same_step else 0] + args
        args += [_ptr(x_hist), _ptr(y_hist), _ptr(out), _ptr(S_out), _ptr(x_hist_out),
                 _ptr(y_hist_out)]
    else:
        args = [variant, int(window)] + args + [_ptr(out), _ptr(S_out)]
    if ws:
        args += [ws_ptr, ws_bytes]
    if fn_name.startswith("falcon_fwd_chunk"):
        args.append(int(chunk))
    args.append(_stream(torch, dev, stream))
    status = getattr(lib, fn_name)(*args)
    _raise(lib, fn_name, status)
    res = (out, S_out) if return_state else (out,)
    if return_history:
        res = res + (x_hist_out, y_hist_out)
    return res if len(res) > 1 else res[0]


def fwd_recurrent(q, k, v, *, variant, beta=0.5, lam=0.0, eps=1e-6, window=1, beta_t=None,
                  k_prev=None, S0=None, out=None, S_out=None, return_state=False, stream=None,
                  x_hist=None, y_hist=None, return_history=False, x_hist_out=None,
                  y_hist_out=None, same_step=False):
    """Recurrent form.  Returns o [B,H,L,dv] float32, then S_L with return_state,
    then the window history after the call (x_hist, y_hist) with return_history.
    x_hist [B,H,window-1,dk] / y_hist [B,H,window-1,dv]: carried window samples of a
    resumed Falcon-3/3A sequence, oldest first.  same_step: x_t = k_t (no k_prev)."""
    return _seq_call("falcon_fwd_recurrent", q, k, v, variant, beta, lam, eps, window, beta_t,
                     k_prev, S0, out, S_out, return_state, None, stream, x_hist, y_hist,
                     return_history, x_hist_out, y_hist_out, same_step)


def fwd_chunk(q, k, v, *, variant, beta=0.5, lam=0.0, eps=1e-6, chunk=64, window=1,
              beta_t=None, k_prev=None, S0=None, out=None, S_out=None, return_state=False,
              stream=None, x_hist=None, y_hist=None, return_history=False, x_hist_out=None,
              y_hist_out=None, same_step=False, workspace="auto"):
    """Chunk-parallel form; results, history and pairing arguments as fwd_recurrent.
    workspace: "auto" (default) allocates the device workspace of the two-kernel
    form where the library has one for the call (falcon_fwd_workspace_bytes > 0),
    a uint8 device tensor supplies it, None runs the single-kernel form."""
    return _seq_call("falcon_fwd_chunk", q, k, v, variant, beta, lam, eps, window, beta_t,
                     k_prev, S0, out, S_out, return_state, chunk, stream, x_hist, y_hist,
                     return_history, x_hist_out, y_hist_out, same_step, workspace)


def fwd_masked(q, k, v, *, variant, beta=0.5, lam=0.0, eps=1e-6, window=1, beta_t=None,
               k_prev=None, S0=None, out=None, S_out=None, return_state=False, stream=None,
               x_hist=None, y_hist=None, return_history=False, x_hist_out=None,
               y_hist_out=None, same_step=False):
    """Masked-parallel form, the whole call one masked system (L <= 64); results,
    history and pairing arguments as fwd_recurrent."""
    return _seq_call("falcon_fwd_masked", q, k, v, variant, beta, lam, eps, window, beta_t,
                     k_prev, S0, out, S_out, return_state, None, stream, x_hist, y_hist,
                     return_history, x_hist_out, y_hist_out, same_step)


def decode_step(S, k_prev, q, k, v, *, variant, beta=0.5, lam=0.0, eps=1e-6, beta_t=None,
                out=None, stream=None, window=1, x_hist=None, y_hist=None, same_step=False):
    """One decode step; updates S and k_prev (and, for window > 1, the window
    history x_hist [N,H,window-1,dk] / y_hist [N,H,window-1,dv]) in place,
    returns o [N,H,dv] float32.  same_step: x = k; k_prev must be None."""
    import torch
    lib = load_library()
    variant = _variant(variant)
    N, H, dv, dk = S.shape
    dev = S.device
    dt = q.dtype
    dcode = _dtype_code(torch, q)
    _check(torch, "S", S, (N, H, dv, dk), torch.float32, dev)
    _check(torch, "k_prev", k_prev, (N, H, dk), dt, dev)
    _check(torch, "q", q, (N, H, dk), dt, dev)
    _check(torch, "k", k, (N, H, dk), dt, dev)
    _check(torch, "v", v, (N, H, dv), dt, dev)
    kind = _BETA_SCALAR
    if beta_t is not None:
        kind = _BETA_TOKEN if beta_t.dim() == 2 else _BETA_CHANNEL
        _check(torch, "beta_t", beta_t, (N, H) if kind == _BETA_TOKEN else (N, H, dv), dt, dev)
    if out is None:
        out = torch.empty((N, H, dv), device=dev, dtype=torch.float32)
    _check(torch, "out", out, (N, H, dv), torch.float32, dev)
    # Falcon-3/3A (any window), a history or the same-step pairing: the extended
    # entry point; the plain one takes the un-windowed variants only
    if (window > 1 or x_hist is not None or y_hist is not None or same_step
            or variant in (FALCON_3, FALCON_3A)):
        _check(torch, "x_hist", x_hist, (N, H, int(window) - 1, dk), dt, dev)
        _check(torch, "y_hist", y_hist, (N, H, int(window) - 1, dv), dt, dev)
        status = lib.falcon_decode_step_ex(
            variant, int(window), SAME_STEP if same_step else 0,
            float(beta if beta is not None else 0.0), _ptr(beta_t), kind, float(lam), float(eps),
            N, H, dk, dv, dcode, _ptr(S), _ptr(k_prev), _ptr(x_hist), _ptr(y_hist), _ptr(q),
            _ptr(k), _ptr(v), _ptr(out), _stream(torch, dev, stream))
        _raise(lib, "falcon_decode_step_ex", status)
        return out
    status = lib.falcon_decode_step(variant, float(beta if beta is not None else 0.0),
                                    _ptr(beta_t), kind, float(lam), float(eps), N, H, dk, dv,
                                    dcode, _ptr(S), _ptr(k_prev), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(out), _stream(torch, dev, stream))
    _raise(lib, "falcon_decode_step", status)
    return out


def bwd_chunk(q, k, v, dO, *, variant, beta=0.5, lam=0.0, eps=1e-6, window=1, beta_t=None,
              k_prev=None, S0=None, dS_L=None, dk_last=None, same_step=False, stream=None,
              _noalloc=False):
    """Gradients of sum <dO, o> + <dS_L, S_L> + <dk_last, k_last> for the chunk form
    (window 1 to 8).  Returns a dict of float32 tensors: dq, dk, dv, and dbeta_t /
    dk_prev / dS0 when beta_t / k_prev / S0 are given."""
    import torch
    lib = load_library()
    variant = _variant(variant)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    dcode = _dtype_code(torch, q)
    f32 = torch.float32
    for name, t, shape, tdt in (("q", q, (B, H, L, dk), dt), ("k", k, (B, H, L, dk), dt),
                                ("v", v, (B, H, L, dv), dt), ("dO", dO, (B, H, L, dv), f32),
                                ("k_prev", k_prev, (B, H, dk), dt), ("S0", S0, (B, H, dv, dk), f32),
                                ("dS_L", dS_L, (B, H, dv, dk), f32),
                                ("dk_last", dk_last, (B, H, dk), f32)):
        _check(torch, name, t, shape, tdt, dev)
    kind = _BETA_SCALAR
    if beta_t is not None:
        kind = _BETA_TOKEN if beta_t.dim() == 3 else _BETA_CHANNEL
        _check(torch, "beta_t", beta_t, (B, H, L) if kind == _BETA_TOKEN else (B, H, L, dv), dt,
               dev)
    out = dict(dq=torch.empty((B, H, L, dk), device=dev, dtype=f32),
               dk=torch.empty((B, H, L, dk), device=dev, dtype=f32),
               dv=torch.empty((B, H, L, dv), device=dev, dtype=f32))
    if beta_t is not None:
        out["dbeta_t"] = torch.empty(beta_t.shape, device=dev, dtype=f32)
    if k_prev is not None and not same_step:
        out["dk_prev"] = torch.empty((B, H, dk), device=dev, dtype=f32)
    if S0 is not None:
        out["dS0"] = torch.empty((B, H, dv, dk), device=dev, dtype=f32)
    if _noalloc:
        status = lib.falcon_bwd_chunk_noalloc(
            variant, int(window), SAME_STEP if same_step else 0,
            float(beta if beta is not None else 0.0), _ptr(beta_t), kind, float(lam), float(eps),
            B, H, L, dk, dv, dcode, _ptr(q), _ptr(k), _ptr(v), _ptr(k_prev), _ptr(S0), _ptr(dO),
            _ptr(dS_L), _ptr(dk_last), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
            _ptr(out.get("dbeta_t")), _ptr(out.get("dk_prev")), _ptr(out.get("dS0")),
            _stream(torch, dev, stream))
        _raise(lib, "falcon_bwd_chunk_noalloc", status)
        return out
    wsb = int(lib.falcon_bwd_workspace_bytes(B, H, L, dk, dv, int(window)))
    ws = torch.empty((max(wsb, 16) // 4 + 4,), device=dev, dtype=f32)
    status = lib.falcon_bwd_chunk(
        variant, int(window), SAME_STEP if same_step else 0, float(beta if beta is not None else 0.0),
        _ptr(beta_t), kind, float(lam), float(eps), B, H, L, dk, dv, dcode, _ptr(q), _ptr(k),
        _ptr(v), _ptr(k_prev), _ptr(S0), _ptr(dO), _ptr(dS_L), _ptr(dk_last), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("dbeta_t")), _ptr(out.get("dk_prev")),
        _ptr(out.get("dS0")), _ptr(ws), wsb, _stream(torch, dev, stream))
    _raise(lib, "falcon_bwd_chunk", status)
    return out


def bwd_chunk_noalloc(q, k, v, dO, **kw):
    """bwd_chunk through falcon_bwd_chunk_noalloc: the library's per-GPU workspace
    array instead of one allocated per call (the outputs are still allocated here;
    a caller that cannot allocate calls the C entry point with its own buffers).
    Calls that overlap in time on one GPU race."""
    return bwd_chunk(q, k, v, dO, _noalloc=True, **kw)

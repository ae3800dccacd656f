"""Host-only checks of the C ABI: the library loads, exports every entry point
declared in include/falcon.h, and rejects bad arguments before any HIP call
(fake, never-dereferenced pointers are enough for that)."""
import ctypes
import os
import re
import subprocess

import pytest

import weight_recurrent_memory_amd as fw
from weight_recurrent_memory_amd import binding

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "falcon.h")
OK, INVALID, UNSUPPORTED = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from weight_recurrent_memory_amd import build_lib
        build_lib.build()
    return fw.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:unsigned\s+long\s+long|\w+)\**\s+\**(falcon_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("falcon_fwd_recurrent", "falcon_fwd_chunk", "falcon_decode_step",
              "falcon_fwd_recurrent_ex", "falcon_fwd_chunk_ex", "falcon_decode_step_ex",
              "falcon_bwd_chunk", "falcon_bwd_workspace_bytes", "falcon_abi_version",
              "falcon_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing but the C interface leaks out of the library
    falcon_syms = {s for s in exported if "falcon" in s}
    assert falcon_syms == set(_declared_functions())


def test_version_and_status_strings(lib):
    assert lib.falcon_abi_version() == 4
    assert lib.falcon_status_string(0) == b"ok"
    assert lib.falcon_status_string(1) == b"invalid argument"
    assert lib.falcon_status_string(2) == b"unsupported configuration"
    assert lib.falcon_status_string(3) == b"HIP launch failure"
    assert lib.falcon_status_string(99) == b"unknown status"


# Fake device addresses: validation must reject every call below before touching them.
P = [0x100000000 + 0x10000000 * i for i in range(12)]


def _seq(lib, fn="falcon_fwd_chunk", **over):
    a = dict(variant=0, window=1, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6,
             batch=1, heads=1, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2],
             k_prev=None, S0=None, o=P[3], S_out=None, chunk=64)
    a.update(over)
    args = [a["variant"], a["window"], a["beta"], a["beta_t"], a["beta_kind"], a["lam"], a["eps"],
            a["batch"], a["heads"], a["seqlen"], a["dk"], a["dv"], a["dtype"], a["q"], a["k"],
            a["v"], a["k_prev"], a["S0"], a["o"], a["S_out"]]
    if fn == "falcon_fwd_chunk":
        args.append(a["chunk"])
    args.append(None)
    return getattr(lib, fn)(*args)


@pytest.mark.parametrize("fn", ["falcon_fwd_chunk", "falcon_fwd_recurrent"])
@pytest.mark.parametrize("over,status", [
    (dict(variant=6), INVALID),
    (dict(variant=-1), INVALID),
    (dict(window=0), INVALID),
    (dict(window=2), INVALID),                       # window > 1 outside Falcon-3/3A
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(q=P[0] + 2), INVALID),                     # misaligned
    (dict(seqlen=0), INVALID),
    (dict(batch=-3), INVALID),
    (dict(lam=-0.1), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(beta=float("inf")), INVALID),
    (dict(beta_kind=1), INVALID),                    # per-token beta without a pointer
    (dict(beta_kind=0, beta_t=P[5]), INVALID),       # pointer with scalar kind
    (dict(beta_kind=2, beta_t=P[5]), INVALID),       # per-channel beta on Falcon-1
    (dict(beta_kind=3, beta_t=P[5]), INVALID),
    (dict(S0=P[6]), INVALID),                        # state without the carried key
    (dict(o=P[0]), INVALID),                         # output aliases q
    (dict(dtype=7), INVALID),
    (dict(dk=48), UNSUPPORTED),
    (dict(dv=256), UNSUPPORTED),
    (dict(variant=2, window=2, k_prev=P[7], S0=P[6]), UNSUPPORTED),  # no window history
])
def test_seq_validation(lib, fn, over, status):
    assert _seq(lib, fn, **over) == status


@pytest.mark.parametrize("over,status", [
    (dict(chunk=0), INVALID),
    (dict(chunk=48), UNSUPPORTED),
    (dict(chunk=128), UNSUPPORTED),
    (dict(dtype=1), UNSUPPORTED),
    (dict(variant=2, window=8), UNSUPPORTED),
    (dict(variant=5, window=17), UNSUPPORTED),       # inner-product windows up to 16
    (dict(variant=5, window=8, dk=32, dv=32), UNSUPPORTED),
    (dict(variant=5, window=8, dv=16), UNSUPPORTED),
    (dict(variant=2, window=32, chunk=16), INVALID),  # window > chunk
])
def test_chunk_only_validation(lib, over, status):
    assert _seq(lib, "falcon_fwd_chunk", **over) == status


def _masked(lib, **over):
    a = dict(variant=0, window=1, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6,
             batch=1, heads=1, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2],
             k_prev=None, S0=None, x_hist=None, y_hist=None, o=P[3], S_out=None, xo=None, yo=None)
    a.update(over)
    return lib.falcon_fwd_masked(a["variant"], a["window"], a["flags"], a["beta"], a["beta_t"],
                                 a["beta_kind"], a["lam"], a["eps"], a["batch"], a["heads"],
                                 a["seqlen"], a["dk"], a["dv"], a["dtype"], a["q"], a["k"], a["v"],
                                 a["k_prev"], a["S0"], a["x_hist"], a["y_hist"], a["o"],
                                 a["S_out"], a["xo"], a["yo"], None)


@pytest.mark.parametrize("over,status", [
    (dict(seqlen=65), UNSUPPORTED),                  # one masked system covers at most 64 steps
    (dict(seqlen=4096), UNSUPPORTED),
    (dict(variant=2, window=9), UNSUPPORTED),
    (dict(variant=0, window=2), INVALID),
    (dict(flags=2), INVALID),
    (dict(flags=1, k_prev=P[7]), INVALID),           # same-step pairing takes no carried key
    (dict(S0=P[6]), INVALID),                        # state without the carried key
    (dict(variant=2, window=3, x_hist=P[8]), INVALID),   # one history pointer without the other
    (dict(variant=2, window=3, k_prev=P[7], S0=P[6]), INVALID),  # windowed state, no history
    (dict(dk=48), UNSUPPORTED),
    (dict(o=P[0]), INVALID),
    (dict(seqlen=0), INVALID),
])
def test_masked_validation(lib, over, status):
    """The masked-parallel entry point validates like the recurrent one and refuses
    sequences longer than one masked system, before any HIP call."""
    assert _masked(lib, **over) == status


def test_masked_max_len():
    text = open(HEADER).read()
    m = re.search(r"#define FALCON_MASKED_MAX_LEN (\d+)", text)
    assert m and int(m.group(1)) == 64


def test_fwd_workspace_bytes(lib):
    # one 12416-byte record per (batch, head) and 16-step sub-chunk, for the
    # regression family with a window of 2 or 4, shared gains, dk 64 / 128, bf16
    def rec(B, H, L):
        return B * H * ((L + 15) // 16) * 12416
    assert lib.falcon_fwd_workspace_bytes(2, 4, 0, 4, 16, 8192, 128, 128, 0) == rec(4, 16, 8192)
    assert lib.falcon_fwd_workspace_bytes(2, 2, 1, 1, 3, 77, 64, 32, 0) == rec(1, 3, 77)
    assert lib.falcon_fwd_workspace_bytes(5, 4, 0, 4, 16, 8192, 128, 128, 0) == 0   # Falcon-3A
    assert lib.falcon_fwd_workspace_bytes(0, 1, 0, 8, 12, 2048, 64, 64, 0) == 0     # window 1
    assert lib.falcon_fwd_workspace_bytes(2, 3, 0, 1, 1, 64, 64, 64, 0) == 0        # window 3
    assert lib.falcon_fwd_workspace_bytes(2, 4, 0, 1, 1, 64, 32, 64, 0) == 0        # dk 32
    assert lib.falcon_fwd_workspace_bytes(2, 4, 0, 1, 1, 64, 64, 64, 1) == 0        # fp32 inputs
    assert lib.falcon_fwd_workspace_bytes(0, 4, 0, 1, 1, 64, 64, 64, 0) == 0        # window on Falcon-1
    assert lib.falcon_fwd_workspace_bytes(2, 4, 0, 0, 1, 64, 64, 64, 0) == 0


def _ws(lib, **over):
    a = dict(variant=2, window=4, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6,
             batch=1, heads=1, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2],
             k_prev=None, S0=None, x_hist=None, y_hist=None, o=P[3], S_out=None, xo=None,
             yo=None, ws=P[8], wsb=1 << 20, chunk=64)
    a.update(over)
    return lib.falcon_fwd_chunk_ws(a["variant"], a["window"], a["flags"], a["beta"], a["beta_t"],
                                   a["beta_kind"], a["lam"], a["eps"], a["batch"], a["heads"],
                                   a["seqlen"], a["dk"], a["dv"], a["dtype"], a["q"], a["k"],
                                   a["v"], a["k_prev"], a["S0"], a["x_hist"], a["y_hist"], a["o"],
                                   a["S_out"], a["xo"], a["yo"], a["ws"], a["wsb"], a["chunk"],
                                   None)


@pytest.mark.parametrize("over,status", [
    (dict(ws=P[8] + 8), INVALID),                    # misaligned workspace
    (dict(ws=P[0]), INVALID),                        # workspace overlaps q
    (dict(ws=P[3] + 4096), INVALID),                 # workspace inside o
    (dict(flags=2), INVALID),
    (dict(chunk=48), UNSUPPORTED),
    (dict(variant=0), INVALID),                      # window 4 on Falcon-1
    (dict(q=None), INVALID),
])
def test_fwd_chunk_ws_validation(lib, over, status):
    """falcon_fwd_chunk_ws validates like falcon_fwd_chunk_ex, and its workspace's
    alignment and overlap, before any HIP call."""
    assert _ws(lib, **over) == status


def test_recurrent_window_limit(lib):
    assert _seq(lib, "falcon_fwd_recurrent", variant=2, window=9) == UNSUPPORTED


def _dec(lib, **over):
    a = dict(variant=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6, nseq=2, heads=2,
             dk=64, dv=64, dtype=0, S=P[0], k_prev=P[1], q=P[2], k=P[3], v=P[4], o=P[5])
    a.update(over)
    return lib.falcon_decode_step(a["variant"], a["beta"], a["beta_t"], a["beta_kind"], a["lam"],
                                  a["eps"], a["nseq"], a["heads"], a["dk"], a["dv"], a["dtype"],
                                  a["S"], a["k_prev"], a["q"], a["k"], a["v"], a["o"], None)


@pytest.mark.parametrize("over,status", [
    (dict(variant=9), INVALID),
    (dict(S=None), INVALID),
    (dict(k_prev=P[3]), INVALID),                    # k_prev aliases k
    (dict(o=P[0]), INVALID),
    (dict(nseq=0), INVALID),
    (dict(beta_kind=2, beta_t=P[6]), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(variant=2), UNSUPPORTED),                  # Falcon-3 needs window history
    (dict(variant=5), UNSUPPORTED),
    (dict(dk=80), UNSUPPORTED),
])
def test_decode_validation(lib, over, status):
    assert _dec(lib, **over) == status


def _seqh(lib, fn="falcon_fwd_chunk_ex", **over):
    a = dict(variant=2, window=3, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6,
             batch=1, heads=1, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2],
             k_prev=P[7], S0=P[6], x_hist=P[8], y_hist=P[9], o=P[3], S_out=None, xo=None,
             yo=None, chunk=64)
    a.update(over)
    args = [a["variant"], a["window"], a["flags"], a["beta"], a["beta_t"], a["beta_kind"],
            a["lam"], a["eps"], a["batch"], a["heads"], a["seqlen"], a["dk"], a["dv"], a["dtype"],
            a["q"], a["k"], a["v"], a["k_prev"], a["S0"], a["x_hist"], a["y_hist"], a["o"],
            a["S_out"], a["xo"], a["yo"]]
    if fn == "falcon_fwd_chunk_ex":
        args.append(a["chunk"])
    args.append(None)
    return getattr(lib, fn)(*args)


@pytest.mark.parametrize("fn", ["falcon_fwd_chunk_ex", "falcon_fwd_recurrent_ex"])
@pytest.mark.parametrize("over,status", [
    (dict(y_hist=None), INVALID),                    # history comes in pairs
    (dict(xo=P[10]), INVALID),                       # so do its outputs
    (dict(variant=0, window=1), INVALID),            # no history with window 1
    (dict(k_prev=None, S0=None), INVALID),           # history needs the carried key
    (dict(x_hist=None, y_hist=None), INVALID),       # a windowed state needs its history
    (dict(x_hist=P[8] + 8), INVALID),                # misaligned
    (dict(x_hist=P[3]), INVALID),                    # history aliases the output
    (dict(xo=P[0], yo=P[10]), INVALID),              # history output aliases q
    (dict(xo=P[8] + 64, yo=P[10]), INVALID),         # partial overlap with the input history
    (dict(variant=0, window=2), INVALID),            # window outside Falcon-3/3A
    (dict(flags=2), INVALID),                        # unknown flag
    (dict(flags=1), INVALID),                        # same-step pairing takes no k_prev
    (dict(flags=1, k_prev=None, x_hist=None, y_hist=None), INVALID),  # windowed S0, no history
])
def test_history_validation(lib, fn, over, status):
    assert _seqh(lib, fn, **over) == status


def _dech(lib, **over):
    a = dict(variant=2, window=3, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6, nseq=2,
             heads=2, dk=64, dv=64, dtype=0, S=P[0], k_prev=P[1], x_hist=P[6], y_hist=P[7],
             q=P[2], k=P[3], v=P[4], o=P[5])
    a.update(over)
    return lib.falcon_decode_step_ex(a["variant"], a["window"], a["flags"], a["beta"],
                                     a["beta_t"], a["beta_kind"], a["lam"], a["eps"], a["nseq"],
                                     a["heads"], a["dk"], a["dv"], a["dtype"], a["S"],
                                     a["k_prev"], a["x_hist"], a["y_hist"], a["q"], a["k"], a["v"],
                                     a["o"], None)


@pytest.mark.parametrize("over,status", [
    (dict(x_hist=None, y_hist=None), INVALID),       # window 3 needs its history
    (dict(window=1), INVALID),                       # window 1 takes none
    (dict(window=0), INVALID),
    (dict(variant=0), INVALID),                      # window > 1 outside Falcon-3/3A
    (dict(y_hist=P[6]), INVALID),                    # x and y history alias
    (dict(x_hist=P[5]), INVALID),                    # history aliases o
    (dict(window=9), UNSUPPORTED),
    (dict(beta_kind=2, beta_t=P[8]), INVALID),       # per-channel gain on Falcon-3
    (dict(flags=1), INVALID),                        # same-step pairing takes no k_prev
    (dict(k_prev=None), INVALID),                    # prefix pairing needs it
    (dict(flags=4, k_prev=None), INVALID),
])
def test_decode_history_validation(lib, over, status):
    assert _dech(lib, **over) == status



def _bwd(lib, **over):
    a = dict(variant=0, window=1, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6, batch=1,
             heads=2, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2], k_prev=None,
             S0=None, dO=P[3], dS_L=None, dk_last=None, dq=P[4], dk_=P[5], dv_=P[6],
             dbeta_t=None, dk_prev=None, dS0=None, ws=P[7], wsb=1 << 26)
    a.update(over)
    return lib.falcon_bwd_chunk(a["variant"], a["window"], a["flags"], a["beta"], a["beta_t"], a["beta_kind"],
                                a["lam"], a["eps"], a["batch"], a["heads"], a["seqlen"], a["dk"],
                                a["dv"], a["dtype"], a["q"], a["k"], a["v"], a["k_prev"], a["S0"],
                                a["dO"], a["dS_L"], a["dk_last"], a["dq"], a["dk_"], a["dv_"],
                                a["dbeta_t"], a["dk_prev"], a["dS0"], a["ws"], a["wsb"], None)


def test_backward_workspace_size(lib):
    # per (batch, head), per slice of min(dv, 32) value rows and per chunk of
    # floor(16 / window) steps: start state, S0 x, Gram (fp32); with two or more
    # slices also their partial dq, dk (L x dk each), dk_prev (dk) and per-token
    # dbeta (L)
    def size(B, H, L, dk, dv, window):
        nch = -(-L // (16 // window))
        rb = min(dv, 32)
        nrg = dv // rb
        rec = B * H * nrg * nch * (rb * dk + 16 * rb + 256)
        part = nrg * B * H * (2 * L * dk + dk + L) if nrg > 1 else 0
        return (rec + part) * 4
    for w in range(1, 9):
        assert lib.falcon_bwd_workspace_bytes(2, 3, 100, 64, 32, w) == size(2, 3, 100, 64, 32, w)
    assert lib.falcon_bwd_workspace_bytes(1, 2, 64, 128, 128, 4) == size(1, 2, 64, 128, 128, 4)
    assert lib.falcon_bwd_workspace_bytes(1, 1, 64, 16, 16, 1) == size(1, 1, 64, 16, 16, 1)
    assert lib.falcon_bwd_workspace_bytes(1, 3, 50, 64, 128, 2) == size(1, 3, 50, 64, 128, 2)
    assert lib.falcon_bwd_workspace_bytes(2, 3, 100, 64, 32, 9) == 0
    assert lib.falcon_bwd_workspace_bytes(0, 3, 100, 64, 32, 1) == 0
    assert lib.falcon_bwd_workspace_bytes(1, 1, 16, 48, 32, 1) == 0


@pytest.mark.parametrize("over,status", [
    (dict(variant=2, window=9), UNSUPPORTED),        # windows 1..8 only
    (dict(variant=5, window=16), UNSUPPORTED),
    (dict(variant=0, window=2), INVALID),            # window > 1 outside Falcon-3/3A
    (dict(variant=2, window=0), INVALID),
    (dict(variant=2, window=2, k_prev=P[8], S0=P[9]), UNSUPPORTED),   # windowed start state
    (dict(dk=256), UNSUPPORTED),
    (dict(flags=2), INVALID),
    (dict(dq=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(wsb=1024), INVALID),                       # workspace too small
    (dict(dbeta_t=P[8]), INVALID),                   # scalar beta has no gradient
    (dict(dk_prev=P[8]), INVALID),                   # no k_prev
    (dict(dS0=P[8]), INVALID),                       # no S0
    (dict(dq=P[0]), INVALID),                        # output aliases q
    (dict(ws=P[4]), INVALID),                        # workspace aliases dq
    (dict(dk_=P[4]), INVALID),                       # two outputs alias
    (dict(S0=P[9]), INVALID),                        # state without the carried key
])
def test_backward_validation(lib, over, status):
    assert _bwd(lib, **over) == status


# fake device addresses 4 GiB apart, for calls whose buffers are larger than P's spacing
BIG = [0x1000000000 + 0x100000000 * i for i in range(12)]


@pytest.mark.parametrize("seqlen,window,variant,status", [
    # dk = dv = 128: a chain's chunk records take 4 (32 * 128 + 16 * 32 + 256) bytes per
    # chunk of floor(16 / window) steps; at 1 GiB and above the call is refused
    (900_000, 1, 0, UNSUPPORTED),
    (860_000, 1, 0, INVALID),          # below the limit: fails later, on the small workspace
    (111_000, 8, 2, UNSUPPORTED),
    (109_000, 8, 2, INVALID),
])
def test_backward_chain_limit(lib, seqlen, window, variant, status):
    """The backward kernel addresses a chain's inputs and records with 32-bit
    offsets; a chain that needs 1 GiB or more of them is refused up front."""
    assert _bwd(lib, batch=1, heads=1, seqlen=seqlen, dk=128, dv=128, window=window,
                variant=variant, q=BIG[0], k=BIG[1], v=BIG[2], dO=BIG[3], dq=BIG[4],
                dk_=BIG[5], dv_=BIG[6], ws=BIG[7], wsb=1 << 26) == status


def _bwd_noalloc(lib, **over):
    a = dict(variant=0, window=1, flags=0, beta=0.5, beta_t=None, beta_kind=0, lam=0.01, eps=1e-6, batch=1,
             heads=2, seqlen=64, dk=64, dv=64, dtype=0, q=P[0], k=P[1], v=P[2], k_prev=None,
             S0=None, dO=P[3], dS_L=None, dk_last=None, dq=P[4], dk_=P[5], dv_=P[6],
             dbeta_t=None, dk_prev=None, dS0=None)
    a.update(over)
    return lib.falcon_bwd_chunk_noalloc(a["variant"], a["window"], a["flags"], a["beta"], a["beta_t"],
                                        a["beta_kind"], a["lam"], a["eps"], a["batch"], a["heads"],
                                        a["seqlen"], a["dk"], a["dv"], a["dtype"], a["q"], a["k"],
                                        a["v"], a["k_prev"], a["S0"], a["dO"], a["dS_L"], a["dk_last"],
                                        a["dq"], a["dk_"], a["dv_"], a["dbeta_t"], a["dk_prev"],
                                        a["dS0"], None)


def test_backward_noalloc_scratch_limit():
    text = open(HEADER).read()
    m = re.search(r"#define FALCON_BWD_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == 64 << 20


@pytest.mark.parametrize("over,status", [
    # the headline backward needs about 276 MB of workspace: beyond the library's array
    (dict(batch=8, heads=12, seqlen=2048), UNSUPPORTED),
    (dict(variant=2, window=9), UNSUPPORTED),
    (dict(variant=0, window=2), INVALID),
    (dict(dq=None), INVALID),
    (dict(dq=P[0]), INVALID),                        # output aliases q
    (dict(dS0=P[8]), INVALID),                       # no S0
    (dict(flags=2), INVALID),
])
def test_backward_noalloc_validation(lib, over, status):
    """The allocation-free backward checks every argument, and its workspace need
    against the array it uses, before any HIP call."""
    assert _bwd_noalloc(lib, **over) == status

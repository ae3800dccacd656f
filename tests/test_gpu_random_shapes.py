"""Seeded random configurations through the recurrent, chunk and masked entry
points, the decode step and the backward, against the fp64 oracle: every
variant, windows 1..8,
both input types where the entry point takes them, L from 1 to 200, dk and dv
from 16 to 128, scalar, per-token and per-channel gains, fresh and carried
starts (key, state and window history), both pairings.  The draws are fixed by
the seed, so every run checks the same configurations; each one is printed
before it is launched."""
import numpy as np
import pytest

from oracle import falcon_oracle as fo
from weight_recurrent_memory_amd.inputs import seq_inputs
from parity_util import TOL_BF16, TOL_FP32_MATH, state_err, to_dev, token_normwise_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_recurrent_memory_amd as fw  # noqa: E402

DIMS = (16, 32, 64, 128)


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        variant = int(rng.integers(0, 6))
        windowed = variant in (fo.FALCON_3, fo.FALCON_3A)
        window = int(rng.integers(1, 9)) if windowed else 1
        per_ch_ok = variant in (fo.FALCON_2, fo.FALCON_2A)
        gains = str(rng.choice(["scalar", "token", "channel"] if per_ch_ok else ["scalar", "token"]))
        same_step = bool(rng.random() < 0.25)
        start = str(rng.choice(["fresh", "key", "state"]))
        if same_step and start == "key":
            start = "fresh"
        L = int(rng.integers(1, 201))
        # fp32 inputs only where the masked form takes them (the chunk form is bf16)
        dtype = str(rng.choice(["bf16", "f32"])) if L <= 64 else "bf16"
        cases.append(dict(
            id=i, variant=variant, window=window, gains=gains, same_step=same_step, start=start,
            L=L, dk=int(rng.choice(DIMS)), dv=int(rng.choice(DIMS)),
            dtype=dtype, chunk=int(rng.choice([16, 32, 64])),
            lam=float(rng.choice([0.0, 0.01, 0.3])), beta=float(rng.uniform(0.3, 1.0)),
            seed=int(rng.integers(0, 1 << 30))))
    return cases


CASES = _draw_cases(160, 20261204)
BWD_CASES = [c for c in _draw_cases(48, 20261205)
             if not (c["window"] > 1 and c["start"] == "state")]   # no windowed start state


def _inputs(c):
    carried_key = c["start"] in ("key", "state") and not c["same_step"]
    with_S0 = c["start"] == "state"
    history = c["window"] - 1 if (c["start"] == "state" and c["window"] > 1) else 0
    return seq_inputs(1, 2, c["L"], c["dk"], c["dv"], seed=c["seed"], dtype=c["dtype"],
                      beta_per_token=c["gains"] == "token",
                      beta_per_channel=c["gains"] == "channel", with_k_prev=carried_key,
                      with_S0=with_S0, s_std=0.2, history=history)


def _run(fn, c, inp, dt):
    up = lambda name: to_dev(torch, inp[name], dt) if name in inp else None
    q, k, v = up("q"), up("k"), up("v")
    kw = dict(variant=c["variant"], beta=c["beta"] if c["gains"] == "scalar" else None,
              lam=c["lam"], eps=1e-6, window=c["window"], beta_t=up("beta_t"),
              k_prev=up("k_prev"), S0=to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None,
              x_hist=up("x_hist"), y_hist=up("y_hist"), return_state=True,
              same_step=c["same_step"])
    if fn is fw.fwd_chunk:
        kw["chunk"] = c["chunk"]
    if fn is fw.fwd_recurrent:
        kw.pop("return_state")
        kw["return_state"] = True
    res = fn(q, k, v, **kw)
    torch.cuda.synchronize()
    return res[0].cpu().numpy(), res[1].cpu().numpy()


def _oracle(c, inp):
    o, S, _ = fo.falcon_recurrence(
        c["variant"], inp["q"], inp["k"], inp["v"],
        beta=c["beta"] if c["gains"] == "scalar" else None, lam=c["lam"], eps=1e-6,
        window=c["window"], beta_t=inp.get("beta_t"), k_prev=inp.get("k_prev"),
        S0=inp.get("S0"), x_hist=inp.get("x_hist"), y_hist=inp.get("y_hist"),
        same_step=c["same_step"])
    return o, S


def _label(c):
    return "case %d: v%d B%d %s %s %s L%d dk%d dv%d %s C%d lam %.2f" % (
        c["id"], c["variant"], c["window"], c["gains"], c["start"],
        "same" if c["same_step"] else "prefix", c["L"], c["dk"], c["dv"], c["dtype"],
        c["chunk"], c["lam"])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fw.load_library()


@pytest.mark.parametrize("c", CASES, ids=[str(c["id"]) for c in CASES])
def test_random_configuration(c):
    inp = _inputs(c)
    o_ref, S_ref = _oracle(c, inp)
    # recurrent form: every configuration, the input type as drawn
    print(_label(c) + " recurrent: launching", flush=True)
    o, S = _run(fw.fwd_recurrent, c, inp, torch.bfloat16 if c["dtype"] == "bf16" else torch.float32)
    err, zok = token_normwise_err(o, o_ref)
    serr = state_err(S, S_ref)
    print("  recurrent o err %.3e S err %.3e" % (err, serr), flush=True)
    assert zok and err <= TOL_FP32_MATH and serr <= TOL_FP32_MATH
    # chunk form: bf16 inputs, window <= chunk, window <= 4 (Falcon-3A with shared
    # gains, dk 64 or 128 and dv a multiple of 32: window <= 16)
    wmax = 16 if (c["variant"] == fo.FALCON_3A and c["gains"] != "channel" and c["dk"] >= 64
                  and c["dv"] % 32 == 0) else 4
    if c["dtype"] == "bf16" and c["window"] <= c["chunk"] and c["window"] <= wmax:
        print(_label(c) + " chunk: launching", flush=True)
        o, S = _run(fw.fwd_chunk, c, inp, torch.bfloat16)
        err, zok = token_normwise_err(o, o_ref)
        serr = state_err(S, S_ref)
        print("  chunk o err %.3e S err %.3e" % (err, serr), flush=True)
        assert zok and err <= TOL_BF16 and serr <= TOL_BF16
    # masked-parallel form: L <= 64, either input type
    if c["L"] <= 64:
        print(_label(c) + " masked: launching", flush=True)
        dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
        o, S = _run(fw.fwd_masked, c, inp, dt)
        err, zok = token_normwise_err(o, o_ref)
        serr = state_err(S, S_ref)
        print("  masked o err %.3e S err %.3e" % (err, serr), flush=True)
        assert zok and err <= TOL_FP32_MATH and serr <= TOL_FP32_MATH


@pytest.mark.parametrize("c", BWD_CASES, ids=[str(c["id"]) for c in BWD_CASES])
def test_random_configuration_backward(c):
    """Gradients of the chunk form (every input, the gains, the carried key and
    state) against the oracle's reverse-mode gradients."""
    inp = _inputs(c)
    B, H, L, dk, dv = 1, 2, c["L"], c["dk"], c["dv"]
    rng = np.random.default_rng(c["seed"] + 1)
    dO = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    dS_L = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
    dk_last = rng.standard_normal((B, H, dk)).astype(np.float32)
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    up = lambda n: to_dev(torch, inp[n], dt) if n in inp else None
    f32 = lambda a: to_dev(torch, a, torch.float32)
    beta = c["beta"] if c["gains"] == "scalar" else None
    print(_label(c) + " backward: launching", flush=True)
    got = fw.bwd_chunk(up("q"), up("k"), up("v"), f32(dO), variant=c["variant"], beta=beta,
                       lam=c["lam"], eps=1e-6, window=c["window"], beta_t=up("beta_t"),
                       k_prev=up("k_prev"),
                       S0=to_dev(torch, inp["S0"], torch.float32) if "S0" in inp else None,
                       dS_L=f32(dS_L), dk_last=f32(dk_last), same_step=c["same_step"])
    torch.cuda.synchronize()
    ref = fo.falcon_backward(c["variant"], inp["q"], inp["k"], inp["v"], dO, beta=beta,
                             lam=c["lam"], eps=1e-6, window=c["window"],
                             beta_t=inp.get("beta_t"), k_prev=inp.get("k_prev"),
                             S0=inp.get("S0"), same_step=c["same_step"], dS_L=dS_L,
                             dk_last=dk_last)
    assert set(got) == set(ref)
    errs = {}
    for n in ref:
        a = np.asarray(got[n].cpu().numpy(), dtype=np.float64)
        b = np.asarray(ref[n], dtype=np.float64)
        errs[n] = float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))
    print("  backward " + " ".join("%s %.2e" % kv for kv in errs.items()), flush=True)
    assert max(errs.values()) <= TOL_FP32_MATH, errs


def _draw_decode(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = int(rng.integers(0, 6))
        windowed = variant in (fo.FALCON_3, fo.FALCON_3A)
        window = int(rng.integers(1, 9)) if windowed else 1
        # the windowed decode step takes a scalar gain
        kinds = ["scalar"] if windowed else (["scalar", "token", "channel"]
                                             if variant in (fo.FALCON_2, fo.FALCON_2A) else ["scalar", "token"])
        out.append(dict(id=i, variant=variant, window=window, gains=str(rng.choice(kinds)),
                        same_step=bool(rng.random() < 0.3), dtype=str(rng.choice(["bf16", "f32"])),
                        dk=int(rng.choice(DIMS)), dv=int(rng.choice(DIMS)),
                        lam=float(rng.choice([0.0, 0.01, 0.3])), beta=float(rng.uniform(0.3, 1.0)),
                        seed=int(rng.integers(0, 1 << 30))))
    return out


DEC_CASES = _draw_decode(40, 20261206)


@pytest.mark.parametrize("c", DEC_CASES, ids=[str(c["id"]) for c in DEC_CASES])
def test_random_decode(c):
    """Five decode steps in place (state, carried key, window history) against the
    oracle's decode step by step."""
    from weight_recurrent_memory_amd.inputs import decode_inputs, to_bf16_values
    steps, N, H, dk, dv, B = 5, 3, 2, c["dk"], c["dv"], c["window"]
    d = decode_inputs(N, H, dk, dv, seed=c["seed"], steps=steps, s_std=0.2, dtype=c["dtype"],
                      beta_per_channel=c["gains"] == "channel", history=B - 1)
    if c["gains"] == "token":
        bt = np.random.default_rng(c["seed"] + 7).uniform(0.2, 1.0, (steps, N, H)).astype(np.float32)
        d["beta_t"] = to_bf16_values(bt) if c["dtype"] == "bf16" else bt
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    S = to_dev(torch, d["S"], torch.float32)
    kp = None if c["same_step"] else to_dev(torch, d["k_prev"], dt)
    xh = to_dev(torch, d["x_hist"], dt) if B > 1 else None
    yh = to_dev(torch, d["y_hist"], dt) if B > 1 else None
    S_r = d["S"].astype(np.float64)
    kp_r = d["k_prev"].astype(np.float64)
    xh_r = d["x_hist"].astype(np.float64) if B > 1 else None
    yh_r = d["y_hist"].astype(np.float64) if B > 1 else None
    print("decode case %d: v%d B%d %s %s %s dk%d dv%d lam %.2f" % (
        c["id"], c["variant"], B, c["gains"], "same" if c["same_step"] else "prefix", c["dtype"],
        dk, dv, c["lam"]), flush=True)
    beta = c["beta"] if c["gains"] == "scalar" else None
    for s_ in range(steps):
        q, k, v = (to_dev(torch, d[n][s_], dt) for n in ("q", "k", "v"))
        bt = to_dev(torch, d["beta_t"][s_], dt) if "beta_t" in d else None
        o = fw.decode_step(S, kp, q, k, v, variant=c["variant"], beta=beta, lam=c["lam"], eps=1e-6,
                           beta_t=bt, window=B, x_hist=xh, y_hist=yh, same_step=c["same_step"])
        if c["variant"] in (fo.FALCON_3, fo.FALCON_3A):   # window 1: no history
            o_r, S_r, kp_r, xh_r, yh_r = fo.falcon_decode_step_window(
                c["variant"], B, S_r, kp_r, xh_r, yh_r, d["q"][s_], d["k"][s_], d["v"][s_],
                beta=beta, lam=c["lam"], eps=1e-6, same_step=c["same_step"])
            if B == 1:
                xh_r = yh_r = None
        else:
            o_r, S_r, kp_r = fo.falcon_decode_step(
                c["variant"], S_r, kp_r, d["q"][s_], d["k"][s_], d["v"][s_], beta=beta,
                lam=c["lam"], eps=1e-6, beta_t=d["beta_t"][s_] if "beta_t" in d else None,
                same_step=c["same_step"])
        torch.cuda.synchronize()
        err, zok = token_normwise_err(o.cpu().numpy(), o_r)
        assert zok and err <= TOL_FP32_MATH, (s_, err)
    serr = state_err(S.cpu().numpy(), S_r)
    print("  decode S err %.3e" % serr, flush=True)
    assert serr <= TOL_FP32_MATH
    if kp is not None:
        np.testing.assert_array_equal(kp.float().cpu().numpy(), kp_r)
    if B > 1:
        np.testing.assert_array_equal(xh.float().cpu().numpy(), xh_r)
        np.testing.assert_array_equal(yh.float().cpu().numpy(), yh_r)

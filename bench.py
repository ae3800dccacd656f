#!/usr/bin/env python3
"""Throughput of the Falcon chunk-parallel forward (and the decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]

A step is one falcon_fwd_chunk call (Falcon-1, the regression update with its
triangular solve: staging, Gram/q.x products, solve, readout and state carry)
over one batch of the headline workload: 8 sequences x 12 heads x 2048 tokens,
dk = dv = 64, chunk 64, bf16 q/k/v (q, k L2-normalized), beta = 0.5,
lambda = 0.01, eps = 1e-6.  Inputs are resident in HBM before the timed region;
launch time is measured with HIP events on the stream the kernel runs on.

Prints one JSON line.  Besides the contract fields it carries
  timing        mean, median and minimum of the timed calls
  roofline      the chunk kernel against HBM bandwidth (algorithmic bytes)
  roofline_mfma the sliding-window forward (Falcon-3, 4 x 16 x 8192, d = 128)
                against the bf16 matrix-core peak, in model flops
  cpu_baseline  the fp64 oracle on the host cores, same workload
  secondary     the other workloads: Falcon-1A, per-channel Falcon-2, windowed
                Falcon-3/3A at d = 128, the backward of the headline workload,
                the decode step (warm, and cold: the state evicted from every
                cache before each step), a copy kernel for attainable bandwidth,
                and model-FLOP utilization.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Falcon chunk fwd tokens/s + MFMA util; decode-step state HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "chunk_traffic.json")
CHUNK_SOURCES = [os.path.join(ROOT, "weight_recurrent_memory_amd", "csrc", f)
                 for f in ("falcon_chunk_wy.hip", "falcon_exact.h", "falcon_mma.h", "falcon_device.h")]
PROFILE_MFMA = os.path.join(ROOT, "profiles", "window_mfma_counters.json")
WINDOW_SOURCES = [os.path.join(ROOT, "weight_recurrent_memory_amd", "csrc", f)
                  for f in ("falcon_chunk_wyb.hip", "falcon_exact.h", "falcon_mma.h", "falcon_device.h")]
HEADLINE_KERNEL = "chunk_wy_kernel<64,true>"
HEADLINE_KERNEL_CHUNK = 32
WINDOW_KERNEL = "chunk_wyb_kernel<128,true,4,true> + wyb_state_kernel<128,4>"


def algorithmic_bytes(batch, heads, L, dk, dv, beta_channel=False, elem=2):
    """Each input read once, o (fp32) written once."""
    per_tok = (2 * dk + dv) * elem + dv * 4 + (dv * elem if beta_channel else 0)
    return batch * heads * L * per_tok


def model_flops_per_head_token(regression, d, C, B=1):
    """Canonical single-level chunk-form model flops per head-token (2 flops per
    multiply-add; triangular products counted on their non-zero part; no
    split-bf16 compensation passes).  Per chunk of C steps with nx = C + B - 1
    keys and C*B window unknowns:
      q.x          C(C+1)/2 + C(B-1) dot products of length d
      S0 q         d^2 per token
      readout P Z  same count as q.x, times d
      carry Z^T X  nx d^2
      regression only: Gram nx(nx-1)/2 dot products, S0 x  nx d^2,
                       triangular solve (CB)(CB-1)/2 times d
    Gives 40,960 (Falcon-1, d = C = 64), 24,704 (Falcon-1A) and 258,956 / 85,248
    (Falcon-3 / 3A, d = 128, C = 64, B = 4)."""
    nx = C + B - 1
    tri_p = C * (C + 1) / 2 + C * (B - 1)
    f = 2 * tri_p * d / C + 2 * d * d + 2 * tri_p * d / C + 2 * nx * d * d / C
    if regression:
        tri_g = nx * (nx - 1) / 2
        tri_s = (C * B) * (C * B - 1) / 2
        f += 2 * tri_g * d / C + 2 * nx * d * d / C + 2 * tri_s * d / C
    return f


def _source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per launch from rocprofv3 counters, if they were taken on the
    current chunk kernel source (else None)."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != _source_hash(CHUNK_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def _mfma_counters():
    """Matrix-core counters of the sliding-window kernel (rocprofv3 --pmc), if they
    were taken on the current kernel source (else None)."""
    try:
        with open(PROFILE_MFMA) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != _source_hash(WINDOW_SOURCES):
        return None
    return rec


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="profiling aid: run only this leg "
                    "(headline|falcon1a|percol|window|masked|backward|decode|copy)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Falcon state update has no cross-GPU "
              "communication in this build; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import weight_recurrent_memory_amd as fw
    from weight_recurrent_memory_amd.inputs import WORKLOADS, decode_inputs, seq_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fw.load_library()

    def up(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(dt)

    def time_calls(fn, steps, warmup, between=None, stats=None):
        """Seconds per call over `steps` timed calls (HIP events on the stream the
        library launches on, torch's current stream).  An event is recorded
        between consecutive calls, so `stats` (a dict) also receives the median and
        minimum single-call times.  `between` runs outside the events before each
        call (the cache-flushing leg); then the per-call times are the only
        measure and the mean is taken over them."""
        for _ in range(warmup):
            if between is not None:
                between()
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        if between is None:
            ev[0].record(s)
            for i in range(steps):
                fn()
                ev[i + 1].record(s)
            torch.cuda.synchronize()
            per = [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(steps)]
            mean = ev[0].elapsed_time(ev[steps]) / 1e3 / steps
        else:
            ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            for i in range(steps):
                between()
                ev[i].record(s)
                fn()
                ev2[i].record(s)
            torch.cuda.synchronize()
            per = [ev[i].elapsed_time(ev2[i]) / 1e3 for i in range(steps)]
            mean = sum(per) / steps
        if stats is not None:
            srt = sorted(per)
            stats.update(median_s=srt[steps // 2] if steps % 2 else 0.5 * (srt[steps // 2 - 1] + srt[steps // 2]),
                         min_s=srt[0], mean_s=mean, calls=steps)
        return mean

    def seq_leg(name, variant, steps, warmup, window=1, stats=None):
        cfg = WORKLOADS[name]
        B, H, L, dk, dv = cfg["shape"]
        per_ch = bool(cfg.get("beta_per_channel"))
        inp = seq_inputs(B, H, L, dk, dv, seed=cfg["seed"], dtype="bf16",
                         beta_per_channel=per_ch)
        q, k, v = (up(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
        bt = up(inp["beta_t"], torch.bfloat16) if per_ch else None
        out = torch.empty((B, H, L, dv), device=dev, dtype=torch.float32)
        beta = cfg["beta"] if cfg["beta"] is not None else 0.0
        fn = lambda: fw.fwd_chunk(q, k, v, variant=variant, beta=beta, lam=cfg["lam"],
                                  eps=cfg["eps"], chunk=cfg["chunk"], window=window,
                                  beta_t=bt, out=out)
        sec = time_calls(fn, steps, warmup, stats=stats)
        nbytes = algorithmic_bytes(B, H, L, dk, dv, beta_channel=per_ch)
        return dict(sec=sec, tokens=B * L, head_tokens=B * H * L, bytes=nbytes, d=dk,
                    chunk=cfg["chunk"], inp=inp, cfg=cfg, out=out)

    out = {}
    # ---------------- headline: Falcon-1 chunk forward, 8 x 12 x 2048 x 64 ----------------
    head_name = "chunk_8x12x2048x64"
    if args.only in (None, "headline"):
        st = {}
        h = seq_leg(head_name, fw.FALCON_1, args.steps, args.warmup, stats=st)
        sec = h["sec"]
        value = h["tokens"] / sec
        achieved = h["bytes"] / sec / 1e9
        mflops = model_flops_per_head_token(True, 64, 64) * h["head_tokens"]
        traffic = _traffic()
        out.update({
            "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": sec * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": head_name, "variant": "falcon1", "batch": 8, "heads": 12,
                       "seq_len": 2048, "dk": 64, "dv": 64, "chunk": 64,
                       "kernel_chunk": HEADLINE_KERNEL_CHUNK, "beta": 0.5,
                       "lambda": 0.01, "eps": 1e-6, "parallelism": "single-gpu"},
            "timing": {"calls": st["calls"], "mean_us": st["mean_s"] * 1e6,
                       "median_us": st["median_s"] * 1e6, "min_us": st["min_s"] * 1e6},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": traffic,
                         "kernel": HEADLINE_KERNEL,
                         "algorithmic_bytes_per_launch": h["bytes"],
                         "avg_launch_us": sec * 1e6},
            "mfma_model_util": {"model_gflop_per_call": mflops / 1e9,
                                "model_tflops": mflops / sec / 1e12,
                                "frac_of_bf16_peak": mflops / sec / 1e12 / BF16_PEAK_TFLOPS,
                                "flop_formula": "canonical single-level chunk form, C = 64"},
        })
        head_inp = h["inp"]
        head_o = h["out"].cpu().numpy()        # outputs of the last timed call
    else:
        head_inp = None

    # ---------------- secondary workloads ----------------
    sec_out = {}
    if not args.no_secondary:
        legs = [("falcon1a", head_name, fw.FALCON_1A, 1),
                ("percol", "chunk_percol_8x12x4096x64", fw.FALCON_2, 1),
                ("window_falcon3", "chunk_window4_4x16x8192x128", fw.FALCON_3, 4),
                ("window_falcon3a", "chunk_window4_4x16x8192x128", fw.FALCON_3A, 4)]
        names = {fw.FALCON_1A: "falcon1a", fw.FALCON_2: "falcon2", fw.FALCON_3: "falcon3",
                 fw.FALCON_3A: "falcon3a"}
        for key, name, variant, win in legs:
            if args.only not in (None, key.split("_")[0]):
                continue
            st = {}
            r = seq_leg(name, variant, 20, 3, window=win, stats=st)
            regression = variant in (fw.FALCON_2, fw.FALCON_3)
            fl = model_flops_per_head_token(regression, r["d"], r["chunk"], win) * r["head_tokens"]
            sec_out[key] = {"workload": name, "variant": names[variant],
                            "tokens_per_s": r["tokens"] / r["sec"], "ms_per_call": r["sec"] * 1e3,
                            "median_ms": st["median_s"] * 1e3, "min_ms": st["min_s"] * 1e3,
                            "hbm_gbs": r["bytes"] / r["sec"] / 1e9,
                            "hbm_frac": r["bytes"] / r["sec"] / 1e9 / HBM_PEAK_GBS,
                            "model_gflop_per_call": fl / 1e9,
                            "model_tflops": fl / r["sec"] / 1e12,
                            "mfma_model_frac": fl / r["sec"] / 1e12 / BF16_PEAK_TFLOPS}
            if key == "window_falcon3":
                # the matrix-core target of the chunk-parallel forward: Falcon-3 at
                # L = 8192, d = 128 (model flops of the canonical C = 64 form)
                achieved_tf = fl / r["sec"] / 1e12
                counters = _mfma_counters()
                out["roofline_mfma"] = {
                    "bound": "mfma", "achieved": achieved_tf, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved_tf / BF16_PEAK_TFLOPS,
                    "workload": name, "variant": "falcon3", "window": 4,
                    "model_gflop_per_call": fl / 1e9, "avg_launch_us": r["sec"] * 1e6,
                    "kernel": WINDOW_KERNEL,
                    "mfma_busy_frac": counters.get("mfma_busy_frac") if counters else None,
                    "issued_tflops": counters.get("issued_tflops") if counters else None,
                    "counters_source": counters.get("source") if counters else None}
            del r
            torch.cuda.empty_cache()
        if args.only in (None, "masked"):
            # short sequences: the masked-parallel form (one masked system per call of
            # 64 steps; falcon_fwd_chunk routes such calls to the same kernel)
            cfg = WORKLOADS["masked_256x12x64x64"]
            B, H, L, dk, dv = cfg["shape"]
            inp = seq_inputs(B, H, L, dk, dv, seed=cfg["seed"], dtype="bf16")
            q, k, v = (up(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
            o = torch.empty((B, H, L, dv), device=dev, dtype=torch.float32)
            kw = dict(variant=fw.FALCON_1, beta=cfg["beta"], lam=cfg["lam"], eps=cfg["eps"], out=o)
            st = {}
            sec = time_calls(lambda: fw.fwd_masked(q, k, v, **kw), 20, 3, stats=st)
            nbytes = algorithmic_bytes(B, H, L, dk, dv)
            sec_out["masked"] = {"workload": "masked_256x12x64x64", "variant": "falcon1",
                                 "kernel": "masked_wy_kernel<64,true,false,false>",
                                 "ms_per_call": sec * 1e3, "median_ms": st["median_s"] * 1e3,
                                 "tokens_per_s": B * L / sec,
                                 "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS}
            del q, k, v, o
            torch.cuda.empty_cache()
        if args.only in (None, "backward"):
            # gradients of the headline workload: q, k, v bf16 and dO fp32 read, dq, dk,
            # dv fp32 written (the per-chunk state checkpoints in the workspace are
            # extra traffic, not counted)
            cfg = WORKLOADS[head_name]
            B, H, L, dk, dv = cfg["shape"]
            inp = head_inp if head_inp is not None else seq_inputs(B, H, L, dk, dv, seed=cfg["seed"],
                                                                  dtype="bf16")
            q, k, v = (up(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
            dO = torch.randn((B, H, L, dv), device=dev, dtype=torch.float32,
                             generator=torch.Generator(device=dev).manual_seed(7))
            fn = lambda: fw.bwd_chunk(q, k, v, dO, variant=fw.FALCON_1, beta=cfg["beta"],
                                      lam=cfg["lam"], eps=cfg["eps"])
            st = {}
            sec = time_calls(fn, 10, 2, stats=st)
            nbytes = B * H * L * ((2 * dk + dv) * 2 + dv * 4 + (2 * dk + dv) * 4)
            sec_out["backward"] = {"workload": head_name, "variant": "falcon1",
                                   "ms_per_call": sec * 1e3, "median_ms": st["median_s"] * 1e3,
                                   "tokens_per_s": B * L / sec,
                                   "hbm_gbs": nbytes / sec / 1e9,
                                   "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes": nbytes}
            # the sliding-window backward (window 4) on the same tokens
            fn = lambda: fw.bwd_chunk(q, k, v, dO, variant=fw.FALCON_3, beta=cfg["beta"],
                                      lam=cfg["lam"], eps=cfg["eps"], window=4)
            sec = time_calls(fn, 4, 1)
            sec_out["backward_window4"] = {"workload": head_name, "variant": "falcon3",
                                           "window": 4, "ms_per_call": sec * 1e3,
                                           "tokens_per_s": B * L / sec,
                                           "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS}
            del q, k, v, dO
            torch.cuda.empty_cache()
        if args.only in (None, "decode"):
            cfg = WORKLOADS["decode_512x12x64"]
            N, H, dk, dv = cfg["shape"]
            pool = 8
            d = decode_inputs(N, H, dk, dv, seed=cfg["seed"], steps=pool)
            S = up(d["S"], torch.float32)
            kp = up(d["k_prev"], torch.bfloat16)
            qs, ks, vs = (up(d[n], torch.bfloat16) for n in ("q", "k", "v"))
            o = torch.empty((N, H, dv), device=dev, dtype=torch.float32)
            it = [0]

            def step():
                p = it[0] % pool
                it[0] += 1
                fw.decode_step(S, kp, qs[p], ks[p], vs[p], variant=fw.FALCON_1, beta=cfg["beta"],
                               lam=cfg["lam"], eps=cfg["eps"], out=o)
            state_bytes = 2 * N * H * dv * dk * 4
            io_bytes = N * H * (3 * dk * 2 + dv * 2 + dv * 4 + dk * 2)  # k_prev r/w, q, k, v, o
            nb = state_bytes + io_bytes
            # warm: back-to-back steps, the 100.7 MB state can stay in the 256 MB
            # Infinity Cache (MALL) between steps
            st = {}
            sec = time_calls(step, args.decode_steps, 20, stats=st)
            # cold: a 1 GiB buffer is written before every timed step (outside its
            # events), which evicts the state from the MALL and the L2s; the step's
            # own time is then what a state that lives in HBM costs
            scratch = torch.empty(1 << 28, device=dev, dtype=torch.float32)
            stc = {}
            sec_cold = time_calls(step, 200, 5, between=lambda: scratch.fill_(1.0), stats=stc)
            # graph: a serving loop's form, `pool` steps captured once in a HIP graph
            # and replayed, so the host launch path leaves the step.  Warm: steps
            # back to back.  Cold: a graph with the 1 GiB fill before every step and
            # a graph of the fills alone; the per-step difference is the step with
            # its state evicted (the fill and the step run one after the other on
            # one stream).
            outs = torch.empty((pool, N, H, dv), device=dev, dtype=torch.float32)

            def capture(with_step, with_fill):
                g = torch.cuda.CUDAGraph()
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    for p in range(pool):
                        if with_fill:
                            scratch.fill_(1.0)
                        if with_step:
                            fw.decode_step(S, kp, qs[p], ks[p], vs[p], variant=fw.FALCON_1,
                                           beta=cfg["beta"], lam=cfg["lam"], eps=cfg["eps"],
                                           out=outs[p])
                return g

            def replay_time(g, reps):
                for _ in range(2):
                    g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / 1e3 / (reps * pool)

            reps = max(1, args.decode_steps // pool)
            g_warm = capture(True, False)
            sec_gw = replay_time(g_warm, reps)
            g_cold, g_fill = capture(True, True), capture(False, True)
            creps = max(1, 200 // pool)
            sec_gc = replay_time(g_cold, creps) - replay_time(g_fill, creps)
            del g_warm, g_cold, g_fill, scratch, outs
            sec_out["decode"] = {"workload": "decode_512x12x64", "variant": "falcon1",
                                 "bytes_per_step": nb,
                                 "warm": {"steps": args.decode_steps, "us_per_step": sec * 1e6,
                                          "median_us": st["median_s"] * 1e6,
                                          "state_gbs": state_bytes / sec / 1e9,
                                          "total_gbs": nb / sec / 1e9,
                                          "frac_of_peak": nb / sec / 1e9 / HBM_PEAK_GBS},
                                 "cold": {"steps": 200, "flush_bytes": 1 << 30,
                                          "us_per_step": sec_cold * 1e6,
                                          "median_us": stc["median_s"] * 1e6,
                                          "total_gbs": nb / stc["median_s"] / 1e9,
                                          "hbm_frac": nb / stc["median_s"] / 1e9 / HBM_PEAK_GBS},
                                 "graph": {"steps_per_graph": pool,
                                           "warm_us_per_step": sec_gw * 1e6,
                                           "warm_total_gbs": nb / sec_gw / 1e9,
                                           "cold_us_per_step": sec_gc * 1e6,
                                           "cold_total_gbs": nb / sec_gc / 1e9,
                                           "cold_hbm_frac": nb / sec_gc / 1e9 / HBM_PEAK_GBS}}
            del S, qs, ks, vs
            torch.cuda.empty_cache()
        if args.only in (None, "copy"):
            # attainable bandwidth: device-to-device copy of 1 GiB (also the known-size
            # kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters)
            a = torch.empty(1 << 28, device=dev, dtype=torch.float32)
            b = torch.empty_like(a)
            sec = time_calls(lambda: b.copy_(a), 20, 3)
            sec_out["copy_1GiB"] = {"gbs": 2 * a.numel() * 4 / sec / 1e9}
            del a, b
    if sec_out:
        out["secondary"] = sec_out
    # the attainable bandwidth of this GPU (the same run's 1 GiB copy) beside the
    # data-sheet peak: each HBM-bound figure as a fraction of both
    copy_gbs = sec_out.get("copy_1GiB", {}).get("gbs")
    if copy_gbs:
        if "roofline" in out:
            out["roofline"]["attainable_gbs"] = copy_gbs
            out["roofline"]["attainable_frac"] = out["roofline"]["achieved"] / copy_gbs
        for leg in sec_out.values():
            if isinstance(leg, dict) and "hbm_gbs" in leg:
                leg["attainable_frac"] = leg["hbm_gbs"] / copy_gbs
        if "decode" in sec_out:
            nb = sec_out["decode"]["bytes_per_step"]
            sec_out["decode"]["cold"]["attainable_frac"] = nb / (sec_out["decode"]["cold"]["median_us"] * 1e-6) / 1e9 / copy_gbs
            sec_out["decode"]["graph"]["cold_attainable_frac"] = sec_out["decode"]["graph"]["cold_total_gbs"] / copy_gbs

    # ---------------- fp64 oracle on the host cores ----------------
    if not args.no_cpu_baseline and args.only is None and head_inp is not None:
        from threadpoolctl import threadpool_info
        from oracle import falcon_oracle as fo
        cfg = WORKLOADS[head_name]
        t = time.perf_counter()
        o_ref = fo.falcon_recurrence(fw.FALCON_1, head_inp["q"], head_inp["k"], head_inp["v"],
                                     beta=cfg["beta"], lam=cfg["lam"], eps=cfg["eps"])[0]
        cpu_sec = time.perf_counter() - t
        # parity of the timed headline call against the oracle (outside the timing):
        # per-token normwise error, max over every (batch, head, token)
        ref_inf = np.max(np.abs(o_ref), axis=-1)
        diff_inf = np.max(np.abs(head_o.astype(np.float64) - o_ref), axis=-1)
        nz = ref_inf > 0
        out["parity"] = {"o_token_normwise_err": float(np.max(diff_inf[nz] / ref_inf[nz])),
                         "zero_rows_exact": bool(np.all(diff_inf[~nz] == 0)),
                         "tolerance": 2e-3, "against": "fp64 oracle, whole headline batch"}
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": 8 * 2048 / cpu_sec, "unit": "tokens/s",
                               "cores": threads, "kind": "oracle",
                               "sample": "the whole headline batch (8 x 12 x 2048 tokens, "
                                         "Falcon-1, fp64 numpy recurrence), %.1f s" % cpu_sec,
                               "cpu_model": _cpu_model(),
                               "host_cpus": len(os.sched_getaffinity(0))}
    print(json.dumps(out))


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of exact tiled attention (forward + backward) on one MI355X.

One step = fa_fwd, then the three backward kernels (row term, dK/dV pass,
dQ pass) on one batch of the 7B-layer attention shape at 8K: bf16, causal,
batch 1, 32 heads, seqlen 8192, head_dim 128, Q/K/V ~ N(0,1)*0.5 and
dO ~ N(0,1) from the seeded generator.  Inputs are resident in HBM before
the timed region.  HIP events on the launch stream bracket every kernel of
every timed step; the wall clock around the K steps gives ms_per_step.

value = algorithmic FLOPs of the step / step time, with forward FLOPs
4*d*P*H and backward 10*d*P*H (P = visible (query, key) pairs per head,
N(N+1)/2 for causal), i.e. two and five d-long contractions per visible
pair.  The roofline object describes the kernel with the largest share of
the step.  The CPU baseline is the fp64 oracle timed on a bounded sample of
the same workload (one head, all rows, forward + backward).

An object "dropout" times the same step with dropout_p = 0.1 (Philox keep
decisions drawn inside the forward, dK/dV and dQ kernels), against the same
algorithmic FLOP count.

A second object, "decode", times the KV-cache decode path on its own
workload (one new token per sequence, GQA 32/8 heads, ragged caches of
16K-32K tokens, d 128, bf16): bytes of the valid K/V cache rows read (plus
q, o and lse) per call / call time, against the 8 TB/s HBM peak.

An object "fp8" times the FP8 forward (fa_fwd_fp8: E4M3 Q, K, V with
per-tensor scales, P rounded to E4M3, bf16 O) on the 8K shape, against the
dense fp8 matrix-core peak.

An object "workloads" times forward and backward (median, minimum and mean
of HIP-event times per call) on the other named workloads: the d=64 causal
batch (4 x 2048, 16 heads), the 32K GQA shape (32 query heads over 8 kv
heads) and the packed sliding-window batch (2 sequences of 8K-16K, window
4096).  "dq_path" names the backward's dQ path ("separate": the deterministic
dQ pass); "atomic_dq" times the opt-in atomic-dQ backward on the 8K and 32K
shapes beside it.  "measured_peak" is the matrix-core rate and shader clock a
calibration kernel of independent MFMA chains sustains on this GPU, the
second denominator next to the published peak; "env" records the software
versions and the GPU.

Prints ONE JSON line.  Only one GPU: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2    # 256 CUs x 8192 dense fp8 FLOP/clk/CU x 2.4 GHz
FP8_WORKLOAD = "fp8_causal_b1_h32_n8192_d128"
WORKLOAD = "bf16_causal_b1_h32_n8192_d128"
METRIC = "attention fwd+bwd TFLOP/s and % MFMA bf16 peak, seq 8192 d128 causal, 1 GPU"
def visible_pairs(p) -> int:
    """Number of visible (query, key) pairs summed over sequences (one head)."""
    lens = p.seqlens if p.seqlens is not None else [p.seqlen_q] * p.batch
    lens_k = p.seqlens if p.seqlens is not None else [p.seqlen_k] * p.batch
    total = 0
    for lq, lk in zip(lens, lens_k):
        i = np.arange(lq, dtype=np.int64)
        pos = i + (lk - lq)
        hi = np.full(lq, lk - 1, dtype=np.int64)
        if p.causal:
            hi = np.minimum(hi, pos)
        if p.window_right >= 0:
            hi = np.minimum(hi, pos + p.window_right)
        lo = np.maximum(0, pos - p.window_left) if p.window_left >= 0 else np.zeros(lq, dtype=np.int64)
        total += int(np.clip(hi - lo + 1, 0, None).sum())
    return total


CPU_SAMPLE_HEADS = 8
# the other named workloads (timed steps each)
OTHER_WORKLOADS = (("bf16_causal_b4_h16_n2048_d64", 20), ("bf16_causal_gqa_b1_h32kv8_n32768_d128", 5),
                   ("fp16_causal_window4096_varlen_b2_h16_d128", 10))
DECODE_WORKLOAD = "bf16_decode_gqa_b8_h32kv8_q1_cache32768_d128"


def decode_bytes(p) -> float:
    """Algorithmic HBM bytes of one decode call: every valid K and V cache row
    of every kv head read once, q read, o written (16-bit), lse written."""
    d = p.head_dim
    kv = 2.0 * sum(p.cache_lens) * p.kv_heads * d * 2
    qo = 2.0 * p.batch * p.seqlen_q * p.heads * d * 2
    return kv + qo + 4.0 * p.batch * p.heads * p.seqlen_q


def bench_decode(fa, synth, torch, steps: int, warmup: int, measured_traffic):
    dev = torch.device("cuda:0")
    p = synth.decode_workload(DECODE_WORKLOAD)
    q, kc, vc = p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev)
    cs = p.cache_seqlens().to(dev)
    plan = fa.DecodePlan(q, kc, vc, cs, causal=p.causal, softmax_scale=p.scale)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(plan.stream)
    for i in range(steps):
        plan.run()
        ev[i + 1].record(plan.stream)
    torch.cuda.synchronize()
    all_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = float(np.mean(all_ms))
    gbs = decode_bytes(p) / (ms / 1e3) / 1e9
    return {"workload": DECODE_WORKLOAD, "ms_per_call": round(ms, 4), "ms_stats": stats(all_ms), "bound": "hbm",
            "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "splits": plan.nsplit,
            "bytes_per_call": int(decode_bytes(p)),
            "traffic": measured_traffic("decode", DECODE_WORKLOAD),
            "tokens_per_s": round(p.batch * p.seqlen_q / (ms / 1e3), 1)}


def bench_fp8(fa, synth, torch, steps: int, warmup: int, measured_traffic):
    dev = torch.device("cuda:0")
    p = synth.workload(FP8_WORKLOAD)
    q, k, v = p.q.to(dev), p.k.to(dev), p.v.to(dev)
    plan = fa.Fp8Plan(q, k, v, p.descale_q, p.descale_k, p.descale_v, causal=p.causal,
                      window_size=(p.window_left, p.window_right), softmax_scale=p.scale)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(plan.stream)
    for i in range(steps):
        plan.run()
        ev[i + 1].record(plan.stream)
    torch.cuda.synchronize()
    all_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = float(np.mean(all_ms))
    flops = 4.0 * p.head_dim * visible_pairs(p) * p.heads
    tf = flops / (ms / 1e3) / 1e12
    return {"workload": FP8_WORKLOAD, "ms": round(ms, 4), "ms_stats": stats(all_ms), "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "traffic": measured_traffic("fwd_fp8", FP8_WORKLOAD)}


def stats(xs):
    xs = [float(x) for x in xs]
    return {"median": round(float(np.median(xs)), 4), "min": round(float(np.min(xs)), 4),
            "mean": round(float(np.mean(xs)), 4)}


def make_plan(fa, p, dev, deterministic=True):
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    cu = p.cu_seqlens()
    cu = cu.to(dev) if cu is not None else None
    return fa.Plan(q, k, v, do, causal=p.causal, window_size=(p.window_left, p.window_right),
                   softmax_scale=p.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
                   max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k, deterministic=deterministic)


def time_plan(plan, steps: int, warmup: int, torch):
    """HIP-event times (ms) of fa_fwd and of the three backward stages, per
    step, on the plan's stream."""
    calls = [plan.fwd, lambda: plan.bwd_stage(0), lambda: plan.bwd_stage(1), lambda: plan.bwd_stage(2)]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(plan.stream)
        for i, c in enumerate(calls):
            c()
            ev[s][i + 1].record(plan.stream)
    torch.cuda.synchronize()
    per = [[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(calls))] for s in range(steps)]
    return {"fwd": [x[0] for x in per], "bwd": [x[1] + x[2] + x[3] for x in per],
            "stages": [[x[i] for x in per] for i in range(1, 4)]}


def note(msg):
    """One progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload_entry(p, t, peak_meas):
    """fwd / bwd times and rates of one workload from time_plan's result."""
    pairs = visible_pairs(p)
    fl = {"fwd": 4.0 * p.head_dim * pairs * p.heads, "bwd": 10.0 * p.head_dim * pairs * p.heads}
    out = {"dtype": p.dtype, "batch": p.batch, "heads": p.heads, "kv_heads": p.kv_heads,
           "seq_len": p.seqlen_q, "head_dim": p.head_dim, "causal": bool(p.causal),
           "window": [p.window_left, p.window_right], "visible_pairs_per_head": pairs}
    if p.seqlens is not None:
        out["seqlens"] = list(p.seqlens)
    for ph in ("fwd", "bwd"):
        st = stats(t[ph])
        tf = fl[ph] / (st["median"] / 1e3) / 1e12
        out[ph] = {"ms": st, "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                   "frac_measured_peak": round(tf / peak_meas, 4) if peak_meas else None}
    return out


def env_info(torch):
    info = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as fh:
            info["rocm"] = fh.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=60)
        info["hipcc"] = next((l.strip() for l in r.stdout.splitlines() if l.startswith("HIP version")), None)
    except (OSError, subprocess.SubprocessError):
        info["hipcc"] = None
    prop = torch.cuda.get_device_properties(0)
    info["gpu"] = torch.cuda.get_device_name(0)
    info["arch"] = getattr(prop, "gcnArchName", None)
    info["compute_units"] = prop.multi_processor_count
    return info


def cpu_baseline(p, threads: int):
    """fp64 oracle, forward + backward for the first CPU_SAMPLE_HEADS kv heads
    (with their query heads) of batch 0 of the workload."""
    import oracle
    oracle.build(force=False)
    pairs = visible_pairs(p)
    d = p.head_dim
    nh = CPU_SAMPLE_HEADS * (p.heads // p.kv_heads)
    flops = (4 + 10) * d * pairs * nh / p.batch
    q, k, v, do = (t[:1].double().numpy() for t in (p.q, p.k, p.v, p.do))
    t0 = time.perf_counter()
    oracle.attention_bwd(q, k, v, do, scale=p.scale, causal=p.causal,
                         window=(p.window_left, p.window_right),
                         kv_heads=list(range(CPU_SAMPLE_HEADS)), threads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{WORKLOAD}: {nh} of {p.heads} heads of batch 0, all {p.seqlen_q} rows, "
                      f"forward + backward in fp64 ({flops / 1e9:.1f} GFLOP)"}


def bench_dropout(fa, p, q, k, v, do, steps: int, warmup: int, flops: float, torch):
    plan = fa.Plan(q, k, v, do, causal=p.causal, window_size=(p.window_left, p.window_right),
                   softmax_scale=p.scale, dropout_p=0.1, dropout_seed=20240601)
    calls = [plan.fwd, lambda: plan.bwd_stage(0), lambda: plan.bwd_stage(1), lambda: plan.bwd_stage(2)]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(plan.stream)
        calls[0]()
        ev[s][1].record(plan.stream)
        for c in calls[1:]:
            c()
        ev[s][2].record(plan.stream)
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    step_ms = fwd_ms + bwd_ms
    return {"dropout_p": 0.1, "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "step_ms": round(step_ms, 4), "tflops": round(flops / (step_ms / 1e3) / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the KV-cache decode measurement")
    ap.add_argument("--no-dropout", action="store_true", help="skip the dropout step measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward measurement")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (default min(16, cores))")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other named workloads")
    ap.add_argument("--no-peak", action="store_true", help="skip the matrix-core calibration")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import synth
    import exact_tiled_attention_10_amd as fa
    from exact_tiled_attention_10_amd.profile_run import measured_traffic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    note(f"main step: {WORKLOAD}, {args.steps} timed steps after {args.warmup}")
    p = synth.workload(WORKLOAD)
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    plan = fa.Plan(q, k, v, do, causal=p.causal, window_size=(p.window_left, p.window_right),
                   softmax_scale=p.scale)
    stream = plan.stream
    names = ["fwd", "bwd_rowdot", "bwd_dkdv", "bwd_dq"]
    calls = [plan.fwd, lambda: plan.bwd_stage(0), lambda: plan.bwd_stage(1), lambda: plan.bwd_stage(2)]

    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev = events[s]
        ev[0].record(stream)
        for i, c in enumerate(calls):
            c()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    kern_all = {n: [events[s][i].elapsed_time(events[s][i + 1]) for s in range(K)] for i, n in enumerate(names)}
    kern_ms = {n: float(np.mean(v)) for n, v in kern_all.items()}
    ev_step_ms = float(np.mean([events[s][0].elapsed_time(events[s][-1]) for s in range(K)]))

    pairs = visible_pairs(p)
    d, H = p.head_dim, p.heads
    fwd_flops = 4.0 * d * pairs * H
    bwd_flops = 10.0 * d * pairs * H
    nrow = p.batch * p.seqlen_q * H
    algo = {  # algorithmic work per launch
        "fwd": ("mfma", fwd_flops),
        "bwd_rowdot": ("hbm", 2.0 * nrow * d * 2 + 4.0 * nrow),
        "bwd_dkdv": ("mfma", 8.0 * d * pairs * H),
        "bwd_dq": ("mfma", 2.0 * d * pairs * H),
    }
    peak = None
    if not args.no_peak:
        note("matrix-core calibration")
        from exact_tiled_attention_10_amd.profile_run import mfma_peak
        tf16, ghz16 = mfma_peak(False)
        tf8, ghz8 = mfma_peak(True)
        peak = {"bf16": {"tflops": round(tf16, 1), "clock_ghz": round(ghz16, 3),
                         "frac_of_published": round(tf16 / PEAK_BF16_TFLOPS, 4)},
                "fp8": {"tflops": round(tf8, 1), "clock_ghz": round(ghz8, 3),
                        "frac_of_published": round(tf8 / PEAK_FP8_TFLOPS, 4)},
                "kernel": "independent 32x32 MFMA chains, 8 waves per CU pair of SIMDs x4, every CU"}
    pk16 = peak["bf16"]["tflops"] if peak else None
    kernels = {}
    for n in names:
        bound, work = algo[n]
        t = kern_ms[n] / 1e3
        if bound == "mfma":
            ach = work / t / 1e12
            kernels[n] = {"ms": round(kern_ms[n], 4), "ms_stats": stats(kern_all[n]), "bound": "mfma",
                          "achieved": round(ach, 2), "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                          "frac_measured_peak": round(ach / pk16, 4) if pk16 else None}
        else:
            ach = work / t / 1e9
            kernels[n] = {"ms": round(kern_ms[n], 4), "ms_stats": stats(kern_all[n]), "bound": "hbm",
                          "achieved": round(ach, 1), "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    dom = max(names, key=lambda n: kern_ms[n])
    kd = kernels[dom]
    roofline = {"bound": kd["bound"], "kernel": dom, "achieved": kd["achieved"],
                "peak": PEAK_BF16_TFLOPS if kd["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": kd["unit"], "frac": kd["frac"], "traffic": measured_traffic(dom.replace("bwd_", ""), WORKLOAD)}

    fwd_ms = kern_ms["fwd"]
    bwd_ms = kern_ms["bwd_rowdot"] + kern_ms["bwd_dkdv"] + kern_ms["bwd_dq"]
    value = (fwd_flops + bwd_flops) / (ms_step / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals)",
        "config": {"workload": WORKLOAD, "batch": p.batch, "heads": H, "kv_heads": p.kv_heads,
                   "seq_len": p.seqlen_q, "head_dim": d, "causal": bool(p.causal),
                   "parallelism": "single GPU"},
        "pct_peak": {"fwd": round(100 * fwd_flops / (fwd_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "bwd": round(100 * bwd_flops / (bwd_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "step": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "pct_measured_peak": None if not pk16 else {
            "fwd": round(100 * fwd_flops / (fwd_ms / 1e3) / 1e12 / pk16, 2),
            "bwd": round(100 * bwd_flops / (bwd_ms / 1e3) / 1e12 / pk16, 2),
            "step": round(100 * value / pk16, 2)},
        "measured_peak": peak,
        "dq_path": "separate",
        "fwd_tflops": round(fwd_flops / (fwd_ms / 1e3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms / 1e3) / 1e12, 2),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "event_ms_per_step": round(ev_step_ms, 4),
        "tokens_per_s": round(p.batch * p.seqlen_q / (ms_step / 1e3), 1),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
        "dropout": None,
        "fp8": None,
        "decode": None,
        "workloads": None,
        "atomic_dq": None,
        "env": env_info(torch),
        "timing": "HIP events on the launch stream, no cache flush between calls; per-kernel mean, "
                  "ms_stats median/min/mean over the timed steps",
    }
    if not args.no_workloads:
        wl = {}
        for name, steps in OTHER_WORKLOADS:
            note(f"workload {name}")
            pw = synth.workload(name)
            plan_w = make_plan(fa, pw, dev)
            wl[name] = workload_entry(pw, time_plan(plan_w, steps, 2, torch), pk16)
            del plan_w
            torch.cuda.empty_cache()
        out["workloads"] = wl
        # the opt-in atomic-dQ backward on the 8K and 32K shapes, same process
        at = {}
        for name, steps in ((WORKLOAD, K), ("bf16_causal_gqa_b1_h32kv8_n32768_d128", 5)):
            note(f"atomic-dQ backward on {name}")
            pw = p if name == WORKLOAD else synth.workload(name)
            plan_a = make_plan(fa, pw, dev, deterministic=False)
            ta = time_plan(plan_a, steps, 2, torch)
            pairs_w = visible_pairs(pw)
            bst = stats(ta["bwd"])
            at[name] = {"bwd_ms": bst, "stages_ms": [stats(x) for x in ta["stages"]],
                        "bwd_tflops": round(10.0 * pw.head_dim * pairs_w * pw.heads / (bst["median"] / 1e3) / 1e12, 1)}
            if name != WORKLOAD:
                plan_d = make_plan(fa, pw, dev, deterministic=True)
                td = time_plan(plan_d, steps, 2, torch)
                at[name]["separate_bwd_ms"] = stats(td["bwd"])
                del plan_d
            else:
                at[name]["separate_bwd_ms"] = stats([sum(x) for x in zip(*(kern_all[n] for n in names[1:]))])
            del plan_a
            torch.cuda.empty_cache()
        out["atomic_dq"] = at
    if not args.no_dropout:
        note("dropout step")
        out["dropout"] = bench_dropout(fa, p, q, k, v, do, K, args.warmup, fwd_flops + bwd_flops, torch)
    if not args.no_fp8:
        note("fp8 forward")
        out["fp8"] = bench_fp8(fa, synth, torch, max(K, 20), max(args.warmup, 3), measured_traffic)
    if not args.no_decode:
        note("decode")
        out["decode"] = bench_decode(fa, synth, torch, max(K, 20), max(args.warmup, 3), measured_traffic)
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        note(f"cpu baseline (oracle, {threads} threads)")
        out["cpu_baseline"] = cpu_baseline(p, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

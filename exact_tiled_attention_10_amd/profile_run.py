"""Profiling entry points for rocprofv3 runs, and the summaries taken from them.

Subcommands (run from anywhere; the repository root is found from this file):

  run     --workload W --kernel {fwd,rowdot,dkdv,dq,decode,fwd_fp8} [--iters N]
          Run one kernel of the library N times on a named synthetic workload
          (after one untimed call of each earlier stage to produce its inputs;
          `decode` runs the KV-cache decode call, split pass and merge, on a
          named decode workload).  Meant to sit under `rocprofv3 --pmc ...`.
  copy    [--mib M] [--iters N]
          Run the calibration copy (libfacalib.so: read M MiB, write M MiB with
          16-byte-per-lane loads and stores of whole lines, as the attention
          kernels do) N times: the reference for the HBM byte counters.
  lds     [--workgroups G] [--iters N]
          Run the LDS calibration (libfacalib.so: conflict-free LDS reads of a
          known number of bytes, b128 reads, then transposing b64 reads) and
          print their times: the reference for the LDS activity counter.
  ldscal  --dir DIR [--workgroups G] [--iters N]
          From a `rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE`
          run of `lds`, print bytes per counter unit and bytes per clock per CU.
  traffic --workload W --kernel K --fetch DIR --write DIR --copy-fetch DIR
          --copy-write DIR [--mib M]
          Read the counter CSVs of four `rocprofv3 --pmc` runs (FETCH_SIZE and
          WRITE_SIZE, for the kernel and for the calibration copy), scale the
          kernel's counts by the copy's known/counted ratio, and record the
          bytes per launch in profiles/traffic.json together with the hash of
          the kernel's sources (bench.py reports the figure only while the
          hash still matches).
  mfma    [--workgroups G] [--iters N]
          Run the matrix-core calibration (libfacalib.so: independent bf16
          32x32x16 and fp8 32x32x64 MFMA chains on every SIMD) and print the
          rate it sustains and the shader clock under that load.
  ldsmfma [--workgroups G] [--iters N]
          Run the LDS-fed matrix-core calibration (every MFMA with a 1 KiB LDS
          read of its own; 32x32x16 at 1 and 2 waves per SIMD, reads 1, 2, 4
          MFMAs ahead; 16x16x32 at 1 to 4 waves per SIMD, reads 4 ahead)
          and print the rate each sustains, as a fraction of the matrix-core
          peak at the clock measured during the run.
  mix     [--workgroups G]
          Run the pipe-mix calibration (the two waves of each SIMD given
          idle / MFMA / FMA / exp2 work) and print each pair's time, its rates
          per SIMD-cycle at the measured clock, and the times of its halves.
  trace   --db FILE --title T --command C
          Print a markdown table of a rocprofv3 kernel-trace database.
  util    --prefix P [--kernels fwd,dkdv,dq,fwd_fp8]
          Print a utilisation table from two counter passes per kernel
          (directories P_<kernel>_1 and P_<kernel>_2, see profiles/).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# Sources each kernel is built from (the hash ties a counter reading to a build).
KERNEL_SOURCES = {
    "fwd": ["fa_fwd.hip", "fa_device.hpp"],
    "rowdot": ["fa_bwd.hip", "fa_device.hpp"],
    "dkdv": ["fa_bwd.hip", "fa_device.hpp"],
    "dq": ["fa_bwd.hip", "fa_device.hpp"],
    "decode": ["fa_decode.hip", "fa_device.hpp"],
    "fwd_fp8": ["fa_fwd_fp8.hip", "fa_device.hpp"],
}
# Patterns (re.search) for the kernel names in rocprofv3 output.
KERNEL_NAMES = {"fwd": "fwd_kernel<", "rowdot": "bwd_rowdot_kernel", "dkdv": "bwd_dkdv_kernel",
                "dq": "bwd_dq_kernel", "decode": "decode_split_kernel", "fwd_fp8": "fwd_fp8_kernel"}
COPY_NAME = "calib_copy_kernel"
CALIB_LIB = os.path.join(HERE, "libfacalib.so")


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed: what the
    compiler sees, so edits to comments keep a counter record valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch recorded for this kernel and workload, or None when
    there is no record or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel)
    if not ent or ent.get("workload") != workload or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def _run(args):
    sys.path.insert(0, ROOT)
    import torch
    import synth
    import exact_tiled_attention_10_amd as fa

    dev = torch.device("cuda:0")
    if args.kernel == "decode":
        p = synth.decode_workload(args.workload)
        cs = p.cache_seqlens().to(dev)
        plan = fa.DecodePlan(p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev), cs, causal=p.causal,
                             softmax_scale=p.scale)
        torch.cuda.synchronize()
        for _ in range(args.iters):
            plan.run()
        torch.cuda.synchronize()
        print(f"ran decode x{args.iters} on {args.workload}", flush=True)
        return
    if args.kernel == "fwd_fp8":
        p = synth.workload(args.workload)
        plan = fa.Fp8Plan(p.q.to(dev), p.k.to(dev), p.v.to(dev), p.descale_q, p.descale_k, p.descale_v,
                          causal=p.causal, window_size=(p.window_left, p.window_right), softmax_scale=p.scale)
        torch.cuda.synchronize()
        for _ in range(args.iters):
            plan.run()
        torch.cuda.synchronize()
        print(f"ran fwd_fp8 x{args.iters} on {args.workload}", flush=True)
        return
    p = synth.workload(args.workload)
    q, k, v, do = (t.to(dev) for t in (p.q, p.k, p.v, p.do))
    cu = p.cu_seqlens()
    cu = cu.to(dev) if cu is not None else None
    plan = fa.Plan(q, k, v, do, causal=p.causal, window_size=(p.window_left, p.window_right),
                   softmax_scale=p.scale, cu_seqlens_q=cu, cu_seqlens_k=cu,
                   max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    stages = {"fwd": plan.fwd, "rowdot": lambda: plan.bwd_stage(0),
              "dkdv": lambda: plan.bwd_stage(1), "dq": lambda: plan.bwd_stage(2)}
    order = ["fwd", "rowdot", "dkdv", "dq"]
    for name in order[:order.index(args.kernel)]:  # inputs of the profiled stage
        stages[name]()
    torch.cuda.synchronize()
    for _ in range(args.iters):
        stages[args.kernel]()
    torch.cuda.synchronize()
    print(f"ran {args.kernel} x{args.iters} on {args.workload}", flush=True)


def _copy(args):
    import ctypes
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is not built; run `python -m exact_tiled_attention_10_amd.build`")
    L = ctypes.CDLL(CALIB_LIB)
    L.fa_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.fa_calib_copy.restype = ctypes.c_int
    nbytes = args.mib * (1 << 20)
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(args.iters):
        rc = L.fa_calib_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), nbytes, 1024, stream)
        if rc != 0:
            raise RuntimeError(f"fa_calib_copy returned {rc}")
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x{args.iters}", flush=True)


def mfma_peak(fp8: bool, workgroups: int = 1024, iters: int = 20000, reps: int = 3):
    """Sustained dense MFMA rate (TFLOP/s) and shader clock (GHz) measured on
    the current device by the calibration kernel: `workgroups` workgroups of
    8 waves, each wave `iters` rounds of 4 independent MFMA chains.  Returns
    (tflops, clock_ghz), the median over `reps` timed launches after one
    untimed launch."""
    import ctypes
    import numpy as np
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is not built; run `python -m exact_tiled_attention_10_amd.build`")
    L = ctypes.CDLL(CALIB_LIB)
    L.fa_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p]
    L.fa_calib_mfma.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def launch():
        rc = L.fa_calib_mfma(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()), workgroups, iters,
                             int(bool(fp8)), sp)
        if rc != 0:
            raise RuntimeError(f"fa_calib_mfma returned {rc}")

    launch()
    torch.cuda.synchronize()
    times, ghz = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
        c = clocks.cpu().numpy().view(np.uint64).reshape(-1, 4).astype(np.float64)
        ok = c[:, 3] > c[:, 2]
        ghz.append(float(np.median((c[ok, 1] - c[ok, 0]) / (c[ok, 3] - c[ok, 2]) * 0.1)))
    flops = workgroups * 8.0 * iters * 4 * (131072 if fp8 else 32768)
    t = float(np.median(times))
    return flops / t / 1e12, float(np.median(ghz))


def _mfma(args):
    sys.path.insert(0, ROOT)
    for fp8 in (False, True):
        tf, ghz = mfma_peak(fp8, args.workgroups, args.iters)
        print(f"{'fp8' if fp8 else 'bf16'}: {tf:.1f} TFLOP/s sustained, shader clock {ghz:.3f} GHz", flush=True)


def _calib_timed(fn, sink, clocks, reps=3):
    """Median time (s) and shader clock (GHz) of `reps` launches of fn() after
    one untimed launch; fn launches a calibration kernel writing `clocks`."""
    import numpy as np
    import torch
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times, ghz = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
        c = clocks.cpu().numpy().view(np.uint64).reshape(-1, 4).astype(np.float64)
        ok = c[:, 3] > c[:, 2]
        ghz.append(float(np.median((c[ok, 1] - c[ok, 0]) / (c[ok, 3] - c[ok, 2]) * 0.1)))
    return float(np.median(times)), float(np.median(ghz))


def _calib_lib():
    import ctypes
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is not built; run `python -m exact_tiled_attention_10_amd.build`")
    L = ctypes.CDLL(CALIB_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.fa_calib_lds_mfma.argtypes = [P, P, I, I, I, I, P]
    L.fa_calib_lds_mfma.restype = I
    L.fa_calib_lds_mfma16.argtypes = [P, P, I, I, I, P]
    L.fa_calib_lds_mfma16.restype = I
    L.fa_calib_mix.argtypes = [P, P, I, I, I, I, I, P]
    L.fa_calib_mix.restype = I
    return L


# gfx950 bf16 32x32x16 MFMA: 32768 FLOP in 32 cycles on one SIMD
_MFMA_FLOP_PER_SIMD_CYCLE = 1024.0


def _ldsmfma(args):
    import ctypes
    import torch
    L = _calib_lib()
    dev = torch.device("cuda:0")
    sink = torch.empty(args.workgroups * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(args.workgroups * 4, dtype=torch.int64, device=dev)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    print("| waves per SIMD | reads ahead | TFLOP/s | clock (GHz) | fraction of the matrix-core peak at that clock |")
    print("|---|---|---|---|---|")
    for wps in (1, 2):
        for pf in (1, 2, 4):
            def fn():
                rc = L.fa_calib_lds_mfma(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                                         args.workgroups, args.iters, wps, pf, sp)
                if rc != 0:
                    raise RuntimeError(f"fa_calib_lds_mfma returned {rc}")
            t, ghz = _calib_timed(fn, sink, clocks)
            flops = args.workgroups * 4.0 * wps * args.iters * 16 * 32768
            frac = flops / t / (_SIMDS * _MFMA_FLOP_PER_SIMD_CYCLE * ghz * 1e9)
            print(f"| {wps} | {pf} | {flops / t / 1e12:.0f} | {ghz:.3f} | {frac:.3f} |", flush=True)
    # the 16x16x32 form: a 1 KiB operand per 16384 FLOP (half the 32x32x16 reuse)
    sink16 = torch.empty(args.workgroups * 1024, dtype=torch.float32, device=dev)
    print()
    print("16x16x32 MFMA, one 1 KiB LDS read each, 4 ahead:")
    print()
    print("| waves per SIMD | TFLOP/s | clock (GHz) | fraction of the matrix-core peak at that clock |")
    print("|---|---|---|---|")
    for wps in (1, 2, 3, 4):
        def fn16():
            rc = L.fa_calib_lds_mfma16(ctypes.c_void_p(sink16.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                                       args.workgroups, args.iters, wps, sp)
            if rc != 0:
                raise RuntimeError(f"fa_calib_lds_mfma16 returned {rc}")
        t, ghz = _calib_timed(fn16, sink16, clocks)
        flops = args.workgroups * 4.0 * wps * args.iters * 32 * 16384
        frac = flops / t / (_SIMDS * _MFMA_FLOP_PER_SIMD_CYCLE * ghz * 1e9)
        print(f"| {wps} | {flops / t / 1e12:.0f} | {ghz:.3f} | {frac:.3f} |", flush=True)


_ROLE = {0: "idle", 1: "MFMA (registers)", 2: "MFMA (1 KiB LDS read each)", 3: "FMA chains", 4: "exp2 chains",
         5: "MFMA + 4 FMAs each, one stream", 6: "MFMA + 4 exp2 each, one stream",
         7: "LDS-fed MFMA + 4 FMAs each, one stream", 8: "LDS-fed MFMA + 4 exp2 each, one stream"}


def _mix(args):
    import ctypes
    import torch
    L = _calib_lib()
    dev = torch.device("cuda:0")
    sink = torch.empty(args.workgroups * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(args.workgroups * 4, dtype=torch.int64, device=dev)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    it_m, it_v = args.iters_mfma, args.iters_valu

    def run(ra, rb):
        def fn():
            rc = L.fa_calib_mix(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                                args.workgroups, it_m, it_v, ra, rb, sp)
            if rc != 0:
                raise RuntimeError(f"fa_calib_mix returned {rc}")
        return _calib_timed(fn, sink, clocks)

    alone = {}
    for r in (1, 2, 3, 4):
        alone[r] = run(r, 0)
    print("| waves 0-3 (one per SIMD) | waves 4-7 (one per SIMD) | time (ms) | clock (GHz) | MFMA fraction of peak "
          "| vector instructions per SIMD-cycle | sum of the halves alone (ms) |")
    print("|---|---|---|---|---|---|---|")
    for ra, rb in ((1, 0), (2, 0), (3, 0), (4, 0), (3, 3), (4, 4), (1, 3), (1, 4), (2, 3), (2, 4),
                   (5, 0), (6, 0), (5, 5), (6, 6), (7, 0), (8, 0), (7, 7), (8, 8)):
        t, ghz = run(ra, rb) if (ra, rb) not in ((r, 0) for r in alone) else alone[ra]
        cyc = t * ghz * 1e9
        mf = sum(4 for r in (ra, rb) if r in (1, 2, 5, 6, 7, 8)) * args.workgroups * it_m * 16 * 32768.0
        vw = sum(4 for r in (ra, rb) if r in (3, 4, 5, 6, 7, 8)) * args.workgroups * it_v * 16.0
        mfrac = mf / (_SIMDS * _MFMA_FLOP_PER_SIMD_CYCLE * cyc) if mf else 0.0
        vrate = vw / (_SIMDS * cyc) if vw else 0.0
        # a mixed role's halves are its MFMA part (role 1) and its vector part (3 or 4)
        parts = [x for r in (ra, rb) if r
                 for x in (((alone[2][0] if r >= 7 else alone[1][0]), alone[3 if r % 2 else 4][0])
                           if r >= 5 else (alone[r][0],))]
        print(f"| {_ROLE[ra]} | {_ROLE[rb]} | {1e3 * t:.3f} | {ghz:.3f} | {mfrac:.3f} | {vrate:.3f} | "
              f"{1e3 * sum(parts):.3f} |", flush=True)


LDS_NAME = "calib_lds_kernel"
_LDS_WAVE_STEP_BYTES = 1024  # bytes one wave reads per step of the LDS calibration


def _lds_bytes(workgroups: int, iters: int) -> int:
    return workgroups * 8 * iters * 8 * _LDS_WAVE_STEP_BYTES


def _lds(args):
    import ctypes
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is not built; run `python -m exact_tiled_attention_10_amd.build`")
    L = ctypes.CDLL(CALIB_LIB)
    L.fa_calib_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.fa_calib_lds.restype = ctypes.c_int
    out = torch.empty(args.workgroups * 512, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for tr in (0, 1):
        for rep in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = L.fa_calib_lds(ctypes.c_void_p(out.data_ptr()), args.workgroups, args.iters, tr,
                                ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"fa_calib_lds returned {rc}")
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            nb = _lds_bytes(args.workgroups, args.iters)
            print(f"lds {'transposing b64' if tr else 'b128'} run {rep}: {ms:.3f} ms, "
                  f"{nb / ms / 1e9:.1f} TB/s", flush=True)


def _ldscal(args):
    """Bytes per SQ_LDS_IDX_ACTIVE unit and LDS read bandwidth per CU and clock,
    per dispatch of the LDS calibration."""
    nb = _lds_bytes(args.workgroups, args.iters)
    idx = _counter_per_dispatch(args.dir, LDS_NAME, "SQ_LDS_IDX_ACTIVE")
    gui = _counter_per_dispatch(args.dir, LDS_NAME, "GRBM_GUI_ACTIVE")
    ins = _counter_per_dispatch(args.dir, LDS_NAME, "SQ_INSTS_LDS")
    for i, (a, g, n) in enumerate(zip(idx, gui, ins)):
        cyc = g / _XCDS
        print(f"dispatch {i}: {nb / a:.1f} bytes per SQ_LDS_IDX_ACTIVE unit, {nb / n:.0f} bytes per LDS "
              f"instruction, {nb / cyc / _CUS:.1f} bytes per clock per CU ({cyc:.3g} cycles per XCD)")


def _counter_per_dispatch(run_dir: str, name_sub: str, counter: str) -> list:
    """Per-dispatch values (summed over the rows rocprofv3 reports for one
    dispatch) of `counter` for kernels whose name matches the pattern name_sub."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(float)
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if re.search(name_sub, r["Kernel_Name"]) and r["Counter_Name"] == counter:
                    per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for kernels matching {name_sub!r} in {run_dir}")
    return [per[d] for d in sorted(per, key=int)]


def _traffic(args):
    kname = KERNEL_NAMES[args.kernel]
    kf = _counter_per_dispatch(args.fetch, kname, "FETCH_SIZE")
    kw = _counter_per_dispatch(args.write, kname, "WRITE_SIZE")
    cf = _counter_per_dispatch(args.copy_fetch, COPY_NAME, "FETCH_SIZE")
    cw = _counter_per_dispatch(args.copy_write, COPY_NAME, "WRITE_SIZE")
    mean = lambda xs: sum(xs) / len(xs)
    known_kib = args.mib * 1024.0
    f_fac = known_kib / mean(cf)  # true bytes per counted byte, reads
    w_fac = known_kib / mean(cw)  # and writes
    fetch_b = mean(kf) * 1024.0 * f_fac
    write_b = mean(kw) * 1024.0 * w_fac
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    data.setdefault("kernels", {})[args.kernel] = {
        "workload": args.workload,
        "source_hash": source_hash(args.kernel),
        "bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes": round(fetch_b),
        "write_bytes": round(write_b),
        "fetch_kib_counted": mean(kf),
        "write_kib_counted": mean(kw),
        "calibration": {"copy_mib": args.mib, "fetch_kib_counted": mean(cf), "write_kib_counted": mean(cw),
                        "fetch_factor": f_fac, "write_factor": w_fac},
    }
    data["method"] = ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (separate runs), KiB per dispatch "
                      "averaged over dispatches, each scaled by known/counted bytes of a plain copy kernel")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(data["kernels"][args.kernel], indent=1))


def _counters_mean(run_dir: str, name_sub: str) -> dict:
    """Mean per dispatch of every counter rocprofv3 recorded for kernels whose
    name matches the pattern name_sub."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    tot, disp = defaultdict(float), defaultdict(set)
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                kn = r["Kernel_Name"]
                if not re.search(name_sub, kn):
                    continue
                tot[r["Counter_Name"]] += float(r["Counter_Value"])
                disp[r["Counter_Name"]].add(r["Dispatch_Id"])
    return {c: tot[c] / len(disp[c]) for c in tot}


# gfx950: 8 XCDs of 32 CUs with 4 SIMDs each
_XCDS, _SIMDS, _CUS = 8, 1024, 256
# SQ_LDS_IDX_ACTIVE advances once per 256 bytes of LDS reads (the LDS
# calibration above), i.e. it counts cycles of the LDS at its full width.
_LDS_BYTES_PER_UNIT = 256


def _util(args):
    """Utilisation table from two counter passes per kernel (run directories
    <prefix>_<kernel>_1 and _2)."""
    rows = ["| kernel | clock cycles per XCD | matrix cores busy | VALU and MFMA co-issue | "
            "waves waiting | LDS instructions | LDS bank-conflict cycles | LDS busy |",
            "|---|---|---|---|---|---|---|---|"]
    for k in args.kernels.split(","):
        c = _counters_mean(f"{args.prefix}_{k}_1", KERNEL_NAMES[k])
        c.update(_counters_mean(f"{args.prefix}_{k}_2", KERNEL_NAMES[k]))
        simd_cycles = c["GRBM_GUI_ACTIVE"] / _XCDS * _SIMDS
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
        coex = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles
        wait = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
        lds = c["SQ_LDS_IDX_ACTIVE"] / (c["GRBM_GUI_ACTIVE"] / _XCDS * _CUS)
        rows.append(f"| {k} | {c['GRBM_GUI_ACTIVE'] / _XCDS:.3g} | {100 * busy:.1f}% | {100 * coex:.1f}% | "
                    f"{100 * wait:.1f}% | {c['SQ_INSTS_LDS']:.3g} | {c['SQ_LDS_BANK_CONFLICT']:.0f} | "
                    f"{100 * lds:.1f}% |")
    print("\n".join(rows))


def _trace(args):
    """Per (kernel, grid) launch statistics of a rocprofv3 kernel-trace
    database: one kernel template serves several workloads, told apart by
    their grids."""
    c = sqlite3.connect(args.db)
    durs = defaultdict(list)
    info = {}
    for r in c.execute("select name, duration, grid_x, grid_y, grid_z, workgroup_x, lds_size, scratch_size "
                       "from kernels order by start"):
        key = (r[0], r[2], r[3], r[4])
        durs[key].append(r[1])
        info[key] = r[5:]
    total = sum(sum(v) for v in durs.values())
    out = [f"# {args.title}", "", "Commands (from the repository root):", "", "```", args.command, "```", "",
           "Per kernel and grid (a grid identifies the workload): all calls, and the mean of the last "
           f"{args.last} (the timed calls).", "",
           f"| kernel | grid | calls | avg (us) | avg last {args.last} (us) | % of traced time | WG | LDS (B) | "
           "scratch (B) |",
           "|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(durs, key=lambda k: -sum(durs[k])):
        n, gx, gy, gz = key
        d = durs[key]
        short = n.replace("fa::(anonymous namespace)::", "").replace("void ", "")
        last = d[-args.last:]
        wg, lds, scr = info[key]
        out.append(f"| `{short}` | {gx}x{gy}x{gz} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                   f"{sum(last) / len(last) / 1e3:.1f} | {100 * sum(d) / total:.1f} | {wg} | {lds} | {scr} |")
    if args.bench_log:
        with open(args.bench_log) as fh:
            line = next((l for l in fh if l.startswith('{"metric"')), None)
        if line:
            d = json.loads(line)
            summary = {"ms_per_step": d["ms_per_step"], "value": d["value"],
                       "kernels_ms": {k: v["ms"] for k, v in d["kernels"].items()}}
            if d.get("decode"):
                summary["decode"] = {k: d["decode"][k] for k in ("workload", "ms_per_call", "achieved", "unit")}
            if d.get("fp8"):
                summary["fp8"] = {k: d["fp8"][k] for k in ("workload", "ms", "achieved", "unit")}
            if d.get("workloads"):
                summary["workloads_median_ms"] = {n: {ph: w[ph]["ms"]["median"] for ph in ("fwd", "bwd")}
                                                  for n, w in d["workloads"].items()}
            if d.get("atomic_dq"):
                summary["atomic_dq_bwd_median_ms"] = {n: e["bwd_ms"]["median"] for n, e in d["atomic_dq"].items()}
            out += ["", "bench.py line of the same run (HIP-event kernel times, ms):", "", "```",
                    json.dumps(summary), "```"]
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--kernel", required=True, choices=list(KERNEL_NAMES))
    r.add_argument("--iters", type=int, default=3)
    cp = sub.add_parser("copy")
    cp.add_argument("--mib", type=int, default=1024)
    cp.add_argument("--iters", type=int, default=3)
    ld = sub.add_parser("lds")
    ld.add_argument("--workgroups", type=int, default=512)
    ld.add_argument("--iters", type=int, default=4096)
    lc = sub.add_parser("ldscal")
    lc.add_argument("--dir", required=True)
    lc.add_argument("--workgroups", type=int, default=512)
    lc.add_argument("--iters", type=int, default=4096)
    mf = sub.add_parser("mfma")
    mf.add_argument("--workgroups", type=int, default=1024)
    mf.add_argument("--iters", type=int, default=20000)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel", required=True, choices=list(KERNEL_NAMES))
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        t.add_argument(a, required=True)
    t.add_argument("--mib", type=int, default=1024)
    u = sub.add_parser("util")
    u.add_argument("--prefix", required=True, help="counter run directories <prefix>_<kernel>_1 and _2")
    u.add_argument("--kernels", default="fwd,dkdv,dq,fwd_fp8")
    lm = sub.add_parser("ldsmfma")
    lm.add_argument("--workgroups", type=int, default=256)
    lm.add_argument("--iters", type=int, default=2000)
    mx = sub.add_parser("mix")
    mx.add_argument("--workgroups", type=int, default=256)
    mx.add_argument("--iters-mfma", type=int, default=500)
    mx.add_argument("--iters-valu", type=int, default=2000)
    tr = sub.add_parser("trace")
    tr.add_argument("--db", required=True)
    tr.add_argument("--title", required=True)
    tr.add_argument("--command", required=True)
    tr.add_argument("--last", type=int, default=5)
    tr.add_argument("--bench-log", default=None)
    args = ap.parse_args(argv)
    {"run": _run, "copy": _copy, "lds": _lds, "ldscal": _ldscal, "traffic": _traffic, "trace": _trace,
     "util": _util, "mfma": _mfma, "ldsmfma": _ldsmfma, "mix": _mix}[args.cmd](args)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the Simple GLA hot path on one MI355X.

One step = one chunked prefill of a lightning layer (B=1, H=32, T=8192,
Dk=Dv=128, bf16 in, fp32 state out) through ``sgla_chunk_fwd``. K timed steps
run back to back after W warm-up steps, bracketed by device synchronisation;
``value`` is prefill tokens/s. Each call is also bracketed by HIP events on the
stream it runs on, which gives the per-call duration used for the roofline.

The fused decode step (256 sequences x 32 heads, Dk=Dv=128, fp32 state in HBM,
64 successive steps) is timed the same way and reported in ``decode``.
``prologue`` reports both again through the entry points that take q and k
before the per-head RMSNorm and RoPE and apply them as the tiles load.

``cpu_baseline`` times the oracle (plain C, fp64, OpenMP over (sequence, head)
units) on the same prefill workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Simple GLA prefill tokens/s @H=32,D=128 bf16 (MFMA %) + decode HBM GB/s"
PREFILL = "prefill_bf16_h32_t8192_d128"
DECODE = "decode_bf16_n256_h32_d128_x64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")

PREFILL_PRO = PREFILL + "+qk_norm_rope"
DECODE_PRO = DECODE + "+qk_norm_rope"
DECODE_BF16 = DECODE + "+bf16_state"
EPILOGUE = "out_norm_gate_bf16_8192x4096"
GDN_PREFILL = "gdn_prefill_bf16_h32_t8192_d128"
GDN_DECODE = "gdn_decode_bf16_n256_h32_d128_x64"
# The kernels of one call of each workload, as rocprofv3 names them.
CALL_KERNELS = {
    PREFILL: ["chunk_mfma_kernel<true, false>", "scan_kernel<128, 128>",
              "chunk_mfma_kernel<false, false>"],
    PREFILL_PRO: ["chunk_mfma_kernel<true, true>", "scan_kernel<128, 128>",
                  "chunk_mfma_kernel<false, true>"],
    DECODE: ["recurrent_step_kernel<unsigned short, 128, 128, false, float>"],
    DECODE_PRO: ["recurrent_step_kernel<unsigned short, 128, 128, true, float>"],
    DECODE_BF16: ["recurrent_step_kernel<unsigned short, 128, 128, false, unsigned short>"],
    EPILOGUE: ["out_norm_gate_kernel<unsigned short, 2>"],
    GDN_PREFILL: ["gdn_prep_kernel", "gdn_chain_kernel", "gdn_output_kernel"],
    GDN_DECODE: ["gdn_step_kernel<unsigned short, 128, 128>"],
}


# The sources each workload's kernels are built from, besides the shared ones
# (headers, the host code that picks launch shapes, the build flags).
WORKLOAD_SOURCES = {
    PREFILL: ["chunk_mfma.hip", "chunk_plan.hip"],
    PREFILL_PRO: ["chunk_mfma.hip", "chunk_plan.hip"],
    DECODE: ["recurrent_step.hip"],
    DECODE_PRO: ["recurrent_step.hip"],
    DECODE_BF16: ["recurrent_step.hip"],
    EPILOGUE: ["out_norm_gate.hip"],
    GDN_PREFILL: ["gdn_chunk.hip"],
    GDN_DECODE: ["gdn_step.hip"],
}
SHARED_SOURCES = ["sgla_internal.h", "mfma_tile.h", "sgla_host.hip", "../build.py"]


def kernel_source_hash(workload):
    """sha256 over the sources of one workload's kernels, to tell whether a
    stored counter record still describes the kernels that are built."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_hybrid_amd", "csrc")
    for name in sorted(WORKLOAD_SOURCES[workload]) + SHARED_SOURCES:
        h.update(name.encode())
        with open(os.path.normpath(os.path.join(csrc, name)), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per call from the committed FETCH_SIZE/WRITE_SIZE record,
    or None when there is none or the kernels changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("bytes_per_call")


def copy_calibration(torch, dev, nbytes=256 << 20, reps=3):
    """An elementwise pass of known size (fp32 negation: nbytes read, nbytes
    written, kernel name containing ``neg_kernel``), so FETCH_SIZE/WRITE_SIZE
    can be scaled to bytes when run under rocprofv3 --pmc."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _counter_rows(run_dir, counter):
    """(kernel name, value) per dispatch from the counter CSVs rocprofv3
    wrote under run_dir (--output-format csv)."""
    import csv
    rows = []
    for path in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                                 recursive=True)):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(name, val) for _, name, val in rows]


def _per_kernel_avg(rows):
    acc = {}
    for name, val in rows:
        acc.setdefault(name, []).append(val)
    return {name: sum(v) / len(v) for name, v in acc.items()}


def record_traffic(fetch_dir, write_dir, calib_bytes=256 << 20):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run of
    ``bench.py --copy-calibration`` into HBM bytes per call.

    Both counters are in KiB per dispatch. Each is scaled by what it reads
    for the fp32 negation pass of known size (calib_bytes read and written),
    averaged per kernel, and summed over the kernels of one call of each
    workload (CALL_KERNELS). Writes profiles/traffic.json keyed by workload,
    with the hash of the kernel sources the counters were taken on."""
    fetch_rows = _counter_rows(fetch_dir, "FETCH_SIZE")
    write_rows = _counter_rows(write_dir, "WRITE_SIZE")

    def calibration(rows):
        # The input generators negate small tensors too; the calibration
        # dispatches are the large ones.
        vals = [v for n, v in rows if "neg_kernel" in n]
        if not vals:
            raise SystemExit("record-traffic: no calibration pass (neg_kernel) in the counter runs")
        big = [v for v in vals if v >= 0.25 * max(vals)]
        return calib_bytes / (sum(big) / len(big) * 1024.0)

    f_scale = calibration(fetch_rows)
    w_scale = calibration(write_rows)
    fetch = _per_kernel_avg(fetch_rows)
    write = _per_kernel_avg(write_rows)

    def find(pattern, table):
        names = [n for n in table if pattern in n]
        return names[0] if len(names) == 1 else None

    rec = {"_calibration": {"fetch_scale": f_scale, "write_scale": w_scale,
                            "pass": "fp32 negation, %d bytes read and written" % calib_bytes}}
    for wl, parts in CALL_KERNELS.items():
        kern = {}
        for pat in parts:
            nf, nw = find(pat, fetch), find(pat, write)
            if nf is None or nw is None:
                kern = None
                break
            kern[nf] = {"fetch": fetch[nf] * 1024.0 * f_scale, "write": write[nw] * 1024.0 * w_scale}
        if kern:
            rec[wl] = {"source_hash": kernel_source_hash(wl), "kernels": kern,
                       "bytes_per_call": sum(v["fetch"] + v["write"] for v in kern.values())}
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


def prefill_bytes(B, T, H, Dk, Dv, elem=2, with_s0=False):
    """Algorithmic HBM bytes of one chunked-forward call: q, k, v read, o
    written, g read (1,028 B per token and head at D=128 bf16), the final
    state written and the initial state read when present."""
    tok = B * T * H * (2 * Dk * elem + Dv * elem + Dv * elem + 4)
    st = B * H * Dk * Dv * 4 * (2 if with_s0 else 1)
    return tok + st


def prefill_flops(B, T, H, Dk, Dv, C=64):
    """Dense-tile flops: QK^T and A.V on 64x64 tiles, Q.S and K^T.V."""
    per_tok = 2 * C * Dk + 2 * C * Dv + 2 * Dk * Dv + 2 * Dk * Dv
    return B * T * H * per_tok


def decode_bytes(N, H, Dk, Dv, elem=2, state_elem=4):
    """One decode step: the state read and written (fp32, or bf16 with
    state_elem=2), q, k, v read, g read, o written."""
    return N * H * (2 * Dk * Dv * state_elem + (2 * Dk + Dv) * elem + 4 + Dv * elem)


def time_calls(fn, steps, warmup, torch, single_reps=20):
    """Time `steps` back-to-back calls between two events on the current
    stream (the stream the library launches on). Returns the host wall time,
    the region's event time (ms) and, from a separate short pass with events
    around each call, single-call times. Events around every call would add
    host time to each step, so the timed region has none."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region = a.elapsed_time(b)
    n1 = min(steps, single_reps)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n1)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n1)]
    for i in range(n1):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in zip(starts, ends)]
    return wall, region, per


def time_flushed(fn, reps, torch, dev, flush_bytes=1 << 30):
    """Per-call times with the caches emptied before each call: a 1 GiB
    buffer is overwritten between calls (outside the timed events), so the
    call's inputs come from HBM rather than the 256 MB memory-side cache."""
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    per = []
    for _ in range(reps):
        flush.fill_(1.0)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    del flush
    return per


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def cpu_baseline(inp, W, min_seconds=10.0, max_reps=500):
    """The oracle on the whole prefill workload, repeated until at least
    ``min_seconds`` of host time have passed (one pass takes a fraction of a
    second on many cores); reports the mean rate."""
    import numpy as np
    import oracle
    q, k, v, g = (W.to_numpy_f32(inp[x]) for x in ("q", "k", "v", "g"))
    threads = oracle.default_threads()
    oracle.build(force=False)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(q, k, v, g, inp["scale"], nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    B, T, H, _ = q.shape
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                     if l.startswith("model name"))
    except Exception:  # pragma: no cover
        model = "unknown"
    return {"value": B * T * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole prefill workload (B=1, T=8192, all 32 heads, 262,144 "
                      "head-tokens), %d passes in %.1f s (%.3f s each), fp64 C oracle, OpenMP over "
                      "(sequence, head) units; host CPU %s" % (reps, dt, dt / reps, model)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-passes", type=int, default=3,
                    help="timed passes of 64 decode steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "prologue", "epilogue",
                                       "bf16-state", "gdn"], default="all")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB elementwise pass (for counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write profiles/traffic.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of this script with --copy-calibration")
    ap.add_argument("--flushed-reps", type=int, default=20,
                    help="calls timed one by one after a cache flush (0: skip)")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(*args.record_traffic)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d (WORLD_SIZE %d) is not "
              "supported. A sequence shards by (sequence, head) units, with a carried-state "
              "exchange for context parallelism; neither is built here." % (args.gpus, world),
              file=sys.stderr)
        return 2

    import torch
    import linear_attention_hybrid_amd as sgla
    import sgla_inputs as W

    sgla.library()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, dev)
    props = torch.cuda.get_device_properties(dev)
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded; q,k unit-RMS + RoPE, v ~ N(0,1), g = log sigmoid(N(4,1)))"}

    if args.only in ("all", "prefill"):
        inp = W.make_workload(PREFILL, seed=args.seed, device=dev)
        B, T, H, Dk = inp["q"].shape
        Dv = inp["v"].shape[-1]
        out = torch.empty_like(inp["v"])
        fs = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)

        def step():
            sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], None, None, inp["scale"],
                           out=out, final_state=fs)

        wall, region, per = time_calls(step, args.steps, args.warmup, torch)
        ms_step = region / args.steps
        per_avg = ms_step
        nbytes = prefill_bytes(B, T, H, Dk, Dv)
        flops = prefill_flops(B, T, H, Dk, Dv)
        achieved = nbytes / (per_avg * 1e-3) / 1e9
        result.update({
            "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step,
            "config": {"workload": PREFILL, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv,
                       "chunk": 64, "scale": inp["scale"], "initial_state": "zero",
                       "final_state": "fp32", "gpu": props.name},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": recorded_traffic(PREFILL),
                         "kernel": "sgla_chunk_fwd (whole call: plan, segment-state, scan and "
                                   "output kernels)",
                         "algorithmic_bytes_per_launch": nbytes,
                         "avg_launch_ms": per_avg},
            "mfma": {"useful_tflops": flops / (per_avg * 1e-3) / 1e12,
                     "useful_frac_of_bf16_peak": flops / (per_avg * 1e-3) / 1e12 /
                     BF16_DENSE_PEAK_TFLOPS,
                     "dense_tile_flops_per_launch": flops},
            "wall_s_timed": wall,
            "per_call_ms": {"mean": per_avg, "median_single": median(per), "min_single": min(per)},
        })
        if args.flushed_reps > 0:
            fl = time_flushed(step, args.flushed_reps, torch, dev)
            result["flushed"] = {
                "note": "each call after a 1 GiB overwrite; inputs read from HBM",
                "reps": len(fl), "median_ms": median(fl), "min_ms": min(fl),
                "tokens_per_s": B * T / (median(fl) * 1e-3),
                "achieved_GBs": nbytes / (median(fl) * 1e-3) / 1e9,
                "frac": nbytes / (median(fl) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(inp, W)
        del inp, out, fs
        torch.cuda.empty_cache()

    if args.only in ("all", "decode"):
        d = W.make_workload(DECODE, seed=4, device=dev)
        steps, N, H, Dk = d["q"].shape
        Dv = d["v"].shape[-1]
        state = d["state"]
        out = torch.empty((N, H, Dv), dtype=d["v"].dtype, device=dev)
        counter = [0]

        def dstep():
            i = counter[0] % steps
            counter[0] += 1
            sgla.recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state,
                                scale=d["scale"], out=out)

        n_timed = steps * args.decode_passes
        wall, region, per = time_calls(dstep, n_timed, steps, torch)
        per_avg = region / n_timed
        nb = decode_bytes(N, H, Dk, Dv)
        gbs = nb / (per_avg * 1e-3) / 1e9
        dec = {"workload": DECODE, "steps_timed": n_timed, "ms_per_step": region / n_timed,
               "tokens_per_s": N / (region / n_timed * 1e-3),
               "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                            "traffic": recorded_traffic(DECODE),
                            "kernel": "sgla_recurrent_step",
                            "algorithmic_bytes_per_launch": nb, "avg_launch_ms": per_avg}}
        result["decode"] = dec
        if args.only == "decode":
            result.update({"value": dec["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": dec["ms_per_step"],
                           "config": {"workload": DECODE}, "roofline": dec["roofline"]})
    if args.only in ("all", "prologue"):
        result["prologue"] = bench_prologue(args, torch, sgla, W, dev)
        if args.only == "prologue":
            pf = result["prologue"]["prefill"]
            result.update({"value": pf["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": pf["ms_per_call"],
                           "config": {"workload": PREFILL + " (raw q/k, RMSNorm + RoPE in-kernel)"},
                           "roofline": pf["roofline"]})
    if args.only in ("all", "bf16-state"):
        result["decode_bf16_state"] = bench_bf16_state(args, torch, sgla, W, dev)
        if args.only == "bf16-state":
            e = result["decode_bf16_state"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_step"],
                           "config": {"workload": e["workload"]}, "roofline": e["roofline"]})
    if args.only in ("all", "epilogue"):
        result["epilogue"] = bench_epilogue(args, torch, sgla, W, dev)
        if args.only == "epilogue":
            e = result["epilogue"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_call"],
                           "config": {"workload": e["workload"]}, "roofline": e["roofline"]})
    if args.only in ("all", "gdn"):
        result["gdn"] = bench_gdn(args, torch, sgla, W, dev)
        if args.only == "gdn":
            e = result["gdn"]["prefill"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_call"],
                           "config": {"workload": e["workload"]}, "roofline": e["roofline"]})
    print(json.dumps(result), flush=True)
    return 0


def bench_gdn(args, torch, sgla, W, dev):
    """The gated delta rule on the same shapes: prefill B=1, T=8192, H=32,
    Dk=Dv=128 (sgla_gdn_chunk_fwd) and the batched decode, 256 x 32 heads,
    64 successive steps (sgla_gdn_recurrent_step); "gdn" inputs (L2-normalised
    q and k, beta = sigmoid(N(0, 1)))."""
    out = {}
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "gdn", seed=args.seed, device=dev,
                         with_beta=True)
    o = torch.empty_like(inp["v"])
    fs = torch.empty((1, 32, 128, 128), dtype=torch.float32, device=dev)

    def step():
        sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                           scale=inp["scale"], out=o, final_state=fs)

    _, region, per = time_calls(step, args.steps, args.warmup, torch)
    per_avg = region / args.steps
    nbytes = prefill_bytes(1, 8192, 32, 128, 128) + 8192 * 32 * 4
    gbs = nbytes / (per_avg * 1e-3) / 1e9
    out["prefill"] = {"workload": GDN_PREFILL, "ms_per_call": region / args.steps,
                      "tokens_per_s": 8192 / (region / args.steps * 1e-3),
                      "per_call_ms": {"mean": per_avg, "median_single": median(per), "min_single": min(per)},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                   "traffic": recorded_traffic(GDN_PREFILL),
                                   "kernel": "sgla_gdn_chunk_fwd (whole call: per-chunk UT "
                                             "transform, state chain, per-chunk output)",
                                   "algorithmic_bytes_per_launch": nbytes,
                                   "avg_launch_ms": per_avg}}
    del inp, o, fs
    torch.cuda.empty_cache()
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "gdn", seed=4, device=dev, with_beta=True)
    dout = torch.empty((256, 32, 128), dtype=torch.bfloat16, device=dev)
    counter = [0]

    def dstep():
        i = counter[0] % 64
        counter[0] += 1
        sgla.gdn_recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["beta"][i],
                                d["state"], scale=d["scale"], out=dout)

    n_timed = 64 * args.decode_passes
    _, region, per = time_calls(dstep, n_timed, 64, torch)
    per_avg = region / n_timed
    nb = decode_bytes(256, 32, 128, 128) + 256 * 32 * 4
    gbs = nb / (per_avg * 1e-3) / 1e9
    out["decode"] = {"workload": GDN_DECODE, "ms_per_step": region / n_timed,
                     "tokens_per_s": 256 / (region / n_timed * 1e-3),
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                  "traffic": recorded_traffic(GDN_DECODE),
                                  "kernel": "sgla_gdn_recurrent_step",
                                  "algorithmic_bytes_per_launch": nb, "avg_launch_ms": per_avg}}
    del d, dout
    torch.cuda.empty_cache()
    return out


def bench_bf16_state(args, torch, sgla, W, dev):
    """The batched decode (256 x 32 heads, D=128, 64 successive steps) with
    the state pool stored in bf16 (sgla_recurrent_step_ex)."""
    d = W.make_workload(DECODE, seed=4, device=dev)
    steps, N, H, Dk = d["q"].shape
    Dv = d["v"].shape[-1]
    state = d["state"].to(torch.bfloat16)
    del d["state"]
    out = torch.empty((N, H, Dv), dtype=d["v"].dtype, device=dev)
    counter = [0]

    def dstep():
        i = counter[0] % steps
        counter[0] += 1
        sgla.recurrent_step_ex(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state,
                               scale=d["scale"], out=out)

    n_timed = steps * args.decode_passes
    _, region, per = time_calls(dstep, n_timed, steps, torch)
    per_avg = region / n_timed
    nb = decode_bytes(N, H, Dk, Dv, state_elem=2)
    gbs = nb / (per_avg * 1e-3) / 1e9
    del d, state, out
    torch.cuda.empty_cache()
    return {"workload": DECODE + " with a bf16 state pool", "steps_timed": n_timed,
            "ms_per_step": region / n_timed, "tokens_per_s": N / (region / n_timed * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(DECODE_BF16),
                         "kernel": "sgla_recurrent_step_ex (bf16 state)",
                         "algorithmic_bytes_per_launch": nb, "avg_launch_ms": per_avg}}


def bench_epilogue(args, torch, sgla, W, dev):
    """The output epilogue (RMSNorm over all 32 heads of a token, sigmoid
    gate) on the prefill's output shape: 8192 tokens x 4096, bf16."""
    rows, width = 8192, 4096
    inp = W.make_epilogue(rows, width, "bf16", seed=args.seed, device=dev)
    out = torch.empty_like(inp["o"])

    def step():
        sgla.out_norm_gate(inp["o"], inp["z"], inp["weight"], out=out)

    _, region, per = time_calls(step, args.steps, args.warmup, torch)
    per_avg = region / args.steps
    nbytes = 3 * rows * width * 2 + width * 4
    gbs = nbytes / (per_avg * 1e-3) / 1e9
    del inp, out
    return {"workload": "out_norm_gate bf16 %d tokens x %d (32 heads x 128)" % (rows, width),
            "ms_per_call": region / args.steps, "tokens_per_s": rows / (region / args.steps * 1e-3),
            "per_call_ms": {"mean": per_avg, "median_single": median(per), "min_single": min(per)},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": recorded_traffic(EPILOGUE),
                         "kernel": "sgla_out_norm_gate",
                         "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": per_avg}}


def bench_prologue(args, torch, sgla, W, dev):
    """Prefill and decode through the q/k-prologue entry points: same shapes
    as the plain lines, q and k drawn before normalisation (the "raw"
    preset), RMSNorm weights 1 + N(0, 0.1^2), RoPE base 10000."""
    out = {}
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "raw", seed=args.seed, device=dev)
    qw, kw = W.norm_weights(128, seed=args.seed, device=dev)
    o = torch.empty_like(inp["v"])
    fs = torch.empty((1, 32, 128, 128), dtype=torch.float32, device=dev)

    def step():
        sgla.chunk_fwd_qk_norm_rope(inp["q"], inp["k"], inp["v"], inp["g"], qw, kw,
                                    scale=inp["scale"], out=o, final_state=fs)

    _, region, per = time_calls(step, args.steps, args.warmup, torch)
    per_avg = region / args.steps
    nbytes = prefill_bytes(1, 8192, 32, 128, 128) + 2 * 128 * 4
    gbs = nbytes / (per_avg * 1e-3) / 1e9
    out["prefill"] = {"workload": PREFILL + " with raw q/k", "ms_per_call": region / args.steps,
                      "tokens_per_s": 8192 / (region / args.steps * 1e-3),
                      "per_call_ms": {"mean": per_avg, "median_single": median(per), "min_single": min(per)},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                   "traffic": recorded_traffic(PREFILL_PRO),
                                   "kernel": "sgla_chunk_fwd_qk_norm_rope (whole call)",
                                   "algorithmic_bytes_per_launch": nbytes,
                                   "avg_launch_ms": per_avg}}
    del inp, o, fs
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "raw", seed=4, device=dev)
    dqw, dkw = W.norm_weights(128, seed=4, device=dev)
    dout = torch.empty((256, 32, 128), dtype=torch.bfloat16, device=dev)
    counter = [0]

    def dstep():
        i = counter[0] % 64
        counter[0] += 1
        sgla.recurrent_step_qk_norm_rope(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["state"],
                                         dqw, dkw, d["pos"][i], scale=d["scale"], out=dout)

    n_timed = 64 * args.decode_passes
    _, region, per = time_calls(dstep, n_timed, 64, torch)
    per_avg = region / n_timed
    nb = decode_bytes(256, 32, 128, 128) + 256 * 4 + 2 * 128 * 4
    gbs = nb / (per_avg * 1e-3) / 1e9
    out["decode"] = {"workload": DECODE + " with raw q/k", "ms_per_step": region / n_timed,
                     "tokens_per_s": 256 / (region / n_timed * 1e-3),
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                  "traffic": recorded_traffic(DECODE_PRO),
                                  "kernel": "sgla_recurrent_step_qk_norm_rope",
                                  "algorithmic_bytes_per_launch": nb, "avg_launch_ms": per_avg}}
    del d, dout
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    sys.exit(main())

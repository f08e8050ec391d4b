#!/usr/bin/env python3
"""Benchmark of the Simple GLA hot path on one MI355X.

One step = one chunked prefill of a lightning layer (B=1, H=32, T=8192,
Dk=Dv=128, bf16 in, fp32 state out) through ``sgla_chunk_fwd_ex`` with a
caller workspace. The headline times each of K calls on its own, after a pass
that reads a 1 GiB buffer so that q, k, v come from HBM and not from the
memory-side cache (read, not written: a written buffer would leave dirty lines
whose write-back lands inside the timed call); ``value`` is prefill tokens/s
over those calls. The same calls back to back are reported in
``back_to_back``.

Also reported, each with its own roofline object: a stream copy on the same
GPU (``stream_copy``), the 65,536-token continuation with an initial state and
its split at 32,768 as two chained calls (``long``), the 524,288-token packed
varlen prefill (``varlen``), the fused decode step (256 sequences x 32 heads,
64 successive steps, ``decode``), a cache-resident prefill that measures the
kernels' compute rate (``mfma.cache_resident``), and the prologue, bf16-state,
epilogue and gated-delta-rule entry points.

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

LONG = "prefill_bf16_h32_t65536_d128_cont"
VARLEN = "varlen_bf16_h32_d128_8seq_512k"
PREFILL_PRO = PREFILL + "+qk_norm_rope"
DECODE_PRO = DECODE + "+qk_norm_rope"
DECODE_BF16 = DECODE + "+bf16_state"
EPILOGUE = "out_norm_gate_bf16_8192x4096"
GDN_PREFILL = "gdn_prefill_bf16_h32_t8192_d128"
GDN_DECODE = "gdn_decode_bf16_n256_h32_d128_x64"
KDA_PREFILL = "kda_prefill_bf16_h32_t8192_d128"
KDA_DECODE = "kda_decode_bf16_n256_h32_d128_x64"
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32, vendor figure: dense matrix cores and vector ALUs alike
# The kernels of one call of each workload, as rocprofv3 names them.
CALL_KERNELS = {
    PREFILL: ["state_halves_kernel", "chunk_halves_kernel"],
    PREFILL_PRO: ["chunk_mfma_kernel<true, true>", "scan_kernel<128, 128>",
                  "chunk_mfma_kernel<false, true>"],
    LONG: ["chunk_mfma_kernel<true, false>", "chunk_halves_kernel"],
    VARLEN: ["plan_kernel", "chunk_mfma_kernel<true, false>", "scan_kernel<128, 128>",
             "chunk_mfma_kernel<false, false>"],
    DECODE: ["recurrent_step_kernel<unsigned short, 128, 128, false, float>"],
    DECODE_PRO: ["recurrent_step_kernel<unsigned short, 128, 128, true, float>"],
    DECODE_BF16: ["recurrent_step_kernel<unsigned short, 128, 128, false, unsigned short>"],
    EPILOGUE: ["out_norm_gate_kernel<unsigned short, 2>"],
    GDN_PREFILL: ["gdn_prep_kernel", "gdn_chain_kernel", "gdn_output_kernel"],
    GDN_DECODE: ["gdn_step_kernel<unsigned short, 128, 128, false>"],
    KDA_PREFILL: ["kda_prep_kernel<unsigned short, 128, 128, false>", "kda_chain_kernel<128, 128>",
                  "kda_output_kernel<unsigned short, 128, 128, false>"],
    KDA_DECODE: ["gdn_step_kernel<unsigned short, 128, 128, true>"],
}


# The sources each workload's kernels are built from, besides the shared ones
# (headers, the host code that picks launch shapes, the build flags).
WORKLOAD_SOURCES = {
    PREFILL: ["chunk_mfma.hip", "chunk_plan.hip", "chunk_halves.hip"],
    LONG: ["chunk_mfma.hip", "chunk_plan.hip", "chunk_halves.hip"],
    VARLEN: ["chunk_mfma.hip", "chunk_plan.hip"],
    PREFILL_PRO: ["chunk_mfma.hip", "chunk_plan.hip"],
    DECODE: ["recurrent_step.hip"],
    DECODE_PRO: ["recurrent_step.hip"],
    DECODE_BF16: ["recurrent_step.hip"],
    EPILOGUE: ["out_norm_gate.hip"],
    GDN_PREFILL: ["gdn_chunk.hip"],
    GDN_DECODE: ["gdn_step.hip"],
    KDA_PREFILL: ["kda_chunk.hip", "chunk_plan.hip"],
    KDA_DECODE: ["gdn_step.hip"],
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


MFMA_RECORD = os.path.join(ROOT, "profiles", "mfma.json")


def recorded_mfma(workload):
    """Matrix-core busy fraction per kernel of one call, from the committed
    counter record (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE cycles of
    every SIMD), or None when there is none or the kernels changed since."""
    try:
        with open(MFMA_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("kernels")


def recorded_issued(workload):
    """Matrix-core flops one call issues (bf16 and fp32), from the committed
    counter record (SQ_INSTS_VALU_MFMA_MOPS_* x 512 summed over the call's
    kernels), or None when there is none or the kernels changed since."""
    try:
        with open(MFMA_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(workload) or "issued" not in entry:
        return None
    return entry["issued"]


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


def _load_record(path):
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def record_traffic(fetch_dir, write_dir, workloads=None, calib_bytes=256 << 20):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run of
    ``bench.py --copy-calibration`` into HBM bytes per call.

    Both counters are in KiB per dispatch. Each is scaled by what it reads
    for the fp32 negation pass of known size (calib_bytes read and written),
    averaged per kernel, and summed over the kernels of one call of each
    workload (CALL_KERNELS). Writes profiles/traffic.json keyed by workload,
    with the hash of the kernel sources the counters were taken on; with
    ``workloads`` only those entries are replaced (the runs then hold only
    their kernels: several workloads share kernel names)."""
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

    rec = _load_record(TRAFFIC_RECORD)
    rec["_calibration"] = {"fetch_scale": f_scale, "write_scale": w_scale,
                           "pass": "fp32 negation, %d bytes read and written" % calib_bytes}
    for wl, parts in CALL_KERNELS.items():
        if workloads and wl not in workloads:
            continue
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


def _update_entry(rec, wl, fields):
    """Merge fields into a workload's entry; an entry taken on other kernel
    sources is dropped first."""
    h = kernel_source_hash(wl)
    entry = rec.get(wl)
    if not entry or entry.get("source_hash") != h:
        entry = {"source_hash": h}
    entry.update(fields)
    rec[wl] = entry


def record_mops(pmc_dir, workloads=None):
    """Matrix-core flops issued by each kernel of a call, from a rocprofv3
    --pmc run with SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_INSTS_VALU_MFMA_MOPS_F32
    (units of 512 flops), averaged per kernel and summed over the call.
    Merged into profiles/mfma.json beside the busy fractions."""
    bf = _per_kernel_avg(_counter_rows(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
    f32 = _per_kernel_avg(_counter_rows(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_F32"))

    def find(pattern):
        names = [n for n in bf if pattern in n and n in f32]
        return names[0] if len(names) == 1 else None

    rec = _load_record(MFMA_RECORD)
    rec["_issued"] = "SQ_INSTS_VALU_MFMA_MOPS_BF16 and _F32 x 512 flops, per kernel and per call"
    for wl, parts in CALL_KERNELS.items():
        if workloads and wl not in workloads:
            continue
        kern = {}
        for pat in parts:
            n = find(pat)
            if n is None:
                kern = None
                break
            kern[pat] = {"bf16": bf[n] * 512.0, "f32": f32[n] * 512.0}
        if kern:
            _update_entry(rec, wl, {"issued": {
                "kernels": kern,
                "bf16_per_call": sum(v["bf16"] for v in kern.values()),
                "f32_per_call": sum(v["f32"] for v in kern.values())}})
    os.makedirs(os.path.dirname(MFMA_RECORD), exist_ok=True)
    with open(MFMA_RECORD, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


def record_mfma(pmc_dir, workloads=None, xcds=8, simds=1024):
    """Matrix-core busy fraction of each kernel of a call, from a rocprofv3
    --pmc run with SQ_VALU_MFMA_BUSY_CYCLES (busy cycles summed over every
    SIMD) and GRBM_GUI_ACTIVE (active cycles summed over the XCDs):
    busy / (active / xcds * simds). Writes profiles/mfma.json keyed by
    workload, with the hash of the kernel sources the counters were taken on."""
    busy = _per_kernel_avg(_counter_rows(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES"))
    active = _per_kernel_avg(_counter_rows(pmc_dir, "GRBM_GUI_ACTIVE"))

    def find(pattern):
        names = [n for n in busy if pattern in n and n in active]
        return names[0] if len(names) == 1 else None

    rec = _load_record(MFMA_RECORD)
    rec["_formula"] = ("SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs * %d SIMDs)"
                       % (xcds, simds))
    for wl, parts in CALL_KERNELS.items():
        if workloads and wl not in workloads:
            continue
        kern = {}
        for pat in parts:
            n = find(pat)
            if n is None:
                kern = None
                break
            kern[pat] = busy[n] / (active[n] / xcds * simds) if active[n] else 0.0
        if kern:
            _update_entry(rec, wl, {"kernels": kern})
    os.makedirs(os.path.dirname(MFMA_RECORD), exist_ok=True)
    with open(MFMA_RECORD, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


def issued_reading(issued, dense_flops, ms):
    """The matrix-core flops a call issues (counter record) as a rate, a
    fraction of the bf16 dense peak, and a multiple of the dense-tile
    algorithmic flops (what the kernels recompute or split into hi/lo pairs)."""
    if not issued:
        return None
    fl = issued["bf16_per_call"]
    return {"bf16_flops_per_call": fl, "tflops": fl / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS,
            "recompute_factor": fl / dense_flops}


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
    """Per-call times with the caches emptied before each call: a 1 GiB buffer
    is read (summed) between calls, outside the timed events, so the call's
    inputs come from HBM rather than the 256 MB memory-side cache. Reading
    leaves the cache full of clean lines; overwriting the buffer instead would
    leave dirty lines, and their write-back during the timed call made every
    kernel measured that way two to three times slower."""
    flush = torch.ones(flush_bytes // 4, dtype=torch.float32, device=dev)
    per = []
    for _ in range(reps):
        sink = flush.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    del flush, sink
    return per


def stream_copy(torch, dev, nbytes=1 << 30, reps=20):
    """A 1 GiB -> 1 GiB fp32 copy (torch's copy kernel), back to back: the
    HBM rate a plain stream reaches on this GPU (2 * nbytes per copy)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes_per_copy": 2 * nbytes, "ms": ms, "GBs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "kernel": "torch copy_ of 1 GiB fp32, back to back"}


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
    ap.add_argument("--steps", type=int, default=50,
                    help="timed prefill calls (each after a cache flush; also back to back)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-passes", type=int, default=3,
                    help="timed passes of 64 decode steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", choices=["all", "prefill", "long", "varlen", "decode", "prologue",
                                       "epilogue", "bf16-state", "gdn", "kda"], default="all")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB elementwise pass (for counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: write profiles/traffic.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of this script with --copy-calibration")
    ap.add_argument("--workloads", nargs="+", metavar="W",
                    help="with --record-traffic / --record-mfma: the workloads the runs hold")
    ap.add_argument("--no-b2b", action="store_true",
                    help="time the prefill only after cache flushes (profiler runs)")
    ap.add_argument("--record-mops", metavar="PMC_DIR",
                    help="write the matrix-core flops issued per call into profiles/mfma.json from a "
                         "rocprofv3 --pmc run with SQ_INSTS_VALU_MFMA_MOPS_BF16 and _F32")
    ap.add_argument("--record-mfma", metavar="PMC_DIR",
                    help="no GPU work: write profiles/mfma.json from a rocprofv3 --pmc run with "
                         "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the 65,536-token workload's split (two chained calls), so that a "
                         "profiler's per-kernel averages hold whole calls only")
    ap.add_argument("--long-steps", type=int, default=5,
                    help="timed calls of the 65,536-token and the packed varlen workloads")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(*args.record_traffic, workloads=args.workloads)
    if args.record_mfma:
        return record_mfma(args.record_mfma, workloads=args.workloads)
    if args.record_mops:
        return record_mops(args.record_mops, workloads=args.workloads)
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
              "data": "synthetic (seeded; q,k rows N(0,1) scaled to unit RMS, isotropic, so the "
                      "RoPE rotation would leave their distribution unchanged and is not applied; "
                      "v ~ N(0,1); g = log sigmoid(N(4,1)))"}

    if args.only in ("all", "prefill"):
        result["stream_copy"] = stream_copy(torch, dev)
        inp = W.make_workload(PREFILL, seed=args.seed, device=dev)
        B, T, H, Dk = inp["q"].shape
        Dv = inp["v"].shape[-1]
        out = torch.empty_like(inp["v"])
        fs = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, sgla.chunk_workspace_size(B, T, H, Dk, Dv)), dtype=torch.uint8,
                         device=dev)

        def step():
            sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], None, None, inp["scale"],
                           out=out, final_state=fs, workspace=ws)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fl = time_flushed(step, args.steps, torch, dev)
        wall = time.perf_counter() - t0
        ms_step = sum(fl) / len(fl)
        if args.no_b2b:
            region, per = float("nan"), [float("nan")]
        else:
            _, region, per = time_calls(step, args.steps, 0, torch)
        b2b = region / args.steps
        nbytes = prefill_bytes(B, T, H, Dk, Dv)
        flops = prefill_flops(B, T, H, Dk, Dv)
        achieved = nbytes / (ms_step * 1e-3) / 1e9
        copy_gbs = result["stream_copy"]["GBs"]
        result.update({
            "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step,
            "config": {"workload": PREFILL, "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv,
                       "chunk": 64, "scale": inp["scale"], "initial_state": "zero",
                       "final_state": "fp32", "timing": "each call after a 1 GiB read pass",
                       "gpu": props.name},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "frac_of_stream_copy": achieved / copy_gbs,
                         "traffic": recorded_traffic(PREFILL),
                         "kernel": "sgla_chunk_fwd_ex (whole call: segment-state and "
                                   "value-half output kernels)",
                         "algorithmic_bytes_per_launch": nbytes,
                         "avg_launch_ms": ms_step},
            "mfma": {"useful_tflops": flops / (ms_step * 1e-3) / 1e12,
                     "useful_frac_of_bf16_peak": flops / (ms_step * 1e-3) / 1e12 /
                     BF16_DENSE_PEAK_TFLOPS,
                     "dense_tile_flops_per_launch": flops,
                     "busy": recorded_mfma(PREFILL),
                     "issued": issued_reading(recorded_issued(PREFILL), flops, ms_step)},
            "wall_s_timed": wall,
            "per_call_ms": {"mean": ms_step, "median": median(fl), "min": min(fl),
                            "max": max(fl)},
            "back_to_back": {"note": "the same calls with no flush between them; q, k, v then "
                                     "stay partly in the 256 MB memory-side cache",
                             "ms_per_call": b2b, "tokens_per_s": B * T / (b2b * 1e-3),
                             "achieved_GBs": nbytes / (b2b * 1e-3) / 1e9,
                             "frac": nbytes / (b2b * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "median_single": median(per), "min_single": min(per)},
        })
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(inp, W)
        del inp, out, fs, ws
        torch.cuda.empty_cache()
        if args.only == "all":
            result["mfma"]["cache_resident"] = bench_cache_resident(args, torch, sgla, W, dev)
    if args.only in ("all", "long"):
        result["long"] = bench_long(args, torch, sgla, W, dev)
        if args.only == "long":
            e = result["long"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_call"], "config": {"workload": LONG},
                           "roofline": e["roofline"]})
    if args.only in ("all", "varlen"):
        result["varlen"] = bench_varlen(args, torch, sgla, W, dev)
        if args.only == "varlen":
            e = result["varlen"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_call"], "config": {"workload": VARLEN},
                           "roofline": e["roofline"]})

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
    if args.only in ("all", "kda"):
        result["kda"] = bench_kda(args, torch, sgla, W, dev)
        if args.only == "kda":
            e = result["kda"]["prefill"]
            result.update({"value": e["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": e["ms_per_call"],
                           "config": {"workload": e["workload"]}, "roofline": e["roofline"]})
    print(json.dumps(result), flush=True)
    return 0


def _prefill_caller(sgla, torch, inp, dev):
    """A prefill call on a named workload's inputs with preallocated outputs
    and workspace, and its algorithmic bytes."""
    B, T, H, Dk = inp["q"].shape
    Dv = inp["v"].shape[-1]
    cu = inp["cu_seqlens"]
    N = B if cu is None else cu.numel() - 1
    Barg = N if cu is not None else B
    out = torch.empty_like(inp["v"])
    fs = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sgla.chunk_workspace_size(Barg, T, H, Dk, Dv, varlen=cu is not None)),
                     dtype=torch.uint8, device=dev)
    s0 = inp["initial_state"]

    def call():
        sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], s0, cu, inp["scale"], out=out,
                       final_state=fs, workspace=ws)

    tokens = B * T * H * (2 * Dk * 2 + 2 * Dv * 2 + 4)
    states = N * H * Dk * Dv * 4 * (2 if s0 is not None else 1)
    return call, tokens + states, out, fs, ws


def _region(fn, n, torch):
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def bench_long(args, torch, sgla, W, dev):
    """The 65,536-token continuation (B=1, H=32, D=128, bf16, fp32 initial
    state ~ N(0, 0.02^2)), and the same tokens as two chained calls split at
    32,768 (the second starts from the first's final state). Its inputs (1.5
    GiB) exceed the memory-side cache, so back-to-back calls read HBM."""
    inp = W.make_workload(LONG, seed=3, device=dev)
    call, nbytes, out, fs, ws = _prefill_caller(sgla, torch, inp, dev)
    T = inp["q"].shape[1]
    call()
    torch.cuda.synchronize()
    ms = _region(call, args.long_steps, torch)
    res = {"workload": LONG, "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "traffic": recorded_traffic(LONG),
                        "kernel": "sgla_chunk_fwd_ex (whole call: segment-state and "
                                  "value-half output kernels)",
                        "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms},
           "mfma_busy": recorded_mfma(LONG),
           "mfma_issued": issued_reading(recorded_issued(LONG),
                                         prefill_flops(1, T, 32, 128, 128), ms)}
    if args.no_split:
        del inp, out, fs, ws
        torch.cuda.empty_cache()
        return res
    t = W.WORKLOADS[LONG]["split"]
    halves = []
    for part in ("a", "b"):
        sl = slice(0, t) if part == "a" else slice(t, T)
        d = {x: inp[x][:, sl].contiguous() for x in ("q", "k", "v", "g")}
        d.update(cu_seqlens=None, scale=inp["scale"],
                 initial_state=inp["initial_state"] if part == "a" else None)
        halves.append(d)
    ca, nba, _, fsa, wsa = _prefill_caller(sgla, torch, halves[0], dev)
    halves[1]["initial_state"] = fsa
    cb, nbb, _, _, wsb = _prefill_caller(sgla, torch, halves[1], dev)

    def chained():
        ca()
        cb()

    chained()
    torch.cuda.synchronize()
    ms2 = _region(chained, args.long_steps, torch)
    res["split"] = {"at": t, "ms_per_pair": ms2, "tokens_per_s": T / (ms2 * 1e-3),
                    "achieved_GBs": (nba + nbb) / (ms2 * 1e-3) / 1e9,
                    "frac": (nba + nbb) / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del inp, out, fs, ws, halves, fsa, wsa, wsb
    torch.cuda.empty_cache()
    return res


def bench_varlen(args, torch, sgla, W, dev):
    """The packed varlen prefill: 8 sequences, 524,288 tokens in total, lengths
    log-uniform in [4096, 262144] rescaled to the total, H=32, D=128, bf16."""
    inp = W.make_workload(VARLEN, seed=5, device=dev)
    call, nbytes, out, fs, ws = _prefill_caller(sgla, torch, inp, dev)
    T = inp["q"].shape[1]
    lengths = (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1]).tolist()
    call()
    torch.cuda.synchronize()
    ms = _region(call, args.long_steps, torch)
    res = {"workload": VARLEN, "lengths": lengths, "ms_per_call": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "traffic": recorded_traffic(VARLEN),
                        "kernel": "sgla_chunk_fwd_ex (whole call: plan, segment-state, scan "
                                  "and output kernels)",
                        "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms},
           "mfma_busy": recorded_mfma(VARLEN)}
    del inp, out, fs, ws
    torch.cuda.empty_cache()
    return res


def bench_cache_resident(args, torch, sgla, W, dev):
    """The prefill kernels' compute rate: B=2, T=2048, H=32, D=128 (64 MiB of
    q, k, v and o) back to back, so every call finds its inputs in the caches
    and the call is bound by the kernels' own work, not by HBM. Reported as
    dense-tile flops per second over the bf16 matrix-core peak."""
    inp = W.make_prefill(2, 2048, 32, 128, 128, "bf16", "lightning", seed=7, device=dev)
    call, nbytes, out, fs, ws = _prefill_caller(sgla, torch, inp, dev)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    ms = _region(call, 50, torch)
    flops = prefill_flops(2, 2048, 32, 128, 128)
    del inp, out, fs, ws
    torch.cuda.empty_cache()
    return {"workload": "prefill B=2 T=2048 H=32 D=128 bf16, back to back (cache-resident)",
            "ms_per_call": ms, "useful_tflops": flops / (ms * 1e-3) / 1e12,
            "useful_frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / BF16_DENSE_PEAK_TFLOPS,
            "achieved_GBs": nbytes / (ms * 1e-3) / 1e9}


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
    ws = torch.empty(sgla.gdn_workspace_size(1, 8192, 32, 128, 128), dtype=torch.uint8, device=dev)

    def step():
        sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                           scale=inp["scale"], out=o, final_state=fs, workspace=ws)

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


def kda_prefill_flops(T, H, D):
    """Algorithmic fp32 FLOPs of the chunked KDA per call (chunks of 64, Dk =
    Dv = D): per chunk and head the per-dim-decayed products M (63 * 64 / 2
    pairs), L (64 * 65 / 2), the triangular W = T X and U = T V (64 * 65 / 2
    rows each), new_v = U - W S, the state update and the inter output (64 x D
    x D each), the intra output L new_v (64 * 65 / 2), at 2 FLOPs per
    multiply-add; the 64 x 64 triangular solve is left out."""
    per = 2 * D * (2016 + 4 * 2080) + 3 * 2 * 64 * D * D
    return per * (T // 64) * H


def bench_kda(args, torch, sgla, W, dev):
    """The gated delta rule with one gate per key dim (KDA) on the same
    shapes: prefill B=1, T=8192, H=32, Dk=Dv=128 (sgla_kda_chunk_fwd, fp32
    contractions on the matrix cores, the pairwise decay factors on the
    vector ALUs) and the batched decode, 256 x 32 heads, 64
    successive steps (sgla_kda_recurrent_step); "kda" inputs (L2-normalised q
    and k, per-dim gates, beta = sigmoid(N(0, 1)))."""
    out = {}
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "kda", seed=args.seed, device=dev,
                         with_beta=True)
    o = torch.empty_like(inp["v"])
    fs = torch.empty((1, 32, 128, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(sgla.kda_workspace_size(1, 8192, 32, 128, 128), dtype=torch.uint8, device=dev)

    def step():
        sgla.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                           scale=inp["scale"], out=o, final_state=fs, workspace=ws)

    _, region, per = time_calls(step, args.steps, args.warmup, torch)
    per_avg = region / args.steps
    flops = kda_prefill_flops(8192, 32, 128)
    tf = flops / (per_avg * 1e-3) / 1e12
    # prefill_bytes counts one gate float per token and head; KDA reads 128,
    # and beta: 128 more floats per token and head.
    nbytes = prefill_bytes(1, 8192, 32, 128, 128) + 8192 * 32 * 128 * 4
    out["prefill"] = {"workload": KDA_PREFILL, "ms_per_call": per_avg,
                      "tokens_per_s": 8192 / (per_avg * 1e-3),
                      "per_call_ms": {"mean": per_avg, "median_single": median(per), "min_single": min(per)},
                      "achieved_GBs": nbytes / (per_avg * 1e-3) / 1e9,
                      "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": tf / FP32_PEAK_TFLOPS,
                                   "traffic": recorded_traffic(KDA_PREFILL),
                                   "kernel": "sgla_kda_chunk_fwd (whole call: per-chunk UT "
                                             "transform, state chain, per-chunk output; fp32)",
                                   "algorithmic_flops_per_launch": flops,
                                   "avg_launch_ms": per_avg}}
    iss = recorded_issued(KDA_PREFILL)
    out["prefill"]["mfma"] = {
        "busy": recorded_mfma(KDA_PREFILL),
        "issued": None if not iss else {
            "f32_flops_per_call": iss["f32_per_call"], "bf16_flops_per_call": iss["bf16_per_call"],
            "f32_tflops": iss["f32_per_call"] / (per_avg * 1e-3) / 1e12,
            "f32_frac_of_peak": iss["f32_per_call"] / (per_avg * 1e-3) / 1e12 / FP32_PEAK_TFLOPS}}
    del inp, o, fs, ws
    torch.cuda.empty_cache()
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "kda", seed=4, device=dev, with_beta=True)
    dout = torch.empty((256, 32, 128), dtype=torch.bfloat16, device=dev)
    counter = [0]

    def dstep():
        i = counter[0] % 64
        counter[0] += 1
        sgla.kda_recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["beta"][i],
                                d["state"], scale=d["scale"], out=dout)

    n_timed = 64 * args.decode_passes
    _, region, per = time_calls(dstep, n_timed, 64, torch)
    per_avg = region / n_timed
    nb = decode_bytes(256, 32, 128, 128) + 256 * 32 * 128 * 4
    gbs = nb / (per_avg * 1e-3) / 1e9
    out["decode"] = {"workload": KDA_DECODE, "ms_per_step": per_avg,
                     "tokens_per_s": 256 / (per_avg * 1e-3),
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                  "traffic": recorded_traffic(KDA_DECODE),
                                  "kernel": "sgla_kda_recurrent_step",
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
    ws = torch.empty(max(1, sgla.chunk_workspace_size(1, 8192, 32, 128, 128, prologue=True)),
                     dtype=torch.uint8, device=dev)

    def step():
        sgla.chunk_fwd_qk_norm_rope(inp["q"], inp["k"], inp["v"], inp["g"], qw, kw,
                                    scale=inp["scale"], out=o, final_state=fs, workspace=ws)

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
                                   "kernel": "sgla_chunk_fwd_ex with the prologue (whole call)",
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

#!/usr/bin/env python3
"""Throughput of the tensor-parallel activation compression hot path on one MI355X.

One step = every rank's compress of its shard (N bf16 shards already resident
in HBM, one compress launch each) followed by the decompress-reduce of the N
compressed shards with re-quantization for the gather stage -- all of the hot
path. Shards rotate over several input sets so that the working set exceeds
the 256 MB Infinity Cache. Kernels are launched eagerly on one stream.

The headline workload is qwen-tp (8 shards of 32768 x 5120 bf16, FP8
dual-scale with the 128-point Hadamard transform, re-quantized to FP8), the
largest configuration that fits one GPU; the other 8-shard workloads (equarx,
flashcomm) are timed in the same run and reported under "workloads".

Per workload:
  * steps for 0.5 s of wall time (the GPU's clocks rise from idle), then the
    W warm-up steps;
  * timed region: K steps between one pair of HIP events, bracketed by
    synchronizations (no event inside it) -> value, ms_per_step;
  * K more steps with an event at every step boundary -> median, p10, p90;
  * K more steps with events between the compress phase (N launches) and the
    reduce -> each kernel's average launch duration in step context (the
    roofline's denominator);
  * the quality check: the compress and the reduce+requantize round trips on
    a seeded sample of row chunks, GPU against the oracle at the same tensor
    scale (the oracle computes it from the whole tensor itself).

value = N * rows * cols * 2 bytes of bf16 input / step time (GB/s).

Prints one JSON line. --gpus above 1 is refused: the benchmark measures one GPU.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
PREWARM_S = 0.5
PEAK_CLOCK_GHZ = 2.4
HEADLINE = "qwen-tp"
EXTRA = "equarx,flashcomm"
FORMAT_NAMES = ["", "FP8 dual-scale", "INT8 sym", "INT4 asym", "INT8 asym", "FP8 E5M2 dual-scale"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default=EXTRA,
                    help="comma-separated workloads timed after the headline one in the same run "
                         "(reported under 'workloads'); 'none' for the headline alone")
    ap.add_argument("--scale-mode", choices=["delayed", "auto", "given"], default="delayed",
                    help="FP8 tensor scale: delayed (abs-max of the previous step, one pass), "
                         "auto (abs-max pre-pass of this tensor) or given (a fixed g, no workspace)")
    ap.add_argument("--launch", choices=["graph", "eager"], default="eager")
    ap.add_argument("--fp8-codes", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 workloads: the code format of the dual-scale codec (E5M2 is the variant "
                         "format 5)")
    ap.add_argument("--prewarm", type=float, default=PREWARM_S,
                    help="seconds of steps before the warm-up steps (0 for profiler counter passes)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-quality", action="store_true", help="skip the GPU-vs-oracle quality check")
    ap.add_argument("--ring", action="store_true",
                    help="INT workloads: also time one quantized ring reduce-scatter hop (taco_ring_hop) at "
                         "full size and run the full-loop and semi-loop rings over the shards for their MSE")
    ap.add_argument("--reorder", action="store_true",
                    help="also time the reordered compress (data-driven reshaping) and compare the rel-MSE with "
                         "and without the reorder, for the workload's codec and for INT8 / INT4 on its data")
    ap.add_argument("--no-consumer", action="store_true",
                    help="skip the consumer measurement (decode + GEMM vs the fused decode-GEMM) of the "
                         "workloads whose gather stage has no Hadamard transform")
    ap.add_argument("--overlap", action="store_true",
                    help="sweep launch caps of the codec beside the bf16 GEMM that produces the next "
                         "activation (workloads with a GEMM, qwen-tp; without the flag only the uncapped "
                         "overlap is measured)")
    ap.add_argument("--rank-share", action="store_true",
                    help="also time the decompress-reduce at one rank's share: (rows / N) x cols from N sources "
                         "(kept out of the default run so the profiled runs hold only full-size launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) for counter calibration")
    ap.add_argument("--summarize", nargs="+", metavar="PATH",
                    help="FETCH_DIR WRITE_DIR TRACE_DIR [TRACE_LOG]: turn rocprofv3 FETCH_SIZE / WRITE_SIZE / "
                         "kernel-trace output (and the bench line printed under the trace) into the "
                         "profiles/ summaries and exit")
    ap.add_argument("--summarize-issue", metavar="DIR",
                    help="turn a rocprofv3 --pmc run of instruction and busy counters (with --kernel-trace) into "
                         "profiles/issue_<kernel>_<workload>.txt and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "NAME"),
                    help="write profiles/kernels_NAME_trace.txt: kernel-trace statistics of every kernel of this "
                         "library in one profiled run (with --command)")
    ap.add_argument("--summarize-consumer", nargs=2, metavar=("TRACE_DIR", "MFMA_DIR"),
                    help="write profiles/consumer_gemm.txt from a kernel trace of the default bench command and "
                         "an MFMA counter pass (then exit)")
    ap.add_argument("--command", default="", help="with --summarize: the profiled command, recorded")
    return ap.parse_args()


def algorithmic_bytes(w):
    """Bytes each kernel must move, from the formats' definitions."""
    n = w.n
    if w.in_format in (1, 5):
        cbytes, meta_in = n, n // w.in_block          # FP8 codes + int8 exponent per block
        hdr = 16
    elif w.in_format == 2:
        cbytes, meta_in, hdr = n, 4 * (n // 64), 0
    else:
        cbytes = n // 2 if w.in_format == 3 else n
        meta_in, hdr = 5 * (n // 128), 0              # float scale + uint8 zero point
    compress = 2 * n + cbytes + meta_in + hdr
    shard = cbytes + meta_in + hdr
    if w.out_format is None:
        out = 4 * n
    elif w.out_format in (1, 5):
        out = n + n // w.out_block + 16
    elif w.out_format == 2:
        out = n + 4 * (n // 64)
    else:
        out = n + 5 * (n // 128)
    reduce = w.shards * shard + out
    return compress, reduce


def decode_bytes(w):
    """Bytes the consumer-side decode of the gather-stage output to bf16 moves."""
    n = w.n
    if w.out_format in (1, 5):
        src = n + n // w.out_block + 16
    elif w.out_format == 2:
        src = n + 4 * (n // 64)
    else:
        src = n + 5 * (n // 128)
    return src + 2 * n


def kernel_patterns(w):
    """Name prefixes (as the profiler prints them) of the compress and reduce
    kernels this workload launches."""
    if w.in_format in (1, 5) and w.hadamard:
        comp = f"k_fp8_had_compress<{7 if w.in_block == 128 else w.in_block.bit_length() - 1}, "
    else:
        comp = f"k_quantize<{w.in_format}, {w.in_block}, false, false, false>"
    nmax = 2 if w.shards <= 2 else 4 if w.shards <= 4 else 8 if w.shards <= 8 else 16
    fout = w.out_format if w.out_format else w.in_format
    bout = w.out_block if w.out_format else w.in_block
    red = f"k_reduce<{w.in_format}, {w.in_block}, {fout}, {bout}, {nmax}>"
    return {"compress": comp, "reduce": red}


def kernel_source_hash():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_compression_tensor_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name, workload, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{name}_{workload}_counters.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_BYTES = 256 << 20


def _csv_rows(d, suffix):
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _trace_stats(trace_dir, concurrent_with, by_grid=()):
    """Per-kernel statistics (calls, average, min, max, total in ns) from the
    per-dispatch kernel trace, leaving out every dispatch that ran at the same
    time as a dispatch of another kernel whose name contains one of the
    patterns in `concurrent_with` (e.g. the codec launches timed beside a
    library GEMM). Kernels whose name contains a pattern in `by_grid` are
    kept apart by grid size (one kernel serving several shapes)."""
    import bisect

    def key(r):
        n = r["Kernel_Name"]
        grid = r.get("Grid_Size_X") or r.get("Grid_Size") or "?"
        return f"{n} [grid {grid}]" if any(p in n for p in by_grid) else n
    rows = [(key(r), int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
            for r in _csv_rows(trace_dir, "kernel_trace.csv")]
    others = sorted((a, b, n) for n, a, b in rows if any(p in n for p in concurrent_with))
    starts = [a for a, _, _ in others]
    ends_max, m = [], 0      # running max of the ends, for the interval test
    for _, b, _ in others:
        m = max(m, b)
        ends_max.append(m)
    stats = {}
    for n, a, b in rows:
        if not any(p in n for p in concurrent_with):
            # the other dispatches that start before this one ends; one of them
            # overlaps it if the latest end among them lies after its start
            i = bisect.bisect_left(starts, b) - 1
            if i >= 0 and ends_max[i] > a:
                continue
        d = b - a
        st = stats.setdefault(n, {"Calls": 0, "TotalDurationNs": 0, "MinNs": d, "MaxNs": d})
        st["Calls"] += 1
        st["TotalDurationNs"] += d
        st["MinNs"] = min(st["MinNs"], d)
        st["MaxNs"] = max(st["MaxNs"], d)
    for st in stats.values():
        st["AverageNs"] = st["TotalDurationNs"] / st["Calls"]
    return stats


def summarize(fetch_dir, write_dir, trace_dir, names, command, trace_log=None):
    """Per-launch HBM bytes of each workload's compress and reduce kernels from
    two counter passes, scaled by what the same counters read for a plain copy
    of COPY_BYTES (read and write), plus the kernel-trace statistics and, when
    the profiled run's output is given, the bench's own event timing in that
    same run; written to profiles/<kernel>_<workload>_counters.txt and
    profiles/kernels_<workload>_trace.txt."""
    import numpy as np
    import workloads as W
    src_hash = kernel_source_hash()
    bench_ms = {}
    if trace_log:
        lines = [l for l in open(trace_log) if l.startswith("{")]
        if lines:
            line = json.loads(lines[-1])
            per = {line["config"]["name"]: line["kernels"]}
            for k, v in (line.get("workloads") or {}).items():
                per[k] = v["kernels"]
            bench_ms = {k: {"compress": v.get("compress_ms"), "reduce": v.get("reduce_ms")} for k, v in per.items()}
    per = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for row in _csv_rows(d, "counter_collection.csv"):
            if row.get("Counter_Name") != cname:
                continue
            per.setdefault((cname, row.get("Kernel_Name", "")), []).append(float(row["Counter_Value"]))
    # the calibration copies are the three largest copy dispatches of the run
    copy_f = sorted((v for (c, k), vs in per.items() if c == "FETCH_SIZE" and "copy" in k.lower() for v in vs),
                    reverse=True)[:3]
    copy_w = sorted((v for (c, k), vs in per.items() if c == "WRITE_SIZE" and "copy" in k.lower() for v in vs),
                    reverse=True)[:3]
    f_fetch = COPY_BYTES / (np.median(copy_f) * 1024) if copy_f else None
    f_write = COPY_BYTES / (np.median(copy_w) * 1024) if copy_w else None
    trace = _trace_stats(trace_dir, concurrent_with=("Cijk",))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for wname in names:
        w = W.WORKLOADS[wname]
        pats = kernel_patterns(w)
        for key, pat in pats.items():
            fk = [(k, vs) for (c, k), vs in per.items() if c == "FETCH_SIZE" and pat in k]
            wk = [(k, vs) for (c, k), vs in per.items() if c == "WRITE_SIZE" and pat in k]
            if not fk or not wk:
                continue
            fk.sort(key=lambda kv: -len(kv[1]))
            wk.sort(key=lambda kv: -len(kv[1]))
            kname = fk[0][0]
            fetch_kib = float(np.median(fk[0][1]))
            write_kib = float(np.median(wk[0][1]))
            hbm = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write if f_fetch and f_write else None
            tr = trace.get(kname)
            path = os.path.join(ROOT, "profiles", f"{key}_{wname}_counters.txt")
            with open(path, "w") as fh:
                fh.write(f"# rocprofv3 hardware counters for {kname}\n")
                fh.write(f"# workload: {wname}\n# command: {command}\n")
                fh.write("# FETCH_SIZE and WRITE_SIZE come from separate --pmc passes (KiB per dispatch,\n"
                         "# median over dispatches); each is scaled by COPY_BYTES / counter of a plain\n"
                         "# device-to-device copy of COPY_BYTES profiled in the same pass.\n")
                fh.write(f"kernel: {kname}\n")
                fh.write(f"source_hash: {src_hash}\n")
                fh.write(f"fetch_kib_per_dispatch: {fetch_kib:.1f}\n")
                fh.write(f"write_kib_per_dispatch: {write_kib:.1f}\n")
                fh.write(f"copy_bytes: {COPY_BYTES}\n")
                fh.write(f"copy_fetch_factor: {f_fetch}\n")
                fh.write(f"copy_write_factor: {f_write}\n")
                fh.write(f"hbm_bytes_per_launch: {hbm}\n")
                fh.write(f"algorithmic_bytes_per_launch: {algorithmic_bytes(w)[0 if key == 'compress' else 1]}\n")
                if tr is not None:
                    fh.write(f"trace_calls: {tr.get('Calls')}\n")
                    fh.write(f"trace_average_ns: {tr.get('AverageNs')}\n")
                    fh.write(f"trace_min_ns: {tr.get('MinNs')}\n")
                    fh.write(f"trace_max_ns: {tr.get('MaxNs')}\n")
                b = bench_ms.get(wname, {}).get(key)
                if b is not None:
                    fh.write("# the bench's own HIP-event average in the profiled run (launches in step\n"
                             "# context, including the gap before each launch, which the profiler widens)\n")
                    fh.write(f"bench_event_average_ns_under_profiler: {b * 1e6:.0f}\n")
            written.append(path)
        if trace:
            # this workload's kernels: its compress, reduce and the decode of its
            # gather-stage format; the device copies are the run's shared reference
            dec = {1: "k_fp8_had_decode", 5: "k_fp8_had_decode"}.get(w.out_format, f"k_dequantize<{w.out_format}, ")
            mine = [n for n in trace if any(p in n for p in pats.values()) or
                    (dec in n and (w.out_format not in (1, 5) or "<7, " + ("true" if w.out_format == 5 else "false") in n))]
            if w.in_format in (1, 5) and w.hadamard:
                mine += [n for n in trace if "k_fp8_had_amax" in n]
            path = os.path.join(ROOT, "profiles", f"kernels_{wname}_trace.txt")
            with open(path, "w") as fh:
                fh.write(f"# rocprofv3 kernel-trace statistics: the kernels of workload {wname}\n"
                         f"# command: {command}\n")
                fh.write("# (kernel durations exclude dispatch gaps; the bench's phase events include them;\n"
                         "# launches that ran at the same time as a library GEMM are left out)\n")
                fh.write(f"source_hash: {src_hash}\n")
                fh.write(f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel\n")
                for name in sorted(set(mine), key=lambda n: -float(trace[n]["TotalDurationNs"])):
                    row = trace[name]
                    fh.write(f"{int(row['Calls']):>6} {float(row['AverageNs']) / 1e3:>9.2f} "
                             f"{float(row['MinNs']) / 1e3:>9.2f} {float(row['MaxNs']) / 1e3:>9.2f}  {name[:160]}\n")
            written.append(path)
    print("\n".join(written))


ISSUE_COUNTERS = ("SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM", "SQ_WAVES",
                  "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE", "GRBM_COUNT")


def summarize_issue(d, names, command):
    """Instruction-issue profile of each workload's compress and reduce: per
    dispatch medians of the SQ / GRBM counters (one --pmc pass with the kernel
    trace, which gives each dispatch's duration), and what follows from them:
    VALU instructions per wave, VALU busy (quad-cycles of VALU work per CU
    over the active cycles of one XCD) and the VALU floor (the VALU
    instructions at one wave64 instruction per 4 cycles on each of the 1024
    SIMDs at the 2.4 GHz peak clock)."""
    import numpy as np
    import workloads as W
    src_hash = kernel_source_hash()
    ctr = {}
    for row in _csv_rows(d, "counter_collection.csv"):
        key = (row.get("Kernel_Name", ""), row.get("Dispatch_Id") or row.get("Correlation_Id"))
        ctr.setdefault(key, {})[row["Counter_Name"]] = ctr.get(key, {}).get(row["Counter_Name"], 0.0) + \
            float(row["Counter_Value"])
    dur = {}
    for row in _csv_rows(d, "kernel_trace.csv"):
        key = (row.get("Kernel_Name", ""), row.get("Dispatch_Id") or row.get("Correlation_Id"))
        dur[key] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    written = []
    for wname in names:
        w = W.WORKLOADS[wname]
        for key, pat in kernel_patterns(w).items():
            rows = [(k, v) for k, v in ctr.items() if pat in k[0]]
            if not rows:
                continue
            kname = rows[0][0][0]
            med = {c: float(np.median([v.get(c, np.nan) for _, v in rows])) for c in ISSUE_COUNTERS}
            ds = [dur[k] for k, _ in rows if k in dur]
            t_ns = float(np.median(ds)) if ds else None
            xcds, cus, simds = 8, 256, 1024
            gui = med["GRBM_GUI_ACTIVE"]
            path = os.path.join(ROOT, "profiles", f"issue_{key}_{wname}.txt")
            with open(path, "w") as fh:
                fh.write(f"# rocprofv3 instruction and busy counters for {kname}\n")
                fh.write(f"# workload: {wname}\n# command: {command}\n")
                fh.write("# per-dispatch medians over the run's dispatches of this kernel; SQ counters are summed\n"
                         "# over shader engines and XCDs, GRBM_GUI_ACTIVE over the 8 XCDs\n")
                fh.write(f"kernel: {kname}\nsource_hash: {src_hash}\ndispatches: {len(rows)}\n")
                for c in ISSUE_COUNTERS:
                    fh.write(f"{c}: {med[c]:.0f}\n")
                floor_ns = med["SQ_INSTS_VALU"] * 4 / simds / PEAK_CLOCK_GHZ
                fh.write(f"valu_floor_ns (SQ_INSTS_VALU * 4 cycles / 1024 SIMDs / 2.4 GHz): {floor_ns:.0f}\n")
                if t_ns:
                    fh.write(f"duration_ns_median: {t_ns:.0f}\n")
                    fh.write(f"duration_over_valu_floor: {t_ns / floor_ns:.3f}\n")
                fh.write(f"valu_insts_per_wave: {med['SQ_INSTS_VALU'] / max(med['SQ_WAVES'], 1):.1f}\n")
                fh.write(f"salu_insts_per_wave: {med['SQ_INSTS_SALU'] / max(med['SQ_WAVES'], 1):.1f}\n")
                fh.write(f"vmem_insts_per_wave: {med['SQ_INSTS_VMEM'] / max(med['SQ_WAVES'], 1):.1f}\n")
                fh.write(f"valu_busy (100 * SQ_ACTIVE_INST_VALU / 256 CUs / (GRBM_GUI_ACTIVE / 8)): "
                         f"{100 * med['SQ_ACTIVE_INST_VALU'] / cus / (gui / xcds):.1f}\n")
            written.append(path)
    print("\n".join(written))


def cpu_baseline(w, seconds):
    """The oracle, as written, on a bounded sample of the same workload: row
    chunks of every shard, compressed and reduced (+ requantized), spread over
    a thread pool (NumPy releases the GIL inside its loops)."""
    import oracle
    from oracle import codecs as cd
    import workloads as W

    cin = cd.Codec(w.in_format, w.in_block, w.hadamard)
    cout = cd.Codec(w.out_format, w.out_block, w.hadamard) if w.out_format else None
    nchunks = (w.rows + W.ROW_CHUNK - 1) // W.ROW_CHUNK
    host_cores = os.cpu_count() or 1
    threads = max(1, min(16, host_cores))

    inputs = {}

    def one(chunk):
        shards = [oracle.compress(cin, inputs[(chunk, r)]) for r in range(w.shards)]
        oracle.decompress_reduce(shards, cout)
        return chunk

    # calibrate on one chunk, then size the sample to the time budget
    for r in range(w.shards):
        inputs[(0, r)] = W.make_shard(w, r, chunks=[0])
    t = time.perf_counter()
    one(0)
    per_chunk = time.perf_counter() - t
    want = max(1, int(seconds * threads / max(per_chunk, 1e-6)))
    chunks = list(range(min(nchunks, max(threads, want))))
    for c in chunks:
        for r in range(w.shards):
            if (c, r) not in inputs:
                inputs[(c, r)] = W.make_shard(w, r, chunks=[c])
    # whole passes over the sample until the time budget is spent (a workload
    # smaller than the budget is run several times over)
    passes = 0
    t = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while True:
            list(ex.map(one, chunks))
            passes += 1
            dt = time.perf_counter() - t
            if dt >= seconds:
                break
    rows = sum(min(W.ROW_CHUNK, w.rows - c * W.ROW_CHUNK) for c in chunks)
    bytes_in = passes * w.shards * rows * w.cols * 2
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = host_cores
    return {"value": round(bytes_in / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host_cores": host_cores, "host_cores_usable": affinity, "threads": threads,
            "sample": f"{rows} of {w.rows} rows of each of the {w.shards} shards ({len(chunks)} chunks of "
                      f"{W.ROW_CHUNK} rows): compress + decompress-reduce"
                      + (" + requantize" if cout else "") + f"; {passes} pass(es), {dt:.1f} s; NumPy float32 "
                      f"oracle over a pool of {threads} threads on a host with {host_cores} cores"}


def oracle_tensor_scale(w, oc, bits):
    """The oracle's data-driven FP8 tensor scale of one whole shard: the abs-max
    of the transformed tensor is the max over row chunks (run in a thread pool),
    and the oracle's own scale rule is applied to it."""
    import numpy as np
    from oracle import codecs as cd
    import workloads as W
    step = W.ROW_CHUNK

    def amax(r0):
        return float(np.max(np.abs(cd.transform(oc, bits[r0:r0 + step]))))

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        A = max(ex.map(amax, range(0, bits.shape[0], step)))
    return cd.auto_tensor_scale(np.float32([A]), oc.format)


def quality(w, ctx):
    """rel-MSE of the compress round trip (shard 0) and of the reduce +
    requantize round trip, GPU against the oracle at the same tensor scale, on
    a seeded sample of row chunks. The GPU compresses the step's first input
    set again with the data-driven tensor scale of each whole tensor (AUTO);
    the oracle computes that scale from the whole tensor itself, so both sides
    quantize the sample rows with the same g and their codes must agree bit for
    bit. The delayed-scale figure (the scale the timed steps used: the previous
    step's abs-max) is reported beside it."""
    import numpy as np
    import torch
    import oracle
    from oracle import codecs as cd
    from oracle.formats import bf16_bits_to_f32
    import quantized_compression_tensor_amd as T
    import workloads as W

    dev = "cuda"
    c_in, c_out = ctx["c_in"], ctx["c_out"]
    oc = cd.Codec(w.in_format, w.in_block, w.hadamard)
    ocout = cd.Codec(w.out_format, w.out_block, w.hadamard) if w.out_format else None
    fp8 = w.in_format in T.FP8_FORMATS
    ch = W.sample_chunks(w, 3, seed=7)
    rows_idx = W.chunk_rows(ch, w.rows)
    ridx = torch.from_numpy(rows_idx).to(dev)
    bits0 = ctx["sets_bits"]
    xs0 = ctx["xs"][0]

    # GPU: AUTO compress of every shard of set 0, reduce + requantize, decodes
    qb = [T.empty_compressed(c_in, w.rows, w.cols, dev) for _ in range(w.shards)]
    for r in range(w.shards):
        wsb = torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) if fp8 else None
        T.taco_compress(c_in, xs0[r], w.rows, w.cols, T.TACO_SCALE_AUTO if fp8 else 1.0, qb[r], workspace=wsb)
    d = torch.empty(w.n, dtype=torch.float32, device=dev)

    def decoded_rows(c, buf):
        T.taco_decompress(c, buf, w.rows, w.cols, d, 0)
        return d.view(w.rows, w.cols)[ridx].cpu().numpy()

    got_c = decoded_rows(c_in, qb[0])
    got_delayed = decoded_rows(c_in, ctx["bufs"][0][0])
    if c_out is not None:
        rq = T.empty_compressed(c_out, w.rows, w.cols, dev)
        T.taco_decompress_reduce(c_in, qb, w.rows, w.cols, None, c_out, rq)
        got_r = decoded_rows(c_out, rq)
    else:
        T.taco_decompress_reduce(c_in, qb, w.rows, w.cols, d)
        got_r = d.view(w.rows, w.cols)[ridx].cpu().numpy()
    torch.cuda.synchronize()

    def gpu_region_rows(c, buf):
        """codes / block metadata / g of the sample rows, parsed by the layout."""
        L = T.taco_layout(c, w.rows, w.cols)
        h = buf.cpu().numpy()
        cb = w.cols // 2 if c.format == T.TACO_FMT_INT4_ASYM else w.cols
        nb = w.cols // c.block
        mb = 1 if c.format in T.FP8_FORMATS else 4
        codes = h[L.codes_off:L.codes_off + L.codes_bytes].reshape(w.rows, cb)[rows_idx]
        meta = h[L.scale_off:L.scale_off + L.scale_bytes].reshape(w.rows, nb * mb)[rows_idx]
        aux = h[L.aux_off:L.aux_off + L.aux_bytes].reshape(w.rows, nb)[rows_idx] if L.aux_bytes else None
        g = h[L.tensor_off:L.tensor_off + 4].view(np.float32)[0] if L.tensor_bytes else None
        return codes, meta, aux, g

    def same(gpu, ref):
        codes, meta, aux, g = gpu
        ok = bool((codes.reshape(-1) == ref.codes.reshape(-1)).all())
        ok &= bool((meta.reshape(-1) == np.ascontiguousarray(ref.scale).view(np.uint8).reshape(-1)).all())
        if aux is not None:
            ok &= bool((aux.reshape(-1) == ref.zero.reshape(-1)).all())
        if g is not None:
            ok &= bool(np.float32(g).view(np.uint32) == np.float32(ref.tensor_scale).view(np.uint32))
        return ok

    # oracle: each shard's scale from its whole tensor, then the sample rows
    t0 = time.perf_counter()
    gs = [oracle_tensor_scale(w, oc, bits0[r]) if fp8 else None for r in range(w.shards)]
    ref_sh = [oracle.compress(oc, bits0[r][rows_idx], tensor_scale=gs[r]) for r in range(w.shards)]
    acc, rq_ref = oracle.decompress_reduce(ref_sh, ocout)
    ref_c = oracle.decode(ref_sh[0])
    ref_r = oracle.decode(rq_ref) if rq_ref is not None else acc
    t_oracle = time.perf_counter() - t0

    x0 = bf16_bits_to_f32(bits0[0][rows_idx])
    exact = np.zeros(x0.shape, np.float64)
    for r in range(w.shards):
        exact += bf16_bits_to_f32(bits0[r][rows_idx]).astype(np.float64)
    rm = oracle.rel_mse
    out = {
        "sample_rows": int(len(rows_idx)),
        "tensor_scale": "data-driven (AUTO) on both sides" if fp8 else "n/a",
        "compress": {"rel_mse_gpu": rm(got_c, x0), "rel_mse_oracle": rm(ref_c, x0),
                     "codes_bit_exact": same(gpu_region_rows(c_in, qb[0]), ref_sh[0])},
        "reduce": {"rel_mse_gpu": rm(got_r, exact), "rel_mse_oracle": rm(ref_r, exact),
                   "against": "exact float64 sum of the bf16 shards",
                   "codes_bit_exact": same(gpu_region_rows(c_out, rq), rq_ref) if c_out is not None else
                   bool((got_r.view(np.uint32) == acc.view(np.uint32)).all())},
        "oracle_seconds": round(t_oracle, 2),
    }
    if fp8:
        g_gpu = [np.float32(T.regions(qb[r], c_in, w.rows, w.cols)[3][0].item()) for r in range(w.shards)]
        out["gpu_g_equals_oracle_g"] = all(g_gpu[r].view(np.uint32) == np.float32(gs[r]).view(np.uint32)
                                           for r in range(w.shards))
        out["delayed_scale"] = {
            "rel_mse_gpu": rm(got_delayed, x0),
            "vs_data_driven": round(rm(got_delayed, x0) / max(rm(got_c, x0), 1e-300), 4),
            "note": "compress round trip of the timed steps' shard 0, whose g is the previous step's abs-max / 448"}
    return out


def setup(w, args):
    """Seeded inputs on the device, compressed buffers and workspaces."""
    import numpy as np
    import torch
    import quantized_compression_tensor_amd as T
    import workloads as W
    dev = "cuda"
    c_in = T.codec(w.in_format, w.in_block, 1 if w.hadamard else 0)
    c_out = T.codec(w.out_format, w.out_block, 1 if w.hadamard else 0) if w.out_format else None
    fp8 = w.in_format in T.FP8_FORMATS
    in_bytes = w.shards * w.n * 2
    nsets = max(2, min(4, -(-2 * MALL_BYTES // in_bytes) + 1))
    sets_bits, xs, bufs, outs = None, [], [], []
    for s in range(nsets):
        bits = [W.make_shard(w, r + 100 * s) for r in range(w.shards)]
        if s == 0:
            sets_bits = bits
        xs.append([torch.from_numpy(b.view(np.int16)).to(dev) for b in bits])
        bufs.append([T.empty_compressed(c_in, w.rows, w.cols, dev) for _ in range(w.shards)])
        outs.append(T.empty_compressed(c_out, w.rows, w.cols, dev) if c_out is not None
                    else torch.empty(w.n, dtype=torch.float32, device=dev))
    wss = [torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) for _ in range(w.shards)]
    scale = {"delayed": T.TACO_SCALE_DELAYED, "auto": T.TACO_SCALE_AUTO, "given": 0.01}[args.scale_mode] \
        if fp8 else 1.0
    torch.cuda.synchronize()
    return dict(c_in=c_in, c_out=c_out, fp8=fp8, nsets=nsets, sets_bits=sets_bits, xs=xs, bufs=bufs, outs=outs,
                wss=wss, scale=scale, use_ws=fp8 and args.scale_mode != "given", in_bytes=in_bytes)


def pctl(v, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(v), q)), 5)


def run_workload(w, args, headline):
    """Time one workload: returns its summary dict (and the step function for
    the optional overlap measurement)."""
    import torch
    import quantized_compression_tensor_amd as T

    dev = "cuda"
    ctx = setup(w, args)
    c_in, c_out, nsets = ctx["c_in"], ctx["c_out"], ctx["nsets"]
    xs, bufs, outs, wss = ctx["xs"], ctx["bufs"], ctx["outs"], ctx["wss"]
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def compress(s):
        for r in range(w.shards):
            T.taco_compress(c_in, xs[s][r], w.rows, w.cols, ctx["scale"], bufs[s][r],
                            workspace=wss[r] if ctx["use_ws"] else None, stream=sh)

    def reduce(s):
        if c_out is not None:
            T.taco_decompress_reduce(c_in, bufs[s], w.rows, w.cols, None, c_out, outs[s], stream=sh)
        else:
            T.taco_decompress_reduce(c_in, bufs[s], w.rows, w.cols, outs[s], stream=sh)

    mk = lambda: torch.cuda.Event(enable_timing=True)
    K = args.steps
    with torch.cuda.stream(stream):
        # first calls seed the delayed-scale history with this data
        for s in range(nsets):
            compress(s)
            reduce(s)
        torch.cuda.synchronize()
        if args.launch == "graph":
            g_step = []
            for s in range(nsets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    compress(s)
                    reduce(s)
                g_step.append(g)

        def step(s):
            if args.launch == "graph":
                g_step[s].replay()
            else:
                compress(s)
                reduce(s)

        # the first steps after the GPU sat idle (while the host generated the
        # inputs) run slower until its clocks rise: before the W warm-up steps,
        # steps run for at least --prewarm seconds of wall time
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < args.prewarm:
            for _ in range(8):
                step(i % nsets)
                i += 1
            torch.cuda.synchronize()
        prewarm_steps = i
        for i in range(args.warmup):
            step(i % nsets)
        torch.cuda.synchronize()

        # timed region: K whole steps between one pair of events (an event
        # record between kernels costs GPU time, so none inside the region)
        ev0, ev1 = mk(), mk()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(K):
            step(i % nsets)
        ev1.record(stream)
        host = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

        # step-time distribution: K more steps, an event at every step boundary
        evs = [mk() for _ in range(K + 1)]
        evs[0].record(stream)
        for i in range(K):
            step(i % nsets)
            evs[i + 1].record(stream)
        # per-kernel launch durations in step context: K more steps with an
        # event before the N compress launches, one between them and the
        # reduce, and one after it; each average includes the short gap
        # before each launch, so it bounds the kernel's own duration from above
        ph = [(mk(), mk(), mk()) for _ in range(K)]
        for i in range(K):
            ph[i][0].record(stream)
            compress(i % nsets)
            ph[i][1].record(stream)
            reduce(i % nsets)
            ph[i][2].record(stream)
        # streaming reference: a plain device copy of one shard (2 B read +
        # 2 B written per element), N per step, back to back. Left out of the
        # counter passes, whose calibration copies must be the only large
        # device copies of the run.
        a_x, b_x = mk(), mk()
        if not args.copy_calibration:
            ref_out = torch.empty(w.n, dtype=torch.int16, device=dev)
            a_x.record(stream)
            for i in range(K):
                for r in range(w.shards):
                    ref_out.copy_(xs[i % nsets][r].reshape(-1))
            b_x.record(stream)
        # the consumer-side decode of the gather-stage output to bf16 (the next
        # GEMM's input; FP8: with the inverse transform), outside the step
        dec_out = torch.empty(w.n, dtype=torch.bfloat16, device=dev) if c_out is not None else None
        a_d, b_d = mk(), mk()
        if dec_out is not None:
            a_d.record(stream)
            for i in range(K):
                T.taco_decompress(c_out, outs[i % nsets], w.rows, w.cols, dec_out, 1, stream=sh)
            b_d.record(stream)
        torch.cuda.synchronize()

    steps_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
    comp_launch = [ph[i][0].elapsed_time(ph[i][1]) / w.shards for i in range(K)]
    red_launch = [ph[i][1].elapsed_time(ph[i][2]) for i in range(K)]
    t_comp = sum(comp_launch) / K
    t_red = sum(red_launch) / K
    t_dec = a_d.elapsed_time(b_d) / K if dec_out is not None else None
    t_ref = a_x.elapsed_time(b_x) / (K * w.shards) if not args.copy_calibration else None
    ms_step = wall * 1e3 / K
    b_comp, b_red = algorithmic_bytes(w)
    comp_gbs = b_comp / (t_comp * 1e-3) / 1e9
    red_gbs = b_red / (t_red * 1e-3) / 1e9
    res = {
        "name": w.name,
        "workload": f"{w.name}: {w.shards} bf16 shards of {w.rows}x{w.cols}; compress {FORMAT_NAMES[w.in_format]} "
                    f"block {w.in_block}{' + Hadamard' if w.hadamard else ''}; decompress-reduce "
                    + (f"-> {FORMAT_NAMES[w.out_format]}" if w.out_format else "-> FP32 sum"),
        "shards": w.shards, "rows": w.rows, "cols": w.cols,
        "value": round(ctx["in_bytes"] / (ms_step * 1e-3) / 1e9, 2),
        "ms_per_step": round(ms_step, 5),
        "step_hbm_frac": round((w.shards * b_comp + b_red) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_ms_distribution": {"median": pctl(steps_ms, 50), "p10": pctl(steps_ms, 10), "p90": pctl(steps_ms, 90),
                                 "note": "K further steps with an event at each step boundary"},
        "kernels": {
            "compress_ms": round(t_comp, 5), "compress_GBs": round(comp_gbs, 1),
            "compress_hbm_frac": round(comp_gbs / HBM_PEAK_GBS, 4),
            "reduce_ms": round(t_red, 5), "reduce_GBs": round(red_gbs, 1),
            "reduce_hbm_frac": round(red_gbs / HBM_PEAK_GBS, 4),
            "compress_ms_p10_p90": [pctl(comp_launch, 10), pctl(comp_launch, 90)],
            "reduce_ms_p10_p90": [pctl(red_launch, 10), pctl(red_launch, 90)],
            **({"decode_bf16_ms": round(t_dec, 5),
                "decode_bf16_GBs": round(decode_bytes(w) / (t_dec * 1e-3) / 1e9, 1)} if t_dec else {}),
            "phases_hbm_frac": round((w.shards * b_comp + b_red) / ((w.shards * t_comp + t_red) * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 4),
            "host_ms_per_step": round(host * 1e3 / K, 5),
            "event_ms_per_step": round(ev0.elapsed_time(ev1) / K, 5),
        },
        "algorithmic_bytes": {"compress": b_comp, "reduce": b_red, "step": w.shards * b_comp + b_red},
        "input_sets": nsets,
        "prewarm_steps": prewarm_steps,
        "tensor_scale": args.scale_mode if ctx["fp8"] else "n/a",
    }
    if t_ref:
        res["copy_reference"] = {
            "kernel": "device copy of one bf16 shard (2 B read + 2 B written per element), timed like the "
                      "compress: the streaming rate this machine reaches at this size",
            "ms": round(t_ref, 5), "GBs": round(4 * w.n / (t_ref * 1e-3) / 1e9, 1),
            "compress_vs_copy": round(comp_gbs / (4 * w.n / (t_ref * 1e-3) / 1e9), 3)}
    if not args.no_quality:
        res["quality"] = quality(w, ctx)
    if not args.no_consumer and c_out is not None:
        res["consumer"] = measure_consumer(w, ctx, stream, K=max(10, K // 2))
    extras = {"stream": stream, "step": lambda s: (compress(s), reduce(s)), "ctx": ctx, "t_comp": t_comp,
              "t_red": t_red, "ms_step": ms_step}
    return res, extras


def measure_consumer(w, ctx, stream, K):
    """The next layer's input: the gather-stage output (the requantized sum,
    resident from the step) times a bf16 weight W [cols, cols] in the layout
    of a linear layer. Unfused: taco_decompress to bf16, then torch.matmul
    (hipBLASLt) on it; fused: taco_decompress_gemm, the decode in the GEMM's
    prologue. Both write bf16 [rows, cols]. Codecs with the Hadamard
    transform are not taken by the fused kernel (reported as such)."""
    import torch
    import quantized_compression_tensor_amd as T
    c = ctx["c_out"]
    if c.hadamard:
        return {"note": "gather codec applies the Hadamard transform: the fused decode-GEMM takes codecs "
                        "without it (the decode + GEMM path is the decode_bf16_ms kernel + a library GEMM)"}
    rows, cols, outs, nsets = w.rows, w.cols, ctx["outs"], ctx["nsets"]
    sh = stream.cuda_stream
    g = torch.Generator(device="cuda").manual_seed(w.seed + 77)
    wt = (torch.randn(cols, cols, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    dec = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    y_unf = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    y_fus = torch.empty_like(y_unf)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def decode(i):
        T.taco_decompress(c, outs[i % nsets], rows, cols, dec, 1, stream=sh)

    def gemm(i):
        torch.matmul(dec, wt.t(), out=y_unf)

    def fused(i):
        T.taco_decompress_gemm(c, outs[i % nsets], rows, cols, wt, cols, y_fus, 1, stream=sh)

    def timed(*fns):
        for i in range(3):
            for f in fns:
                f(i)
        a, b = mk(), mk()
        a.record(stream)
        for i in range(K):
            for f in fns:
                f(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    with torch.cuda.stream(stream):
        # three interleaved rounds, the fastest of each (clock drift between
        # the measurements would otherwise favour one side)
        runs = {"dec": [], "gemm": [], "both": [], "fused": []}
        for _ in range(3):
            runs["dec"].append(timed(decode))
            runs["gemm"].append(timed(gemm))
            runs["both"].append(timed(decode, gemm))
            runs["fused"].append(timed(fused))
        t_dec, t_gemm, t_both, t_fused = (min(runs[k]) for k in ("dec", "gemm", "both", "fused"))
        decode(0)
        gemm(0)
        fused(0)
        torch.cuda.synchronize()
        ref = y_unf.float()
        ref_max = float(ref.abs().max())
        diff = (y_fus.float() - ref).abs()
        rel = float(diff.max()) / ref_max if ref_max > 0 else float("nan")
        differ = float((diff > 0).float().mean())
    flops = 2.0 * rows * cols * cols
    return {"shape": f"[{rows}, {cols}] x [{cols}, {cols}]^T, bf16 out",
            "decode_bf16_ms": round(t_dec, 5), "gemm_ms": round(t_gemm, 5),
            "gemm_tflops": round(flops / t_gemm / 1e9, 1),
            "decode_then_gemm_ms": round(t_both, 5), "fused_ms": round(t_fused, 5),
            "fused_tflops": round(flops / t_fused / 1e9, 1),
            "fused_speedup_vs_decode_then_gemm": round(t_both / t_fused, 3),
            "max_rel_diff_vs_unfused": float(f"{rel:.3g}"), "max_abs_output": float(f"{ref_max:.4g}"),
            "outputs_differing_frac": round(differ, 4)}


def measure_rank_share(w, xs, stream, K):
    """The decompress-reduce at one rank's share of the step: with N ranks a rank
    reduces the (rows / N) x cols row chunk it owns, from N sources (one
    compressed chunk per rank), and re-quantizes it for the gather stage. The
    N source chunks are compressed here from row chunks of the workload's
    shards; enough independent sets rotate that they exceed twice the
    Infinity Cache, so the chunks come from HBM as the full-size kernels' do."""
    import torch
    import quantized_compression_tensor_amd as T
    dev = "cuda"
    rows = w.rows // w.shards
    ws_ = dataclasses.replace(w, rows=rows)
    c_in = T.codec(w.in_format, w.in_block, int(w.hadamard))
    c_out = T.codec(w.out_format, w.out_block, int(w.hadamard)) if w.out_format else None
    fp8 = w.in_format in T.FP8_FORMATS
    per_set = w.shards * T.taco_compressed_bytes(c_in, rows, w.cols)
    nsets = max(2, -(-2 * MALL_BYTES // per_set))
    sh = stream.cuda_stream
    sets, outs = [], []
    with torch.cuda.stream(stream):
        for j in range(nsets):
            bufs = []
            for r in range(w.shards):
                x = xs[j % len(xs)][r].reshape(-1)[:rows * w.cols]
                b = T.empty_compressed(c_in, rows, w.cols, dev)
                wsb = torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) if fp8 else None
                T.taco_compress(c_in, x, rows, w.cols, T.TACO_SCALE_AUTO if fp8 else 1.0, b, workspace=wsb, stream=sh)
                bufs.append(b)
            sets.append(bufs)
            outs.append(T.empty_compressed(c_out, rows, w.cols, dev) if c_out is not None
                        else torch.empty(rows * w.cols, dtype=torch.float32, device=dev))

        def red(j):
            if c_out is not None:
                T.taco_decompress_reduce(c_in, sets[j], rows, w.cols, None, c_out, outs[j], stream=sh)
            else:
                T.taco_decompress_reduce(c_in, sets[j], rows, w.cols, outs[j], stream=sh)

        for j in range(nsets):
            red(j)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(K):
            red(i % nsets)
        b.record(stream)
        torch.cuda.synchronize()
    t = a.elapsed_time(b) / K
    _, b_red = algorithmic_bytes(ws_)
    gbs = b_red / (t * 1e-3) / 1e9
    return {"rows": rows, "cols": w.cols, "sources": w.shards, "input_sets": nsets, "reduce_ms": round(t, 5),
            "reduce_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": b_red}


def measure_ring(w, xs, stream, K):
    """One hop of the quantized ring (dequantize the incoming shard, add the
    local bf16 shard, quantize for the next hop) timed at full size, and the
    whole rings over the workload's shards: the full loop (N - 1 hops in one
    direction, then the gather) and the semi-loop (each chunk gathered from both
    ends towards the middle: two chains of about N/2 hops, joined by one more
    hop), each decoded and compared with the exact sum, next to quantizing the
    exact sum once (the all-gather alone)."""
    import torch
    import quantized_compression_tensor_amd as T
    c_out = T.codec(w.out_format, w.out_block, 0)
    dev = "cuda"
    N = len(xs)
    sh = stream.cuda_stream
    bufs = [T.empty_compressed(c_out, w.rows, w.cols, dev) for _ in range(3)]

    def decoded(buf):
        o = torch.empty(w.n, dtype=torch.float32, device=dev)
        T.taco_decompress(c_out, buf, w.rows, w.cols, o, 0, stream=sh)
        return o

    with torch.cuda.stream(stream):
        # full loop: the first rank quantizes its shard, every later rank adds its own
        T.taco_ring_hop(c_out, None, xs[0], w.rows, w.cols, None, c_out, bufs[0], stream=sh)
        for r in range(1, N):
            T.taco_ring_hop(c_out, bufs[(r - 1) % 2], xs[r], w.rows, w.cols, None, c_out, bufs[r % 2], stream=sh)
        ring = decoded(bufs[(N - 1) % 2])
        # semi-loop: ranks 0 .. h-1 chain forwards, ranks N-1 .. h backwards,
        # and the last rank of the backward chain adds the forward partial sum
        h = N // 2
        fwd = [T.empty_compressed(c_out, w.rows, w.cols, dev) for _ in range(2)]
        bwd = [T.empty_compressed(c_out, w.rows, w.cols, dev) for _ in range(2)]
        T.taco_ring_hop(c_out, None, xs[0], w.rows, w.cols, None, c_out, fwd[0], stream=sh)
        for r in range(1, h):
            T.taco_ring_hop(c_out, fwd[(r - 1) % 2], xs[r], w.rows, w.cols, None, c_out, fwd[r % 2], stream=sh)
        f_last = fwd[(h - 1) % 2]
        T.taco_ring_hop(c_out, None, xs[N - 1], w.rows, w.cols, None, c_out, bwd[0], stream=sh)
        j = 0
        for r in range(N - 2, h - 1, -1):
            T.taco_ring_hop(c_out, bwd[j % 2], xs[r], w.rows, w.cols, None, c_out, bwd[(j + 1) % 2], stream=sh)
            j += 1
        b_last = bwd[j % 2]
        # join: dequantize both partial sums and requantize their sum (a
        # two-source decompress-reduce in the gather codec)
        semi_q = T.empty_compressed(c_out, w.rows, w.cols, dev)
        T.taco_decompress_reduce(c_out, [f_last, b_last], w.rows, w.cols, None, c_out, semi_q, stream=sh)
        semi = decoded(semi_q)
        exact = torch.zeros(w.n, dtype=torch.float64, device=dev)
        for x in xs:
            exact += x.view(torch.bfloat16).reshape(-1).to(torch.float64)
        once_q = T.empty_compressed(c_out, w.rows, w.cols, dev)
        T.taco_requantize(c_out, exact.to(torch.float32), w.rows, w.cols, 1.0, once_q, stream=sh)
        once = decoded(once_q)
        # timing: K hops back to back between one pair of events
        for i in range(3):
            T.taco_ring_hop(c_out, bufs[i % 2], xs[i % N], w.rows, w.cols, None, c_out, bufs[2], stream=sh)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(K):
            T.taco_ring_hop(c_out, bufs[i % 2], xs[i % N], w.rows, w.cols, None, c_out, bufs[2], stream=sh)
        b.record(stream)
    torch.cuda.synchronize()
    hop_ms = a.elapsed_time(b) / K
    n = w.n
    qb = n + (4 * (n // 64) if w.out_format == 2 else 5 * (n // 128))   # INT8 codes + metadata
    hop_bytes = qb + 2 * n + qb
    mse = lambda v: float(((v.double() - exact) ** 2).mean())
    return {"hop_ms": round(hop_ms, 5), "hop_GBs": round(hop_bytes / (hop_ms * 1e-3) / 1e9, 1),
            "hop_hbm_frac": round(hop_bytes / (hop_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "hop_algorithmic_bytes": hop_bytes, "ranks": N, "hops": N - 1,
            "ring_mse": mse(ring), "semi_loop_mse": mse(semi), "all_gather_only_mse": mse(once),
            "semi_loop": f"ranks 0..{h - 1} forwards, {N - 1}..{h} backwards, joined by one two-source reduce",
            "ring_codec_in": "INT8 (gather codec)"}


def measure_reorder(w, ctx, stream, K):
    """The data-driven reshaping (taco_chunk_order, taco_compress_reordered):
    the order of the 8-channel groups comes from another input set of the
    workload (an earlier step's activation of rank 0). Reported: the reordered
    compress's launch time beside the plain one, and the compress round trip's
    rel-MSE with and without the reorder on a seeded sample of rows, for the
    workload's codec and for the INT8 (block 64) and INT4 (group 128) codecs on
    the same data, the GPU's figure checked against the oracle's."""
    import numpy as np
    import torch
    import oracle
    from oracle import codecs as cd
    from oracle.formats import bf16_bits_to_f32
    import quantized_compression_tensor_amd as T
    import workloads as W
    dev = "cuda"
    xs, bits0 = ctx["xs"], ctx["sets_bits"]
    order = torch.empty(w.cols // 8, dtype=torch.int32, device=dev)
    T.taco_chunk_order(xs[1][0], w.rows, w.cols, order, stream=stream.cuda_stream)
    torch.cuda.synchronize()
    o = order.cpu().numpy().astype(np.int64)
    c_in = ctx["c_in"]
    fp8 = ctx["fp8"]
    sh = stream.cuda_stream
    wss = [torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) for _ in range(w.shards)]
    bufs = ctx["bufs"][0]
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def run(reordered):
        for i in range(K):
            r = i % w.shards
            s = i % ctx["nsets"]
            if reordered:
                T.taco_compress_reordered(c_in, xs[s][r], w.rows, w.cols, T.TACO_SCALE_DELAYED if fp8 else 1.0,
                                          bufs[r], order, workspace=wss[r] if fp8 else None, stream=sh)
            else:
                T.taco_compress(c_in, xs[s][r], w.rows, w.cols, T.TACO_SCALE_DELAYED if fp8 else 1.0, bufs[r],
                                workspace=wss[r] if fp8 else None, stream=sh)

    times = {}
    with torch.cuda.stream(stream):
        for reordered in (False, True, False, True):
            run(reordered)
            a, b = mk(), mk()
            a.record(stream)
            run(reordered)
            b.record(stream)
            torch.cuda.synchronize()
            times.setdefault(reordered, []).append(a.elapsed_time(b) / K)
    t_plain, t_re = min(times[False]), min(times[True])
    # the decode to bf16, plain and restoring the channel order
    dec = torch.empty(w.n, dtype=torch.bfloat16, device=dev)

    def run_dec(reordered):
        for i in range(K):
            src = bufs[i % w.shards]
            if reordered:
                T.taco_decompress_reordered(c_in, src, w.rows, w.cols, dec, order, 1, stream=sh)
            else:
                T.taco_decompress(c_in, src, w.rows, w.cols, dec, 1, stream=sh)

    dtimes = {}
    with torch.cuda.stream(stream):
        for reordered in (False, True, False, True):
            run_dec(reordered)
            a, b = mk(), mk()
            a.record(stream)
            run_dec(reordered)
            b.record(stream)
            torch.cuda.synchronize()
            dtimes.setdefault(reordered, []).append(a.elapsed_time(b) / K)
    td_plain, td_re = min(dtimes[False]), min(dtimes[True])
    del dec
    b_comp, _ = algorithmic_bytes(w)
    # quality on sampled rows, GPU and oracle, plain and reordered
    ch = W.sample_chunks(w, 3, seed=7)
    idx = W.chunk_rows(ch, w.rows)
    it = torch.from_numpy(idx).to(dev)
    x0 = bits0[0][idx]
    xf = bf16_bits_to_f32(x0)
    codecs = [(cd.Codec(w.in_format, w.in_block, w.hadamard), "workload codec"),
              (cd.Codec.int8_sym(), "INT8 sym 64"), (cd.Codec.int4_asym(), "INT4 asym 128")]
    if w.in_format == 2:
        codecs = codecs[:1] + codecs[2:]
    elif w.in_format == 3:
        codecs = codecs[:2]
    q = []
    d = torch.empty(w.n, dtype=torch.float32, device=dev)
    for oc, label in codecs:
        c = T.codec(oc.format, oc.block, int(oc.hadamard))
        f8 = oc.format in cd.FP8_FORMATS
        buf = T.empty_compressed(c, w.rows, w.cols, dev)
        row = {"codec": label}
        for reordered in (False, True):
            ws = torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) if f8 else None
            g = np.float32(2.0 ** -9)     # a given tensor scale keeps the oracle to the sampled rows
            if reordered:
                T.taco_compress_reordered(c, xs[0][0], w.rows, w.cols, float(g) if f8 else 1.0, buf, order,
                                          workspace=ws)
                T.taco_decompress_reordered(c, buf, w.rows, w.cols, d, order, 0)
                ref = oracle.decode_reordered(oracle.compress_reordered(oc, x0, o, tensor_scale=g if f8 else None), o)
            else:
                T.taco_compress(c, xs[0][0], w.rows, w.cols, float(g) if f8 else 1.0, buf, workspace=ws)
                T.taco_decompress(c, buf, w.rows, w.cols, d, 0)
                ref = oracle.decode(oracle.compress(oc, x0, tensor_scale=g if f8 else None))
            got = d.view(w.rows, w.cols)[it].cpu().numpy()
            key = "reordered" if reordered else "plain"
            row[f"rel_mse_{key}"] = oracle.rel_mse(got, xf)
            row[f"gpu_equals_oracle_{key}"] = bool((got.view(np.uint32) == ref.reshape(got.shape).view(np.uint32)).all())
        row["reordered_over_plain"] = round(row["rel_mse_reordered"] / row["rel_mse_plain"], 4)
        q.append(row)
    return {"order_from": "input set 1, rank 0 (an earlier step's activation)",
            "compress_ms_plain": round(t_plain, 5), "compress_ms_reordered": round(t_re, 5),
            "compress_hbm_frac_reordered": round(b_comp / (t_re * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_bf16_ms_plain": round(td_plain, 5), "decode_bf16_ms_reordered": round(td_re, 5),
            "sample_rows": int(len(idx)), "tensor_scale": "given 2^-9 (FP8 codecs)", "quality": q}


def measure_overlap(w, step_fn, nsets, stream, K, ctx, caps=(0, 1024, 512, 256, 128, 64)):
    """The bf16 GEMM [rows, cols] x [cols, cols]^T (a weight in linear-layer layout) that produces the next activation,
    alone and concurrently with the codec step on a second stream (default
    priority), with the codec's launches capped at each of `caps` workgroups
    (taco_set_launch_limit; 0 = uncapped). Per cap: the codec step alone, both
    together, and the fraction of the shorter of the two that the overlap hid.
    Also the consumer side: the decode of the gather-stage output to bf16
    followed by the GEMM on it, against the GEMM alone (the decode's share of
    the consumer's time)."""
    import torch
    import quantized_compression_tensor_amd as T
    g_stream = torch.cuda.Stream()
    a = torch.randn(w.rows, w.cols, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(w.cols, w.cols, dtype=torch.bfloat16, device="cuda")   # a weight [N, K], linear-layer layout
    c = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    def gemm(i):
        with torch.cuda.stream(g_stream):
            torch.matmul(a, b.t(), out=c)

    def codec(i):
        with torch.cuda.stream(stream):
            step_fn(i % nsets)

    def both(i):
        gemm(i)
        codec(i)

    for _ in range(3):
        gemm(0)
    gemm_ms = timed(gemm)
    flops = 2.0 * w.rows * w.cols * w.cols
    rows = []
    for cap in caps:
        with T.launch_limit(cap):
            for i in range(3):
                codec(i)
            codec_ms = timed(codec)
            both_ms = timed(both)
        serial = gemm_ms + codec_ms
        rows.append({"codec_workgroup_cap": cap, "codec_ms": round(codec_ms, 4), "both_ms": round(both_ms, 4),
                     "serial_ms": round(serial, 4),
                     "hidden_frac": round((serial - both_ms) / min(gemm_ms, codec_ms), 3)})
    best = min(rows, key=lambda r: r["both_ms"])
    # consumer: decode the gather-stage output to bf16, then the GEMM on it
    dec = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device="cuda")
    c_out = ctx["c_out"]

    def consumer(i):
        with torch.cuda.stream(g_stream):
            T.taco_decompress(c_out, ctx["outs"][i % nsets], w.rows, w.cols, dec, 1, stream=g_stream.cuda_stream)
            torch.matmul(dec, b.t(), out=c)

    def decode_only(i):
        with torch.cuda.stream(g_stream):
            T.taco_decompress(c_out, ctx["outs"][i % nsets], w.rows, w.cols, dec, 1, stream=g_stream.cuda_stream)

    consumer(0)
    cons_ms = timed(consumer)
    dec_ms = timed(decode_only)
    gemm2_ms = timed(gemm)
    return {"gemm_ms": round(gemm_ms, 4), "gemm_tflops": round(flops / gemm_ms / 1e9, 1), "by_cap": rows,
            "best": best,
            "consumer": {"decode_bf16_ms": round(dec_ms, 4), "gemm_ms": round(gemm2_ms, 4),
                         "decode_then_gemm_ms": round(cons_ms, 4),
                         "decode_share": round((cons_ms - gemm2_ms) / cons_ms, 4)}}


def _short(name):
    """A kernel name cut to 100 characters, keeping a trailing [grid ...] tag."""
    if " [grid " in name:
        base, tag = name.rsplit(" [grid ", 1)
        return f"{base[:100]} [grid {tag}"
    return name[:140]


def summarize_trace(trace_dir, name, command):
    """Kernel-trace statistics of every kernel of this library in one profiled
    run (e.g. `--reorder`, whose reordered and plain kernels run side by side),
    written to profiles/kernels_<name>_trace.txt."""
    lines = [f"# rocprofv3 kernel-trace statistics of this library's kernels: {name}",
             f"# command: {command}",
             f"source_hash: {kernel_source_hash()}",
             " calls    avg_us    min_us    max_us  kernel"]
    stats = _trace_stats(trace_dir, concurrent_with=("Cijk",))
    for n, r in sorted(stats.items(), key=lambda kv: -float(kv[1]["AverageNs"])):
        if "taco::" in n:
            lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                         f"{float(r['MaxNs']) / 1e3:9.2f}  {_short(n)}")
    path = os.path.join(ROOT, "profiles", f"kernels_{name}_trace.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def summarize_consumer(trace_dir, mfma_dir, command):
    """Kernel-trace statistics of the consumer kernels (the fused decode-GEMM,
    the library GEMM, the bf16 decode) and the fused kernel's MFMA counters:
    MFMA pipe busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs * GRBM_GUI_ACTIVE
    / 8 XCDs), and the other VALU instructions per MFMA instruction."""
    keep = ("k_dequant_gemm", "Cijk", "k_dequantize")
    lines = ["# consumer kernels: the gather-stage output times a bf16 weight W [cols, cols] (linear-layer layout)",
             f"# command: {command}",
             f"source_hash: {kernel_source_hash()}",
             " calls    avg_us    min_us    max_us  kernel"]
    stats = _trace_stats(trace_dir, concurrent_with=("k_fp8_had_compress", "k_reduce", "k_quantize"),
                         by_grid=("Cijk", "k_dequant_gemm"))
    for n, r in sorted(stats.items(), key=lambda kv: -float(kv[1]["AverageNs"])):
        if any(k in n for k in keep) and ("k_dequantize" not in n or ", true, false>" in n):
            lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                         f"{float(r['MaxNs']) / 1e3:9.2f}  {_short(n)}")
    per = {}
    for row in _csv_rows(mfma_dir, "counter_collection.csv"):
        n = row.get("Kernel_Name", "")
        if "k_dequant_gemm" not in n:
            continue
        d = per.setdefault(n, {}).setdefault(row["Dispatch_Id"], {})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    for n, disp in per.items():
        last = disp[max(disp, key=int)]
        busy = last.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * last.get("GRBM_GUI_ACTIVE", 1.0) / 8)
        lines += [f"kernel: {n[:140]}",
                  *[f"  {k}: {v:.6g}" for k, v in sorted(last.items())],
                  f"  mfma_busy_frac: {busy:.3f}",
                  # SQ_INSTS_VALU counts the MFMA instructions too
                  f"  other_valu_per_mfma: {(last.get('SQ_INSTS_VALU', 0.0) - last.get('SQ_INSTS_MFMA', 0.0)) / max(1.0, last.get('SQ_INSTS_MFMA', 1.0)):.2f}"]
    path = os.path.join(ROOT, "profiles", "consumer_gemm.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def main():
    args = parse()
    if args.summarize_consumer:
        summarize_consumer(*args.summarize_consumer, args.command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command)
        return
    if args.summarize_issue:
        names = [args.workload] + [x for x in args.extra.split(",") if x and x != "none"]
        summarize_issue(args.summarize_issue, names, args.command)
        return
    if args.summarize:
        if len(args.summarize) not in (3, 4):
            sys.exit("--summarize takes FETCH_DIR WRITE_DIR TRACE_DIR [TRACE_LOG]")
        fetch, write, trace = args.summarize[:3]
        log = args.summarize[3] if len(args.summarize) == 4 else None
        names = [args.workload] + [x for x in args.extra.split(",") if x and x != "none"]
        summarize(fetch, write, trace, names, args.command, log)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is designed, not implemented: one GPU is measured)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_compression_tensor_amd as T
    import workloads as W

    def resolve(name):
        w = W.WORKLOADS[name]
        if args.fp8_codes == "e5m2" and w.in_format == T.TACO_FMT_FP8_DUAL:
            w = dataclasses.replace(w, in_format=T.TACO_FMT_FP8E5_DUAL,
                                    out_format=T.TACO_FMT_FP8E5_DUAL if w.out_format else None)
        return w

    torch.cuda.set_device(0)
    w = resolve(args.workload)
    head, ex = run_workload(w, args, True)
    src_hash = kernel_source_hash()
    kern = head["kernels"]
    t_comp, t_red = ex["t_comp"], ex["t_red"]
    b_comp, b_red = algorithmic_bytes(w)
    dominant = "compress" if w.shards * t_comp >= t_red else "reduce"
    ach = kern["compress_GBs"] if dominant == "compress" else kern["reduce_GBs"]
    bytes_launch = b_comp if dominant == "compress" else b_red
    traffic = read_traffic(dominant, w.name, src_hash)

    rank_share = measure_rank_share(w, ex["ctx"]["xs"], ex["stream"], K=max(20, args.steps // 2)) \
        if args.rank_share else None
    ring = None
    if args.ring:
        if w.in_format in T.FP8_FORMATS:
            sys.exit("--ring applies to the INT workloads (the FP8 codec is not a ring codec)")
        ring = measure_ring(w, ex["ctx"]["xs"][0], ex["stream"], K=max(10, args.steps // 4))
    reorder = measure_reorder(w, ex["ctx"], ex["stream"], K=max(16, args.steps)) if args.reorder else None
    overlap = None
    if args.overlap or w.gemm:
        # the workload's GEMM alone, the codec step alone and both on two streams; --overlap adds the sweep
        # of launch caps
        overlap = measure_overlap(w, step_fn=ex["step"], nsets=ex["ctx"]["nsets"], stream=ex["stream"],
                                  K=max(10, args.steps // 2), ctx=ex["ctx"],
                                  caps=(0, 1024, 512, 256, 128, 64) if args.overlap else (0,))
    del ex
    torch.cuda.empty_cache()

    extras = {}
    for name in [x for x in args.extra.split(",") if x and x != "none" and x != args.workload]:
        r, e = run_workload(resolve(name), args, False)
        del e
        torch.cuda.empty_cache()
        extras[name] = r

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None if args.no_cpu else cpu_baseline(w, args.cpu_seconds)
    eight = {x["name"]: x["step_hbm_frac"] for x in [head] + list(extras.values()) if x["shards"] == 8}

    out = {
        "metric": "compress+reduce GB/s of bf16 input (fraction of HBM peak); quant rel-MSE",
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": head["workload"], "name": w.name,
            "shards": w.shards, "rows": w.rows, "cols": w.cols,
            "input_dtype": "bf16", "arithmetic": "f32 (bf16 widened exactly; sums and transform in f32)",
            "tensor_scale": head["tensor_scale"], "launch": args.launch, "input_sets": head["input_sets"],
        },
        "roofline": {
            "bound": "hbm", "kernel": dominant, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_launch,
            "launch_ms": kern["compress_ms"] if dominant == "compress" else kern["reduce_ms"],
            **({"copy_reference": head["copy_reference"]} if "copy_reference" in head else {}),
        },
        "step_hbm_frac": head["step_hbm_frac"],
        "step_ms_distribution": head["step_ms_distribution"],
        "kernels": kern,
        "algorithmic_bytes": head["algorithmic_bytes"],
        **({"quality": head["quality"]} if "quality" in head else {}),
        **({"consumer": head["consumer"]} if "consumer" in head else {}),
        "cpu_baseline": cpu,
        "eight_shard_step_hbm_frac": eight,
        "workloads": extras,
        **({"rank_share": rank_share} if rank_share else {}),
        **({"overlap": overlap} if overlap else {}),
        **({"reorder": reorder} if reorder else {}),
        **({"ring": ring} if ring else {}),
        "source_hash": src_hash,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

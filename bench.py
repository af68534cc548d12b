#!/usr/bin/env python3
"""Throughput of the tensor-parallel activation compression hot path on one MI355X.

One step = every rank's compress of its shard (N bf16 shards already resident
in HBM, one compress launch each) followed by the decompress-reduce of the N
compressed shards with re-quantization for the gather stage -- all of the hot
path. Shards rotate over several input sets so that the working set exceeds
the 256 MB Infinity Cache. Kernels are launched eagerly on one stream; the
timed region has one pair of HIP events per step. Each kernel's average launch
duration (for the roofline) comes from the same launches repeated right after,
each between its own pair of events on the launch stream. --launch graph
replays the step from HIP graphs instead (slower here: the runtime leaves gaps
between graph launches).

value = N * rows * cols * 2 bytes of bf16 input / step time (GB/s).

Prints one JSON line. --gpus above 1 is refused: this build measures one GPU.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt-tp")
    ap.add_argument("--scale-mode", choices=["delayed", "auto", "given"], default="delayed",
                    help="FP8 tensor scale: delayed (abs-max of the previous step, one pass), "
                         "auto (abs-max pre-pass of this tensor) or given (a fixed g, no workspace)")
    ap.add_argument("--launch", choices=["graph", "eager"], default="eager")
    ap.add_argument("--fp8-codes", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 workloads: the code format of the dual-scale codec (E5M2 is the variant "
                         "format 5)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--ring", action="store_true",
                    help="INT workloads: also time one quantized ring reduce-scatter hop (taco_ring_hop) at "
                         "full size and run the whole full-loop ring over the shards for its MSE")
    ap.add_argument("--overlap", action="store_true",
                    help="qwen-tp: also run the step concurrently with the bf16 GEMM that produces the "
                         "next activation, on a second stream, and report the overlap")
    ap.add_argument("--rank-share", action="store_true",
                    help="also time the decompress-reduce at one rank's share: (rows / N) x cols from N sources "
                         "(kept out of the default run so the profiled runs hold only full-size launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) for counter calibration")
    ap.add_argument("--summarize", nargs="+", metavar="PATH",
                    help="FETCH_DIR WRITE_DIR TRACE_DIR [TRACE_LOG]: turn rocprofv3 FETCH_SIZE / WRITE_SIZE / "
                         "kernel-trace output (and the bench line printed under the trace) into the "
                         "profiles/ summaries and exit")
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
    """One hop of the full-loop ring (dequantize the incoming shard, add the
    local bf16 shard, quantize for the next hop) timed at full size, and the
    whole ring over the workload's shards: its MSE against the exact sum, next
    to the MSE of quantizing the exact sum once (the all-gather alone)."""
    import torch
    import quantized_compression_tensor_amd as T
    c_in = T.codec(w.in_format, w.in_block, 0)
    c_out = T.codec(w.out_format, w.out_block, 0)
    dev = "cuda"
    N = len(xs)
    sh = stream.cuda_stream
    bufs = [T.empty_compressed(c_out, w.rows, w.cols, dev) for _ in range(3)]
    with torch.cuda.stream(stream):
        # the ring: the first rank quantizes its shard, every later rank adds its own
        T.taco_ring_hop(c_out, None, xs[0], w.rows, w.cols, None, c_out, bufs[0], stream=sh)
        for r in range(1, N):
            T.taco_ring_hop(c_out, bufs[(r - 1) % 2], xs[r], w.rows, w.cols, None, c_out, bufs[r % 2], stream=sh)
        ring = torch.empty(w.n, dtype=torch.float32, device=dev)
        T.taco_decompress(c_out, bufs[(N - 1) % 2], w.rows, w.cols, ring, 0, stream=sh)
        exact = torch.zeros(w.n, dtype=torch.float64, device=dev)
        for x in xs:
            exact += x.view(torch.bfloat16).reshape(-1).to(torch.float64)
        once_q = T.empty_compressed(c_out, w.rows, w.cols, dev)
        T.taco_requantize(c_out, exact.to(torch.float32), w.rows, w.cols, 1.0, once_q, stream=sh)
        once = torch.empty(w.n, dtype=torch.float32, device=dev)
        T.taco_decompress(c_out, once_q, w.rows, w.cols, once, 0, stream=sh)
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
    mse_ring = float(((ring.double() - exact) ** 2).mean())
    mse_once = float(((once.double() - exact) ** 2).mean())
    return {"hop_ms": round(hop_ms, 5), "hop_GBs": round(hop_bytes / (hop_ms * 1e-3) / 1e9, 1),
            "hop_hbm_frac": round(hop_bytes / (hop_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "hop_algorithmic_bytes": hop_bytes, "ranks": N, "hops": N - 1,
            "ring_mse": mse_ring, "all_gather_only_mse": mse_once, "ring_codec_in": "INT8 (gather codec)"}


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
KERNEL_KEYS = {"compress": ("k_fp8_had_compress", "k_quantize"), "reduce": ("k_reduce",)}


def _csv_rows(d, suffix):
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def summarize(fetch_dir, write_dir, trace_dir, workload, command, trace_log=None):
    """Per-launch HBM bytes of the hot kernels from two counter passes, scaled by
    what the same counters read for a plain copy of COPY_BYTES (read and write),
    plus the kernel-trace averages and, when the profiled run's output is given,
    the bench's own event timing in that same run; written to
    profiles/<kernel>_<workload>_*.txt."""
    import numpy as np
    src_hash = kernel_source_hash()
    bench_ms = {}
    if trace_log:
        lines = [l for l in open(trace_log) if l.startswith("{")]
        if lines:
            k = json.loads(lines[-1]).get("kernels", {})
            bench_ms = {"compress": k.get("compress_ms"), "reduce": k.get("reduce_ms")}
    per = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for row in _csv_rows(d, "counter_collection.csv"):
            if row.get("Counter_Name") != cname:
                continue
            name = row.get("Kernel_Name", "")
            per.setdefault((cname, name), []).append(float(row["Counter_Value"]))
    # the calibration copies are the three largest copy dispatches of the run
    copy_f = sorted((v for (c, k), vs in per.items() if c == "FETCH_SIZE" and "copy" in k.lower() for v in vs),
                    reverse=True)[:3]
    copy_w = sorted((v for (c, k), vs in per.items() if c == "WRITE_SIZE" and "copy" in k.lower() for v in vs),
                    reverse=True)[:3]
    f_fetch = COPY_BYTES / (np.median(copy_f) * 1024) if copy_f else None
    f_write = COPY_BYTES / (np.median(copy_w) * 1024) if copy_w else None
    trace = {}
    for row in _csv_rows(trace_dir, "kernel_stats.csv"):
        trace[row["Name"]] = row
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for key, subs in KERNEL_KEYS.items():
        fk = [(k, vs) for (c, k), vs in per.items() if c == "FETCH_SIZE" and any(t in k for t in subs)]
        wk = [(k, vs) for (c, k), vs in per.items() if c == "WRITE_SIZE" and any(t in k for t in subs)]
        fk.sort(key=lambda kv: -len(kv[1]))
        wk.sort(key=lambda kv: -len(kv[1]))
        if not fk or not wk:
            continue
        kname = fk[0][0]
        fetch_kib = float(np.median(fk[0][1]))
        write_kib = float(np.median(wk[0][1]))
        hbm = None
        if f_fetch and f_write:
            hbm = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
        tr = next((v for n, v in trace.items() if n == kname), None)
        path = os.path.join(ROOT, "profiles", f"{key}_{workload}_counters.txt")
        with open(path, "w") as fh:
            fh.write(f"# rocprofv3 hardware counters for {kname}\n")
            fh.write(f"# workload: {workload}\n# command: {command}\n")
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
            if tr is not None:
                fh.write(f"trace_calls: {tr.get('Calls')}\n")
                fh.write(f"trace_average_ns: {tr.get('AverageNs')}\n")
                fh.write(f"trace_min_ns: {tr.get('MinNs')}\n")
                fh.write(f"trace_max_ns: {tr.get('MaxNs')}\n")
            if bench_ms.get(key) is not None:
                fh.write("# the bench's own HIP-event average in the profiled run (back-to-back launches,\n"
                         "# including the gap before each launch, which the profiler widens)\n")
                fh.write(f"bench_event_average_ns_under_profiler: {bench_ms[key] * 1e6:.0f}\n")
        written.append(path)
    if trace:
        path = os.path.join(ROOT, "profiles", f"kernels_{workload}_trace.txt")
        with open(path, "w") as fh:
            fh.write(f"# rocprofv3 kernel-trace statistics, workload {workload}\n# command: {command}\n")
            fh.write("# (kernel durations exclude dispatch gaps; the bench's step events include them)\n")
            fh.write(f"source_hash: {src_hash}\n")
            fh.write(f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel\n")
            for name, row in sorted(trace.items(), key=lambda kv: -float(kv[1]["TotalDurationNs"])):
                fh.write(f"{int(row['Calls']):>6} {float(row['AverageNs']) / 1e3:>9.2f} "
                         f"{float(row['MinNs']) / 1e3:>9.2f} {float(row['MaxNs']) / 1e3:>9.2f}  {name[:160]}\n")
        written.append(path)
    print("\n".join(written))


def cpu_baseline(w, seconds):
    """The oracle, as written, on a bounded sample of the same workload: row
    chunks of every shard, compressed and reduced (+ requantized), spread over
    a thread pool (NumPy releases the GIL inside its loops)."""
    import numpy as np
    import oracle
    from oracle import codecs as cd
    import workloads as W

    cin = cd.Codec(w.in_format, w.in_block, w.hadamard)
    cout = cd.Codec(w.out_format, w.out_block, w.hadamard) if w.out_format else None
    nchunks = (w.rows + W.ROW_CHUNK - 1) // W.ROW_CHUNK
    threads = max(1, min(16, os.cpu_count() or 1))

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
    return {"value": round(bytes_in / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {w.rows} rows of each of the {w.shards} shards ({len(chunks)} chunks of "
                      f"{W.ROW_CHUNK} rows): compress + decompress-reduce"
                      + (" + requantize" if cout else "") + f"; {passes} pass(es), {dt:.1f} s"}


def quality(w, bufs, sets_bits, c_in):
    """rel-MSE of the compress round trip of shard 0 (set 0) on a seeded sample of
    row chunks: the GPU's (decoded on the GPU) next to the oracle's own."""
    import numpy as np
    import torch
    import oracle
    from oracle import codecs as cd
    from oracle.formats import bf16_bits_to_f32
    import quantized_compression_tensor_amd as T
    import workloads as W

    ch = W.sample_chunks(w, 3, seed=7)
    rows_idx = W.chunk_rows(ch, w.rows)
    d = torch.empty(w.n, dtype=torch.float32, device="cuda")
    T.taco_decompress(c_in, bufs[0][0], w.rows, w.cols, d, 0)
    torch.cuda.synchronize()
    x = sets_bits[0][0][rows_idx]
    got = d.view(w.rows, w.cols)[torch.from_numpy(rows_idx).cuda()].cpu().numpy()
    xf = bf16_bits_to_f32(x)
    oc = cd.Codec(w.in_format, w.in_block, w.hadamard)
    ref = oracle.decode(oracle.compress(oc, x))
    return {"rel_mse_gpu": oracle.rel_mse(got, xf), "rel_mse_oracle": oracle.rel_mse(ref, xf),
            "sample_rows": int(len(rows_idx))}


def measure_overlap(w, step_fn, nsets, stream, codec_ms, K):
    """The bf16 GEMM [rows, cols] x [cols, cols] that produces the next activation,
    alone and concurrently with the codec step on a second stream (default
    priority). Reported: GEMM alone, codec alone (the timed step), both together,
    and how much of the shorter one the overlap hid."""
    import torch
    g_stream = torch.cuda.Stream()
    a = torch.randn(w.rows, w.cols, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(w.cols, w.cols, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(w.rows, w.cols, dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(g_stream):
        for _ in range(3):
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(g_stream):
        for _ in range(K):
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    gemm_ms = (time.perf_counter() - t0) * 1e3 / K
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        with torch.cuda.stream(g_stream):
            torch.matmul(a, b, out=c)
        with torch.cuda.stream(stream):
            step_fn(i % nsets)
    torch.cuda.synchronize()
    both_ms = (time.perf_counter() - t0) * 1e3 / K
    flops = 2.0 * w.rows * w.cols * w.cols
    serial = gemm_ms + codec_ms
    return {"gemm_ms": round(gemm_ms, 4), "gemm_tflops": round(flops / gemm_ms / 1e9, 1),
            "codec_ms": round(codec_ms, 4), "both_ms": round(both_ms, 4), "serial_ms": round(serial, 4),
            "hidden_frac": round((serial - both_ms) / min(gemm_ms, codec_ms), 3)}


def main():
    args = parse()
    if args.summarize:
        if len(args.summarize) not in (3, 4):
            sys.exit("--summarize takes FETCH_DIR WRITE_DIR TRACE_DIR [TRACE_LOG]")
        fetch, write, trace = args.summarize[:3]
        log = args.summarize[3] if len(args.summarize) == 4 else None
        summarize(fetch, write, trace, args.workload, args.command, log)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is a design, not part of this build)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import quantized_compression_tensor_amd as T
    import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.fp8_codes == "e5m2" and w.in_format == T.TACO_FMT_FP8_DUAL:
        w = dataclasses.replace(w, in_format=T.TACO_FMT_FP8E5_DUAL,
                                out_format=T.TACO_FMT_FP8E5_DUAL if w.out_format else None)
    torch.cuda.set_device(0)
    dev = "cuda"
    c_in = T.codec(w.in_format, w.in_block, 1 if w.hadamard else 0)
    c_out = T.codec(w.out_format, w.out_block, 1 if w.hadamard else 0) if w.out_format else None
    fp8 = w.in_format in T.FP8_FORMATS
    scale = {"delayed": T.TACO_SCALE_DELAYED, "auto": T.TACO_SCALE_AUTO, "given": 0.01}[args.scale_mode] \
        if fp8 else 1.0
    use_ws = fp8 and args.scale_mode != "given"

    in_bytes = w.shards * w.n * 2
    nsets = max(2, min(4, -(-2 * MALL_BYTES // in_bytes) + 1))
    sets_bits, xs, bufs, outs = [], [], [], []
    for s in range(nsets):
        bits = [W.make_shard(w, r + 100 * s) for r in range(w.shards)]
        sets_bits.append(bits if s == 0 else None)
        xs.append([torch.from_numpy(b.view(np.int16)).to(dev) for b in bits])
        bufs.append([T.empty_compressed(c_in, w.rows, w.cols, dev) for _ in range(w.shards)])
        if c_out is not None:
            outs.append(T.empty_compressed(c_out, w.rows, w.cols, dev))
        else:
            outs.append(torch.empty(w.n, dtype=torch.float32, device=dev))
    wss = [torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=dev) for _ in range(w.shards)]
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def compress_one(s, r):
        T.taco_compress(c_in, xs[s][r], w.rows, w.cols, scale, bufs[s][r],
                        workspace=wss[r] if use_ws else None, stream=sh)

    def compress(s):
        for r in range(w.shards):
            compress_one(s, r)

    def reduce(s):
        if c_out is not None:
            T.taco_decompress_reduce(c_in, bufs[s], w.rows, w.cols, None, c_out, outs[s], stream=sh)
        else:
            T.taco_decompress_reduce(c_in, bufs[s], w.rows, w.cols, outs[s], stream=sh)

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

        for i in range(args.warmup):
            step(i % nsets)
        torch.cuda.synchronize()

        K = args.steps
        mk = lambda: torch.cuda.Event(enable_timing=True)
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

        # per-kernel launch durations (roofline): the same launches again, each
        # kernel's K steps' worth back to back between one pair of events on the
        # launch stream; the average includes the short gap between dependent
        # launches, so it is an upper bound on the kernel's own duration
        a_c, b_c, a_r, b_r = mk(), mk(), mk(), mk()
        a_c.record(stream)
        for i in range(K):
            compress(i % nsets)
        b_c.record(stream)
        a_r.record(stream)
        for i in range(K):
            reduce(i % nsets)
        b_r.record(stream)
        # streaming reference: a plain device copy of each shard (2 B read +
        # 2 B written per element), timed like the compress. Left out of the
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

    t_comp = a_c.elapsed_time(b_c) / (K * w.shards)   # ms per compress launch
    t_red = a_r.elapsed_time(b_r) / K                 # ms per reduce call
    t_dec = a_d.elapsed_time(b_d) / K if dec_out is not None else None
    t_ref = a_x.elapsed_time(b_x) / (K * w.shards) if not args.copy_calibration else None
    ms_step = wall * 1e3 / K
    gpu_ms_step = ev0.elapsed_time(ev1) / K
    value = in_bytes / (ms_step * 1e-3) / 1e9

    b_comp, b_red = algorithmic_bytes(w)
    comp_gbs = b_comp / (t_comp * 1e-3) / 1e9
    red_gbs = b_red / (t_red * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    dominant = "compress" if w.shards * t_comp >= t_red else "reduce"
    if dominant == "compress":
        ach, bytes_launch, kname = comp_gbs, b_comp, "compress"
    else:
        ach, bytes_launch, kname = red_gbs, b_red, "reduce"
    traffic = read_traffic(kname, w.name, src_hash)

    rank_share = measure_rank_share(w, xs, stream, K=max(20, K // 2)) if args.rank_share else None

    ring = None
    if args.ring:
        if w.in_format in T.FP8_FORMATS:
            sys.exit("--ring applies to the INT workloads (the FP8 codec is not a ring codec)")
        ring = measure_ring(w, xs[0], stream, K=max(10, K // 4))

    overlap = None
    if args.overlap:
        overlap = measure_overlap(w, step_fn=lambda s: (compress(s), reduce(s)), nsets=nsets, stream=stream,
                                  codec_ms=ms_step, K=max(5, K // 5))

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    q = quality(w, bufs, sets_bits, c_in)
    cpu = None if args.no_cpu else cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "compress+reduce GB/s of bf16 input (fraction of HBM peak); quant rel-MSE",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.shards} bf16 shards of {w.rows}x{w.cols}; "
                        f"compress {['', 'FP8 dual-scale', 'INT8 sym', 'INT4 asym', 'INT8 asym', 'FP8 E5M2 dual-scale'][w.in_format]} "
                        f"block {w.in_block}{' + Hadamard' if w.hadamard else ''}; decompress-reduce "
                        + (f"-> {['', 'FP8 dual-scale', 'INT8 sym', 'INT4 asym', 'INT8 asym', 'FP8 E5M2 dual-scale'][w.out_format]}"
                           if w.out_format else "-> FP32 sum"),
            "shards": w.shards, "rows": w.rows, "cols": w.cols,
            "tensor_scale": args.scale_mode if fp8 else "n/a",
            "launch": args.launch, "input_sets": nsets,
        },
        "roofline": {
            "bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_launch,
            "copy_reference": {
                "kernel": "device copy of one bf16 shard (2 B read + 2 B written per element), timed like "
                          "the compress: the streaming rate this machine reaches at this size",
                "ms": round(t_ref, 5), "GBs": round(4 * w.n / (t_ref * 1e-3) / 1e9, 1),
                "compress_vs_copy": round(comp_gbs / (4 * w.n / (t_ref * 1e-3) / 1e9), 3),
            } if t_ref else None,
        },
        "kernels": {
            "compress_ms": round(t_comp, 5), "compress_GBs": round(comp_gbs, 1),
            "reduce_ms": round(t_red, 5), "reduce_GBs": round(red_gbs, 1),
            **({"decode_bf16_ms": round(t_dec, 5),
                "decode_bf16_GBs": round(decode_bytes(w) / (t_dec * 1e-3) / 1e9, 1)} if t_dec else {}),
            "step_hbm_frac": round((w.shards * b_comp + b_red) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "host_ms_per_step": round(host * 1e3 / K, 5),
            "event_ms_per_step": round(gpu_ms_step, 5),
        },
        **({"rank_share": rank_share} if rank_share else {}),
        "quality": q,
        "cpu_baseline": cpu,
        **({"overlap": overlap} if overlap else {}),
        **({"ring": ring} if ring else {}),
        "source_hash": src_hash,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

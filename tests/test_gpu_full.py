"""GPU parity at the full workload sizes, in the launch configuration the bench
times: the whole tensors go through the GPU; the oracle recomputes a seeded
sample of row chunks (first, last and random ones) of every shard, which must
match bit for bit, and properties that hold at any size are checked on the
whole output."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
from oracle.formats import bf16_bits_to_f32
import quantized_compression_tensor_amd as T
import dataclasses

import workloads as W
from tests.gpu_util import DEV, ccodec, new_workspace, same_f32_bits

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def rows_of(buf, oc, rows, cols, idx):
    """Codes / scales / zero points of the selected rows of a GPU buffer."""
    codes, sc, aux, ten = T.regions(buf, ccodec(oc), rows, cols)
    it = torch.from_numpy(idx).to(DEV)
    cpr = cols // 2 if oc.format == cd.INT4_ASYM else cols
    bpr = cols // oc.block
    out = dict(codes=codes.view(rows, cpr)[it].cpu().numpy().reshape(-1),
               scale=sc.view(rows, bpr)[it].cpu().numpy().reshape(-1),
               zero=aux.view(rows, bpr)[it].cpu().numpy().reshape(-1) if aux.numel() else None,
               g=np.float32(ten.cpu().numpy()[0]) if ten.numel() else None)
    return out


def check_rows(got, ref, where):
    assert (got["codes"] == ref.codes).all(), f"{where}: {(got['codes'] != ref.codes).sum()} codes differ"
    if ref.codec.format in cd.FP8_FORMATS:
        assert (got["scale"].astype(np.int8) == ref.scale.astype(np.int8)).all(), f"{where}: exponents differ"
        assert got["g"] == ref.tensor_scale, f"{where}: g {got['g']} vs {ref.tensor_scale}"
    else:
        assert (got["scale"].view(np.uint32) == ref.scale.view(np.uint32)).all(), f"{where}: scales differ"
    if ref.zero is not None:
        assert (got["zero"] == ref.zero).all(), f"{where}: zero points differ"


def _workload(name):
    if name == "gpt-tp-e5m2":   # the gpt-tp tensors through the E5M2 variant of the FP8 codec
        return dataclasses.replace(W.WORKLOADS["gpt-tp"], name=name, in_format=cd.FP8E5_DUAL,
                                   out_format=cd.FP8E5_DUAL)
    return W.WORKLOADS[name]


@pytest.mark.parametrize("name", ["gpt-tp", "equarx", "flashcomm", "qwen-tp", "gpt-tp-e5m2"])
def test_full_size_workload(name):
    w = _workload(name)
    cin = cd.Codec(w.in_format, w.in_block, w.hadamard)
    cout = cd.Codec(w.out_format, w.out_block, w.hadamard)
    fp8 = cin.format in cd.FP8_FORMATS
    chunks = W.sample_chunks(w, 2, seed=11)
    idx = W.chunk_rows(chunks, w.rows)
    print(f"[{name}] {w.shards} x {w.rows}x{w.cols}, sampled rows {len(idx)}", flush=True)

    # GPU: whole tensors, one compress per shard exactly as the bench launches it
    # (a fresh workspace in delayed-scale mode has no history, so g = 1)
    bufs, exact = [], None
    for r in range(w.shards):
        bits = W.make_shard(w, r)
        x = torch.from_numpy(bits.view(np.int16)).to(DEV)
        buf = T.empty_compressed(ccodec(cin), w.rows, w.cols, DEV)
        if fp8:
            T.taco_compress(ccodec(cin), x, w.rows, w.cols, T.TACO_SCALE_DELAYED, buf, workspace=new_workspace())
        else:
            T.taco_compress(ccodec(cin), x, w.rows, w.cols, 1.0, buf)
        xf = x.view(torch.bfloat16).to(torch.float64)
        exact = xf if exact is None else exact + xf
        del x, xf
        bufs.append(buf)
    s = torch.empty(w.n, dtype=torch.float32, device=DEV)
    out = T.empty_compressed(ccodec(cout), w.rows, w.cols, DEV)
    T.taco_decompress_reduce(ccodec(cin), bufs, w.rows, w.cols, s, ccodec(cout), out)
    dec = torch.empty(w.n, dtype=torch.float32, device=DEV)
    T.taco_decompress(ccodec(cout), out, w.rows, w.cols, dec, 0)
    torch.cuda.synchronize()

    # oracle on the sampled rows of every shard
    refs = []
    for r in range(w.shards):
        sb = W.make_shard(w, r, chunks=chunks)
        ref = oracle.compress(cin, sb, tensor_scale=np.float32(1.0) if fp8 else None)
        check_rows(rows_of(bufs[r], cin, w.rows, w.cols, idx), ref, f"{name} shard {r}")
        refs.append(ref)
    acc, rq = oracle.decompress_reduce(refs, cout)
    it = torch.from_numpy(idx).to(DEV)
    assert same_f32_bits(s.view(w.rows, w.cols)[it].cpu().numpy(), acc).all(), f"{name}: FP32 sum differs"
    check_rows(rows_of(out, cout, w.rows, w.cols, idx), rq, f"{name} requantized")

    # whole-tensor properties: the gather-stage output decodes to the exact sum
    # of the bf16 shards within the codec's error, in every row
    err = (dec.view(w.rows, w.cols).double() - exact.view(w.rows, w.cols))
    num = (err * err).sum(dim=1)
    den = (exact.view(w.rows, w.cols) ** 2).sum(dim=1)
    worst = float((num / den).max())
    total = float(num.sum() / den.sum())
    # per-row sanity bounds: FP8 ~7e-4 per quantization, INT8 ~5e-5, INT4 ~1e-2
    limit = {cd.FP8_DUAL: 1e-2, cd.FP8E5_DUAL: 4e-2, cd.INT8_SYM: 1e-3, cd.INT8_ASYM: 1e-1}[cout.format]
    print(f"[{name}] requantized sum rel-MSE {total:.3e} (worst row {worst:.3e})", flush=True)
    assert worst < limit and np.isfinite(worst)
    if fp8:
        assert rows_of(out, cout, w.rows, w.cols, idx[:1])["g"] == np.float32(w.shards)   # g' = sum of g_r = N


# A reduce launch covers at most 2^28 elements; the host splits larger tensors
# into pieces over offset pointers. 65600 x 4096 is 262144 elements past 2^28,
# so the second piece holds the last 64 rows.
PIECE_PAIRS = [
    (cd.Codec(cd.FP8_DUAL, 128, True), cd.Codec(cd.FP8_DUAL, 128, True), "normal"),
    (cd.Codec(cd.INT8_SYM, 64, False), cd.Codec(cd.INT8_SYM, 64, False), "normal"),
    (cd.Codec(cd.INT4_ASYM, 128, False), cd.Codec(cd.INT8_ASYM, 128, False), "t3"),
    (cd.Codec(cd.INT8_ASYM, 128, False), cd.Codec(cd.INT8_ASYM, 128, False), "t3"),
]


@pytest.mark.parametrize("cin,cout,body", PIECE_PAIRS,
                         ids=lambda p: f"fmt{p.format}" if isinstance(p, cd.Codec) else p)
def test_reduce_split_into_pieces(cin, cout, body):
    rows, cols, shards = 65600, 4096, 2
    assert rows * cols > (1 << 28)
    w = W.Workload("piece-split", rows, cols, shards, 6000 + cin.format, body, 0.02,
                   cin.format, cin.block, cin.hadamard, cout.format, cout.block)
    fp8 = cin.format == cd.FP8_DUAL
    g = np.float32(0.0125)
    n_chunks = (rows + W.ROW_CHUNK - 1) // W.ROW_CHUNK
    chunks = [0, (1 << 28) // cols // W.ROW_CHUNK - 1, n_chunks - 1]   # first, last of piece 0, piece 1
    idx = W.chunk_rows(chunks, rows)
    print(f"[piece-split {cin.format}->{cout.format}] n = {rows * cols}, sampled rows {len(idx)}", flush=True)
    bufs = []
    for r in range(shards):
        x = torch.from_numpy(W.make_shard(w, r).view(np.int16)).to(DEV)
        buf = T.empty_compressed(ccodec(cin), rows, cols, DEV)
        T.taco_compress(ccodec(cin), x, rows, cols, float(g) if fp8 else 1.0, buf)
        del x
        bufs.append(buf)
    s = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    out = T.empty_compressed(ccodec(cout), rows, cols, DEV)
    T.taco_decompress_reduce(ccodec(cin), bufs, rows, cols, s, ccodec(cout), out)
    torch.cuda.synchronize()

    refs = []
    for r in range(shards):
        ref = oracle.compress(cin, W.make_shard(w, r, chunks=chunks), tensor_scale=g if fp8 else None)
        check_rows(rows_of(bufs[r], cin, rows, cols, idx), ref, f"shard {r}")
        refs.append(ref)
    acc, rq = oracle.decompress_reduce(refs, cout)
    it = torch.from_numpy(idx).to(DEV)
    assert same_f32_bits(s.view(rows, cols)[it].cpu().numpy(), acc).all(), "FP32 sum differs"
    check_rows(rows_of(out, cout, rows, cols, idx), rq, "requantized")
    if fp8:
        assert rows_of(out, cout, rows, cols, idx[:1])["g"] == np.float32(g + g)   # written once, by piece 0

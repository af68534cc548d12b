"""GPU parity of the data-driven reshaping (taco_chunk_order,
taco_compress_reordered, taco_decompress_reordered) against the oracle's
chunk_order, compress_reordered and decode_reordered: orders equal, codes and
scales bit-exact, decodes bit-exact, for every format, on ragged and
multi-tile shapes, through a whole reduce, under a launch cap, and with order
entries out of range (clamped into the row)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
from oracle.formats import f32_to_bf16_bits
import quantized_compression_tensor_amd as T
import workloads as W
from tests.gpu_util import DEV, ccodec, upload_bits, new_workspace, parse, assert_same, same_f32_bits

pytestmark = pytest.mark.gpu

CODECS = [cd.Codec.fp8(128, True), cd.Codec.fp8e5(128, True), cd.Codec.fp8(128, False), cd.Codec.int8_sym(),
          cd.Codec.int4_asym(), cd.Codec.int8_asym()]
# Compress and decode stage whole rows through LDS in units of the fewest rows
# that hold at least 8192 elements, at most 16384, and whole tiles (1024
# elements for the INT codecs, 512 for the FP8 Hadamard kernels); other rows
# are gathered from global memory. The shapes take partial last units (1 x 512,
# 3 x 1024, 37 x 1536), 9728 (INT: gathered, no unit of whole tiles fits;
# FP8: one row), one 16384-column row (a 64 KiB float32 unit) and 16896,
# gathered throughout.
SHAPES = [(1, 512), (3, 1024), (37, 1536), (300, 4096), (64, 5120), (7, 9728), (2, 16384), (3, 16896)]


def cid(oc):
    return f"f{oc.format}-b{oc.block}" + ("-h" if oc.hadamard else "")


def gpu_order(bits):
    rows, cols = bits.shape
    o = torch.empty(cols // 8, dtype=torch.int32, device=DEV)
    T.taco_chunk_order(upload_bits(bits) if rows else torch.empty(16, dtype=torch.int16, device=DEV), rows, cols, o)
    torch.cuda.synchronize()
    return o


def outlier_bits(shape, seed):
    rng = np.random.default_rng(seed)
    x = (0.02 * rng.standard_t(3, size=shape)).astype(np.float32)
    ch = rng.choice(shape[1], size=max(1, shape[1] // 100), replace=False)
    x[:, ch] *= np.float32(100.0)
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("shape", SHAPES + [(0, 1024), (2000, 512), (3, 131072), (0, 131072)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_chunk_order_matches_oracle(shape):
    bits = outlier_bits(shape, seed=shape[0] + shape[1]) if shape[0] else np.zeros(shape, np.uint16)
    got = gpu_order(bits).cpu().numpy()
    assert (got == oracle.chunk_order(bits)).all()


def test_chunk_order_ties_zeros_and_nan():
    x = np.zeros((5, 1024), np.float32)
    x[:, 8:16] = 3.0                       # groups 1 and 7 tie
    x[2, 56:64] = -3.0
    x[4, 100] = np.nan                     # group 12: NaN ranks as the largest (like infinity)
    x[1, 200] = np.inf                     # group 25 ties with it
    x[3, 1000] = 1e-30
    bits = f32_to_bf16_bits(x)
    got = gpu_order(bits).cpu().numpy()
    assert (got == oracle.chunk_order(bits)).all()
    assert got[:4].tolist() == [12, 25, 1, 7]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("oc", CODECS, ids=cid)
def test_compress_and_decode_reordered(oc, shape):
    rows, cols = shape
    x = outlier_bits(shape, seed=31 * rows + oc.format)
    stats = outlier_bits(shape, seed=31 * rows + oc.format + 7)
    order = gpu_order(stats)
    o = order.cpu().numpy().astype(np.int64)
    assert (o == oracle.chunk_order(stats)).all()
    c = ccodec(oc)
    fp8 = oc.format in cd.FP8_FORMATS
    buf = T.empty_compressed(c, rows, cols)
    ws = new_workspace() if fp8 else None
    T.taco_compress_reordered(c, upload_bits(x), rows, cols, T.TACO_SCALE_AUTO if fp8 else 1.0, buf, order, workspace=ws)
    d32 = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    d16 = torch.empty(rows * cols, dtype=torch.int16, device=DEV)
    T.taco_decompress_reordered(c, buf, rows, cols, d32, order, 0)
    T.taco_decompress_reordered(c, buf, rows, cols, d16, order, 1)
    torch.cuda.synchronize()
    ref = oracle.compress_reordered(oc, x, o)
    assert_same(parse(buf, oc, rows, cols), ref, "reordered compress")
    assert same_f32_bits(d32.cpu().numpy(), oracle.decode_reordered(ref, o)).all(), "decode f32"
    assert (d16.cpu().numpy().view(np.uint16) == oracle.decode_reordered(ref, o, "bf16").reshape(-1)).all(), \
        "decode bf16"


def _random_shapes(seed, count):
    """Seeded (rows, cols): cols a multiple of 512 up to 20480 (staged units of
    1 to 16 rows, and a few gathered widths), rows 1 to 40 (partial last
    units of every size)."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 41)), 512 * int(rng.integers(1, 41))) for _ in range(count)]


@pytest.mark.parametrize("oc", [cd.Codec.fp8(128, True), cd.Codec.int8_sym(), cd.Codec.int4_asym(),
                                cd.Codec.int8_asym()], ids=cid)
def test_reordered_random_shapes(oc):
    """Compress and both decodes, reordered, on seeded random shapes against
    the oracle, bit for bit (the FP8 codec with its data-driven tensor scale,
    so the abs-max pre-pass runs too)."""
    fp8 = oc.format in cd.FP8_FORMATS
    c = ccodec(oc)
    for rows, cols in _random_shapes(1000 + oc.format, 10):
        print(f"[reorder random] {cid(oc)} {rows}x{cols}", flush=True)
        x = outlier_bits((rows, cols), seed=rows * cols + oc.format)
        order = gpu_order(outlier_bits((rows, cols), seed=rows * cols + 1))
        o = order.cpu().numpy().astype(np.int64)
        buf = T.empty_compressed(c, rows, cols)
        T.taco_compress_reordered(c, upload_bits(x), rows, cols, T.TACO_SCALE_AUTO if fp8 else 1.0, buf, order,
                                  workspace=new_workspace() if fp8 else None)
        d32 = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
        d16 = torch.empty(rows * cols, dtype=torch.int16, device=DEV)
        T.taco_decompress_reordered(c, buf, rows, cols, d32, order, 0)
        T.taco_decompress_reordered(c, buf, rows, cols, d16, order, 1)
        torch.cuda.synchronize()
        ref = oracle.compress_reordered(oc, x, o)
        assert_same(parse(buf, oc, rows, cols), ref, f"reordered compress {rows}x{cols}")
        assert same_f32_bits(d32.cpu().numpy(), oracle.decode_reordered(ref, o)).all(), f"decode f32 {rows}x{cols}"
        assert (d16.cpu().numpy().view(np.uint16) == oracle.decode_reordered(ref, o, "bf16").reshape(-1)).all(), \
            f"decode bf16 {rows}x{cols}"


@pytest.mark.parametrize("oc", [cd.Codec.fp8(128, True), cd.Codec.int8_sym(), cd.Codec.int4_asym()], ids=cid)
def test_reordered_shards_through_the_reduce(oc):
    # every rank compresses its shard in the shared order; the reduce and the
    # requantization run on the reordered tensors unchanged; the consumer
    # decodes with the inverse order
    rows, cols, n = 64, 4096, 4
    xs = [outlier_bits((rows, cols), seed=400 + r) for r in range(n)]
    order = gpu_order(outlier_bits((rows, cols), seed=499))
    o = order.cpu().numpy().astype(np.int64)
    c = ccodec(oc)
    go = cd.Codec.int8_asym() if oc.format == cd.INT4_ASYM else oc
    co = ccodec(go)
    fp8 = oc.format in cd.FP8_FORMATS
    bufs = []
    for r in range(n):
        b = T.empty_compressed(c, rows, cols)
        T.taco_compress_reordered(c, upload_bits(xs[r]), rows, cols, 0.01 if fp8 else 1.0, b, order)
        bufs.append(b)
    out = T.empty_compressed(co, rows, cols)
    T.taco_decompress_reduce(c, bufs, rows, cols, None, co, out)
    dec = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    T.taco_decompress_reordered(co, out, rows, cols, dec, order, 0)
    torch.cuda.synchronize()
    refs = [oracle.compress_reordered(oc, xs[r], o, tensor_scale=np.float32(0.01) if fp8 else None) for r in range(n)]
    _, rq = oracle.decompress_reduce(refs, go)
    assert_same(parse(out, go, rows, cols), rq, "requantized sum")
    assert same_f32_bits(dec.cpu().numpy(), oracle.decode_reordered(rq, o)).all()


@pytest.mark.parametrize("oc", [cd.Codec.fp8(128, True), cd.Codec.int4_asym()], ids=cid)
def test_reordered_under_a_launch_cap(oc):
    rows, cols = 300, 5120
    x = outlier_bits((rows, cols), seed=77)
    order = gpu_order(outlier_bits((rows, cols), seed=78))
    c = ccodec(oc)
    fp8 = oc.format in cd.FP8_FORMATS
    outs = []
    for lim in (0, 1, 5):
        b = T.empty_compressed(c, rows, cols)
        d = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
        with T.launch_limit(lim):
            T.taco_compress_reordered(c, upload_bits(x), rows, cols, T.TACO_SCALE_AUTO if fp8 else 1.0, b, order,
                                      workspace=new_workspace() if fp8 else None)
            T.taco_decompress_reordered(c, b, rows, cols, d, order, 0)
        torch.cuda.synchronize()
        outs.append((parse(b, oc, rows, cols), d.cpu().numpy()))
    for p, d in outs[1:]:
        assert (p["codes"] == outs[0][0]["codes"]).all() and (p["scale"].view(np.uint8) == outs[0][0]["scale"].view(np.uint8)).all()
        assert (d.view(np.uint32) == outs[0][1].view(np.uint32)).all()


def test_order_entries_out_of_range_are_clamped_into_the_row():
    # a caller's order that is not a permutation reads no memory outside the
    # row: entries below 0 read group 0, entries past the end the last group
    oc = cd.Codec.int8_sym()
    rows, cols = 8, 1024
    x = outlier_bits((rows, cols), seed=5)
    bad = np.arange(cols // 8, dtype=np.int32)
    bad[3], bad[10], bad[100] = -7, 10 ** 6, 128
    order = torch.from_numpy(bad).to(DEV)
    c = ccodec(oc)
    b = T.empty_compressed(c, rows, cols)
    T.taco_compress_reordered(c, upload_bits(x), rows, cols, 1.0, b, order)
    torch.cuda.synchronize()
    clamped = np.clip(bad, 0, cols // 8 - 1).astype(np.int64)
    cmap = (clamped[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    assert_same(parse(b, oc, rows, cols), oracle.compress(oc, x[:, cmap]), "clamped order")
    # the decode of such an order writes unspecified values but stays inside
    # its row and its output (INT: gathered through the order's inverse; FP8
    # with the transform: scattered through the order)
    for dc in (oc, cd.Codec.fp8(128, True)):
        cc = ccodec(dc)
        bb = T.empty_compressed(cc, rows, cols)
        T.taco_compress(cc, upload_bits(x), rows, cols, 0.01 if dc.format in cd.FP8_FORMATS else 1.0, bb)
        guard = torch.full((3 * rows * cols,), 7.0, dtype=torch.float32, device=DEV)
        out = guard[rows * cols:2 * rows * cols]
        T.taco_decompress_reordered(cc, bb, rows, cols, out, order, 0)
        torch.cuda.synchronize()
        g = guard.cpu().numpy()
        assert (g[:rows * cols] == 7.0).all() and (g[2 * rows * cols:] == 7.0).all(), cid(dc)


def test_full_size_reordered_compress_sampled_rows():
    # qwen-tp shape: the order from another shard, the whole tensor through the
    # GPU (compress, then the bf16 and float32 decodes: at this size each
    # workgroup walks many staged units, with the next one's loads in flight),
    # sampled row chunks through the oracle with the same order
    w = W.WORKLOADS["qwen-tp"]
    oc = cd.Codec.fp8(128, True)
    c = ccodec(oc)
    order = torch.empty(w.cols // 8, dtype=torch.int32, device=DEV)
    stats = W.make_shard(w, 1, chunks=list(range(8)))
    T.taco_chunk_order(upload_bits(stats), stats.shape[0], w.cols, order)
    x = W.make_shard(w, 0)
    buf = T.empty_compressed(c, w.rows, w.cols)
    T.taco_compress_reordered(c, upload_bits(x), w.rows, w.cols, 0.0078125, buf, order)
    torch.cuda.synchronize()
    o = order.cpu().numpy().astype(np.int64)
    assert (o == oracle.chunk_order(stats)).all()
    chunks = W.sample_chunks(w, 2, seed=3)
    idx = W.chunk_rows(chunks, w.rows)
    ref = oracle.compress_reordered(oc, x[idx], o, tensor_scale=np.float32(0.0078125))
    codes, k, _, _ = T.regions(buf, c, w.rows, w.cols)
    it = torch.from_numpy(idx).to(DEV)
    assert (codes.view(w.rows, w.cols)[it].cpu().numpy().reshape(-1) == ref.codes).all()
    assert (k.view(w.rows, w.cols // 128)[it].cpu().numpy().reshape(-1) == ref.scale).all()
    del x
    dec = torch.empty(w.rows * w.cols, dtype=torch.int16, device=DEV)
    T.taco_decompress_reordered(c, buf, w.rows, w.cols, dec, order, 1)
    torch.cuda.synchronize()
    got_d = dec.view(w.rows, w.cols)[it].cpu().numpy().view(np.uint16).reshape(-1)
    assert (got_d == oracle.decode_reordered(ref, o, "bf16").reshape(-1)).all(), "decode"
    del dec
    d32 = torch.empty(w.rows * w.cols, dtype=torch.float32, device=DEV)
    T.taco_decompress_reordered(c, buf, w.rows, w.cols, d32, order, 0)
    torch.cuda.synchronize()
    got_f = d32.view(w.rows, w.cols)[it].cpu().numpy().reshape(-1)
    assert same_f32_bits(got_f, oracle.decode_reordered(ref, o).reshape(-1)).all(), "decode f32"


@pytest.mark.parametrize("name", ["equarx", "flashcomm"])
def test_full_size_staged_reorder_sampled_rows(name):
    """The INT codecs' reordered compress and bf16 decode at the workload's full
    size (rows staged through LDS: two rows per unit at 5120 columns, one at
    8192), sampled row chunks against the oracle with the same order."""
    w = W.WORKLOADS[name]
    oc = cd.Codec(w.in_format, w.in_block, False)
    c = ccodec(oc)
    print(f"full-size staged reorder {name}: {w.rows}x{w.cols}", flush=True)
    order = torch.empty(w.cols // 8, dtype=torch.int32, device=DEV)
    stats = W.make_shard(w, 1, chunks=list(range(4)))
    T.taco_chunk_order(upload_bits(stats), stats.shape[0], w.cols, order)
    x = W.make_shard(w, 0)
    buf = T.empty_compressed(c, w.rows, w.cols)
    T.taco_compress_reordered(c, upload_bits(x), w.rows, w.cols, 1.0, buf, order)
    dec = torch.empty(w.rows * w.cols, dtype=torch.int16, device=DEV)
    T.taco_decompress_reordered(c, buf, w.rows, w.cols, dec, order, 1)
    torch.cuda.synchronize()
    o = order.cpu().numpy().astype(np.int64)
    assert (o == oracle.chunk_order(stats)).all()
    idx = W.chunk_rows(W.sample_chunks(w, 2, seed=11), w.rows)
    ref = oracle.compress_reordered(oc, x[idx], o)
    codes, sc, aux, _ = T.regions(buf, c, w.rows, w.cols)
    it = torch.from_numpy(idx).to(DEV)
    per_row = w.cols // (2 if oc.format == cd.INT4_ASYM else 1)
    assert (codes.view(w.rows, per_row)[it].cpu().numpy().reshape(-1) == ref.codes).all(), "codes"
    got_s = sc.view(w.rows, w.cols // oc.block)[it].cpu().numpy().reshape(-1)
    assert (got_s.view(np.uint32) == ref.scale.astype(np.float32).view(np.uint32)).all(), "scales"
    if ref.zero is not None:
        assert (aux.view(w.rows, w.cols // oc.block)[it].cpu().numpy().reshape(-1) == ref.zero).all(), "zero points"
    got_d = dec.view(w.rows, w.cols)[it].cpu().numpy().view(np.uint16).reshape(-1)
    assert (got_d == oracle.decode_reordered(ref, o, "bf16").reshape(-1)).all(), "decode"


@pytest.mark.parametrize("oc", [cd.Codec.fp8(128, True), cd.Codec.int8_sym()], ids=cid)
def test_reordered_graph_replays_match_eager(oc):
    """The reordered compress (FP8: with the delayed tensor scale, so the
    workspace protocol runs in the graph) and both decodes, captured once in a
    HIP graph and replayed on three inputs copied in eagerly between the
    replays, write exactly what the same calls write eagerly."""
    rows, cols = 300, 5120
    fp8 = oc.format in cd.FP8_FORMATS
    c = ccodec(oc)
    order = gpu_order(outlier_bits((rows, cols), seed=901))
    xs = [upload_bits(outlier_bits((rows, cols), seed=910 + i)) for i in range(3)]
    scale = T.TACO_SCALE_DELAYED if fp8 else 1.0

    def calls(x, ws, buf, d32, d16, stream=None):
        sh = None if stream is None else stream.cuda_stream
        T.taco_compress_reordered(c, x, rows, cols, scale, buf, order, workspace=ws, stream=sh)
        T.taco_decompress_reordered(c, buf, rows, cols, d32, order, 0, stream=sh)
        T.taco_decompress_reordered(c, buf, rows, cols, d16, order, 1, stream=sh)

    def alloc():
        return (new_workspace() if fp8 else None, T.empty_compressed(c, rows, cols),
                torch.empty(rows * cols, dtype=torch.float32, device=DEV),
                torch.empty(rows * cols, dtype=torch.int16, device=DEV))

    eager = []
    ws, buf, d32, d16 = alloc()
    for x in xs:
        calls(x, ws, buf, d32, d16)
        torch.cuda.synchronize()
        eager.append((buf.clone(), d32.clone(), d16.clone()))
    ws, buf, d32, d16 = alloc()
    x_in = torch.empty_like(xs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        calls(x_in, ws, buf, d32, d16, stream=st)
    for i, x in enumerate(xs):
        x_in.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eb, e32, e16 = eager[i]
        got, want = T.regions(buf, c, rows, cols), T.regions(eb, c, rows, cols)
        for k in range(3):   # codes, scales, zero points
            assert torch.equal(got[k], want[k]), f"replay {i}: region {k}"
        assert torch.equal(got[3][:1], want[3][:1]), f"replay {i}: tensor scale"
        assert torch.equal(d32.view(torch.int32), e32.view(torch.int32)), f"replay {i}: float32 decode"
        assert torch.equal(d16, e16), f"replay {i}: bf16 decode"

"""Memory safety at ragged ends: every entry point reads and writes only inside
the buffers it is given.

Each buffer sits in the middle of a larger allocation whose guard bytes before
and after it hold a fixed pattern; after the call the guards must be unchanged.
The shapes end in partial 1024-element wave tiles (the last one shorter than
half a tile) and partial FP8 chunks, where lanes and unrolled tiles reach past
the end and the kernels' clipped buffer accesses must drop the stores. The
overrun any such lane could make is a few KiB, well inside the 64 KiB guards.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as cd
import quantized_compression_tensor_amd as T
import workloads as W
from tests.gpu_util import DEV, ccodec

pytestmark = pytest.mark.gpu

GUARD = 1 << 16
PATTERN = 0xA5
CODECS = [cd.Codec.fp8(128, True), cd.Codec.fp8(64, False), cd.Codec.fp8e5(128, True),
          cd.Codec.int8_sym(), cd.Codec.int4_asym(), cd.Codec.int8_asym()]
SHAPES = [(3, 1152), (5, 1664), (1, 128), (9, 2944)]   # n = 3456, 8320, 128, 26496


class Arena:
    """nbytes of buffer between two guards of GUARD bytes, all set to PATTERN."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.t = torch.full((2 * GUARD + ((self.n + 255) & ~255),), PATTERN, dtype=torch.uint8, device=DEV)

    def buf(self, dtype=torch.uint8):
        return self.t[GUARD:GUARD + self.n].view(dtype)

    def fill(self, host_bytes):
        self.buf().copy_(torch.from_numpy(np.ascontiguousarray(host_bytes).view(np.uint8).reshape(-1)))
        return self

    def assert_guards(self, what):
        torch.cuda.synchronize()
        t = self.t.cpu().numpy()
        head, tail = t[:GUARD], t[GUARD + self.n:]
        bad_head, bad_tail = np.flatnonzero(head != PATTERN), np.flatnonzero(tail != PATTERN)
        assert bad_head.size == 0, f"{what}: wrote {bad_head.size} bytes before the buffer (first at -{GUARD - bad_head[-1]})"
        assert bad_tail.size == 0, f"{what}: wrote {bad_tail.size} bytes past the end (first at +{bad_tail[0]})"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("oc", CODECS, ids=lambda oc: f"f{oc.format}-b{oc.block}" + ("-h" if oc.hadamard else ""))
def test_writes_stay_inside_buffers(oc, shape):
    rows, cols = shape
    n = rows * cols
    c = ccodec(oc)
    fp8 = oc.format in cd.FP8_FORMATS
    nbytes = T.taco_compressed_bytes(c, rows, cols)
    body = "t3" if oc.format in (cd.INT4_ASYM, cd.INT8_ASYM) else "normal"
    scale = T.TACO_SCALE_AUTO if fp8 else 1.0
    print(f"bounds: codec {oc} shape {shape}", flush=True)

    # compress three shards (FP8 with the data-driven scale and a workspace)
    shards, xs = [], []
    for r in range(3):
        bits = W.random_bits(shape, seed=40 + r, sigma=0.05, body=body)
        x = Arena(2 * n).fill(bits)
        ws = Arena(T.TACO_WORKSPACE_BYTES).fill(np.zeros(T.TACO_WORKSPACE_BYTES, np.uint8)) if fp8 else None
        out = Arena(nbytes)
        T.taco_compress(c, x.buf(), rows, cols, scale, out.buf(), workspace=ws.buf() if ws else None)
        out.assert_guards(f"compress shard {r}")
        x.assert_guards(f"compress input {r}")
        if ws:
            ws.assert_guards(f"compress workspace {r}")
        shards.append(out)
        xs.append(x)

    # the debug hook's pre-rounding values
    pre = Arena(4 * n)
    dbg = Arena(nbytes)
    T.taco_compress_debug(c, xs[0].buf(), rows, cols, 0.01 if fp8 else 1.0, dbg.buf(), pre.buf(torch.float32))
    pre.assert_guards("compress_debug prequant")
    dbg.assert_guards("compress_debug output")

    # decode to float32 and bf16
    for dt, es in ((0, 4), (1, 2)):
        o = Arena(es * n)
        T.taco_decompress(c, shards[0].buf(), rows, cols, o.buf(), dt)
        o.assert_guards(f"decompress out_dtype={dt}")

    # decompress-reduce: FP32 sum and re-quantization
    cout = {cd.INT4_ASYM: cd.Codec.int8_asym()}.get(oc.format, oc)
    co = ccodec(cout)
    s = Arena(4 * n)
    rq = Arena(T.taco_compressed_bytes(co, rows, cols))
    T.taco_decompress_reduce(c, [a.buf() for a in shards], rows, cols, s.buf(torch.float32), co, rq.buf())
    s.assert_guards("reduce sum")
    rq.assert_guards("reduce requant")
    for a in shards:
        a.assert_guards("reduce input")

    # stand-alone requantization of the FP32 sum
    rq2 = Arena(T.taco_compressed_bytes(co, rows, cols))
    T.taco_requantize(co, s.buf(torch.float32), rows, cols, 0.01 if cout.format in cd.FP8_FORMATS else 1.0,
                      rq2.buf())
    rq2.assert_guards("requantize")

    # one ring hop (integer formats): incoming shard + local bf16
    if not fp8:
        hs = Arena(4 * n)
        hq = Arena(T.taco_compressed_bytes(co, rows, cols))
        T.taco_ring_hop(c, shards[1].buf(), xs[2].buf(), rows, cols, hs.buf(torch.float32), co, hq.buf())
        hs.assert_guards("ring hop sum")
        hq.assert_guards("ring hop requant")


@pytest.mark.parametrize("shape", [(128, 128, 128), (384, 256, 640), (512, 384, 256)], ids=str)
@pytest.mark.parametrize("oc", [cd.Codec.fp8(32, False), cd.Codec.int8_sym(), cd.Codec.int4_asym(),
                                cd.Codec.int8_asym()], ids=lambda oc: f"f{oc.format}-b{oc.block}")
@pytest.mark.parametrize("out_dtype", [0, 1], ids=["f32", "bf16"])
def test_decompress_gemm_stays_inside_buffers(oc, shape, out_dtype):
    """The fused decode-GEMM reads its compressed A and its weight, and writes its
    output, only inside the buffers given (both tile sizes: (512, 384, 256) runs
    the 256 x 256 tiles); the inputs are left unchanged."""
    M, K, N = shape
    c = ccodec(oc)
    print(f"bounds: decode-GEMM codec {oc} shape {shape} out {out_dtype}", flush=True)
    body = "t3" if oc.format in (cd.INT4_ASYM, cd.INT8_ASYM) else "normal"
    bits = W.random_bits((M, K), seed=91, sigma=0.05, body=body)
    x = Arena(2 * M * K).fill(bits)
    a = Arena(T.taco_compressed_bytes(c, M, K))
    T.taco_compress(c, x.buf(), M, K, 0.05, a.buf())
    a.assert_guards("compress of the activation")
    a_before = a.buf().clone()
    w = Arena(2 * N * K).fill(W.random_bits((N, K), seed=92, sigma=0.05))
    w_before = w.buf().clone()
    out = Arena(M * N * (2 if out_dtype else 4))
    T.taco_decompress_gemm(c, a.buf(), M, K, w.buf(), N, out.buf(), out_dtype)
    out.assert_guards("decode-GEMM output")
    a.assert_guards("decode-GEMM activation")
    w.assert_guards("decode-GEMM weight")
    assert torch.equal(a.buf(), a_before) and torch.equal(w.buf(), w_before), "an input was written"


@pytest.mark.parametrize("shape", [(1, 512), (3, 1536), (7, 9728), (2, 16896)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("oc", [cd.Codec.fp8(128, True), cd.Codec.fp8(128, False), cd.Codec.int8_sym(),
                                cd.Codec.int4_asym(), cd.Codec.int8_asym()],
                         ids=lambda oc: f"f{oc.format}-b{oc.block}" + ("-h" if oc.hadamard else ""))
def test_reordered_entry_points_stay_inside_buffers(oc, shape):
    """The group order, the reordered compress (FP8: with the data-driven scale,
    so its abs-max pre-pass runs too) and both reordered decodes, at widths that
    are staged through LDS in partial units (512, 1536, 9728) and gathered
    (16896)."""
    rows, cols = shape
    n = rows * cols
    c = ccodec(oc)
    fp8 = oc.format in cd.FP8_FORMATS
    print(f"bounds (reordered): codec {oc} shape {shape}", flush=True)
    stats = Arena(2 * n).fill(W.random_bits(shape, seed=70, sigma=0.05))
    order = Arena(4 * (cols // 8))
    T.taco_chunk_order(stats.buf(), rows, cols, order.buf(torch.int32))
    order.assert_guards("chunk_order")
    stats.assert_guards("chunk_order statistics")
    body = "t3" if oc.format in (cd.INT4_ASYM, cd.INT8_ASYM) else "normal"
    x = Arena(2 * n).fill(W.random_bits(shape, seed=71, sigma=0.05, body=body))
    ws = Arena(T.TACO_WORKSPACE_BYTES).fill(np.zeros(T.TACO_WORKSPACE_BYTES, np.uint8)) if fp8 else None
    out = Arena(T.taco_compressed_bytes(c, rows, cols))
    T.taco_compress_reordered(c, x.buf(), rows, cols, T.TACO_SCALE_AUTO if fp8 else 1.0, out.buf(),
                              order.buf(torch.int32), workspace=ws.buf() if ws else None)
    out.assert_guards("compress_reordered")
    x.assert_guards("compress_reordered input")
    if ws:
        ws.assert_guards("compress_reordered workspace")
    for dt, es in ((0, 4), (1, 2)):
        o = Arena(es * n)
        T.taco_decompress_reordered(c, out.buf(), rows, cols, o.buf(), order.buf(torch.int32), dt)
        o.assert_guards(f"decompress_reordered out_dtype={dt}")
    order.assert_guards("order after use")

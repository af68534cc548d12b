"""The launch cap (taco_set_launch_limit) changes grids, never results: every
entry point gives the same bytes under caps of 1, 3 and 64 workgroups as
uncapped, including the FP8 tensor-scale workspace history; and the codec
capped beside a concurrent bf16 GEMM at the qwen-tp shape (the overlap of
the TACO abstract) matches the oracle on sampled rows."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
import quantized_compression_tensor_amd as T
import workloads as W
from tests.gpu_util import DEV, ccodec, upload_bits, upload_f32, new_workspace, parse, assert_same, same_buffers

pytestmark = pytest.mark.gpu

CODECS = [cd.Codec.fp8(128, True), cd.Codec.fp8e5(128, True), cd.Codec.fp8(64, False), cd.Codec.int8_sym(),
          cd.Codec.int4_asym(), cd.Codec.int8_asym()]
LIMITS = [1, 3, 64]


def cid(oc):
    return f"f{oc.format}-b{oc.block}" + ("-h" if oc.hadamard else "")


def gather_codec(oc):
    return cd.Codec.int8_asym() if oc.format == cd.INT4_ASYM else oc


def run_all(oc, xs, rows, cols):
    """Every entry point once (FP8: AUTO then DELAYED on one workspace);
    returns the output tensors."""
    c, co = ccodec(oc), ccodec(gather_codec(oc))
    fp8 = oc.format in cd.FP8_FORMATS
    ws = new_workspace() if fp8 else None
    bufs = [T.empty_compressed(c, rows, cols) for _ in xs]
    for r, x in enumerate(xs):
        T.taco_compress(c, x, rows, cols, (T.TACO_SCALE_AUTO if r == 0 else T.TACO_SCALE_DELAYED) if fp8 else 1.0,
                        bufs[r], workspace=ws)
    pre = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    dbuf = T.empty_compressed(c, rows, cols)
    T.taco_compress_debug(c, xs[0], rows, cols, 0.25 if fp8 else 1.0, dbuf, pre)
    s = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    rq = T.empty_compressed(co, rows, cols)
    T.taco_decompress_reduce(c, bufs, rows, cols, s, co, rq)
    dec32 = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
    dec16 = torch.empty(rows * cols, dtype=torch.int16, device=DEV)
    T.taco_decompress(co, rq, rows, cols, dec32, 0)
    T.taco_decompress(c, bufs[1], rows, cols, dec16, 1)
    rq2 = T.empty_compressed(co, rows, cols)
    T.taco_requantize(co, s, rows, cols, 0.5 if fp8 else 1.0, rq2)
    out = {"bufs": bufs, "dbuf": dbuf, "pre": pre, "sum": s, "rq": rq, "dec32": dec32, "dec16": dec16, "rq2": rq2}
    if not fp8:
        hop_s = torch.empty(rows * cols, dtype=torch.float32, device=DEV)
        hop_q = T.empty_compressed(co, rows, cols)
        T.taco_ring_hop(co, rq, xs[1], rows, cols, hop_s, co, hop_q)
        out.update(hop_s=hop_s, hop_q=hop_q)
    return out


@pytest.mark.parametrize("oc", CODECS, ids=cid)
def test_every_entry_point_is_the_same_under_a_launch_cap(oc):
    rows, cols = 300, 4096          # 1200 wave tiles of 1024, a ragged last FP8 chunk
    xs = [upload_bits(W.random_bits((rows, cols), seed=6100 + 7 * r + oc.format, sigma=0.05, body="t3"))
          for r in range(3)]
    ref = run_all(oc, xs, rows, cols)
    torch.cuda.synchronize()
    go = gather_codec(oc)
    for lim in LIMITS:
        with T.launch_limit(lim):
            got = run_all(oc, xs, rows, cols)
        torch.cuda.synchronize()
        for r in range(3):
            assert same_buffers(got["bufs"][r], ref["bufs"][r], oc, rows, cols), f"cap {lim}: compress {r}"
        assert same_buffers(got["dbuf"], ref["dbuf"], oc, rows, cols), f"cap {lim}: debug compress"
        assert same_buffers(got["rq"], ref["rq"], go, rows, cols), f"cap {lim}: requantized sum"
        assert same_buffers(got["rq2"], ref["rq2"], go, rows, cols), f"cap {lim}: requantize"
        for k in ("pre", "sum", "dec32", "dec16", "hop_s"):
            if k in ref:
                assert torch.equal(got[k].view(torch.int32 if got[k].dtype == torch.float32 else torch.int16),
                                   ref[k].view(torch.int32 if ref[k].dtype == torch.float32 else torch.int16)), \
                    f"cap {lim}: {k}"
        if "hop_q" in ref:
            assert same_buffers(got["hop_q"], ref["hop_q"], go, rows, cols), f"cap {lim}: ring hop"
    # and the uncapped run itself against the oracle (compress of shard 0)
    want = oracle.compress(oc, W.random_bits((rows, cols), seed=6100 + oc.format, sigma=0.05, body="t3"))
    assert_same(parse(ref["bufs"][0], oc, rows, cols), want, "uncapped compress vs oracle")


def test_capped_codec_beside_the_gemm_at_full_size():
    """qwen-tp: 8 shards of 32768 x 5120, FP8 dual-scale with the transform and
    a given tensor scale per shard, compressed and reduced with an FP8 gather
    stage on one stream, capped at 128 workgroups, while the bf16 GEMM
    [32768 x 5120] x [5120 x 5120] runs on another; codes, exponents and the
    requantized sum of sampled rows against the oracle."""
    w = W.WORKLOADS["qwen-tp"]
    oc = cd.Codec.fp8(128, True)
    c = ccodec(oc)
    gs = [np.float32(2.0 ** -9 * (1 + r / 8)) for r in range(w.shards)]
    chunks = W.sample_chunks(w, 2, seed=11)
    idx = W.chunk_rows(chunks, w.rows)
    print(f"[overlap] qwen-tp full size, sample rows {len(idx)}", flush=True)
    xs = [upload_bits(W.make_shard(w, r)) for r in range(w.shards)]
    bufs = [T.empty_compressed(c, w.rows, w.cols) for _ in range(w.shards)]
    out = T.empty_compressed(c, w.rows, w.cols)
    a = torch.randn(w.rows, w.cols, dtype=torch.bfloat16, device=DEV)
    b = torch.randn(w.cols, w.cols, dtype=torch.bfloat16, device=DEV)
    gstream, cstream = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        for _ in range(3):
            y = torch.matmul(a, b)
    with torch.cuda.stream(cstream), T.launch_limit(128):
        for r in range(w.shards):
            T.taco_compress(c, xs[r], w.rows, w.cols, float(gs[r]), bufs[r])
        T.taco_decompress_reduce(c, bufs, w.rows, w.cols, None, c, out)
    torch.cuda.synchronize()
    it = torch.from_numpy(idx).to(DEV)
    refs = [oracle.compress(oc, W.make_shard(w, r, chunks=chunks), tensor_scale=gs[r]) for r in range(w.shards)]
    nb = w.cols // oc.block
    for r in range(w.shards):
        codes, k, _, g = T.regions(bufs[r], c, w.rows, w.cols)
        assert (codes.view(w.rows, w.cols)[it].cpu().numpy().reshape(-1) == refs[r].codes).all(), f"shard {r} codes"
        assert (k.view(w.rows, nb)[it].cpu().numpy().reshape(-1) == refs[r].scale).all(), f"shard {r} exponents"
        assert g[0].item() == gs[r]
    _, rq = oracle.decompress_reduce(refs, oc)
    codes, k, _, g = T.regions(out, c, w.rows, w.cols)
    assert (codes.view(w.rows, w.cols)[it].cpu().numpy().reshape(-1) == rq.codes).all(), "requantized codes"
    assert (k.view(w.rows, nb)[it].cpu().numpy().reshape(-1) == rq.scale).all(), "requantized exponents"
    assert np.float32(g[0].item()).view(np.uint32) == rq.tensor_scale.view(np.uint32)
    del y

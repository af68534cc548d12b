"""GPU parity of the ring hop (taco_ring_hop) against the oracle's ring_hop
([EQuARX] "What carries the argument": dequantize the received shard to FP32,
add the local contribution, quantize the partial sum for the next hop)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
import quantized_compression_tensor_amd as T
import workloads as W
from tests.gpu_util import DEV, ccodec, upload_bits, gpu_compress, parse, assert_same, same_f32_bits

pytestmark = pytest.mark.gpu

PAIRS = [(cd.Codec(cd.INT8_SYM, 64, False), cd.Codec(cd.INT8_SYM, 64, False)),
         (cd.Codec(cd.INT4_ASYM, 128, False), cd.Codec(cd.INT8_ASYM, 128, False)),
         (cd.Codec(cd.INT8_ASYM, 128, False), cd.Codec(cd.INT8_ASYM, 128, False))]
PIDS = ["i8s", "i4a-i8a", "i8a"]
SHAPES = [(1, 128), (3, 384), (37, 1024), (5, 2560), (64, 4096)]


def gpu_hop(cin, cout, incoming, local_dev, shape, want_sum=True, want_rq=True):
    rows, cols = shape
    s = torch.empty(rows * cols, dtype=torch.float32, device=DEV) if want_sum else None
    out = T.empty_compressed(ccodec(cout), rows, cols, DEV) if want_rq else None
    T.taco_ring_hop(ccodec(cin), incoming, local_dev, rows, cols, s, ccodec(cout) if want_rq else None, out)
    torch.cuda.synchronize()
    return s, out


@pytest.mark.parametrize("cin,cout", PAIRS, ids=PIDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_hop(cin, cout, shape):
    if shape[1] % cin.block:
        pytest.skip("cols not a multiple of block")
    body = "t3" if cin.format != cd.INT8_SYM else "normal"
    a = W.random_bits(shape, seed=shape[0] * 13 + cin.format, sigma=0.05, body=body)
    x = W.random_bits(shape, seed=shape[0] * 17 + cin.format + 1, sigma=0.05, body=body)
    inc_buf, _ = gpu_compress(cin, a, 1.0)
    inc_ref = oracle.compress(cin, a)
    acc, rq = oracle.ring_hop(inc_ref, x, cout)
    s, out = gpu_hop(cin, cout, inc_buf, upload_bits(x), shape)
    assert same_f32_bits(s.cpu().numpy(), acc).all(), "sum differs"
    assert_same(parse(out, cout, *shape), rq, "requantized")


@pytest.mark.parametrize("cin,cout", PAIRS, ids=PIDS)
def test_first_hop_and_single_outputs(cin, cout):
    shape = (37, 1024)
    x = W.random_bits(shape, seed=99 + cin.format, sigma=0.05)
    acc, rq = oracle.ring_hop(None, x, cout, in_codec=cin)
    s, out = gpu_hop(cin, cout, None, upload_bits(x), shape)
    assert same_f32_bits(s.cpu().numpy(), acc).all()
    assert_same(parse(out, cout, *shape), rq, "first hop")
    s2, _ = gpu_hop(cin, cout, None, upload_bits(x), shape, want_rq=False)
    assert same_f32_bits(s2.cpu().numpy(), acc).all()
    _, out2 = gpu_hop(cin, cout, None, upload_bits(x), shape, want_sum=False)
    assert_same(parse(out2, cout, *shape), rq, "requantize only")


def test_hop_edge_values():
    # zero blocks, a huge block and exact ties in the incoming and local shards
    cin = cout = cd.Codec(cd.INT8_SYM, 64, False)
    shape = (4, 256)
    vals = np.zeros(shape, np.float32)
    vals[1] = np.linspace(-3.0e38, 3.0e38, 256, dtype=np.float32)
    vals[2, :64] = 1.0
    vals[3] = (np.arange(256) % 7 - 3) * 0.5
    from oracle.formats import f32_to_bf16_bits
    a = f32_to_bf16_bits(vals)
    x = f32_to_bf16_bits(vals[::-1].copy())
    inc_buf, _ = gpu_compress(cin, a, 1.0)
    acc, rq = oracle.ring_hop(oracle.compress(cin, a), x, cout)
    s, out = gpu_hop(cin, cout, inc_buf, upload_bits(x), shape)
    assert same_f32_bits(s.cpu().numpy(), acc).all()
    assert_same(parse(out, cout, *shape), rq, "edge values")


def test_full_loop_ring_matches_oracle_at_every_hop():
    # 8 ranks of N(0, 1) data; the chunk travels 7 hops, each re-quantized,
    # and the last hop's output is what the all-gather sends.
    N, shape = 8, (64, 1024)
    codec = cd.Codec(cd.INT8_SYM, 64, False)
    from oracle.formats import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(1234)
    xs = [f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)) for _ in range(N)]
    ref, buf = None, None
    for r in range(N):
        acc, ref = oracle.ring_hop(ref, xs[r], codec, in_codec=codec)
        _, buf = gpu_hop(codec, codec, buf, upload_bits(xs[r]), shape, want_sum=False)
        assert_same(parse(buf, codec, *shape), ref, f"hop {r}")
    exact = sum(bf16_bits_to_f32(x).astype(np.float64) for x in xs)
    mse = float(((oracle.dequantize(ref).reshape(shape) - exact) ** 2).mean())
    print(f"[ring] 8-rank full-loop INT8 block-64 MSE {mse:.3e} (EQuARX page: 0.0014)", flush=True)
    assert 0.00105 < mse < 0.00175


@pytest.mark.parametrize("codec", [cd.Codec(cd.INT8_SYM, 64, False), cd.Codec(cd.INT8_ASYM, 128, False)],
                         ids=["i8s", "i8a"])
@pytest.mark.parametrize("N", [2, 5, 8])
def test_semi_loop_ring_matches_oracle_at_every_step(codec, N):
    # the semi-loop: ranks 0 .. h-1 chain one way, ranks N-1 .. h the other
    # (taco_ring_hop at every link), and the two partial sums meet in a
    # two-source taco_decompress_reduce that quantizes for the all-gather
    shape = (64, 1024)
    from oracle.formats import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(4321 + N)
    xs = [f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)) for _ in range(N)]
    h = N // 2
    chains = [list(range(h)), list(range(N - 1, h - 1, -1))]
    ends = []
    for ci, chain in enumerate(chains):
        ref, buf = None, None
        for r in chain:
            _, ref = oracle.ring_hop(ref, xs[r], codec, in_codec=codec)
            _, buf = gpu_hop(codec, codec, buf, upload_bits(xs[r]), shape, want_sum=False)
            assert_same(parse(buf, codec, *shape), ref, f"chain {ci}, rank {r}")
        ends.append(buf)
    c = ccodec(codec)
    out = T.empty_compressed(c, *shape, DEV)
    T.taco_decompress_reduce(c, ends, *shape, None, c, out)
    torch.cuda.synchronize()
    want = oracle.semi_loop_ring(xs, codec)
    assert_same(parse(out, codec, *shape), want, "join")
    if N == 8 and codec.format == cd.INT8_SYM:
        exact = sum(bf16_bits_to_f32(x).astype(np.float64) for x in xs)
        mse = float(((oracle.dequantize(want).reshape(shape) - exact) ** 2).mean())
        print(f"[ring] 8-rank semi-loop INT8 block-64 MSE {mse:.3e} (EQuARX page: 0.001)", flush=True)
        assert 0.00075 < mse < 0.00125


def test_full_size_hop_sampled_rows():
    # the equarx shape (8192 x 5120): whole tensors through the GPU, the oracle on
    # sampled row chunks, bit for bit
    cin = cout = cd.Codec(cd.INT8_SYM, 64, False)
    w = W.WORKLOADS["equarx"]
    chunks = W.sample_chunks(w, 3, seed=5)
    idx = W.chunk_rows(chunks, w.rows)
    a = W.make_shard(w, 0)
    x = W.make_shard(w, 1)
    inc_buf, _ = gpu_compress(cin, a, 1.0)
    s, out = gpu_hop(cin, cout, inc_buf, upload_bits(x), (w.rows, w.cols))
    ref_in = oracle.compress(cin, W.make_shard(w, 0, chunks=chunks))
    acc, rq = oracle.ring_hop(ref_in, W.make_shard(w, 1, chunks=chunks), cout)
    it = torch.from_numpy(idx).to(DEV)
    assert same_f32_bits(s.view(w.rows, w.cols)[it].cpu().numpy(), acc).all()
    codes, sc, _, _ = T.regions(out, ccodec(cout), w.rows, w.cols)
    bpr = w.cols // cout.block
    assert (codes.view(w.rows, w.cols)[it].cpu().numpy().reshape(-1) == rq.codes).all()
    assert (sc.view(w.rows, bpr)[it].cpu().numpy().reshape(-1).view(np.uint32) == rq.scale.view(np.uint32)).all()

"""Parity of the decode fused into the consumer's GEMM (taco_decompress_gemm)
with the oracle's decode(A) @ W^T, through the C ABI.

Shapes with M and N multiples of 256 run the 256 x 256 tiles, the others
the 128 x 128 ones; (2304, 512, 768) has nine tile rows (a group of eight
and a group of one). Three kinds of check:
 * a permutation weight: every output is one decoded activation value times
   1.0, so the result is exact and is compared value for value with the
   oracle's bf16 decode (this pins the in-kernel decode, its bf16 rounding and
   every row / column index);
 * dense weights against the oracle's float64 product, within the float32
   accumulation bound (K / 4) * 2^-24 * sum |a| |w| (plus half a bf16 ulp
   for bf16 output);
 * the full consumer sizes of the INT8 gather stages on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
import quantized_compression_tensor_amd as T
import workloads as W
from tests.gpu_util import DEV, ccodec, upload_bits, upload_compressed

pytestmark = pytest.mark.gpu

CODECS = [cd.Codec.int8_sym(), cd.Codec.int8_asym(), cd.Codec.int4_asym(),
          cd.Codec.fp8(32, False), cd.Codec.fp8(64, False), cd.Codec.fp8(128, False),
          cd.Codec.fp8e5(128, False)]


def cid(c):
    return f"f{c.format}b{c.block}"


def _activation(oc, M, K, seed):
    """An oracle-compressed activation (t-distributed body for the asymmetric
    formats, normal otherwise) with two all-zero rows (zero-scale blocks)."""
    body = "t3" if oc.format in (cd.INT4_ASYM, cd.INT8_ASYM) else "normal"
    bits = W.random_bits((M, K), seed=seed, sigma=0.05, body=body)
    bits[1] = 0
    bits[M - 2] = 0
    ts = np.float32(0.05) if oc.format in cd.FP8_FORMATS else None
    return oracle.compress(oc, bits, tensor_scale=ts)


def _run(oc, ref, w_bits, N, out_dtype):
    M, K = ref.rows, ref.cols
    a = upload_compressed(ref)
    w = upload_bits(w_bits)
    out = torch.empty(M * N, dtype=torch.bfloat16 if out_dtype else torch.float32, device=DEV)
    T.taco_decompress_gemm(ccodec(oc), a, M, K, w, N, out, out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(M, N)


def _tolerance(ref, mag, K, out_dtype):
    tol = (K / 4) * 2.0 ** -24 * mag + 2.0 ** -126
    if out_dtype:
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    return tol


@pytest.mark.parametrize("M", [384, 512], ids=["tiles128", "tiles256"])
@pytest.mark.parametrize("out_dtype", [0, 1], ids=["f32", "bf16"])
@pytest.mark.parametrize("oc", CODECS, ids=cid)
def test_permutation_weight_is_exact(oc, out_dtype, M):
    K = 512
    ref = _activation(oc, M, K, seed=50 + oc.format + oc.block)
    perm = np.random.default_rng(7).permutation(K)
    w_bits = np.zeros((K, K), np.uint16)
    w_bits[np.arange(K), perm] = 0x3F80   # bf16 1.0: output n is input column perm[n]
    got = _run(oc, ref, w_bits, K, out_dtype)
    a = oracle.bf16_bits_to_f32(oracle.decode(ref, "bf16")).astype(np.float64)
    want = a[:, perm]
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ; first at {np.argwhere(bad)[:4].tolist()}"


@pytest.mark.parametrize("shape", [(256, 384, 256), (2304, 512, 768), (1152, 640, 640), (128, 128, 1280)], ids=str)
@pytest.mark.parametrize("out_dtype", [0, 1], ids=["f32", "bf16"])
@pytest.mark.parametrize("oc", CODECS, ids=cid)
def test_dense_weight_matches_oracle(oc, out_dtype, shape):
    M, K, N = shape
    ref = _activation(oc, M, K, seed=90 + oc.format + oc.block + M)
    w_bits = W.random_bits((N, K), seed=17 + N, sigma=0.05)
    got = _run(oc, ref, w_bits, N, out_dtype)
    want, mag = oracle.decode_gemm(ref, w_bits)
    err = np.abs(got - want)
    tol = _tolerance(want, mag, K, out_dtype)
    assert (err <= tol).all(), f"max excess {float((err - tol).max())}, max |ref| {float(np.abs(want).max())}"
    # the check is not vacuous: outputs are far from zero relative to the tolerance
    assert np.median(np.abs(want)) > 100 * np.median(tol)


def _handmade_int8(oc, M, K, seed):
    """Random INT8 codes with plausible scales (and zero points) for the
    full-size check: the oracle never compresses the whole tensor."""
    rng = np.random.default_rng(seed)
    nb = M * K // oc.block
    scale = (rng.random(nb, dtype=np.float32) * np.float32(0.02) + np.float32(1e-3)).astype(np.float32)
    if oc.format == cd.INT8_SYM:
        codes = rng.integers(-127, 128, M * K, dtype=np.int8).view(np.uint8)
        return cd.Compressed(oc, M, K, codes, scale)
    codes = rng.integers(0, 256, M * K, dtype=np.uint8)
    zero = rng.integers(0, 256, nb, dtype=np.uint8)
    return cd.Compressed(oc, M, K, codes, scale, zero)


def _rows_of(c: cd.Compressed, rows):
    per = c.cols // c.codec.block
    codes = c.codes.reshape(c.rows, c.cols)[rows].reshape(-1)
    scale = c.scale.reshape(c.rows, per)[rows].reshape(-1)
    zero = None if c.zero is None else c.zero.reshape(c.rows, per)[rows].reshape(-1)
    return cd.Compressed(c.codec, len(rows), c.cols, codes, scale, zero, c.tensor_scale)


@pytest.mark.parametrize("name,oc", [("equarx", cd.Codec.int8_sym()), ("flashcomm", cd.Codec.int8_asym())])
def test_full_size_sampled_rows(name, oc):
    """The consumer of each workload's gather stage at its full size
    ([rows, cols] activation, [cols, cols] weight), bf16 output as the bench
    runs it; 34 rows (first, last and 32 seeded ones) against the oracle."""
    w = W.WORKLOADS[name]
    M, K, N = w.rows, w.cols, w.cols
    print(f"full-size decode-GEMM {name}: M={M} K={K} N={N}", flush=True)
    c = _handmade_int8(oc, M, K, seed=w.seed)
    w_bits = W.random_bits((N, K), seed=w.seed + 1, sigma=0.02)
    got = _run(oc, c, w_bits, N, 1)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(w.seed).choice(M, 32, replace=False)]))
    want, mag = oracle.decode_gemm(_rows_of(c, rows), w_bits)
    err = np.abs(got[rows] - want)
    tol = _tolerance(want, mag, K, 1)
    assert (err <= tol).all(), f"max excess {float((err - tol).max())}"


def test_graph_replays_match_eager():
    """The fused decode-GEMM captured once in a HIP graph and replayed on three
    different activations (copied in eagerly between the replays) writes exactly
    what the eager calls write."""
    oc, M, K, N = cd.Codec.int8_asym(), 512, 512, 256
    c = ccodec(oc)
    acts = [upload_compressed(_activation(oc, M, K, seed=300 + s)) for s in range(3)]
    w = upload_bits(W.random_bits((N, K), seed=301, sigma=0.05))
    eager = []
    for a in acts:
        out = torch.empty(M * N, dtype=torch.bfloat16, device=DEV)
        T.taco_decompress_gemm(c, a, M, K, w, N, out, 1)
        torch.cuda.synchronize()
        eager.append(out)
    a_dev = torch.empty_like(acts[0])
    a_dev.copy_(acts[0])
    out = torch.zeros(M * N, dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        T.taco_decompress_gemm(c, a_dev, M, K, w, N, out, 1, stream=st.cuda_stream)
    for s in (1, 0, 2):
        a_dev.copy_(acts[s])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[s]), f"replay on activation {s}"

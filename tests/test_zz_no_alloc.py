"""taco_compress_noalloc, the compress that allocates nothing (its FP8
tensor-scale workspace is the library's per-GPU scratch array), against
taco_compress with a caller-owned workspace: two calls in a row on the same
scratch, the second with a smaller input, must give the same bytes. The
oracle checks the first call's codes as well."""

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as cd
import quantized_compression_tensor_amd as T
import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CODECS = [cd.Codec.fp8(128, True), cd.Codec.fp8e5(128, True), cd.Codec.fp8(64, False), cd.Codec.int8_sym(),
          cd.Codec.int4_asym()]


def cid(oc):
    return f"f{oc.format}-b{oc.block}" + ("-h" if oc.hadamard else "")


@pytest.mark.parametrize("oc", CODECS, ids=cid)
def test_noalloc_matches_workspace_compress(oc):
    big, small = (300, 4096), (37, 1024)
    a = W.random_bits(big, seed=7100 + oc.format, sigma=0.02)
    b = W.random_bits(small, seed=7200 + oc.format, sigma=0.5)
    c = U.ccodec(oc)
    fp8 = oc.format in cd.FP8_FORMATS
    first = T.TACO_SCALE_AUTO if fp8 else 1.0
    second = T.TACO_SCALE_DELAYED if fp8 else 1.0
    xa, xb = U.upload_bits(a), U.upload_bits(b)
    ws = U.new_workspace()
    ref_a, ref_b = T.empty_compressed(c, *big), T.empty_compressed(c, *small)
    got_a, got_b = T.empty_compressed(c, *big), T.empty_compressed(c, *small)
    # AUTO first (its pre-pass records this tensor's abs-max whatever the
    # scratch held before), then DELAYED on the smaller tensor: the second call
    # takes its tensor scale from the first call's record in both paths
    T.taco_compress(c, xa, *big, first, ref_a, workspace=ws)
    T.taco_compress(c, xb, *small, second, ref_b, workspace=ws)
    T.taco_compress_noalloc(c, xa, *big, first, got_a)
    T.taco_compress_noalloc(c, xb, *small, second, got_b)
    torch.cuda.synchronize()
    assert U.same_buffers(got_a, ref_a, oc, *big), "first call differs from taco_compress"
    assert U.same_buffers(got_b, ref_b, oc, *small), "second (smaller) call differs from taco_compress"
    U.assert_same(U.parse(got_a, oc, *big), oracle.compress(oc, a), "first call vs oracle")
    if fp8:
        g_prev = cd.auto_tensor_scale(cd.transform(oc, a), oc.format)
        U.assert_same(U.parse(got_b, oc, *small), oracle.compress(oc, b, tensor_scale=g_prev),
                      "second call vs oracle with the first tensor's scale")
    else:
        U.assert_same(U.parse(got_b, oc, *small), oracle.compress(oc, b), "second call vs oracle")


def test_noalloc_given_scale_and_empty():
    oc = cd.Codec.fp8(128, True)
    c = U.ccodec(oc)
    x = W.random_bits((64, 2048), seed=7300, sigma=0.02)
    got = T.empty_compressed(c, 64, 2048)
    T.taco_compress_noalloc(c, U.upload_bits(x), 64, 2048, 0.0078125, got)
    T.taco_compress_noalloc(c, U.upload_bits(x), 0, 2048, T.TACO_SCALE_DELAYED, got)   # empty: nothing enqueued
    torch.cuda.synchronize()
    U.assert_same(U.parse(got, oc, 64, 2048), oracle.compress(oc, x, tensor_scale=np.float32(0.0078125)),
                  "given tensor scale")

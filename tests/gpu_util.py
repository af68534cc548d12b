"""Helpers for the GPU parity tests: run the C ABI through the binding and turn
its output buffers into the oracle's representation for comparison."""

import numpy as np
import torch

import oracle
from oracle import codecs as cd
import quantized_compression_tensor_amd as T

DEV = "cuda"


def ccodec(oc: cd.Codec):
    return T.codec(oc.format, oc.block, 1 if oc.hadamard else 0)


def upload_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def upload_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def new_workspace():
    return torch.zeros(T.TACO_WORKSPACE_BYTES // 4, dtype=torch.int32, device=DEV)


def gpu_compress(oc, bits, scale=1.0, ws=None, debug=False, xdev=None):
    """Compress with the GPU; scale is the tensor_scale argument (FP8)."""
    rows, cols = bits.shape
    c = ccodec(oc)
    x = upload_bits(bits) if xdev is None else xdev
    buf = T.empty_compressed(c, rows, cols)
    pre = None
    if debug:
        pre = torch.empty(max(1, rows * cols), dtype=torch.float32, device=DEV)
        T.taco_compress_debug(c, x, rows, cols, scale, buf, pre, workspace=ws)
    else:
        T.taco_compress(c, x, rows, cols, scale, buf, workspace=ws)
    torch.cuda.synchronize()
    return buf, pre


def parse(buf, oc, rows, cols):
    """GPU buffer -> dict(codes, scale, zero, g) as numpy arrays."""
    codes, sc, aux, ten = T.regions(buf, ccodec(oc), rows, cols)
    out = dict(codes=codes.cpu().numpy(), scale=sc.cpu().numpy(),
               zero=aux.cpu().numpy() if aux.numel() else None,
               g=np.float32(ten.cpu().numpy()[0]) if ten.numel() else None)
    return out


def assert_same(gpu, ref: oracle.Compressed, where=""):
    """Codes and every scale bit-exact. NaN codes compare as a class."""
    gc, rc = gpu["codes"], ref.codes
    assert gc.shape == rc.shape, where
    bad = gc != rc
    if ref.codec.format == cd.FP8_DUAL:
        bad &= ~(((gc & 0x7F) == 0x7F) & ((rc & 0x7F) == 0x7F))
    if ref.codec.format == cd.FP8E5_DUAL:
        def e5_nan(c):
            return ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0)
        bad &= ~(e5_nan(gc) & e5_nan(rc))
    nbad = int(bad.sum())
    assert nbad == 0, f"{where}: {nbad} of {gc.size} codes differ; first at {np.flatnonzero(bad)[:8]}"
    if ref.codec.format in cd.FP8_FORMATS:
        assert (gpu["scale"].astype(np.int8) == ref.scale.astype(np.int8)).all(), f"{where}: block exponents differ"
        assert gpu["g"].view(np.uint32) == np.float32(ref.tensor_scale).view(np.uint32), \
            f"{where}: g {gpu['g']!r} vs {ref.tensor_scale!r}"
    else:
        s_bad = gpu["scale"].view(np.uint32) != ref.scale.astype(np.float32).view(np.uint32)
        assert not s_bad.any(), f"{where}: {int(s_bad.sum())} scales differ"
    if ref.zero is not None:
        assert (gpu["zero"] == ref.zero).all(), f"{where}: zero points differ"


def same_f32_bits(a, b):
    a = np.ascontiguousarray(a, np.float32).reshape(-1)
    b = np.ascontiguousarray(b, np.float32).reshape(-1)
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def same_buffers(b1, b2, oc, rows, cols):
    """Two compressed buffers hold the same codes, scales, zero points and g
    (the padding between 256-byte aligned regions is never written)."""
    p1, p2 = parse(b1, oc, rows, cols), parse(b2, oc, rows, cols)
    for k in ("codes", "scale", "zero"):
        if p1[k] is None:
            assert p2[k] is None
        elif not (p1[k].view(np.uint8) == p2[k].view(np.uint8)).all():
            return False
    g1, g2 = p1["g"], p2["g"]
    return (g1 is None and g2 is None) or (np.float32(g1).view(np.uint32) == np.float32(g2).view(np.uint32))


def upload_compressed(ref: oracle.Compressed):
    """A device buffer in the library's layout holding an oracle shard (codes,
    scales, zero points and, for FP8, the tensor scale g); bytes between the
    regions are zero."""
    c = ccodec(ref.codec)
    buf = T.empty_compressed(c, ref.rows, ref.cols)
    buf.zero_()
    codes, sc, aux, ten = T.regions(buf, c, ref.rows, ref.cols)
    codes.copy_(torch.from_numpy(np.ascontiguousarray(ref.codes, np.uint8)))
    if ref.codec.format in cd.FP8_FORMATS:
        sc.copy_(torch.from_numpy(np.ascontiguousarray(ref.scale, np.int8)))
        ten[0] = float(np.float32(ref.tensor_scale))
    else:
        sc.copy_(torch.from_numpy(np.ascontiguousarray(ref.scale, np.float32)))
    if ref.zero is not None:
        aux.copy_(torch.from_numpy(np.ascontiguousarray(ref.zero, np.uint8)))
    return buf

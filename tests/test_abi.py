"""The C ABI without a GPU: the library loads, exports every entry point its
header declares, computes layouts, names status codes, and rejects bad
arguments before anything is enqueued (none of these calls touches HIP)."""

import ctypes
import os
import re

import pytest

import quantized_compression_tensor_amd as T
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "taco.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(taco_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(T.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(T.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in [(0, "TACO_OK"), (-1, "TACO_ERR_INVALID_ARG"), (-2, "TACO_ERR_SHAPE"),
                       (-3, "TACO_ERR_FORMAT"), (-4, "TACO_ERR_ALIGN"), (-5, "TACO_ERR_WORKSPACE"),
                       (-6, "TACO_ERR_HIP"), (-99, "TACO_ERR_UNKNOWN")]:
        assert T.taco_status_string(code) == name


FP8 = T.codec(T.TACO_FMT_FP8_DUAL, 128, 1)
I8S = T.codec(T.TACO_FMT_INT8_SYM, 64)
I4A = T.codec(T.TACO_FMT_INT4_ASYM, 128)
I8A = T.codec(T.TACO_FMT_INT8_ASYM, 128)
E5 = T.codec(T.TACO_FMT_FP8E5_DUAL, 128, 1)


def test_layouts_by_hand():
    L = T.taco_layout(FP8, 4096, 4096).as_dict()
    n = 4096 * 4096
    assert L == dict(codes_off=0, codes_bytes=n, scale_off=n, scale_bytes=n // 128,
                     aux_off=n + n // 128, aux_bytes=0, tensor_off=n + n // 128, tensor_bytes=16,
                     total_bytes=n + n // 128 + 256)
    L = T.taco_layout(I4A, 3, 384).as_dict()          # n = 1152: 576 code bytes, 9 groups
    assert L["codes_bytes"] == 576 and L["scale_off"] == 768 and L["scale_bytes"] == 36
    assert L["aux_off"] == 1024 and L["aux_bytes"] == 9 and L["tensor_off"] == 1280
    assert L["tensor_bytes"] == 0 and L["total_bytes"] == 1280
    L = T.taco_layout(I8S, 1, 64).as_dict()
    assert L["codes_bytes"] == 64 and L["scale_off"] == 256 and L["scale_bytes"] == 4
    assert L["total_bytes"] == 512
    assert T.taco_compressed_bytes(I8A, 0, 128) == 0
    assert T.taco_workspace_bytes(FP8, 1, 128) == T.TACO_WORKSPACE_BYTES
    assert T.taco_workspace_bytes(E5, 1, 128) == T.TACO_WORKSPACE_BYTES
    assert T.taco_workspace_bytes(I8S, 1, 64) == 0
    assert T.taco_layout(E5, 4096, 4096).as_dict() == T.taco_layout(FP8, 4096, 4096).as_dict()


@pytest.mark.parametrize("c,cols,err", [
    (T.codec(T.TACO_FMT_FP8_DUAL, 128, 1), 100, T.TACO_ERR_SHAPE),
    (T.codec(T.TACO_FMT_FP8_DUAL, 96, 1), 96, T.TACO_ERR_SHAPE),
    (T.codec(T.TACO_FMT_FP8_DUAL, 128, 2), 128, T.TACO_ERR_FORMAT),
    (T.codec(T.TACO_FMT_FP8E5_DUAL, 96, 0), 96, T.TACO_ERR_SHAPE),
    (T.codec(T.TACO_FMT_FP8E5_DUAL, 128, 3), 128, T.TACO_ERR_FORMAT),
    (T.codec(T.TACO_FMT_INT8_SYM, 128), 128, T.TACO_ERR_SHAPE),
    (T.codec(T.TACO_FMT_INT8_SYM, 64, 1), 64, T.TACO_ERR_FORMAT),
    (T.codec(T.TACO_FMT_INT4_ASYM, 64), 128, T.TACO_ERR_SHAPE),
    (T.codec(9, 128), 128, T.TACO_ERR_FORMAT),
    (T.codec(T.TACO_FMT_FP8_DUAL, 128, 1), 0, T.TACO_ERR_INVALID_ARG),
])
def test_layout_rejects(c, cols, err):
    with pytest.raises(T.TacoError) as e:
        T.taco_layout(c, 4, cols)
    assert e.value.status == err
    assert T.lib().taco_compressed_bytes(c, 4, cols) == err


def _st(fn, *a):
    try:
        fn(*a)
    except T.TacoError as e:
        return e.status
    return 0


A = 4096          # a fake, 16-byte aligned "device" address: never dereferenced,
B_ = 1 << 20      # every call below fails validation before any launch


def test_compress_validation():
    comp = T.taco_compress
    assert _st(comp, FP8, None, 2, 128, 1.0, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 1.0, None) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A + 2, 2, 128, 1.0, B_) == T.TACO_ERR_ALIGN
    assert _st(comp, FP8, A, 2, 128, 1.0, B_ + 8) == T.TACO_ERR_ALIGN
    assert _st(comp, FP8, A, -1, 128, 1.0, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 1 << 22, 1 << 14, 1.0, B_) == T.TACO_ERR_INVALID_ARG   # 2^36 elements: too large
    assert _st(comp, FP8, A, 2, 100, 1.0, B_) == T.TACO_ERR_SHAPE
    assert _st(comp, FP8, A, 2, 128, 0.0, B_) == T.TACO_ERR_WORKSPACE          # auto needs a workspace
    assert _st(comp, FP8, A, 2, 128, -1.0, B_) == T.TACO_ERR_WORKSPACE         # delayed needs one too
    assert _st(comp, FP8, A, 2, 128, 0.0, B_, 3 * B_, 16) == T.TACO_ERR_WORKSPACE  # too small
    assert _st(comp, FP8, A, 2, 128, float("nan"), B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 2.0 ** 61, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 2.0 ** -61, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 1.0, A) == T.TACO_ERR_INVALID_ARG         # output overlaps input
    assert _st(comp, FP8, A, 0, 128, 1.0, B_) == 0                             # empty: nothing to do
    assert _st(comp, I8S, A, 2, 96, 1.0, B_) == T.TACO_ERR_SHAPE
    assert _st(T.taco_compress_debug, FP8, A, 2, 128, 1.0, B_, None) == T.TACO_ERR_INVALID_ARG


def test_noalloc_compress_validation():
    """The allocation-free compress checks its arguments as taco_compress does,
    before it looks up (or clears) its scratch array; it takes no workspace."""
    comp = T.taco_compress_noalloc
    assert _st(comp, FP8, None, 2, 128, 0.0, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, -1.0, None) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A + 2, 2, 128, 0.0, B_) == T.TACO_ERR_ALIGN
    assert _st(comp, FP8, A, 2, 100, 0.0, B_) == T.TACO_ERR_SHAPE
    assert _st(comp, FP8, A, 1 << 22, 1 << 14, 0.0, B_) == T.TACO_ERR_INVALID_ARG   # 2^36 elements: too large
    assert _st(comp, FP8, A, 2, 128, float("inf"), B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 2.0 ** 61, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(comp, FP8, A, 2, 128, 0.0, A) == T.TACO_ERR_INVALID_ARG          # output overlaps input
    assert _st(comp, E5, A, 0, 128, -1.0, B_) == 0                             # empty: nothing to do
    assert _st(comp, I4A, A, 2, 96, 1.0, B_) == T.TACO_ERR_SHAPE


def test_reduce_validation():
    red = T.taco_decompress_reduce
    shards = [A, A + (1 << 16)]
    assert _st(red, I8S, [], 4, 64, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(red, I8S, [A] * 17, 4, 64, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(red, I8S, shards, 4, 64, None, None, None) == T.TACO_ERR_INVALID_ARG   # no output
    assert _st(red, I8S, [A, None], 4, 64, B_) == T.TACO_ERR_INVALID_ARG
    assert _st(red, I8S, [A, A + 4], 4, 64, B_) == T.TACO_ERR_ALIGN
    assert _st(red, I8S, shards, 4, 128, None, I8A, B_) == T.TACO_ERR_FORMAT
    assert _st(red, I8S, shards, 4, 64, None, I8A, B_) == T.TACO_ERR_SHAPE          # 64 cols: no 128 group
    assert _st(red, I4A, shards, 4, 128, None, I4A, B_) == T.TACO_ERR_FORMAT
    assert _st(red, FP8, shards, 4, 128, None, T.codec(T.TACO_FMT_FP8_DUAL, 64, 1), B_) == T.TACO_ERR_FORMAT
    assert _st(red, FP8, shards, 4, 128, None, T.codec(T.TACO_FMT_FP8_DUAL, 128, 0), B_) == T.TACO_ERR_FORMAT
    assert _st(red, FP8, shards, 4, 128, None, E5, B_) == T.TACO_ERR_FORMAT            # E4M3 -> E5M2 is no pair
    assert _st(red, E5, shards, 4, 128, None, FP8, B_) == T.TACO_ERR_FORMAT
    assert _st(red, I8S, shards, 4, 64, A) == T.TACO_ERR_INVALID_ARG               # sum overlaps a shard
    assert _st(red, I8S, shards, 0, 64, B_) == 0


def test_ring_hop_validation():
    hop = T.taco_ring_hop
    L = A + (1 << 16)
    assert _st(hop, I8S, A, None, 4, 64, B_) == T.TACO_ERR_INVALID_ARG             # no local shard
    assert _st(hop, I8S, A, L, 4, 64, None, None, None) == T.TACO_ERR_INVALID_ARG  # no output
    assert _st(hop, FP8, A, L, 4, 128, B_) == T.TACO_ERR_FORMAT                    # FP8 is not a ring codec
    assert _st(hop, E5, A, L, 4, 128, B_) == T.TACO_ERR_FORMAT
    assert _st(hop, I8S, A, L, 4, 64, None, FP8, B_) == T.TACO_ERR_SHAPE           # 64 cols: no 128 block
    assert _st(hop, I8S, A, L, 4, 128, None, FP8, B_) == T.TACO_ERR_FORMAT
    assert _st(hop, I4A, A, L, 4, 128, None, I4A, B_) == T.TACO_ERR_FORMAT         # the gather stage is INT8
    assert _st(hop, I8S, A + 4, L, 4, 64, B_) == T.TACO_ERR_ALIGN
    assert _st(hop, I8S, A, L + 2, 4, 64, B_) == T.TACO_ERR_ALIGN
    assert _st(hop, I8S, A, L, 4, 64, A) == T.TACO_ERR_INVALID_ARG                 # sum overlaps the incoming
    assert _st(hop, I8S, A, L, 4, 64, L + 64) == T.TACO_ERR_INVALID_ARG            # sum overlaps the local
    assert _st(hop, I8S, None, L, 0, 64, B_) == 0                                  # empty: nothing to do
    assert _st(hop, I8S, None, L, 4, 96, B_) == T.TACO_ERR_SHAPE


def test_other_entry_points_validation():
    assert _st(T.taco_decompress, I8S, A, 4, 64, B_, 2) == T.TACO_ERR_INVALID_ARG
    assert _st(T.taco_decompress, I8S, A, 4, 64, None, 0) == T.TACO_ERR_INVALID_ARG
    assert _st(T.taco_decompress, I8S, A + 1, 4, 64, B_, 0) == T.TACO_ERR_ALIGN
    assert _st(T.taco_requantize, I8S, A, 4, 96, 1.0, B_) == T.TACO_ERR_SHAPE
    assert _st(T.taco_requantize, FP8, A, 4, 128, 0.0, B_) == T.TACO_ERR_WORKSPACE
    assert _st(T.taco_e4m3_encode, A, None, 16) == T.TACO_ERR_INVALID_ARG
    assert _st(T.taco_e4m3_encode, A, B_, -1) == T.TACO_ERR_INVALID_ARG
    assert _st(T.taco_e4m3_encode, A, A + 16, 64) == T.TACO_ERR_INVALID_ARG       # overlap
    assert _st(T.taco_e4m3_encode, A, B_, 0) == 0
    assert _st(T.taco_e5m2_encode, A, None, 16) == T.TACO_ERR_INVALID_ARG
    assert _st(T.taco_e5m2_encode, A, A + 16, 64) == T.TACO_ERR_INVALID_ARG       # overlap
    assert _st(T.taco_e5m2_encode, A, B_, 0) == 0


def test_reordered_calls_validation():
    comp, dec, order_fn = T.taco_compress_reordered, T.taco_decompress_reordered, T.taco_chunk_order
    O = A + (1 << 20)
    assert _st(comp, FP8, A, 2, 1024, 1.0, B_, None) == T.TACO_ERR_INVALID_ARG          # no order
    assert _st(comp, FP8, A, 2, 384, 1.0, B_, O) == T.TACO_ERR_SHAPE                    # cols not a multiple of 512
    assert _st(comp, I8S, A, 1, 262144, 1.0, B_, O) == T.TACO_ERR_SHAPE                 # cols above 131072
    assert _st(comp, T.codec(T.TACO_FMT_FP8_DUAL, 64, 1), A, 2, 1024, 1.0, B_, O) == T.TACO_ERR_SHAPE   # block 64
    assert _st(comp, FP8, A, 2, 1024, 1.0, B_, O + 4) == T.TACO_ERR_ALIGN
    assert _st(comp, FP8, A, 2, 1024, 1.0, B_, B_ + 256) == T.TACO_ERR_INVALID_ARG      # order overlaps the output
    assert _st(comp, FP8, A, 2, 1024, 0.0, B_, O) == T.TACO_ERR_WORKSPACE               # auto needs a workspace
    assert _st(comp, I4A, A, 0, 1024, 1.0, B_, O) == 0                                  # empty: nothing to do
    assert _st(dec, I8S, A, 2, 1024, B_, None, 0) == T.TACO_ERR_INVALID_ARG
    assert _st(dec, I8S, A, 2, 1000, B_, O, 0) == T.TACO_ERR_SHAPE
    assert _st(dec, I8S, A, 2, 1024, B_, O, 2) == T.TACO_ERR_INVALID_ARG
    assert _st(dec, I8S, A, 2, 1024, B_, B_ + 64, 1) == T.TACO_ERR_INVALID_ARG          # order overlaps the output
    assert _st(order_fn, A, 2, 1000, O) == T.TACO_ERR_SHAPE
    assert _st(order_fn, A, 2, 1024, None) == T.TACO_ERR_INVALID_ARG
    assert _st(order_fn, A, -1, 1024, O) == T.TACO_ERR_INVALID_ARG
    assert _st(order_fn, A, 2, 1024, O + 8) == T.TACO_ERR_ALIGN
    assert _st(order_fn, A, 2, 1024, A + 16) == T.TACO_ERR_INVALID_ARG                  # order overlaps the statistics


def test_decompress_gemm_validation():
    g = T.taco_decompress_gemm
    Wt, O = A + (1 << 24), A + (1 << 26)
    I8A = T.codec(T.TACO_FMT_INT8_ASYM, 128)
    assert _st(g, FP8, A, 128, 128, Wt, 128, O) == T.TACO_ERR_FORMAT                     # Hadamard codec
    assert _st(g, T.codec(T.TACO_FMT_FP8_DUAL, 16, 0), A, 128, 128, Wt, 128, O) == T.TACO_ERR_SHAPE
    assert _st(g, I8A, A, 100, 128, Wt, 128, O) == T.TACO_ERR_SHAPE                      # M
    assert _st(g, I8A, A, 128, 192, Wt, 128, O) == T.TACO_ERR_SHAPE                      # K
    assert _st(g, I8A, A, 128, 128, Wt, 64, O) == T.TACO_ERR_SHAPE                       # N
    assert _st(g, I8A, A, 128, (1 << 20) + 128, Wt, 128, O) == T.TACO_ERR_SHAPE          # K above 2^20
    assert _st(g, I8A, A, 128, 128, Wt, 0, O) == T.TACO_ERR_INVALID_ARG
    assert _st(g, I8A, A, -128, 128, Wt, 128, O) == T.TACO_ERR_INVALID_ARG
    assert _st(g, I8A, A, 1 << 20, 1 << 16, Wt, 128, O) == T.TACO_ERR_INVALID_ARG        # 2^36 activation elements
    assert _st(g, I8A, A, 1 << 18, 128, Wt, 1 << 18, O) == T.TACO_ERR_INVALID_ARG        # 2^36 outputs
    assert _st(g, I8A, A, 128, 128, Wt, 128, O, 2) == T.TACO_ERR_INVALID_ARG             # out_dtype
    assert _st(g, I8A, None, 128, 128, Wt, 128, O) == T.TACO_ERR_INVALID_ARG
    assert _st(g, I8A, A, 128, 128, None, 128, O) == T.TACO_ERR_INVALID_ARG
    assert _st(g, I8A, A, 128, 128, Wt, 128, None) == T.TACO_ERR_INVALID_ARG
    assert _st(g, I8A, A + 8, 128, 128, Wt, 128, O) == T.TACO_ERR_ALIGN
    assert _st(g, I8A, A, 128, 128, Wt + 8, 128, O) == T.TACO_ERR_ALIGN
    assert _st(g, I8A, A, 128, 128, Wt, 128, O + 8) == T.TACO_ERR_ALIGN
    assert _st(g, I8A, A, 128, 128, Wt, 128, A + 1024) == T.TACO_ERR_INVALID_ARG         # out overlaps A
    assert _st(g, I8A, A, 128, 128, Wt, 128, Wt + 1024) == T.TACO_ERR_INVALID_ARG        # out overlaps W
    assert _st(g, I8A, None, 0, 128, None, 128, None) == 0                               # M = 0: nothing to do


def test_launch_limit_is_per_thread_and_restorable():
    import threading
    assert T.taco_set_launch_limit(0) == 0
    assert _st(T.taco_set_launch_limit, -1) == T.TACO_ERR_INVALID_ARG
    assert T.taco_set_launch_limit(7) == 0
    seen = []
    th = threading.Thread(target=lambda: seen.append(T.taco_set_launch_limit(3)))
    th.start()
    th.join()
    assert seen == [0]                       # another thread starts without a cap
    with T.launch_limit(64):
        assert T.taco_set_launch_limit(64) == 64
    assert T.taco_set_launch_limit(0) == 7   # the context manager restored 7


def test_one_hip_runtime_in_the_process():
    """The binding must leave exactly one HIP runtime mapped (torch's), whatever
    was imported first: a second runtime cannot use torch's streams or memory."""
    import subprocess
    import sys
    code = ("import quantized_compression_tensor_amd, torch\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len(set(l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l)))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.stdout.strip() == "1", out.stdout + out.stderr

"""Python binding of the C ABI declared in include/taco.h.

Argument marshalling only: every function below forwards to the function of
the same name in libtaco.so (hand-written gfx950 HIP kernels). Tensors may be
passed as torch tensors (their data_ptr is used) or as raw integer addresses;
the stream defaults to torch's current HIP stream. A nonzero status raises
TacoError. There is no fallback path: if the library cannot be built or
loaded, importing this package fails.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtaco.so")

TACO_OK = 0
TACO_ERR_INVALID_ARG = -1
TACO_ERR_SHAPE = -2
TACO_ERR_FORMAT = -3
TACO_ERR_ALIGN = -4
TACO_ERR_WORKSPACE = -5
TACO_ERR_HIP = -6

TACO_FMT_FP8_DUAL = 1
TACO_FMT_INT8_SYM = 2
TACO_FMT_INT4_ASYM = 3
TACO_FMT_INT8_ASYM = 4
TACO_FMT_FP8E5_DUAL = 5
FP8_FORMATS = (TACO_FMT_FP8_DUAL, TACO_FMT_FP8E5_DUAL)

TACO_SCALE_AUTO = 0.0
TACO_SCALE_DELAYED = -1.0
TACO_MAX_SHARDS = 16
TACO_WORKSPACE_BYTES = 32768

# Entry points declared in include/taco.h (checked by the ABI tests).
EXPORTS = (
    "taco_layout", "taco_compressed_bytes", "taco_workspace_bytes", "taco_compress",
    "taco_compress_debug", "taco_decompress_reduce", "taco_ring_hop", "taco_requantize", "taco_decompress",
    "taco_e4m3_encode", "taco_e5m2_encode", "taco_status_string", "taco_compress_noalloc",
    "taco_set_launch_limit", "taco_chunk_order", "taco_compress_reordered", "taco_decompress_reordered",
    "taco_decompress_gemm",
)


class taco_codec(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("block", ctypes.c_int32),
                ("hadamard", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def __repr__(self):
        return f"taco_codec(format={self.format}, block={self.block}, hadamard={self.hadamard})"


class taco_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "codes_off", "codes_bytes", "scale_off", "scale_bytes", "aux_off", "aux_bytes",
        "tensor_off", "tensor_bytes", "total_bytes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


def codec(fmt, block, hadamard=0):
    return taco_codec(int(fmt), int(block), int(hadamard), 0)


class TacoError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {taco_status_string(status)} ({status})")


def _load():
    # torch ships its own HIP runtime (same soname as /opt/rocm's). Loading it
    # first makes libtaco.so bind to that one runtime; loading libtaco.so first
    # would map a second runtime that does not know torch's streams or memory.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    C = taco_codec
    sig = {
        "taco_layout": (ctypes.c_int, [C, I64, I64, ctypes.POINTER(taco_layout_t)]),
        "taco_compressed_bytes": (I64, [C, I64, I64]),
        "taco_workspace_bytes": (SZ, [C, I64, I64]),
        "taco_compress": (ctypes.c_int, [C, P, I64, I64, F32, P, P, SZ, P]),
        "taco_compress_noalloc": (ctypes.c_int, [C, P, I64, I64, F32, P, P]),
        "taco_compress_debug": (ctypes.c_int, [C, P, I64, I64, F32, P, P, SZ, P, P]),
        "taco_decompress_reduce": (ctypes.c_int, [C, ctypes.POINTER(P), I32, I64, I64, P, C, P, P]),
        "taco_ring_hop": (ctypes.c_int, [C, P, P, I64, I64, P, C, P, P]),
        "taco_requantize": (ctypes.c_int, [C, P, I64, I64, F32, P, P, SZ, P]),
        "taco_decompress": (ctypes.c_int, [C, P, I64, I64, P, I32, P]),
        "taco_e4m3_encode": (ctypes.c_int, [P, P, I64, P]),
        "taco_e5m2_encode": (ctypes.c_int, [P, P, I64, P]),
        "taco_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "taco_set_launch_limit": (ctypes.c_int, [I32, ctypes.POINTER(I32)]),
        "taco_chunk_order": (ctypes.c_int, [P, I64, I64, P, P]),
        "taco_compress_reordered": (ctypes.c_int, [C, P, I64, I64, F32, P, P, SZ, P, P]),
        "taco_decompress_reordered": (ctypes.c_int, [C, P, I64, I64, P, I32, P, P]),
        "taco_decompress_gemm": (ctypes.c_int, [C, P, I64, I64, P, I64, P, I32, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available() and torch.cuda.is_initialized():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(status, where):
    if status != TACO_OK:
        raise TacoError(status, where)
    return status


# ------------------------------------------------------------- host only --

def taco_status_string(status):
    return _lib.taco_status_string(int(status)).decode()


def taco_layout(c, rows, cols):
    L = taco_layout_t()
    _check(_lib.taco_layout(c, rows, cols, ctypes.byref(L)), "taco_layout")
    return L


def taco_compressed_bytes(c, rows, cols):
    n = _lib.taco_compressed_bytes(c, rows, cols)
    if n < 0:
        raise TacoError(int(n), "taco_compressed_bytes")
    return n


def taco_workspace_bytes(c, rows, cols):
    return _lib.taco_workspace_bytes(c, rows, cols)


def taco_set_launch_limit(max_workgroups):
    """Cap the workgroups of every later launch from this host thread (0 = no
    cap); returns the cap that was in force."""
    prev = ctypes.c_int32(0)
    _check(_lib.taco_set_launch_limit(int(max_workgroups), ctypes.byref(prev)), "taco_set_launch_limit")
    return prev.value


class launch_limit:
    """Context manager: ``with launch_limit(k): ...`` runs the block's calls on
    grids of at most k workgroups and restores the previous cap after."""

    def __init__(self, max_workgroups):
        self.k = max_workgroups

    def __enter__(self):
        self.prev = taco_set_launch_limit(self.k)
        return self

    def __exit__(self, *exc):
        taco_set_launch_limit(self.prev)
        return False


# ------------------------------------------------------------ device ops --

def taco_compress(c, x_bf16, rows, cols, tensor_scale, out, workspace=None, ws_bytes=None, stream=None):
    wsb = ws_bytes if ws_bytes is not None else (TACO_WORKSPACE_BYTES if workspace is not None else 0)
    return _check(_lib.taco_compress(c, _ptr(x_bf16), rows, cols, float(tensor_scale), _ptr(out),
                                     _ptr(workspace), wsb, _stream(stream)), "taco_compress")


def taco_compress_noalloc(c, x_bf16, rows, cols, tensor_scale, out, stream=None):
    return _check(_lib.taco_compress_noalloc(c, _ptr(x_bf16), rows, cols, float(tensor_scale), _ptr(out),
                                             _stream(stream)), "taco_compress_noalloc")


def taco_compress_debug(c, x_bf16, rows, cols, tensor_scale, out, prequant, workspace=None, ws_bytes=None,
                        stream=None):
    wsb = ws_bytes if ws_bytes is not None else (TACO_WORKSPACE_BYTES if workspace is not None else 0)
    return _check(_lib.taco_compress_debug(c, _ptr(x_bf16), rows, cols, float(tensor_scale), _ptr(out),
                                           _ptr(workspace), wsb, _ptr(prequant), _stream(stream)),
                  "taco_compress_debug")


def taco_decompress_reduce(c_in, shards, rows, cols, sum_fp32=None, c_out=None, requant_out=None, stream=None):
    arr = (ctypes.c_void_p * max(1, len(shards)))(*[_ptr(s) for s in shards])
    co = c_out if c_out is not None else taco_codec(0, 0, 0, 0)
    return _check(_lib.taco_decompress_reduce(c_in, arr, len(shards), rows, cols, _ptr(sum_fp32), co,
                                              _ptr(requant_out), _stream(stream)), "taco_decompress_reduce")


def taco_ring_hop(c_in, incoming, local_bf16, rows, cols, sum_fp32=None, c_out=None, requant_out=None,
                  stream=None):
    co = c_out if c_out is not None else taco_codec(0, 0, 0, 0)
    return _check(_lib.taco_ring_hop(c_in, _ptr(incoming), _ptr(local_bf16), rows, cols, _ptr(sum_fp32), co,
                                     _ptr(requant_out), _stream(stream)), "taco_ring_hop")


def taco_requantize(c_out, x_fp32, rows, cols, tensor_scale, out, workspace=None, ws_bytes=None, stream=None):
    wsb = ws_bytes if ws_bytes is not None else (TACO_WORKSPACE_BYTES if workspace is not None else 0)
    return _check(_lib.taco_requantize(c_out, _ptr(x_fp32), rows, cols, float(tensor_scale), _ptr(out),
                                       _ptr(workspace), wsb, _stream(stream)), "taco_requantize")


def taco_decompress(c, inp, rows, cols, out, out_dtype=0, stream=None):
    return _check(_lib.taco_decompress(c, _ptr(inp), rows, cols, _ptr(out), int(out_dtype), _stream(stream)),
                  "taco_decompress")


def taco_chunk_order(stats_bf16, rows, cols, order, stream=None):
    return _check(_lib.taco_chunk_order(_ptr(stats_bf16), rows, cols, _ptr(order), _stream(stream)),
                  "taco_chunk_order")


def taco_compress_reordered(c, x_bf16, rows, cols, tensor_scale, out, order, workspace=None, ws_bytes=None,
                            stream=None):
    wsb = ws_bytes if ws_bytes is not None else (TACO_WORKSPACE_BYTES if workspace is not None else 0)
    return _check(_lib.taco_compress_reordered(c, _ptr(x_bf16), rows, cols, float(tensor_scale), _ptr(out),
                                               _ptr(workspace), wsb, _ptr(order), _stream(stream)),
                  "taco_compress_reordered")


def taco_decompress_reordered(c, inp, rows, cols, out, order, out_dtype=0, stream=None):
    return _check(_lib.taco_decompress_reordered(c, _ptr(inp), rows, cols, _ptr(out), int(out_dtype), _ptr(order),
                                                 _stream(stream)), "taco_decompress_reordered")


def taco_decompress_gemm(c, a, M, K, w_bf16, N, out, out_dtype=0, stream=None):
    """out[M, N] = decode(a)[M, K] @ w_bf16[N, K]^T, the decode fused into the GEMM."""
    return _check(_lib.taco_decompress_gemm(c, _ptr(a), M, K, _ptr(w_bf16), N, _ptr(out), int(out_dtype),
                                            _stream(stream)), "taco_decompress_gemm")


def taco_e4m3_encode(x, codes, n, stream=None):
    return _check(_lib.taco_e4m3_encode(_ptr(x), _ptr(codes), n, _stream(stream)), "taco_e4m3_encode")


def taco_e5m2_encode(x, codes, n, stream=None):
    return _check(_lib.taco_e5m2_encode(_ptr(x), _ptr(codes), n, _stream(stream)), "taco_e5m2_encode")


# ------------------------------------------------- buffer plumbing (torch) --

def empty_compressed(c, rows, cols, device="cuda"):
    """A uint8 device tensor sized for one compressed [rows, cols] tensor."""
    import torch
    return torch.empty(max(1, taco_compressed_bytes(c, rows, cols)), dtype=torch.uint8, device=device)


def regions(buf, c, rows, cols):
    """Views of a compressed buffer's regions (codes, scale, aux, tensor), as laid
    out by taco_layout: codes uint8; scale int8 (FP8) or float32; aux uint8;
    tensor float32[4] (FP8) -- for tests and inspection."""
    import torch
    L = taco_layout(c, rows, cols)
    codes = buf[L.codes_off:L.codes_off + L.codes_bytes]
    sc = buf[L.scale_off:L.scale_off + L.scale_bytes]
    sc = sc.view(torch.int8) if c.format in FP8_FORMATS else sc.view(torch.float32)
    aux = buf[L.aux_off:L.aux_off + L.aux_bytes]
    ten = buf[L.tensor_off:L.tensor_off + L.tensor_bytes].view(torch.float32)
    return codes, sc, aux, ten


WS_TICKET_GROUPS = 64   # workspace ticket counters (kernel-side constants)
WS_BANK_LINES = 32      # workspace record lines per bank (three banks)
WS_LINE = 32            # uint32 words per 128-byte line
WS_SHARE_SHIFT = 24     # each call adds 2^24 to every ticket counter


def workspace_history(ws):
    """Read an FP8 tensor-scale workspace (a device tensor of
    TACO_WORKSPACE_BYTES) between calls: returns (calls made, abs-max recorded
    by the most recent call, that call's bank). Layout (uint32 words, 32 per
    line): line 0 unused; line 1 + g, words 0-1: ticket counter g (64, uint64);
    line 65 + 32 b + l, word 0: record line l of bank b (3 banks of 32).
    Inspection only."""
    import numpy as np
    w = ws.detach().cpu().numpy().view(np.uint32).reshape(-1)
    calls = int(w[WS_LINE:WS_LINE + 2].view(np.uint64)[0]) >> WS_SHARE_SHIFT
    if calls == 0:
        return 0, 0.0, None
    bank = (calls - 1) % 3
    amax = bank_lines(w)[bank].copy().view(np.float32).max()
    return calls, float(amax), bank


def bank_lines(words):
    """The record words of a workspace given as uint32 words: [3 banks, 32 lines]."""
    base = WS_LINE * (1 + WS_TICKET_GROUPS)
    return words[base: base + WS_LINE * 3 * WS_BANK_LINES].reshape(3, WS_BANK_LINES, WS_LINE)[:, :, 0]

// The C ABI: validation, buffer layout and kernel dispatch; all checks run
// before any work is enqueued. Apart from the allocation-free compress's
// scratch array (and the fill kernel that clears it once per device),
// everything here is host code.
#include <math.h>
#include <string.h>

#include <mutex>

#include "taco.h"
#include "taco_internal.h"

namespace {

using namespace taco;

// Largest tensor (rows * cols) a call accepts: 2^35 elements keeps every
// one-wave-per-tile grid under 2^32 threads.
constexpr int64_t kMaxElems = int64_t(1) << 35;

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_fp8_format(int32_t f) { return f == TACO_FMT_FP8_DUAL || f == TACO_FMT_FP8E5_DUAL; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int check_codec(const taco_codec& c) {
  if (c.reserved != 0) return TACO_ERR_INVALID_ARG;
  switch (c.format) {
    case TACO_FMT_FP8_DUAL:
    case TACO_FMT_FP8E5_DUAL:
      if (c.hadamard != 0 && c.hadamard != 1) return TACO_ERR_FORMAT;
      if (c.block != 16 && c.block != 32 && c.block != 64 && c.block != 128) return TACO_ERR_SHAPE;
      return TACO_OK;
    case TACO_FMT_INT8_SYM:
      if (c.hadamard != 0) return TACO_ERR_FORMAT;
      return c.block == 64 ? TACO_OK : TACO_ERR_SHAPE;
    case TACO_FMT_INT4_ASYM:
    case TACO_FMT_INT8_ASYM:
      if (c.hadamard != 0) return TACO_ERR_FORMAT;
      return c.block == 128 ? TACO_OK : TACO_ERR_SHAPE;
    default:
      return TACO_ERR_FORMAT;
  }
}

int check_shape(const taco_codec& c, int64_t rows, int64_t cols) {
  int st = check_codec(c);
  if (st != TACO_OK) return st;
  if (rows < 0 || cols <= 0) return TACO_ERR_INVALID_ARG;
  if (cols % c.block != 0) return TACO_ERR_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return TACO_ERR_INVALID_ARG;
  return TACO_OK;
}

void layout_of(const taco_codec& c, int64_t n, taco_layout_t* L) {
  const int64_t nb = n / c.block;
  L->codes_off = 0;
  L->codes_bytes = c.format == TACO_FMT_INT4_ASYM ? n / 2 : n;
  L->scale_off = align256(L->codes_bytes);
  L->scale_bytes = is_fp8_format(c.format) ? nb : 4 * nb;
  L->aux_off = align256(L->scale_off + L->scale_bytes);
  L->aux_bytes = (c.format == TACO_FMT_INT4_ASYM || c.format == TACO_FMT_INT8_ASYM) ? nb : 0;
  L->tensor_off = align256(L->aux_off + L->aux_bytes);
  L->tensor_bytes = is_fp8_format(c.format) ? 16 : 0;
  L->total_bytes = align256(L->tensor_off + L->tensor_bytes);
}

int log2_block(int b) { return b == 16 ? 4 : b == 32 ? 5 : b == 64 ? 6 : 7; }

// FP8 tensor-scale mode: 0 = given g, 1 = auto (pre-pass), 2 = delayed.
// internal_ws: the workspace is the library's own scratch array (no
// workspace argument to check).
int scale_mode(const taco_codec& c, float ts, void* ws, size_t ws_bytes, bool internal_ws, int* mode) {
  *mode = 0;
  if (!is_fp8_format(c.format)) return TACO_OK;
  if (isnan(ts) || isinf(ts)) return TACO_ERR_INVALID_ARG;
  if (ts > 0.0f) {
    if (ts < kGMin || ts > kGMax) return TACO_ERR_INVALID_ARG;
  } else {
    *mode = (ts == 0.0f) ? 1 : 2;
    if (!internal_ws && (ws == nullptr || ws_bytes < TACO_WORKSPACE_BYTES)) return TACO_ERR_WORKSPACE;
  }
  if (!internal_ws && ws != nullptr && (ws_bytes < TACO_WORKSPACE_BYTES || !aligned16(ws))) return TACO_ERR_WORKSPACE;
  return TACO_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TACO_OK : TACO_ERR_HIP; }

// A launch's status is read with hipGetLastError afterwards, so drop any error an
// earlier, unrelated runtime call on this thread left behind.
void clear_stale_error() { (void)hipGetLastError(); }

struct Regions {
  uint8_t* codes;
  void* scale;
  uint8_t* aux;
  float* tensor;
};

Regions regions_of(void* buf, const taco_layout_t& L) {
  uint8_t* b = static_cast<uint8_t*>(buf);
  return Regions{b + L.codes_off, b + L.scale_off, b + L.aux_off, reinterpret_cast<float*>(b + L.tensor_off)};
}

int scratch_workspace(hipStream_t stream, void** ws);

// internal_ws: the FP8 workspace is the device's scratch array (fetched, and
// cleared on its first use, only after every argument has been checked).
// Shapes the channel-group reorder supports: cols a multiple of 512 and at
// most 131072 (the order fits LDS as int16), FP8 block 128.
int check_reorder(const taco_codec& c, int64_t cols) {
  if (cols % kReorderColsMultiple != 0 || cols > kReorderMaxCols) return TACO_ERR_SHAPE;
  if (is_fp8_format(c.format) && c.block != 128) return TACO_ERR_SHAPE;
  return TACO_OK;
}

// internal_ws: the FP8 workspace is the device's scratch array (fetched, and
// cleared on its first use, only after every argument has been checked).
// order: channel-group reorder of the bf16 input (null: none).
int quantize_common(taco_codec c, const void* x, bool f32_in, int64_t rows, int64_t cols, float ts, void* out,
                    void* ws, size_t ws_bytes, float* dbg, hipStream_t stream, bool internal_ws = false,
                    const int32_t* order = nullptr, bool reordered = false) {
  int st = check_shape(c, rows, cols);
  if (st != TACO_OK) return st;
  if (reordered) {
    st = check_reorder(c, cols);
    if (st != TACO_OK) return st;
    if (order == nullptr) return TACO_ERR_INVALID_ARG;
  }
  int mode = 0;
  st = scale_mode(c, ts, ws, ws_bytes, internal_ws, &mode);
  if (st != TACO_OK) return st;
  const int64_t n = rows * cols;
  if (n == 0) return TACO_OK;
  if (x == nullptr || out == nullptr) return TACO_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out) || (dbg && !aligned16(dbg)) || (order && !aligned16(order)))
    return TACO_ERR_ALIGN;
  taco_layout_t L;
  layout_of(c, n, &L);
  const int64_t in_bytes = n * (f32_in ? 4 : 2);
  if (overlaps(x, in_bytes, out, L.total_bytes)) return TACO_ERR_INVALID_ARG;
  if (order && overlaps(order, 4 * (cols / 8), out, L.total_bytes)) return TACO_ERR_INVALID_ARG;
  if (dbg && (overlaps(dbg, 4 * n, x, in_bytes) || overlaps(dbg, 4 * n, out, L.total_bytes)))
    return TACO_ERR_INVALID_ARG;
  if (internal_ws && is_fp8_format(c.format)) {
    st = scratch_workspace(stream, &ws);
    if (st != TACO_OK) return st;
  }
  Regions R = regions_of(out, L);
  if (is_fp8_format(c.format) && c.hadamard == 1 && !f32_in) {
    FP8HadArgs a;
    a.x = x; a.codes = R.codes; a.kexp = static_cast<int8_t*>(R.scale); a.g_hdr = R.tensor;
    a.nblocks = n / c.block; a.logb = log2_block(c.block); a.e5 = c.format == TACO_FMT_FP8E5_DUAL;
    a.g = mode == 0 ? ts : 1.0f; a.g_from_ws = mode != 0; a.auto_prepass = mode == 1;
    a.ws = ws; a.dbg = dbg; a.ro = make_reorder(order, cols);
    clear_stale_error();
    return hip_status(launch_fp8_had_compress(a, stream));
  }
  QuantArgs a;
  a.fmt = c.format; a.block = c.block; a.f32_in = f32_in; a.x = x; a.n = n;
  a.codes = R.codes; a.scale = R.scale; a.zero = R.aux; a.g_hdr = R.tensor;
  a.g = mode == 0 ? ts : 1.0f; a.g_from_ws = mode != 0; a.auto_prepass = mode == 1;
  a.ws = is_fp8_format(c.format) ? ws : nullptr; a.dbg = dbg; a.ro = make_reorder(order, cols);
  clear_stale_error();
  return hip_status(launch_quantize(a, stream));
}

// ---------------------------------------------------------------- scratch --
// The FP8 tensor-scale workspace of taco_compress_noalloc: one array per GPU,
// in the library's own device memory, so that call allocates nothing. Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device, and is kept per device.
constexpr int kScratchWords = TACO_WORKSPACE_BYTES / 4;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint32_t scratch[kScratchWords];

__global__ __launch_bounds__(256) void k_clear_words(uint32_t* p, int nwords) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < nwords) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch array. The first call on a device looks up its
// address and clears it on `stream` (a fill kernel, ordered before the
// compress that follows on the same stream); later calls reuse the address.
int scratch_workspace(hipStream_t stream, void** ws) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TACO_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return TACO_ERR_HIP;
    clear_stale_error();
    hipLaunchKernelGGL(k_clear_words, dim3((kScratchWords + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ptr), kScratchWords);
    if (hipGetLastError() != hipSuccess) return TACO_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *ws = g_scratch_ptr[dev];
  return TACO_OK;
}

}  // namespace

namespace taco {

thread_local int32_t t_launch_limit = 0;
int launch_limit() { return t_launch_limit; }

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

int resident_groups(const void* kernel, size_t lds) {
  struct Entry {
    const void* kernel;
    size_t lds;
    int dev, groups;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].kernel == kernel && cache[i].lds == lds && cache[i].dev == dev) return cache[i].groups;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, lds) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 1;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (used < 64) cache[used++] = Entry{kernel, lds, dev, n};
  return n;
}

}  // namespace taco

namespace {

bool pair_allowed(const taco_codec& i, const taco_codec& o) {
  if (is_fp8_format(i.format))
    return o.format == i.format && o.block == i.block && o.hadamard == i.hadamard;
  if (i.format == TACO_FMT_INT8_SYM) return o.format == TACO_FMT_INT8_SYM;
  if (i.format == TACO_FMT_INT4_ASYM) return o.format == TACO_FMT_INT8_ASYM;
  if (i.format == TACO_FMT_INT8_ASYM) return o.format == TACO_FMT_INT8_ASYM;
  return false;
}

}  // namespace

extern "C" {

int taco_layout(taco_codec c, int64_t rows, int64_t cols, taco_layout_t* out) {
  if (out == nullptr) return TACO_ERR_INVALID_ARG;
  int st = check_shape(c, rows, cols);
  if (st != TACO_OK) return st;
  layout_of(c, rows * cols, out);
  return TACO_OK;
}

int64_t taco_compressed_bytes(taco_codec c, int64_t rows, int64_t cols) {
  taco_layout_t L;
  int st = taco_layout(c, rows, cols, &L);
  return st == TACO_OK ? L.total_bytes : (int64_t)st;
}

size_t taco_workspace_bytes(taco_codec c, int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return is_fp8_format(c.format) ? TACO_WORKSPACE_BYTES : 0;
}

int taco_compress(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale, void* out,
                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  return quantize_common(c, x_bf16, false, rows, cols, tensor_scale, out, workspace, ws_bytes, nullptr, stream);
}

int taco_compress_noalloc(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale,
                          void* out, hipStream_t stream) {
  return quantize_common(c, x_bf16, false, rows, cols, tensor_scale, out, nullptr, 0, nullptr, stream, true);
}

int taco_compress_debug(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale, void* out,
                        void* workspace, size_t ws_bytes, float* prequant, hipStream_t stream) {
  if (prequant == nullptr) return TACO_ERR_INVALID_ARG;
  return quantize_common(c, x_bf16, false, rows, cols, tensor_scale, out, workspace, ws_bytes, prequant, stream);
}

int taco_requantize(taco_codec c_out, const float* x_fp32, int64_t rows, int64_t cols, float tensor_scale, void* out,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  return quantize_common(c_out, x_fp32, true, rows, cols, tensor_scale, out, workspace, ws_bytes, nullptr, stream);
}

int taco_decompress_reduce(taco_codec c_in, const void* const* shards, int32_t n, int64_t rows, int64_t cols,
                           float* sum_fp32, taco_codec c_out, void* requant_out, hipStream_t stream) {
  int st = check_shape(c_in, rows, cols);
  if (st != TACO_OK) return st;
  if (requant_out != nullptr) {
    st = check_shape(c_out, rows, cols);
    if (st != TACO_OK) return st;
    if (!pair_allowed(c_in, c_out)) return TACO_ERR_FORMAT;
  }
  if (shards == nullptr || n < 1 || n > TACO_MAX_SHARDS) return TACO_ERR_INVALID_ARG;
  if (sum_fp32 == nullptr && requant_out == nullptr) return TACO_ERR_INVALID_ARG;
  const int64_t elems = rows * cols;
  taco_layout_t Li, Lo;
  layout_of(c_in, elems, &Li);
  layout_of(requant_out ? c_out : c_in, elems, &Lo);
  for (int r = 0; r < n; ++r) {
    if (shards[r] == nullptr) return TACO_ERR_INVALID_ARG;
    if (!aligned16(shards[r])) return TACO_ERR_ALIGN;
  }
  if ((sum_fp32 && !aligned16(sum_fp32)) || (requant_out && !aligned16(requant_out))) return TACO_ERR_ALIGN;
  for (int r = 0; r < n; ++r) {
    if (sum_fp32 && overlaps(shards[r], Li.total_bytes, sum_fp32, 4 * elems)) return TACO_ERR_INVALID_ARG;
    if (requant_out && overlaps(shards[r], Li.total_bytes, requant_out, Lo.total_bytes)) return TACO_ERR_INVALID_ARG;
  }
  if (sum_fp32 && requant_out && overlaps(sum_fp32, 4 * elems, requant_out, Lo.total_bytes))
    return TACO_ERR_INVALID_ARG;
  if (elems == 0) return TACO_OK;
  ReduceArgs a;
  memset(&a, 0, sizeof(a));
  a.fin = c_in.format; a.bin = c_in.block;
  a.fout = requant_out ? c_out.format : c_in.format; a.bout = requant_out ? c_out.block : c_in.block;
  a.nshards = n; a.n = elems;
  for (int r = 0; r < n; ++r) {
    Regions R = regions_of(const_cast<void*>(shards[r]), Li);
    a.in.codes[r] = R.codes; a.in.scale[r] = R.scale; a.in.zero[r] = R.aux; a.in.g[r] = R.tensor;
  }
  a.sum = sum_fp32;
  if (requant_out) {
    Regions O = regions_of(requant_out, Lo);
    a.rq_codes = O.codes; a.rq_scale = O.scale; a.rq_zero = O.aux; a.rq_g_hdr = O.tensor;
  }
  clear_stale_error();
  return hip_status(launch_reduce(a, stream));
}

int taco_ring_hop(taco_codec c_in, const void* incoming, const void* local_bf16, int64_t rows, int64_t cols,
                  float* sum_fp32, taco_codec c_out, void* requant_out, hipStream_t stream) {
  int st = check_shape(c_in, rows, cols);
  if (st != TACO_OK) return st;
  if (is_fp8_format(c_in.format)) return TACO_ERR_FORMAT;
  if (requant_out != nullptr) {
    st = check_shape(c_out, rows, cols);
    if (st != TACO_OK) return st;
    if (!pair_allowed(c_in, c_out)) return TACO_ERR_FORMAT;
  }
  if (local_bf16 == nullptr || (sum_fp32 == nullptr && requant_out == nullptr)) return TACO_ERR_INVALID_ARG;
  if ((incoming && !aligned16(incoming)) || !aligned16(local_bf16) || (sum_fp32 && !aligned16(sum_fp32)) ||
      (requant_out && !aligned16(requant_out)))
    return TACO_ERR_ALIGN;
  const int64_t elems = rows * cols;
  taco_layout_t Li, Lo;
  layout_of(c_in, elems, &Li);
  layout_of(requant_out ? c_out : c_in, elems, &Lo);
  const void* outs[2] = {sum_fp32, requant_out};
  const int64_t out_bytes[2] = {4 * elems, Lo.total_bytes};
  for (int k = 0; k < 2; ++k) {
    if (outs[k] == nullptr) continue;
    if (incoming && overlaps(incoming, Li.total_bytes, outs[k], out_bytes[k])) return TACO_ERR_INVALID_ARG;
    if (overlaps(local_bf16, 2 * elems, outs[k], out_bytes[k])) return TACO_ERR_INVALID_ARG;
  }
  if (sum_fp32 && requant_out && overlaps(sum_fp32, 4 * elems, requant_out, Lo.total_bytes))
    return TACO_ERR_INVALID_ARG;
  if (elems == 0) return TACO_OK;
  HopArgs a;
  memset(&a, 0, sizeof(a));
  a.fin = c_in.format; a.bin = c_in.block;
  a.fout = requant_out ? c_out.format : c_in.format; a.bout = requant_out ? c_out.block : c_in.block;
  a.n = elems;
  if (incoming) {
    Regions R = regions_of(const_cast<void*>(incoming), Li);
    a.codes = R.codes; a.scale = R.scale; a.zero = R.aux;
  }
  a.local = static_cast<const uint16_t*>(local_bf16);
  a.sum = sum_fp32;
  if (requant_out) {
    Regions O = regions_of(requant_out, Lo);
    a.rq_codes = O.codes; a.rq_scale = O.scale; a.rq_zero = O.aux;
  }
  clear_stale_error();
  return hip_status(launch_ring_hop(a, stream));
}

namespace {
int decompress_common(taco_codec c, const void* in, int64_t rows, int64_t cols, void* out, int32_t out_dtype,
                      const int32_t* order, bool reordered, hipStream_t stream) {
  int st = check_shape(c, rows, cols);
  if (st != TACO_OK) return st;
  if (reordered) {
    st = check_reorder(c, cols);
    if (st != TACO_OK) return st;
    if (order == nullptr) return TACO_ERR_INVALID_ARG;
  }
  if (out_dtype != 0 && out_dtype != 1) return TACO_ERR_INVALID_ARG;
  const int64_t n = rows * cols;
  if (n == 0) return TACO_OK;
  if (in == nullptr || out == nullptr) return TACO_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out) || (order && !aligned16(order))) return TACO_ERR_ALIGN;
  taco_layout_t L;
  layout_of(c, n, &L);
  const int64_t out_bytes = n * (out_dtype ? 2 : 4);
  if (overlaps(in, L.total_bytes, out, out_bytes)) return TACO_ERR_INVALID_ARG;
  if (order && overlaps(order, 4 * (cols / 8), out, out_bytes)) return TACO_ERR_INVALID_ARG;
  Regions R = regions_of(const_cast<void*>(in), L);
  if (is_fp8_format(c.format) && c.hadamard == 1) {
    FP8HadDecodeArgs a;
    a.codes = R.codes; a.kexp = static_cast<const int8_t*>(R.scale); a.g_hdr = R.tensor;
    a.nblocks = n / c.block; a.logb = log2_block(c.block); a.e5 = c.format == TACO_FMT_FP8E5_DUAL;
    a.bf16_out = out_dtype == 1; a.out = out; a.ro = make_reorder(order, cols);
    clear_stale_error();
    return hip_status(launch_fp8_had_decode(a, stream));
  }
  DequantArgs a;
  a.fmt = c.format; a.block = c.block; a.codes = R.codes; a.scale = R.scale; a.zero = R.aux; a.g_hdr = R.tensor;
  a.n = n; a.bf16_out = out_dtype == 1; a.out = out; a.ro = make_reorder(order, cols);
  clear_stale_error();
  return hip_status(launch_dequantize(a, stream));
}
}  // namespace

int taco_decompress(taco_codec c, const void* in, int64_t rows, int64_t cols, void* out, int32_t out_dtype,
                    hipStream_t stream) {
  return decompress_common(c, in, rows, cols, out, out_dtype, nullptr, false, stream);
}

int taco_decompress_reordered(taco_codec c, const void* in, int64_t rows, int64_t cols, void* out, int32_t out_dtype,
                              const int32_t* order, hipStream_t stream) {
  return decompress_common(c, in, rows, cols, out, out_dtype, order, true, stream);
}

int taco_compress_reordered(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale,
                            void* out, void* workspace, size_t ws_bytes, const int32_t* order, hipStream_t stream) {
  return quantize_common(c, x_bf16, false, rows, cols, tensor_scale, out, workspace, ws_bytes, nullptr, stream,
                         false, order, true);
}

int taco_decompress_gemm(taco_codec c, const void* a, int64_t M, int64_t K, const void* w_bf16, int64_t N, void* out,
                         int32_t out_dtype, hipStream_t stream) {
  int st = check_codec(c);
  if (st != TACO_OK) return st;
  if (c.hadamard != 0) return TACO_ERR_FORMAT;
  if (is_fp8_format(c.format) && c.block < 32) return TACO_ERR_SHAPE;
  if (M < 0 || N <= 0 || K <= 0) return TACO_ERR_INVALID_ARG;
  if (M % 128 != 0 || N % 128 != 0 || K % 128 != 0 || K > (int64_t(1) << 20)) return TACO_ERR_SHAPE;
  if (K > kMaxElems / N || (M > 0 && (K > kMaxElems / M || N > kMaxElems / M))) return TACO_ERR_INVALID_ARG;
  // M * N <= 2^35 keeps the grid, one workgroup per 128 x 128 tile, below 2^21
  if (out_dtype != 0 && out_dtype != 1) return TACO_ERR_INVALID_ARG;
  if (M == 0) return TACO_OK;
  if (a == nullptr || w_bf16 == nullptr || out == nullptr) return TACO_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w_bf16) || !aligned16(out)) return TACO_ERR_ALIGN;
  taco_layout_t L;
  layout_of(c, M * K, &L);
  const int64_t out_bytes = M * N * (out_dtype ? 2 : 4);
  if (overlaps(a, L.total_bytes, out, out_bytes) || overlaps(w_bf16, 2 * N * K, out, out_bytes))
    return TACO_ERR_INVALID_ARG;
  Regions R = regions_of(const_cast<void*>(a), L);
  DGemmArgs d;
  d.fmt = c.format; d.block = c.block; d.codes = R.codes; d.scale = R.scale; d.zero = R.aux; d.g_hdr = R.tensor;
  d.w = static_cast<const uint16_t*>(w_bf16); d.M = M; d.N = N; d.K = K; d.bf16_out = out_dtype == 1; d.out = out;
  d.neg_zero = -0.0f;
  clear_stale_error();
  return hip_status(launch_dequant_gemm(d, stream));
}

int taco_chunk_order(const void* stats_bf16, int64_t rows, int64_t cols, int32_t* order, hipStream_t stream) {
  if (rows < 0 || cols <= 0) return TACO_ERR_INVALID_ARG;
  if (cols % kReorderColsMultiple != 0 || cols > kReorderMaxCols) return TACO_ERR_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return TACO_ERR_INVALID_ARG;
  if (order == nullptr || (rows > 0 && stats_bf16 == nullptr)) return TACO_ERR_INVALID_ARG;
  if (!aligned16(order) || (stats_bf16 && !aligned16(stats_bf16))) return TACO_ERR_ALIGN;
  if (stats_bf16 && overlaps(stats_bf16, 2 * rows * cols, order, 4 * (cols / 8))) return TACO_ERR_INVALID_ARG;
  clear_stale_error();
  return hip_status(launch_chunk_order(stats_bf16, rows, cols, order, stream));
}

namespace {
int fp8_encode(bool e5, const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  if (n < 0 || n > kMaxElems) return TACO_ERR_INVALID_ARG;
  if (n == 0) return TACO_OK;
  if (x == nullptr || codes == nullptr) return TACO_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return TACO_ERR_ALIGN;
  if (overlaps(x, 4 * n, codes, n)) return TACO_ERR_INVALID_ARG;
  clear_stale_error();
  return hip_status(launch_fp8_encode(e5, x, codes, n, stream));
}
}  // namespace

int taco_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  return fp8_encode(false, x, codes, n, stream);
}

int taco_e5m2_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
  return fp8_encode(true, x, codes, n, stream);
}

int taco_set_launch_limit(int32_t max_workgroups, int32_t* previous) {
  if (max_workgroups < 0) return TACO_ERR_INVALID_ARG;
  if (previous != nullptr) *previous = taco::t_launch_limit;
  taco::t_launch_limit = max_workgroups;
  return TACO_OK;
}

const char* taco_status_string(int status) {
  switch (status) {
    case TACO_OK: return "TACO_OK";
    case TACO_ERR_INVALID_ARG: return "TACO_ERR_INVALID_ARG";
    case TACO_ERR_SHAPE: return "TACO_ERR_SHAPE";
    case TACO_ERR_FORMAT: return "TACO_ERR_FORMAT";
    case TACO_ERR_ALIGN: return "TACO_ERR_ALIGN";
    case TACO_ERR_WORKSPACE: return "TACO_ERR_WORKSPACE";
    case TACO_ERR_HIP: return "TACO_ERR_HIP";
    default: return "TACO_ERR_UNKNOWN";
  }
}

}  // extern "C"

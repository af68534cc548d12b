// Transform-free codecs and the decompress-reduce kernel.
//
// Sources (Pith review pages):
// * "EQuARX: Efficient Quantized AllReduce in XLA for Distributed Machine
//   Learning Acceleration" -- "What carries the argument": block-wise
//   symmetric int8 with an abs-max scale, one FP32 scale per 64 entries, and
//   every received shard dequantized to FP32 before it is added.
// * "Flash Communication: Reducing Tensor Parallelization Bottleneck for Fast
//   Large Language Model Inference" -- "What carries the argument":
//   asymmetric group-128 quantization, local FP32 sum of the chunks, INT8
//   re-quantization for the gather stage; Algorithm 1: dequantization from
//   codes, zero point and scale.
// * "TACO: ..." -- Fig. 7 dual-scale FP8 quantization (used here with the
//   transform off, or on float32 values that are already transformed).
//
// Wave layout: a wave holds 1024 consecutive elements, 16 per lane; a block of
// B elements spans B/16 consecutive lanes, so block reductions are DPP steps
// inside a quad or half-row.
#include "device_common.h"
#include "taco_internal.h"

namespace taco {

constexpr int kLaneElems = 16;
constexpr int kWaveElems = kWave * kLaneElems;   // 1024

// ----------------------------------------------------------- lane loads --

template <bool F32IN>
TACO_DEV void load_lane(const void* x, int64_t e0, float* a) {
  if constexpr (F32IN) {
    const float* p = static_cast<const float*>(x) + e0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 w = ld16_nt(p + 4 * q);
      a[4 * q + 0] = __uint_as_float(w.x); a[4 * q + 1] = __uint_as_float(w.y);
      a[4 * q + 2] = __uint_as_float(w.z); a[4 * q + 3] = __uint_as_float(w.w);
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + e0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 w = ld16_nt(p + 8 * q);
      a[8 * q + 0] = bf16_lo(w.x); a[8 * q + 1] = bf16_hi(w.x);
      a[8 * q + 2] = bf16_lo(w.y); a[8 * q + 3] = bf16_hi(w.y);
      a[8 * q + 4] = bf16_lo(w.z); a[8 * q + 5] = bf16_hi(w.z);
      a[8 * q + 6] = bf16_lo(w.w); a[8 * q + 7] = bf16_hi(w.w);
    }
  }
}

TACO_DEV float absmax16(const float* a) { return fmaxf(absmax8(a), absmax8(a + 8)); }

TACO_DEV float max16(const float* a) {
  float m = a[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fmaxf(m, a[i]);
  return m;
}

TACO_DEV float min16(const float* a) {
  float m = a[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = fminf(m, a[i]);
  return m;
}

TACO_DEV uint32_t pack_u8x4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)d << 24);
}

TACO_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// --------------------------------------------------------- quantization --
//
// Per-lane result of quantizing 16 values: code bytes (INT4: 8 bytes in
// words x, y) and the block metadata, valid in every lane of the block.
struct LaneCodes {
  uint4 q;
  float s;      // INT scale, or unused
  int k;        // FP8 block exponent
  int z;        // asymmetric zero point
};

// FP8 dual-scale on values already in the codec's domain. m = max|a| / g,
// k = block exponent, each value scaled by the exact (1/g) * 2^k; an exact
// zero becomes +0 through the +0 addend of the fused multiply-add.
template <int B>
TACO_DEV LaneCodes quant_fp8(float* a, float inv_g, float* pre) {
  constexpr int G = B / kLaneElems;
  LaneCodes r;
  const float M = group_max<G>(absmax16(a));
  const float m = M * inv_g;
  r.k = block_exponent(m);
  const float c = inv_g * pow2f(r.k);
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = fmaf(a[i], c, 0.0f);
  if (__builtin_expect(m * pow2f(r.k) > kE4M3Max, 0)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = sat448(a[i]);
  }
  if (pre) {
#pragma unroll
    for (int i = 0; i < 16; ++i) pre[i] = a[i];
  }
  r.q.x = e4m3_pack4(a[0], a[1], a[2], a[3]);
  r.q.y = e4m3_pack4(a[4], a[5], a[6], a[7]);
  r.q.z = e4m3_pack4(a[8], a[9], a[10], a[11]);
  r.q.w = e4m3_pack4(a[12], a[13], a[14], a[15]);
  r.s = 0.0f; r.z = 0;
  return r;
}

// Symmetric INT8 over a block of 64: s = A/127, q = round(a * (127/A)).
TACO_DEV LaneCodes quant_int8_sym(const float* a, float* pre) {
  LaneCodes r;
  const float A = group_max<4>(absmax16(a));
  const bool live = A >= kTiny;
  r.s = live ? A / 127.0f : 0.0f;
  const float inv = live ? 127.0f / A : 0.0f;
  int q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float t = a[i] * inv;
    if (pre) pre[i] = t;
    q[i] = clampi(rne_int(t), -127, 127);
  }
  r.q.x = pack_u8x4(q[0], q[1], q[2], q[3]);
  r.q.y = pack_u8x4(q[4], q[5], q[6], q[7]);
  r.q.z = pack_u8x4(q[8], q[9], q[10], q[11]);
  r.q.w = pack_u8x4(q[12], q[13], q[14], q[15]);
  r.k = 0; r.z = 0;
  return r;
}

// Asymmetric min/max over a group of 128, BITS = 4 or 8.
template <int BITS>
TACO_DEV LaneCodes quant_asym(const float* a, float* pre) {
  constexpr int QMAX = (1 << BITS) - 1;
  LaneCodes r;
  const float lo = fminf(group_min<8>(min16(a)), 0.0f);
  const float hi = fmaxf(group_max<8>(max16(a)), 0.0f);
  const float rg = hi - lo;
  const bool live = rg >= kTiny;
  r.s = live ? rg / (float)QMAX : 0.0f;
  const float inv = live ? (float)QMAX / rg : 0.0f;
  r.z = clampi(rne_int((-lo) * inv), 0, QMAX);
  int q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float t = a[i] * inv;
    if (pre) pre[i] = t;
    q[i] = clampi(rne_int(t) + r.z, 0, QMAX);
  }
  if constexpr (BITS == 4) {
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j] = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) w[j] |= (uint32_t)q[8 * j + b] << (4 * b);
    }
    r.q = make_uint4(w[0], w[1], 0, 0);
  } else {
    r.q.x = pack_u8x4(q[0], q[1], q[2], q[3]);
    r.q.y = pack_u8x4(q[4], q[5], q[6], q[7]);
    r.q.z = pack_u8x4(q[8], q[9], q[10], q[11]);
    r.q.w = pack_u8x4(q[12], q[13], q[14], q[15]);
  }
  r.k = 0;
  return r;
}

template <int FMT, int B>
TACO_DEV LaneCodes quant_lane(float* a, float inv_g, float* pre) {
  if constexpr (FMT == kFP8) return quant_fp8<B>(a, inv_g, pre);
  else if constexpr (FMT == kINT8S) return quant_int8_sym(a, pre);
  else if constexpr (FMT == kINT4A) return quant_asym<4>(a, pre);
  else return quant_asym<8>(a, pre);
}

// Store one lane's codes; the first lane of each block stores the metadata.
template <int FMT, int B>
TACO_DEV void store_lane(const LaneCodes& r, int64_t e0, uint8_t* codes, void* scale, uint8_t* zero) {
  constexpr int G = B / kLaneElems;
  if constexpr (FMT == kINT4A) {
    *reinterpret_cast<uint2*>(codes + e0 / 2) = make_uint2(r.q.x, r.q.y);
  } else {
    *reinterpret_cast<uint4*>(codes + e0) = r.q;
  }
  if (((threadIdx.x & (kWave - 1)) & (G - 1)) == 0) {
    const int64_t blk = e0 / B;
    if constexpr (FMT == kFP8) {
      static_cast<int8_t*>(scale)[blk] = (int8_t)r.k;
    } else {
      static_cast<float*>(scale)[blk] = r.s;
      if constexpr (FMT == kINT4A || FMT == kINT8A) zero[blk] = (uint8_t)r.z;
    }
  }
}

// ------------------------------------------------------- dequantization --

template <int FMT, int B>
struct LaneIn {
  uint4 q;
  float s;   // INT scale, FP8 combined scale g * 2^-k
  float zf;  // zero point as float
};

template <int FMT, int B>
TACO_DEV LaneIn<FMT, B> load_in(const uint8_t* codes, const void* scale, const uint8_t* zero, const float* g_hdr,
                                int64_t e0) {
  LaneIn<FMT, B> r;
  const int64_t blk = e0 / B;
  if constexpr (FMT == kINT4A) {
    uint2 w = *reinterpret_cast<const uint2*>(codes + e0 / 2);
    r.q = make_uint4(w.x, w.y, 0, 0);
  } else {
    r.q = *reinterpret_cast<const uint4*>(codes + e0);
  }
  if constexpr (FMT == kFP8) {
    const int k = static_cast<const int8_t*>(scale)[blk];
    r.s = (*g_hdr) * pow2f(-k);
    r.zf = 0.0f;
  } else {
    r.s = static_cast<const float*>(scale)[blk];
    r.zf = (FMT == kINT8S) ? 0.0f : (float)zero[blk];
  }
  return r;
}

// Dequantized values of one lane: FP8 dec(q) * (g * 2^-k) (dec(q) * 2^-k is
// exact, so this is the single rounding of dec(q) * 2^-k * g); INT8 q * s;
// asymmetric (q - z) * s with q - z an exact small integer.
template <int FMT, int B>
TACO_DEV void dequant_lane(const LaneIn<FMT, B>& in, float* d) {
  if constexpr (FMT == kFP8) {
    e4m3_unpack4(in.q.x, d); e4m3_unpack4(in.q.y, d + 4);
    e4m3_unpack4(in.q.z, d + 8); e4m3_unpack4(in.q.w, d + 12);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = d[i] * in.s;
  } else if constexpr (FMT == kINT8S) {
    const uint32_t w[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = (float)(int)(int8_t)((w[j] >> (8 * b)) & 0xFF) * in.s;
  } else if constexpr (FMT == kINT8A) {
    const uint32_t w[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = ((float)((w[j] >> (8 * b)) & 0xFF) - in.zf) * in.s;
  } else {
    const uint32_t w[2] = {in.q.x, in.q.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        d[8 * j + 2 * b] = ((float)((lo >> (8 * b)) & 0xFF) - in.zf) * in.s;
        d[8 * j + 2 * b + 1] = ((float)((hi >> (8 * b)) & 0xFF) - in.zf) * in.s;
      }
    }
  }
}

// ---------------------------------------------------------------- kernels --

struct QuantK {
  const void* x;
  int64_t n;
  uint8_t* codes;
  void* scale;
  uint8_t* zero;
  float* g_hdr;
  float g;
  int g_from_ws;
  Workspace* ws;
  float* dbg;
};

template <int FMT, int B, bool F32IN>
__global__ __launch_bounds__(kBlockThreads) void k_quantize(QuantK a) {
  __shared__ float lds4[4];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tile = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
  const bool valid = e0 < a.n;   // n is a multiple of B, B a multiple of 16
  float inv_g = 0.0f;
  if constexpr (FMT == kFP8) {
    const float g = a.g_from_ws ? tensor_scale_from_amax(ws_load_amax_last(a.ws)) : a.g;
    inv_g = 1.0f / g;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.g_hdr = g;
  }
  float v[16];
  if (valid) load_lane<F32IN>(a.x, e0, v);
  else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }
  const float amax = (FMT == kFP8) ? absmax16(v) : 0.0f;
  float pre[16];
  LaneCodes r = quant_lane<FMT, B>(v, inv_g, a.dbg ? pre : nullptr);
  if (valid) {
    store_lane<FMT, B>(r, e0, a.codes, a.scale, a.zero);
    if (a.dbg) {
      float4* d = reinterpret_cast<float4*>(a.dbg + e0);
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = make_float4(pre[4 * q], pre[4 * q + 1], pre[4 * q + 2], pre[4 * q + 3]);
    }
  }
  if constexpr (FMT == kFP8) {
    if (a.ws != nullptr) {
      const float wg = block_max(amax, lds4);
      if (threadIdx.x == 0) ws_publish_amax(a.ws, wg, gridDim.x);
    }
  }
}

// Abs-max pre-pass (FP8 without transform, data-driven tensor scale).
template <bool F32IN>
__global__ __launch_bounds__(kBlockThreads) void k_amax(const void* x, int64_t n, Workspace* ws) {
  __shared__ float lds4[4];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tile = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
  float m = 0.0f;
  if (e0 < n) {
    float v[16];
    load_lane<F32IN>(x, e0, v);
    m = absmax16(v);
  }
  const float wg = block_max(m, lds4);
  if (threadIdx.x == 0) ws_publish_amax(ws, wg, gridDim.x);
}

struct DequantK {
  const uint8_t* codes;
  const void* scale;
  const uint8_t* zero;
  const float* g_hdr;
  int64_t n;
  void* out;
};

template <int FMT, int B, bool BF16OUT>
__global__ __launch_bounds__(kBlockThreads) void k_dequantize(DequantK a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tile = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
  if (e0 >= a.n) return;
  LaneIn<FMT, B> in = load_in<FMT, B>(a.codes, a.scale, a.zero, a.g_hdr, e0);
  float d[16];
  dequant_lane<FMT, B>(in, d);
  if constexpr (BF16OUT) {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + e0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      o[q] = make_uint4(f32_to_bf16(d[8 * q]) | (f32_to_bf16(d[8 * q + 1]) << 16),
                        f32_to_bf16(d[8 * q + 2]) | (f32_to_bf16(d[8 * q + 3]) << 16),
                        f32_to_bf16(d[8 * q + 4]) | (f32_to_bf16(d[8 * q + 5]) << 16),
                        f32_to_bf16(d[8 * q + 6]) | (f32_to_bf16(d[8 * q + 7]) << 16));
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(a.out) + e0);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = make_float4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
  }
}

// Decompress N shards, sum in float32 in shard order, then optionally store
// the sum and/or re-quantize it (FP8: g' = g_0 + ... + g_{N-1}, clamped).
template <int FIN, int BIN, int FOUT, int BOUT>
__global__ __launch_bounds__(kBlockThreads) void k_reduce(ReduceArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tile = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
  const bool valid = e0 < a.n;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  if (valid) {
    int r = 0;
    for (; r + 4 <= a.nshards; r += 4) {
      LaneIn<FIN, BIN> in[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        in[u] = load_in<FIN, BIN>(a.in.codes[r + u], a.in.scale[r + u], a.in.zero[r + u], a.in.g[r + u], e0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float d[16];
        dequant_lane<FIN, BIN>(in[u], d);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
      }
    }
    for (; r < a.nshards; ++r) {
      LaneIn<FIN, BIN> in = load_in<FIN, BIN>(a.in.codes[r], a.in.scale[r], a.in.zero[r], a.in.g[r], e0);
      float d[16];
      dequant_lane<FIN, BIN>(in, d);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
    }
    if (a.sum != nullptr) {
      float4* o = reinterpret_cast<float4*>(a.sum + e0);
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
  }
  if (a.rq_codes != nullptr) {
    float inv_g = 0.0f;
    if constexpr (FOUT == kFP8) {
      float gs = 0.0f;
      for (int r = 0; r < a.nshards; ++r) gs = gs + *a.in.g[r];
      gs = fminf(fmaxf(gs, kGMin), kGMax);
      inv_g = 1.0f / gs;
      if (blockIdx.x == 0 && threadIdx.x == 0) *a.rq_g_hdr = gs;
    }
    LaneCodes rq = quant_lane<FOUT, BOUT>(acc, inv_g, nullptr);
    if (valid) store_lane<FOUT, BOUT>(rq, e0, a.rq_codes, a.rq_scale, a.rq_zero);
  }
}

// Test hook: the device E4M3 encoder alone (four values per lane).
__global__ __launch_bounds__(kBlockThreads) void k_e4m3_encode(const float* x, uint8_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kBlockThreads + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < 4 && i + j < n; ++j) v[j] = x[i + j];
  const uint32_t w = e4m3_pack4(v[0], v[1], v[2], v[3]);
  for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = (uint8_t)(w >> (8 * j));
}

// ------------------------------------------------------------ launchers --

static dim3 grid_for(int64_t n) {
  const int64_t tiles = (n + kWaveElems - 1) / kWaveElems;
  return dim3((unsigned)((tiles + 3) / 4));
}

template <int FMT, int B>
static void launch_q(const QuantArgs& a, const QuantK& k, hipStream_t s) {
  dim3 grid = grid_for(a.n), block(kBlockThreads);
  if (a.f32_in) hipLaunchKernelGGL((k_quantize<FMT, B, true>), grid, block, 0, s, k);
  else hipLaunchKernelGGL((k_quantize<FMT, B, false>), grid, block, 0, s, k);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  QuantK k{a.x, a.n, a.codes, a.scale, a.zero, a.g_hdr, a.g, a.g_from_ws ? 1 : 0,
           static_cast<Workspace*>(a.ws), a.dbg};
  if (a.fmt == kFP8 && a.auto_prepass) {
    dim3 grid = grid_for(a.n), block(kBlockThreads);
    if (a.f32_in) hipLaunchKernelGGL((k_amax<true>), grid, block, 0, s, a.x, a.n, k.ws);
    else hipLaunchKernelGGL((k_amax<false>), grid, block, 0, s, a.x, a.n, k.ws);
  }
  switch (a.fmt) {
    case kFP8:
      switch (a.block) {
        case 16: launch_q<kFP8, 16>(a, k, s); break;
        case 32: launch_q<kFP8, 32>(a, k, s); break;
        case 64: launch_q<kFP8, 64>(a, k, s); break;
        case 128: launch_q<kFP8, 128>(a, k, s); break;
        default: return hipErrorInvalidValue;
      }
      break;
    case kINT8S: launch_q<kINT8S, 64>(a, k, s); break;
    case kINT4A: launch_q<kINT4A, 128>(a, k, s); break;
    case kINT8A: launch_q<kINT8A, 128>(a, k, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int B>
static void launch_dq(const DequantArgs& a, hipStream_t s) {
  DequantK k{a.codes, a.scale, a.zero, a.g_hdr, a.n, a.out};
  dim3 grid = grid_for(a.n), block(kBlockThreads);
  if (a.bf16_out) hipLaunchKernelGGL((k_dequantize<FMT, B, true>), grid, block, 0, s, k);
  else hipLaunchKernelGGL((k_dequantize<FMT, B, false>), grid, block, 0, s, k);
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  switch (a.fmt) {
    case kFP8:
      switch (a.block) {
        case 16: launch_dq<kFP8, 16>(a, s); break;
        case 32: launch_dq<kFP8, 32>(a, s); break;
        case 64: launch_dq<kFP8, 64>(a, s); break;
        case 128: launch_dq<kFP8, 128>(a, s); break;
        default: return hipErrorInvalidValue;
      }
      break;
    case kINT8S: launch_dq<kINT8S, 64>(a, s); break;
    case kINT4A: launch_dq<kINT4A, 128>(a, s); break;
    case kINT8A: launch_dq<kINT8A, 128>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FIN, int BIN, int FOUT, int BOUT>
static void launch_r(const ReduceArgs& a, hipStream_t s) {
  dim3 grid = grid_for(a.n), block(kBlockThreads);
  hipLaunchKernelGGL((k_reduce<FIN, BIN, FOUT, BOUT>), grid, block, 0, s, a);
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.fin == kFP8) {
    switch (a.bin) {
      case 16: launch_r<kFP8, 16, kFP8, 16>(a, s); break;
      case 32: launch_r<kFP8, 32, kFP8, 32>(a, s); break;
      case 64: launch_r<kFP8, 64, kFP8, 64>(a, s); break;
      case 128: launch_r<kFP8, 128, kFP8, 128>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.fin == kINT8S) {
    launch_r<kINT8S, 64, kINT8S, 64>(a, s);
  } else if (a.fin == kINT4A) {
    launch_r<kINT4A, 128, kINT8A, 128>(a, s);
  } else if (a.fin == kINT8A) {
    launch_r<kINT8A, 128, kINT8A, 128>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* x, uint8_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t groups = (n + 4LL * kBlockThreads - 1) / (4LL * kBlockThreads);
  hipLaunchKernelGGL(k_e4m3_encode, dim3((unsigned)groups), dim3(kBlockThreads), 0, s, x, out, n);
  return hipGetLastError();
}

}  // namespace taco

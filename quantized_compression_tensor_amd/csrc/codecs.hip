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
template <int B, bool E5>
TACO_DEV LaneCodes quant_fp8(float* a, float inv_g, float* pre) {
  using F = Fp8Code<E5>;
  constexpr int G = B / kLaneElems;
  LaneCodes r;
  const float M = group_max<G>(absmax16(a));
  const float m = M * inv_g;
  r.k = block_exponent<E5>(m);
  const float c = inv_g * pow2f(r.k);
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = fmaf(a[i], c, 0.0f);
  if (__builtin_expect(m * pow2f(r.k) > F::kMax, 0)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = sat_fp8<E5>(a[i]);
  }
  if (pre) {
#pragma unroll
    for (int i = 0; i < 16; ++i) pre[i] = a[i];
  }
  r.q.x = F::pack4(a[0], a[1], a[2], a[3]);
  r.q.y = F::pack4(a[4], a[5], a[6], a[7]);
  r.q.z = F::pack4(a[8], a[9], a[10], a[11]);
  r.q.w = F::pack4(a[12], a[13], a[14], a[15]);
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
  if constexpr (is_fp8(FMT)) return quant_fp8<B, FMT == kFP8E5>(a, inv_g, pre);
  else if constexpr (FMT == kINT8S) return quant_int8_sym(a, pre);
  else if constexpr (FMT == kINT4A) return quant_asym<4>(a, pre);
  else return quant_asym<8>(a, pre);
}

// ------------------------------------------------------- dequantization --

template <int FMT, int B>
struct LaneIn {
  uint4 q;
  float s;      // INT scale, FP8 combined scale g * 2^-k
  uint32_t z;   // asymmetric zero point; in the reduce, FP8: the dword holding k
  uint32_t sh;  // in the reduce, FP8: bit offset of k in z
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
  r.z = 0;
  r.sh = 0;
  if constexpr (is_fp8(FMT)) {
    const int k = static_cast<const int8_t*>(scale)[blk];
    r.s = (*g_hdr) * pow2f(-k);
  } else {
    r.s = static_cast<const float*>(scale)[blk];
    if constexpr (FMT == kINT4A || FMT == kINT8A) r.z = zero[blk];
  }
  return r;
}

// Byte b of w as a float: unsigned (one v_cvt_f32_ubyte{b}) or signed (one
// v_cvt_f32_i32 with a sign-extended byte operand).
TACO_DEV float ubyte(uint32_t w, int b) { return (float)((w >> (8 * b)) & 0xFFu); }
TACO_DEV float sbyte(uint32_t w, int b) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * b)); }

// Dequantized values of one lane. Every result is the single rounding of the
// exact product, for every finite scale:
//  FP8:  dec(q) * (g * 2^-k); dec(q) * 2^-k is exact, so this is the single
//        rounding of dec(q) * 2^-k * g.
//  INT8 symmetric: q * s, q converted from its signed byte (exact).
//  INT4 asymmetric: (q - z) * s. For four codes at once the bytes
//        ((q | 0x80) - z) ^ 0x80 are formed on a packed word: q + 128 - z lies
//        in [113, 143], so no byte borrows from its neighbour, and the xor
//        turns it into q - z as a signed byte, converted exactly.
//  INT8 asymmetric: (q - z) * s with q - z formed in float (exact).
template <int FMT, int B>
TACO_DEV void dequant_lane(const LaneIn<FMT, B>& in, float* d) {
  if constexpr (is_fp8(FMT)) {
    using F = Fp8Code<FMT == kFP8E5>;
    F::unpack4(in.q.x, d); F::unpack4(in.q.y, d + 4);
    F::unpack4(in.q.z, d + 8); F::unpack4(in.q.w, d + 12);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = d[i] * in.s;
  } else if constexpr (FMT == kINT8S) {
    const uint32_t w[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = sbyte(w[j], b) * in.s;
  } else if constexpr (FMT == kINT8A) {
    const uint32_t w[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
    const float zf = (float)in.z;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = (ubyte(w[j], b) - zf) * in.s;
  } else {
    // 128 - z in every byte (v_perm with selector 0 copies byte 0 of z into all four)
    const uint32_t zrep = 0x80808080u - __builtin_amdgcn_perm(in.z, in.z, 0u);
    uint32_t t[4];
    t[0] = ((in.q.x & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;          // elements 0, 2, 4, 6
    t[1] = (((in.q.x >> 4) & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;   // elements 1, 3, 5, 7
    t[2] = ((in.q.y & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;
    t[3] = (((in.q.y >> 4) & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        d[8 * j + 2 * b] = sbyte(t[2 * j], b) * in.s;
        d[8 * j + 2 * b + 1] = sbyte(t[2 * j + 1], b) * in.s;
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

// Store one lane's codes (streaming stores, as for the buffer stores); the
// first lane of each block stores the metadata.
template <int FMT, int B>
TACO_DEV void store_lane(const LaneCodes& r, int64_t e0, uint8_t* codes, void* scale, uint8_t* zero) {
  constexpr int G = B / kLaneElems;
  if constexpr (FMT == kINT4A) {
    u32x2 w = {r.q.x, r.q.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(codes + e0 / 2));
  } else {
    u32x4 w = {r.q.x, r.q.y, r.q.z, r.q.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(codes + e0));
  }
  if (((threadIdx.x & (kWave - 1)) & (G - 1)) == 0) {
    const int64_t blk = e0 / B;
    if constexpr (is_fp8(FMT)) {
      static_cast<int8_t*>(scale)[blk] = (int8_t)r.k;
    } else {
      static_cast<float*>(scale)[blk] = r.s;
      if constexpr (FMT == kINT4A || FMT == kINT8A) zero[blk] = (uint8_t)r.z;
    }
  }
}

// Quantization without a transform. Grid-stride over 1024-element wave tiles,
// no explicit prefetch: the launch gives every wave one tile and relies on
// full occupancy for the loads in flight (measured faster than a two-buffer
// pipeline on a persistent grid).
template <int FMT, int B, bool F32IN, bool DEBUG>
__global__ __launch_bounds__(kBlockThreads) void k_quantize(QuantK a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ntiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  float inv_g = 0.0f;
  uint32_t e = 0;
  if constexpr (is_fp8(FMT)) {
    __shared__ uint32_t lds_e;
    __shared__ float lds_g;
    float g = a.g;
    if (a.ws != nullptr) {
      if (wave_in_group() == 0) {
        const uint32_t ee = ws_bank_of(ws_ticket(a.ws));
        float gg = a.g;
        if (a.g_from_ws) gg = tensor_scale_from_amax<FMT == kFP8E5>(ws_prev_amax(a.ws, ee));
        if (blockIdx.x == 0) ws_clear_next(a.ws, ee);
        if (lane == 0) { lds_e = ee; lds_g = gg; }
      }
      lds_barrier();
      e = lds_e;
      if (a.g_from_ws) g = lds_g;
    }
    inv_g = 1.0f / g;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.g_hdr = g;
  }
  float run_max = 0.0f;
  for (int64_t tile = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); tile < ntiles;
       tile += stride) {
    const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
    const bool valid = e0 < a.n;   // n is a multiple of B, B a multiple of 16
    float v[16];
    if (valid) load_lane<F32IN>(a.x, e0, v);
    else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    if constexpr (is_fp8(FMT)) run_max = fmaxf(run_max, absmax16(v));
    float pre[16];
    LaneCodes r = quant_lane<FMT, B>(v, inv_g, DEBUG ? pre : nullptr);
    if (valid) {
      store_lane<FMT, B>(r, e0, a.codes, a.scale, a.zero);
      if constexpr (DEBUG) {
        float4* d = reinterpret_cast<float4*>(a.dbg + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = make_float4(pre[4 * q], pre[4 * q + 1], pre[4 * q + 2], pre[4 * q + 3]);
      }
    }
  }
  if constexpr (is_fp8(FMT)) {
    if (a.ws != nullptr) {
      __shared__ float lds_m[kBlockThreads / kWave];
      ws_record_group(a.ws, e, run_max, lds_m);
    }
  }
}

// Abs-max pre-pass (FP8 without transform, data-driven tensor scale).
template <bool F32IN>
__global__ __launch_bounds__(kBlockThreads) void k_amax(const void* x, int64_t n, Workspace* ws) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ntiles = (n + kWaveElems - 1) / kWaveElems;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  float m = 0.0f;
  for (int64_t tile = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); tile < ntiles;
       tile += stride) {
    const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
    if (e0 < n) {
      float v[16];
      load_lane<F32IN>(x, e0, v);
      m = fmaxf(m, absmax16(v));
    }
  }
  __shared__ float lds_m[kBlockThreads / kWave];
  __shared__ uint32_t lds_e;
  if (wave_in_group() == 0) {
    const uint32_t e = ws_bank_of(ws_ticket(ws));
    if (blockIdx.x == 0) ws_clear_next(ws, e);
    if (lane == 0) lds_e = e;
  }
  lds_barrier();
  ws_record_group(ws, lds_e, m, lds_m);
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
//
// Persistent grid over 1024-element wave tiles. A wave walks a flat sequence
// of steps -- (tile, group of up to four shards), the groups of a tile in
// shard order -- with two register sets used alternately: the loads of the
// next step are issued before the current step is dequantized and added, so
// one step's loads are always in flight. All NMAX shard slots are read
// through buffer resources; slots r >= N get an empty resource, load zeros and
// add an exact +0 (acc is never -0), so the instruction stream is the same for
// every N <= NMAX. Steps past the last tile load nothing (their offsets lie
// outside every resource). A launch covers at most kReducePiece elements (the
// host splits larger tensors), so every byte offset fits 32 bits.
// Two resources per shard: the codes, and the block metadata -- the scales,
// followed (asymmetric formats) by the zero points a.zero_rel bytes after the
// first scale byte, the same distance in every shard.
template <int FMT, int B>
struct ShardRsrc {
  rsrc_t codes, meta;
};

// n <= kReducePiece, so every size below is under 2^31.
template <int FMT, int B>
TACO_DEV ShardRsrc<FMT, B> shard_rsrc(const ReduceArgs& a, int r, int n) {
  const bool live = r < a.nshards;
  const int nb = n / B;
  constexpr bool ASYM = FMT == kINT4A || FMT == kINT8A;
  ShardRsrc<FMT, B> s;
  s.codes = make_rsrc32(a.in.codes[r], live ? (FMT == kINT4A ? n / 2 : n) : 0);
  s.meta = make_rsrc32(a.in.scale[r], live ? (is_fp8(FMT) ? (nb + 3) & ~3 : (ASYM ? a.zero_rel + nb : 4 * nb)) : 0);
  return s;
}

// One lane's codes and block metadata of one shard. FP8: g is the shard's
// tensor scale (0 for an empty slot).
template <int FMT, int B>
// FP8 leaves the exponent dword in z and its bit offset in sh: the scale is
// formed when the lane is added (fp8_reduce_scale), so nothing here waits for
// the loads.
TACO_DEV LaneIn<FMT, B> load_in_buf(const ShardRsrc<FMT, B>& s, int e0, int zero_rel) {
  LaneIn<FMT, B> r;
  const int blk = e0 / B;
  if constexpr (FMT == kINT4A) {
    uint2 w = bload64<kNT>(s.codes, e0 / 2, 0);
    r.q = make_uint4(w.x, w.y, 0, 0);
  } else {
    r.q = bload128<kNT>(s.codes, e0, 0);
  }
  r.z = 0;
  r.sh = 0;
  r.s = 0.0f;
  if constexpr (is_fp8(FMT)) {
    // the aligned dword holding the exponent byte (the resource is rounded up
    // to whole dwords, inside the region's padding)
    r.z = bload32(s.meta, blk & ~3, 0);
    r.sh = 8 * (blk & 3);
  } else {
    r.s = __uint_as_float(bload32(s.meta, blk * 4, 0));
    if constexpr (FMT == kINT4A || FMT == kINT8A) r.z = bload8(s.meta, blk, zero_rel);
  }
  return r;
}

template <int FIN, int BIN, int NMAX>
struct ReduceGroup {
  // shards per step: four for FP8 from eight shards on (more bytes per step
  // measured faster), two otherwise (fewer registers, more resident waves)
  static constexpr int GRP = NMAX == 2 ? 1 : (is_fp8(FIN) && NMAX >= 8 ? 4 : 2);
  static constexpr int NG = NMAX / GRP;                 // steps per tile (>= 2)
  LaneIn<FIN, BIN> in[GRP];

  // Issue the loads of shard group `grp` of the tile at element e0 (FP8: the
  // scale is formed when the step is added).
  TACO_DEV void load(const ReduceArgs& a, int grp, int e0, int n) {
    // With more than two groups the compiler would hoist every shard's
    // resources out of the loop and spill them; an opaque group index keeps
    // each step building only its own group's.
    if constexpr (NG > 2) asm volatile("" : "+s"(grp));
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      const int r = grp * GRP + u;
      in[u] = load_in_buf<FIN, BIN>(shard_rsrc<FIN, BIN>(a, r, n), e0, a.zero_rel);
    }
  }

  // Dequantize and add group `grp` (a compile-time step index). glane: lane r
  // holds shard r's FP8 tensor scale g_r; the FP8 scale is g_r * 2^-k (exact).
  TACO_DEV void add_to(float* acc, int grp, float glane) const {
#pragma unroll
    for (int u = 0; u < GRP; ++u) {
      LaneIn<FIN, BIN> x = in[u];
      if constexpr (is_fp8(FIN)) {
        const int k = (int)(int8_t)(uint8_t)(x.z >> x.sh);
        x.s = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(glane), grp * GRP + u)) * pow2f(-k);
      }
      float d[16];
      dequant_lane<FIN, BIN>(x, d);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
    }
  }
};

template <int FIN, int BIN, int FOUT, int BOUT, int NMAX>
__global__ __launch_bounds__(kBlockThreads) void k_reduce(ReduceArgs a) {
  using RG = ReduceGroup<FIN, BIN, NMAX>;
  constexpr int NG = RG::NG;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = (int)a.n;   // <= kReducePiece
  const int ntiles = (n + kWaveElems - 1) / kWaveElems;
  const int stride = (int)gridDim.x * (kBlockThreads / kWave);
  const bool rq = a.rq_codes != nullptr;
  // FP8: lane r < nshards points at shard r's tensor scale, every other lane at
  // shard 0's (always present; empty slots load zero codes, so the scale they
  // pick up multiplies zeros). The scales come in with
  // one gather load issued behind the first step's data loads: a chain of
  // dependent scalar loads here would hold every wave's first loads back, and
  // an unconditional load keeps the wait counts exact.
  typedef __attribute__((address_space(1))) const float* gfloat_ptr;
  gfloat_ptr gp = (gfloat_ptr)a.in.g[0];
  if constexpr (is_fp8(FIN)) {
#pragma unroll
    for (int r = 1; r < NMAX; ++r) {
      // the opaque copy keeps the selection in registers (the compiler would
      // otherwise turn it into a load of the pointer array from memory)
      gfloat_ptr pr = (gfloat_ptr)a.in.g[r];
      asm volatile("" : "+s"(pr));
      gp = (lane == r && r < a.nshards) ? pr : gp;
    }
  }
  float glane = 0.0f;
  const int nb_out = n / BOUT;
  const rsrc_t r_sum = make_rsrc32(a.sum, a.sum ? 4 * n : 0);
  const rsrc_t r_qc = make_rsrc32(a.rq_codes, rq ? n : 0);
  const rsrc_t r_qs = make_rsrc32(a.rq_scale, rq ? (is_fp8(FOUT) ? nb_out : 4 * nb_out) : 0);
  const rsrc_t r_qz = make_rsrc32(a.rq_zero, rq && FOUT == kINT8A ? nb_out : 0);

  // the finished sum of a tile: store it and/or re-quantize it
  auto finish = [&](int t, float* acc) {
    const int e0 = t * kWaveElems + lane * kLaneElems;
    if (a.sum != nullptr) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bstore128(make_uint4(__float_as_uint(acc[4 * q]), __float_as_uint(acc[4 * q + 1]),
                             __float_as_uint(acc[4 * q + 2]), __float_as_uint(acc[4 * q + 3])),
                  r_sum, e0 * 4 + 16 * q, 0);
    }
    if (rq) {
      // FP8: g' = g_0 + ... + g_{N-1} in shard order, clamped
      float inv_g = 0.0f;
      if constexpr (is_fp8(FOUT)) {
        float gs = 0.0f;
        for (int r = 0; r < a.nshards; ++r)
          gs = gs + __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(glane), r));
        gs = fminf(fmaxf(gs, kGMin), kGMax);
        inv_g = 1.0f / gs;
        if (blockIdx.x == 0 && threadIdx.x == 0 && a.write_g) *a.rq_g_hdr = gs;
      }
      // lanes beyond the tensor quantize zeros; their stores fall outside the
      // resources and are dropped
      LaneCodes q = quant_lane<FOUT, BOUT>(acc, inv_g, nullptr);
      const int blk = e0 / BOUT;
      bstore128(q.q, r_qc, e0, 0);
      if constexpr (is_fp8(FOUT)) {
        bstore8((uint32_t)q.k, r_qs, blk, 0);
      } else {
        bstore32(__float_as_uint(q.s), r_qs, blk * 4, 0);
        if constexpr (FOUT == kINT8A) bstore8((uint32_t)q.z, r_qz, blk, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  };

  // One loop iteration covers one tile: its NG >= 2 shard groups, one step
  // each. The two register sets alternate by step; the loads of step k + 1
  // (the next group, or the first group of the wave's next tile) are issued,
  // and kept ahead of the arithmetic by a scheduling barrier, before step k is
  // added. The last iteration's look-ahead lies past the end: it loads zeros.
  static_assert(NG >= 2 && NG % 2 == 0, "an even number of steps per tile");
  int t = (int)blockIdx.x * (kBlockThreads / kWave) + wave_in_group();
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  RG buf[2];
  buf[0].load(a, 0, t * kWaveElems + lane * kLaneElems, n);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (is_fp8(FIN)) glane = *gp;   // lanes >= nshards: shard 0's g, read by no live step
  for (; t < ntiles; t += stride) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int tn = k + 1 < NG ? t : t + stride;   // tile and group of step k + 1
      const int gn = (k + 1) % NG;
      buf[(k + 1) & 1].load(a, gn, tn * kWaveElems + lane * kLaneElems, n);
      __builtin_amdgcn_sched_barrier(0);
      buf[k & 1].add_to(acc, k, glane);
    }
    finish(t, acc);
  }
}

// One hop of a quantized ring reduce-scatter: acc = (0 + dequant(incoming)) +
// local, one float32 rounding per add, then the FP32 sum and/or the partial sum
// quantized for the next hop. Grid-stride over 1024-element wave tiles, one
// tile per wave as launched (as the quantize kernel; 16 values per lane).
template <int FIN, int BIN, int FOUT, int BOUT>
__global__ __launch_bounds__(kBlockThreads) void k_ring_hop(HopArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ntiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  for (int64_t tile = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); tile < ntiles;
       tile += stride) {
    const int64_t e0 = tile * kWaveElems + (int64_t)lane * kLaneElems;
    const bool valid = e0 < a.n;   // n is a multiple of the block, a multiple of 16
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    if (valid) {
      if (a.codes != nullptr) {
        const LaneIn<FIN, BIN> in = load_in<FIN, BIN>(a.codes, a.scale, a.zero, nullptr, e0);
        float d[16];
        dequant_lane<FIN, BIN>(in, d);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
      }
      float x[16];
      load_lane<false>(a.local, e0, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc[i] + x[i];
      if (a.sum != nullptr) {
        float4* o = reinterpret_cast<float4*>(a.sum + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
      }
    }
    if (a.rq_codes != nullptr) {
      // every lane takes part in the block reductions; lanes past the end
      // quantize zeros and store nothing
      const LaneCodes q = quant_lane<FOUT, BOUT>(acc, 0.0f, nullptr);
      if (valid) store_lane<FOUT, BOUT>(q, e0, a.rq_codes, a.rq_scale, a.rq_zero);
    }
  }
}

// Test hook: the device FP8 encoder alone (four values per lane).
template <bool E5>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_encode(const float* x, uint8_t* out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * kBlockThreads + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < 4 && i + j < n; ++j) v[j] = x[i + j];
  const uint32_t w = Fp8Code<E5>::pack4(v[0], v[1], v[2], v[3]);
  for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = (uint8_t)(w >> (8 * j));
}

// ------------------------------------------------------------ launchers --

static dim3 grid_for(int64_t n) {
  const int64_t tiles = (n + kWaveElems - 1) / kWaveElems;
  return dim3((unsigned)((tiles + 3) / 4));
}

// One wave per tile and as many workgroups as that takes: the hardware keeps
// every CU at full occupancy as waves retire (5-8 % faster than a grid capped
// at 4 workgroups per CU on the INT8 and INT4 compress).
static dim3 quant_grid(const QuantArgs& a) { return grid_for(a.n); }

template <int FMT, int B>
static void launch_q(const QuantArgs& a, const QuantK& k, hipStream_t s) {
  dim3 grid = quant_grid(a), block(kBlockThreads);
  if (a.dbg) {
    if (a.f32_in) hipLaunchKernelGGL((k_quantize<FMT, B, true, true>), grid, block, 0, s, k);
    else hipLaunchKernelGGL((k_quantize<FMT, B, false, true>), grid, block, 0, s, k);
  } else {
    if (a.f32_in) hipLaunchKernelGGL((k_quantize<FMT, B, true, false>), grid, block, 0, s, k);
    else hipLaunchKernelGGL((k_quantize<FMT, B, false, false>), grid, block, 0, s, k);
  }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  QuantK k{a.x, a.n, a.codes, a.scale, a.zero, a.g_hdr, a.g, a.g_from_ws ? 1 : 0,
           static_cast<Workspace*>(a.ws), a.dbg};
  if (is_fp8(a.fmt) && a.auto_prepass) {
    dim3 grid = quant_grid(a), block(kBlockThreads);
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
    case kFP8E5:
      switch (a.block) {
        case 16: launch_q<kFP8E5, 16>(a, k, s); break;
        case 32: launch_q<kFP8E5, 32>(a, k, s); break;
        case 64: launch_q<kFP8E5, 64>(a, k, s); break;
        case 128: launch_q<kFP8E5, 128>(a, k, s); break;
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
    case kFP8E5:
      switch (a.block) {
        case 16: launch_dq<kFP8E5, 16>(a, s); break;
        case 32: launch_dq<kFP8E5, 32>(a, s); break;
        case 64: launch_dq<kFP8E5, 64>(a, s); break;
        case 128: launch_dq<kFP8E5, 128>(a, s); break;
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

// Reduce grid. The FP8 and INT8-symmetric inputs are bound by memory: a
// workgroup per 4 * kReduceTilesPerWave tiles, dispatched by the hardware as
// CUs free up, keeps every CU streaming until the end. The asymmetric inputs
// do several times more arithmetic per byte: a persistent grid of
// kReduceGroupsPerCU workgroups per CU spreads each wave's setup over many
// tiles.
template <int FIN, int BIN, int FOUT, int BOUT, int NMAX>
static void launch_r(const ReduceArgs& a, hipStream_t s) {
  constexpr bool ALU_BOUND = FIN == kINT4A || FIN == kINT8A;
  const int64_t tiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t per_group = 4 * (ALU_BOUND ? 1 : kReduceTilesPerWave);
  dim3 grid((unsigned)((tiles + per_group - 1) / per_group)), block(kBlockThreads);
  const unsigned cap = (unsigned)(device_cu_count() * kReduceGroupsPerCU);
  if (ALU_BOUND && grid.x > cap) grid.x = cap;
  hipLaunchKernelGGL((k_reduce<FIN, BIN, FOUT, BOUT, NMAX>), grid, block, 0, s, a);
}

template <int FIN, int BIN, int FOUT, int BOUT>
static void launch_rn(const ReduceArgs& a, hipStream_t s) {
  if (a.nshards <= 2) launch_r<FIN, BIN, FOUT, BOUT, 2>(a, s);
  else if (a.nshards <= 4) launch_r<FIN, BIN, FOUT, BOUT, 4>(a, s);
  else if (a.nshards <= 8) launch_r<FIN, BIN, FOUT, BOUT, 8>(a, s);
  else launch_r<FIN, BIN, FOUT, BOUT, 16>(a, s);
}

static hipError_t launch_reduce_piece(const ReduceArgs& a, hipStream_t s) {
  if (a.fin == kFP8) {
    switch (a.bin) {
      case 16: launch_rn<kFP8, 16, kFP8, 16>(a, s); break;
      case 32: launch_rn<kFP8, 32, kFP8, 32>(a, s); break;
      case 64: launch_rn<kFP8, 64, kFP8, 64>(a, s); break;
      case 128: launch_rn<kFP8, 128, kFP8, 128>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.fin == kFP8E5) {
    switch (a.bin) {
      case 16: launch_rn<kFP8E5, 16, kFP8E5, 16>(a, s); break;
      case 32: launch_rn<kFP8E5, 32, kFP8E5, 32>(a, s); break;
      case 64: launch_rn<kFP8E5, 64, kFP8E5, 64>(a, s); break;
      case 128: launch_rn<kFP8E5, 128, kFP8E5, 128>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.fin == kINT8S) {
    launch_rn<kINT8S, 64, kINT8S, 64>(a, s);
  } else if (a.fin == kINT4A) {
    launch_rn<kINT4A, 128, kINT8A, 128>(a, s);
  } else if (a.fin == kINT8A) {
    launch_rn<kINT8A, 128, kINT8A, 128>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int64_t code_bytes(int fmt, int64_t elems) { return fmt == kINT4A ? elems / 2 : elems; }
static int64_t scale_bytes(int fmt, int64_t blocks) { return is_fp8(fmt) ? blocks : 4 * blocks; }

// Split the tensor into pieces of at most kReducePiece elements; each piece is
// one launch over offset pointers (blocks never straddle pieces).
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  for (int64_t e = 0; e < a.n; e += kReducePiece) {
    ReduceArgs p = a;
    p.n = (a.n - e < kReducePiece) ? a.n - e : kReducePiece;
    p.write_g = (e == 0);
    const int64_t bi = e / a.bin, bo = e / a.bout;
    p.zero_rel = 0;
    for (int r = 0; r < a.nshards; ++r) {
      p.in.codes[r] = a.in.codes[r] + code_bytes(a.fin, e);
      p.in.scale[r] = static_cast<const uint8_t*>(a.in.scale[r]) + scale_bytes(a.fin, bi);
      p.in.zero[r] = a.in.zero[r] + bi;
      if (a.fin == kINT4A || a.fin == kINT8A) {
        // the zero points follow the scales at one distance in every shard
        const int64_t rel = p.in.zero[r] - static_cast<const uint8_t*>(p.in.scale[r]);
        if (rel < 4 * (p.n / a.bin) || rel + p.n / a.bin > 0x7FFFFFF0 || (r > 0 && rel != p.zero_rel))
          return hipErrorInvalidValue;
        p.zero_rel = (int)rel;
      }
    }
    if (a.sum) p.sum = a.sum + e;
    if (a.rq_codes) {
      p.rq_codes = a.rq_codes + e;
      p.rq_scale = static_cast<uint8_t*>(a.rq_scale) + scale_bytes(a.fout, bo);
      p.rq_zero = a.rq_zero + bo;
    }
    hipError_t err = launch_reduce_piece(p, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int FIN, int BIN, int FOUT, int BOUT>
// One wave per tile, as the quantize kernel (5-9 % faster than a grid capped
// at 4 workgroups per CU).
static void launch_hop(const HopArgs& a, hipStream_t s) {
  dim3 grid = grid_for(a.n), block(kBlockThreads);
  hipLaunchKernelGGL((k_ring_hop<FIN, BIN, FOUT, BOUT>), grid, block, 0, s, a);
}

hipError_t launch_ring_hop(const HopArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.fin == kINT8S) launch_hop<kINT8S, 64, kINT8S, 64>(a, s);
  else if (a.fin == kINT4A) launch_hop<kINT4A, 128, kINT8A, 128>(a, s);
  else if (a.fin == kINT8A) launch_hop<kINT8A, 128, kINT8A, 128>(a, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fp8_encode(bool e5, const float* x, uint8_t* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t groups = (n + 4LL * kBlockThreads - 1) / (4LL * kBlockThreads);
  if (e5) hipLaunchKernelGGL(k_fp8_encode<true>, dim3((unsigned)groups), dim3(kBlockThreads), 0, s, x, out, n);
  else hipLaunchKernelGGL(k_fp8_encode<false>, dim3((unsigned)groups), dim3(kBlockThreads), 0, s, x, out, n);
  return hipGetLastError();
}

}  // namespace taco

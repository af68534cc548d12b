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


// max |a|, max a and min a over a lane's V = 8 or 16 values
template <int V>
TACO_DEV float absmax_v(const float* a) {
  if constexpr (V == 8) return absmax8(a);
  else return fmaxf(absmax8(a), absmax8(a + 8));
}

template <int V>
TACO_DEV float max_v(const float* a) {
  float m = a[0];
#pragma unroll
  for (int i = 1; i < V; ++i) m = fmaxf(m, a[i]);
  return m;
}

template <int V>
TACO_DEV float min_v(const float* a) {
  float m = a[0];
#pragma unroll
  for (int i = 1; i < V; ++i) m = fminf(m, a[i]);
  return m;
}

TACO_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// --------------------------------------------------------- quantization --
//
// Per-lane result of quantizing V = 8 or 16 consecutive values (a block of B
// spans B / V lanes): code bytes in words x, y, z, w from the first (INT4:
// V / 2 bytes) and the block metadata, valid in every lane of the block.
struct LaneCodes {
  uint4 q;
  float s;      // INT scale, or unused
  int k;        // FP8 block exponent
  int z;        // asymmetric zero point
};

// FP8 dual-scale on values already in the codec's domain. m = max|a| / g,
// k = block exponent, each value scaled by the exact (1/g) * 2^k; an exact
// zero becomes +0 through the +0 addend of the fused multiply-add.
template <int B, bool E5, int V>
TACO_DEV LaneCodes quant_fp8(float* a, float inv_g, float* pre) {
  using F = Fp8Code<E5>;
  constexpr int G = B / V;
  LaneCodes r;
  const float M = group_max<G>(absmax_v<V>(a));
  const float m = M * inv_g;
  r.k = block_exponent<E5>(m);
  const float c = inv_g * pow2f(r.k);
#pragma unroll
  for (int i = 0; i < V; ++i) a[i] = fmaf(a[i], c, 0.0f);
  if (__builtin_expect(m * pow2f(r.k) > F::kMax, 0)) {
#pragma unroll
    for (int i = 0; i < V; ++i) a[i] = sat_fp8<E5>(a[i]);
  }
  if (pre) {
#pragma unroll
    for (int i = 0; i < V; ++i) pre[i] = a[i];
  }
  r.q = make_uint4(0, 0, 0, 0);
  r.q.x = F::pack4(a[0], a[1], a[2], a[3]);
  r.q.y = F::pack4(a[4], a[5], a[6], a[7]);
  if constexpr (V == 16) {
    r.q.z = F::pack4(a[8], a[9], a[10], a[11]);
    r.q.w = F::pack4(a[12], a[13], a[14], a[15]);
  }
  r.s = 0.0f; r.z = 0;
  return r;
}

// Scale and reciprocal of a block from its statistic m (INT8 symmetric: the
// abs-max; asymmetric: the range hi - lo): s = m / QMAX and inv = QMAX / m,
// both 0 for a block with m < 2^-100 (which then quantizes to zeros).
template <int QMAX>
TACO_DEV void block_scales(float m, float& s, float& inv) {
  const bool live = m >= kTiny;
  s = live ? m / (float)QMAX : 0.0f;
  inv = live ? (float)QMAX / m : 0.0f;
}

// The same for the two blocks a lane holds in the two-half tile layout, with
// one division per quantity: the lanes with bit 2 set divide for the second
// half, the others for the first, and each takes the other result from its
// mirror lane (lane ^ 7 within its eight-lane half-row), which lies in the
// same block of both halves when a block spans at least eight lanes.
template <int QMAX>
TACO_DEV void block_scales_pair(float m0, float m1, float* s, float* inv) {
  const bool upper = (threadIdx.x & 4) != 0;
  float sm, im;
  block_scales<QMAX>(upper ? m1 : m0, sm, im);
  constexpr int kMirror = 0x141;   // DPP row_half_mirror
  const float so = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sm), kMirror, 0xF, 0xF, false));
  const float io = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(im), kMirror, 0xF, 0xF, false));
  s[0] = upper ? so : sm; s[1] = upper ? sm : so;
  inv[0] = upper ? io : im; inv[1] = upper ? im : io;
}

// The same with one division per lane, for a block of G = 4 or 8 lanes that
// all hold its statistic m and are all active: the lanes with bit G/2 set
// divide for the reciprocal, the others for the scale, and each takes the
// other result from its mirror lane (lane ^ (G - 1) inside the block: a quad
// permute for 4 lanes, the half-row mirror for 8).
template <int QMAX, int G>
TACO_DEV void block_scales_split(float m, float& s, float& inv) {
  static_assert(G == 4 || G == 8, "a block of 4 or 8 lanes");
  constexpr int kMirror = G == 8 ? 0x141 : 0x1B;   // DPP row_half_mirror / quad_perm [3, 2, 1, 0]
  const bool upper = (threadIdx.x & (G / 2)) != 0;
  const bool live = m >= kTiny;
  const float num = upper ? (float)QMAX : m, den = upper ? m : (float)QMAX;
  const float mine = live ? num / den : 0.0f;
  const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mine), kMirror, 0xF, 0xF, false));
  s = upper ? other : mine;
  inv = upper ? mine : other;
}

// Four bytes (the low byte of each value) into one word.
TACO_DEV uint32_t pack_bytes(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);   // a.b0, b.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x04000c0cu);   // 0, 0, c.b0, d.b0
  return lo | hi;
}

// Eight 4-bit values in [0, 15] into one word, element 0 in the low nibble:
// one shift-or per value (a chain the compiler would otherwise rebalance into
// separate shifts and three-way ors).
TACO_DEV uint32_t pack_nibbles(const int* q) {
  uint32_t w = (uint32_t)q[0];
#pragma unroll
  for (int b = 1; b < 8; ++b)
    asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(w) : "v"(q[b]), "i"(4 * b), "v"(w));
  return w;
}

// Symmetric INT8 over a block of 64: q = round(a * inv), given the block's
// s = A/127 and inv = 127/A.
template <int V>
TACO_DEV LaneCodes int8_sym_encode(const float* a, float s, float inv, float* pre) {
  LaneCodes r;
  r.s = s;
  int q[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float t = a[i] * inv;
    if (pre) pre[i] = t;
    q[i] = clampi(rne_int(t), -127, 127);
  }
  r.q = make_uint4(0, 0, 0, 0);
  r.q.x = pack_bytes(q[0], q[1], q[2], q[3]);
  r.q.y = pack_bytes(q[4], q[5], q[6], q[7]);
  if constexpr (V == 16) {
    r.q.z = pack_bytes(q[8], q[9], q[10], q[11]);
    r.q.w = pack_bytes(q[12], q[13], q[14], q[15]);
  }
  r.k = 0; r.z = 0;
  return r;
}

template <int V>
TACO_DEV float int8_sym_stat(const float* a) { return group_max<64 / V>(absmax_v<V>(a)); }

template <int V>
TACO_DEV LaneCodes quant_int8_sym(const float* a, float* pre) {
  float s, inv;
  if constexpr (64 / V == 4 || 64 / V == 8) block_scales_split<127, 64 / V>(int8_sym_stat<V>(a), s, inv);
  else block_scales<127>(int8_sym_stat<V>(a), s, inv);
  return int8_sym_encode<V>(a, s, inv, pre);
}

// Asymmetric min/max over a group of 128, BITS = 4 or 8: lo = min(min a, 0),
// hi = max(max a, 0); the statistic is the range hi - lo.
template <int V>
TACO_DEV float asym_stat(const float* a, float& lo) {
  constexpr int G = 128 / V;
  lo = fminf(group_min<G>(min_v<V>(a)), 0.0f);
  const float hi = fmaxf(group_max<G>(max_v<V>(a)), 0.0f);
  return hi - lo;
}

// z = clamp(round(-lo * inv)), q = clamp(round(a * inv) + z).
template <int BITS, int V>
TACO_DEV LaneCodes asym_encode(const float* a, float lo, float s, float inv, float* pre) {
  constexpr int QMAX = (1 << BITS) - 1;
  LaneCodes r;
  r.s = s;
  r.z = clampi(rne_int((-lo) * inv), 0, QMAX);
  r.q = make_uint4(0, 0, 0, 0);
  if constexpr (BITS == 8) {
    // rne(t) + z is an exact integer in float; v_cvt_pk_u8_f32 clamps it to
    // [0, 255] (it saturates, and rounds to nearest even, which leaves an
    // integer unchanged) and writes it into its byte of the word
    const float zf = (float)r.z;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float t = a[i] * inv;
      if (pre) pre[i] = t;
      w[i / 4] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(t) + zf, i % 4, w[i / 4]);
    }
    r.q = make_uint4(w[0], w[1], w[2], w[3]);
    r.k = 0;
    return r;
  }
  int q[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float t = a[i] * inv;
    if (pre) pre[i] = t;
    q[i] = clampi(rne_int(t) + r.z, 0, QMAX);
  }
  if constexpr (BITS == 4) {
    r.q.x = pack_nibbles(q);
    if constexpr (V == 16) r.q.y = pack_nibbles(q + 8);
  } else {
    r.q.x = pack_bytes(q[0], q[1], q[2], q[3]);
    r.q.y = pack_bytes(q[4], q[5], q[6], q[7]);
    if constexpr (V == 16) {
      r.q.z = pack_bytes(q[8], q[9], q[10], q[11]);
      r.q.w = pack_bytes(q[12], q[13], q[14], q[15]);
    }
  }
  r.k = 0;
  return r;
}

template <int BITS, int V>
TACO_DEV LaneCodes quant_asym(const float* a, float* pre) {
  float lo, s, inv;
  if constexpr (128 / V == 4 || 128 / V == 8) block_scales_split<(1 << BITS) - 1, 128 / V>(asym_stat<V>(a, lo), s, inv);
  else block_scales<(1 << BITS) - 1>(asym_stat<V>(a, lo), s, inv);
  return asym_encode<BITS, V>(a, lo, s, inv, pre);
}

template <int FMT, int B, int V = kLaneElems>
TACO_DEV LaneCodes quant_lane(float* a, float inv_g, float* pre) {
  if constexpr (is_fp8(FMT)) return quant_fp8<B, FMT == kFP8E5, V>(a, inv_g, pre);
  else if constexpr (FMT == kINT8S) return quant_int8_sym<V>(a, pre);
  else if constexpr (FMT == kINT4A) return quant_asym<4, V>(a, pre);
  else return quant_asym<8, V>(a, pre);
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
// V = 16 (codes in q.x .. q.w; INT4 in q.x, q.y) or V = 8 (q.x, q.y; INT4 q.x).
template <int FMT, int B, int V = kLaneElems>
TACO_DEV void dequant_lane(const LaneIn<FMT, B>& in, float* d) {
  const uint32_t w[4] = {in.q.x, in.q.y, in.q.z, in.q.w};
  if constexpr (is_fp8(FMT)) {
    using F = Fp8Code<FMT == kFP8E5>;
#pragma unroll
    for (int j = 0; j < V / 4; ++j) F::unpack4(w[j], d + 4 * j);
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = d[i] * in.s;
  } else if constexpr (FMT == kINT8S) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = sbyte(w[j], b) * in.s;
  } else if constexpr (FMT == kINT8A) {
    const float zf = (float)in.z;
#pragma unroll
    for (int j = 0; j < V / 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = (ubyte(w[j], b) - zf) * in.s;
  } else {
    // 128 - z in every byte (v_perm with selector 0 copies byte 0 of z into all four)
    const uint32_t zrep = 0x80808080u - __builtin_amdgcn_perm(in.z, in.z, 0u);
#pragma unroll
    for (int j = 0; j < V / 8; ++j) {
      const uint32_t even = ((w[j] & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;          // elements 0, 2, 4, 6
      const uint32_t odd = (((w[j] >> 4) & 0x0F0F0F0Fu) + zrep) ^ 0x80808080u;    // elements 1, 3, 5, 7
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        d[8 * j + 2 * b] = sbyte(even, b) * in.s;
        d[8 * j + 2 * b + 1] = sbyte(odd, b) * in.s;
      }
    }
  }
}

// INT4 asymmetric, the reduce's form: the same values as dequant_lane, in
// half the instructions. Two codes share one dword as 16-bit halves holding
// c = q + 16 - z in [1, 31] (no half borrows from or carries into the other);
// read as a half-precision subnormal, a half is c * 2^-24 (or, for the codes
// left in bits 4-8 of their half, 16 c * 2^-24) exactly, and one mixed-
// precision fused multiply-add per value forms (q - z) * s = c * s - 16 s
// with a single rounding: c * 2^-24 * (s * 2^24) is the exact product and
// 16 s is exact. Valid when every zero point is at most 15 (what the
// compressor writes, and a stated precondition for buffers read back) and
// |s| < 2^100 (s * 2^24 finite); int4_fast_ok tells the latter.
TACO_DEV float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
TACO_DEV float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

template <int B>
TACO_DEV bool int4_fast_ok(const LaneIn<kINT4A, B>& in) {
  return fabsf(in.s) < 0x1p100f;
}

template <int B>
TACO_DEV void dequant_int4_fast(const LaneIn<kINT4A, B>& in, float* d) {
  const uint32_t zr = 0x00100010u - in.z * 0x00010001u;   // 16 - z in each half
  const uint32_t zr16 = zr << 4;
  const float s24 = in.s * 0x1p24f, s20 = in.s * 0x1p20f, m16 = in.s * -16.0f;
  const uint32_t w[2] = {in.q.x, in.q.y};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t a = (w[j] & 0x000F000Fu) + zr;            // elements 0 and 4 of the dword
    const uint32_t b = (w[j] & 0x00F000F0u) + zr16;          // 1 and 5, times 16
    const uint32_t c = ((w[j] >> 8) & 0x000F000Fu) + zr;     // 2 and 6
    const uint32_t e = ((w[j] >> 8) & 0x00F000F0u) + zr16;   // 3 and 7, times 16
    float* o = d + 8 * j;
    o[0] = fmaf(half_lo(a), s24, m16); o[4] = fmaf(half_hi(a), s24, m16);
    o[1] = fmaf(half_lo(b), s20, m16); o[5] = fmaf(half_hi(b), s20, m16);
    o[2] = fmaf(half_lo(c), s24, m16); o[6] = fmaf(half_hi(c), s24, m16);
    o[3] = fmaf(half_lo(e), s20, m16); o[7] = fmaf(half_hi(e), s20, m16);
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
  ReorderArgs ro;
};

// Store one lane's codes (streaming stores, as for the buffer stores); the
// first lane of each block stores the metadata.

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

// Quantization of the two halves of a wave tile (lane layout of k_quantize):
// the integer formats share one division per scale between the halves.
template <int FMT, int B>
TACO_DEV void quant_halves(float (*v)[8], float inv_g, float (*pre)[8], LaneCodes* r) {
  constexpr int V = 8;
  if constexpr (FMT == kINT8S) {
    static_assert(64 / V >= 8, "a block spans the mirror pairs of block_scales_pair");
    float s[2], inv[2];
    block_scales_pair<127>(int8_sym_stat<V>(v[0]), int8_sym_stat<V>(v[1]), s, inv);
#pragma unroll
    for (int h = 0; h < 2; ++h) r[h] = int8_sym_encode<V>(v[h], s[h], inv[h], pre ? pre[h] : nullptr);
  } else if constexpr (FMT == kINT4A || FMT == kINT8A) {
    static_assert(128 / V >= 8, "a block spans the mirror pairs of block_scales_pair");
    constexpr int BITS = FMT == kINT4A ? 4 : 8;
    float lo[2], s[2], inv[2];
    const float m0 = asym_stat<V>(v[0], lo[0]);
    const float m1 = asym_stat<V>(v[1], lo[1]);
    block_scales_pair<(1 << BITS) - 1>(m0, m1, s, inv);
#pragma unroll
    for (int h = 0; h < 2; ++h) r[h] = asym_encode<BITS, V>(v[h], lo[h], s[h], inv[h], pre ? pre[h] : nullptr);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) r[h] = quant_lane<FMT, B, V>(v[h], inv_g, pre ? pre[h] : nullptr);
  }
}

// Quantization without a transform. Each wave tile of 1024 elements is two
// halves of 512, and a lane holds 8 consecutive elements of each half, so
// every load instruction of a wave reads one contiguous run (1 KiB of bf16;
// measured 7 % faster than 16 consecutive elements per lane, whose two loads
// each touch every other 16 bytes). A block of B elements spans B / 8 lanes of
// one half. Each tile's accesses go through buffer resources clipped at the
// tensor's end (a ragged tail loads zeros and its stores are dropped). The
// launch gives every wave one tile and relies on full occupancy for the loads
// in flight; the loop only matters for grids smaller than that.
template <int FMT, int B, bool F32IN, bool DEBUG, bool REORD = false>
__global__ __launch_bounds__(kBlockThreads) void k_quantize(QuantK a) {
  static_assert(!(REORD && (F32IN || DEBUG)), "the reordering compress takes bf16 input");
  extern __shared__ __attribute__((aligned(16))) int16_t lds_order[];
  if constexpr (REORD) load_order_lds(a.ro, lds_order);
  constexpr int V = 8;                      // elements per lane and half
  constexpr int HALF = kWaveElems / 2;      // 512
  constexpr int ES = F32IN ? 4 : 2;         // input bytes per element
  constexpr int NQ = V * ES / 16;           // 16-byte loads per lane and half
  constexpr int G = B / V;                  // lanes per block
  constexpr int BPH = HALF / B;             // blocks per half
  constexpr int CB = FMT == kINT4A ? 2 : 1; // elements per code byte
  constexpr int MB = is_fp8(FMT) ? 1 : 4;   // bytes per block scale
  constexpr bool ASYM = FMT == kINT4A || FMT == kINT8A;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ntiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  // elements of the last (possibly partial) tile; a multiple of B, so each
  // lane's run lies wholly inside or outside the tensor
  const int tail = (int)(a.n - (ntiles - 1) * kWaveElems);
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
  // quantize and store tile `base` (rt elements) from its loaded lanes
  auto finish = [&](int64_t base, int rt, uint4 (&raw)[2][NQ]) {
    float v[2][V];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (F32IN) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          v[h][4 * q + 0] = __uint_as_float(raw[h][q].x); v[h][4 * q + 1] = __uint_as_float(raw[h][q].y);
          v[h][4 * q + 2] = __uint_as_float(raw[h][q].z); v[h][4 * q + 3] = __uint_as_float(raw[h][q].w);
        }
      } else {
        const uint4 w = raw[h][0];
        v[h][0] = bf16_lo(w.x); v[h][1] = bf16_hi(w.x); v[h][2] = bf16_lo(w.y); v[h][3] = bf16_hi(w.y);
        v[h][4] = bf16_lo(w.z); v[h][5] = bf16_hi(w.z); v[h][6] = bf16_lo(w.w); v[h][7] = bf16_hi(w.w);
      }
      if constexpr (is_fp8(FMT)) run_max = fmaxf(run_max, absmax_v<V>(v[h]));
    }
    float pre[2][V];
    LaneCodes r[2];
    quant_halves<FMT, B>(v, inv_g, DEBUG ? pre : nullptr, r);
    const rsrc_t rc = make_rsrc32(a.codes + base / CB, rt / CB);
    const rsrc_t rs = make_rsrc32(static_cast<uint8_t*>(a.scale) + (base / B) * MB, (rt / B) * MB);
    const rsrc_t rz = make_rsrc32(ASYM ? a.zero + base / B : a.codes, ASYM ? rt / B : 0);
    const int blk = lane / G;   // every lane of a block stores the same metadata
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (FMT == kINT4A) bstore32(r[h].q.x, rc, lane * (V / 2), h * HALF / 2);
      else bstore64(make_uint2(r[h].q.x, r[h].q.y), rc, lane * V, h * HALF);
      if constexpr (is_fp8(FMT)) {
        bstore8((uint32_t)r[h].k, rs, blk, h * BPH);
      } else {
        bstore32(__float_as_uint(r[h].s), rs, 4 * blk, 4 * h * BPH);
        if constexpr (ASYM) bstore8((uint32_t)r[h].z, rz, blk, h * BPH);
      }
      if constexpr (DEBUG) {
        const rsrc_t rd = make_rsrc32(a.dbg + base, rt * 4);
#pragma unroll
        for (int q = 0; q < V / 4; ++q)
          bstore128(make_uint4(__float_as_uint(pre[h][4 * q]), __float_as_uint(pre[h][4 * q + 1]),
                               __float_as_uint(pre[h][4 * q + 2]), __float_as_uint(pre[h][4 * q + 3])),
                    rd, lane * V * 4 + 16 * q, h * HALF * 4);
      }
    }
  };
  bool done = false;
  if constexpr (REORD) {
    if (a.ro.staged) {
      // rows through LDS in units of stage_rows rows (whole 1024-element
      // tiles, at most kStageMaxElems elements): a unit is loaded
      // contiguously, then each lane reads group order[j] of its span's row
      // from LDS; the unit's tiles are the tensor's tiles. The next unit's
      // loads are issued into registers before this unit's tiles are
      // quantized, so they are in flight during the arithmetic.
      uint16_t* rows_lds = reinterpret_cast<uint16_t*>(lds_order) + reorder_stage_offset(a.ro);
      const int cols = a.ro.cols;
      const auto* x = static_cast<const uint16_t*>(a.x);
      const StageUnits su(a.n, cols, a.ro.stage_rows);
      uint4 next[8];
      stage_issue(x, su, blockIdx.x, next);
      for (int64_t u = blockIdx.x; u < su.count; u += gridDim.x) {
        const int64_t pbase = su.base(u);
        const int pelems = su.elems(u);
        stage_commit(next, reinterpret_cast<uint4*>(rows_lds), pelems);
        __syncthreads();
        stage_issue(x, su, u + gridDim.x, next);
        for (int lt = wave_in_group(); lt * kWaveElems < pelems; lt += kBlockThreads / kWave) {
          const int64_t base = pbase + (int64_t)lt * kWaveElems;
          const int rt = a.n - base < kWaveElems ? (int)(a.n - base) : kWaveElems;
          uint4 raw[2][NQ];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int e0 = lt * kWaveElems + h * HALF;   // span start inside the unit
            const bool live = e0 < pelems;
            const int lrow = e0 / cols, col0 = e0 - lrow * cols;   // row inside the unit
            const int src = live ? lds_order[(col0 >> 3) + lane] : 0;
            raw[h][0] = live ? *reinterpret_cast<const uint4*>(rows_lds + lrow * cols + src * kGroupElems)
                             : make_uint4(0, 0, 0, 0);
          }
          finish(base, rt, raw);
        }
        __syncthreads();   // the unit's LDS rows are read before the next unit's are written
      }
      done = true;
    }
  }
  for (int64_t t = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); !done && t < ntiles; t += stride) {
    const int64_t base = t * kWaveElems;
    const int rt = t == ntiles - 1 ? tail : kWaveElems;   // elements of this tile
    const rsrc_t rx = make_rsrc32(static_cast<const uint8_t*>(a.x) + base * ES, rt * ES);
    uint4 raw[2][NQ];
    if constexpr (REORD) {
      // each half is one 512-element span of a row; the lane holding group j
      // of it loads group order[j] of that row
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // the second half of a ragged last tile lies past the end: empty
        // resource, no lookup
        const int64_t e0 = base + h * HALF;
        const bool live = e0 < a.n;
        const SpanPos p = live ? span_pos(a.ro, e0) : SpanPos{0u, 0u};
        const rsrc_t rr = make_rsrc32(static_cast<const uint16_t*>(a.x) + (int64_t)p.row * a.ro.cols,
                                      live ? a.ro.cols * 2 : 0);
        raw[h][0] = bload128<kNT>(rr, live ? reordered_group(lds_order, p, lane) * kGroupElems * 2 : 0, 0);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < NQ; ++q) raw[h][q] = bload128<kNT>(rx, lane * V * ES + 16 * q, h * HALF * ES);
    }
    finish(base, rt, raw);
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
  constexpr int ES = F32IN ? 4 : 2;
  constexpr int NQ = kLaneElems * ES / 16;   // 16-byte loads per lane; load q reads bytes [1024 q, 1024 q + 1024)
  float m = 0.0f;
  for (int64_t t = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); t < ntiles; t += stride) {
    const int64_t base = t * kWaveElems;
    const rsrc_t rx = make_rsrc(static_cast<const uint8_t*>(x) + base * ES, (n - base) * ES);
    float v[16];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint4 w = bload128<kNT>(rx, lane * 16, q * 1024);
      if constexpr (F32IN) {
        v[4 * q + 0] = __uint_as_float(w.x); v[4 * q + 1] = __uint_as_float(w.y);
        v[4 * q + 2] = __uint_as_float(w.z); v[4 * q + 3] = __uint_as_float(w.w);
      } else {
        v[8 * q + 0] = bf16_lo(w.x); v[8 * q + 1] = bf16_hi(w.x); v[8 * q + 2] = bf16_lo(w.y);
        v[8 * q + 3] = bf16_hi(w.y); v[8 * q + 4] = bf16_lo(w.z); v[8 * q + 5] = bf16_hi(w.z);
        v[8 * q + 6] = bf16_lo(w.w); v[8 * q + 7] = bf16_hi(w.w);
      }
    }
    m = fmaxf(m, absmax_v<16>(v));   // a ragged tail loads zeros
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
  ReorderArgs ro;
};

// Decode to float32 or bf16: 1024-element tiles in the two-half lane layout of
// k_quantize (8 consecutive elements of each half per lane), one per wave as
// launched (a smaller grid walks them with a stride of the grid). The output
// uses ordinary stores: the consumer reads it next.
template <int FMT, int B, bool BF16OUT, bool REORD = false>
__global__ __launch_bounds__(kBlockThreads) void k_dequantize(DequantK a) {
  extern __shared__ __attribute__((aligned(16))) int16_t lds_order[];
  if constexpr (REORD) load_order_lds(a.ro, lds_order);
  constexpr int V = 8;
  constexpr int HALF = kWaveElems / 2;
  constexpr int G = B / V, BPH = HALF / B;
  constexpr int CB = FMT == kINT4A ? 2 : 1;
  constexpr int MB = is_fp8(FMT) ? 1 : 4;
  constexpr bool ASYM = FMT == kINT4A || FMT == kINT8A;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t ntiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  float g = 0.0f;
  if constexpr (is_fp8(FMT)) g = *a.g_hdr;
  constexpr int OB = BF16OUT ? 2 : 4;   // output bytes per element
  // the lane's codes, scale and zero point of half h of tile `base` (rt elements)
  auto load_in = [&](int64_t base, int rt, int h) {
    const rsrc_t rc = make_rsrc32(a.codes + base / CB, rt / CB);
    const rsrc_t rs = make_rsrc32(static_cast<const uint8_t*>(a.scale) + (base / B) * MB, (rt / B) * MB);
    const rsrc_t rz = make_rsrc32(ASYM ? a.zero + base / B : a.codes, ASYM ? rt / B : 0);
    LaneIn<FMT, B> in;
    if constexpr (FMT == kINT4A) in.q = make_uint4(bload32(rc, lane * 4, h * HALF / 2), 0, 0, 0);
    else {
      const uint2 c = bload64<kNT>(rc, lane * 8, h * HALF);
      in.q = make_uint4(c.x, c.y, 0, 0);
    }
    in.z = 0;
    in.sh = 0;
    if constexpr (is_fp8(FMT)) {
      const int k = (int)(int8_t)(uint8_t)bload8(rs, lane / G, h * BPH);
      in.s = g * pow2f(-k);
    } else {
      in.s = __uint_as_float(bload32(rs, 4 * (lane / G), 4 * h * BPH));
      if constexpr (ASYM) in.z = bload8(rz, lane / G, h * BPH);
    }
    return in;
  };
  // the lane's 8 decoded values of half h of tile `base`
  auto decode = [&](int64_t base, int rt, int h, float* d) { dequant_lane<FMT, B, V>(load_in(base, rt, h), d); };
  // the output bytes of 8 values: one 16-byte word (bf16) or two (float32)
  auto out_words = [&](const float* d, uint4* w) {
    if constexpr (BF16OUT) {
      w[0] = make_uint4(f32_to_bf16(d[0]) | (f32_to_bf16(d[1]) << 16), f32_to_bf16(d[2]) | (f32_to_bf16(d[3]) << 16),
                        f32_to_bf16(d[4]) | (f32_to_bf16(d[5]) << 16), f32_to_bf16(d[6]) | (f32_to_bf16(d[7]) << 16));
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        w[q] = make_uint4(__float_as_uint(d[4 * q]), __float_as_uint(d[4 * q + 1]), __float_as_uint(d[4 * q + 2]),
                          __float_as_uint(d[4 * q + 3]));
    }
  };
  constexpr int NW = BF16OUT ? 1 : 2;
  if constexpr (REORD) {
    if (a.ro.staged) {
      // rows in units of stage_rows rows (at most kStageMaxElems elements):
      // a unit's codes are copied into LDS contiguously; the lane that writes
      // output group g of a 512-element span reads the codes of reordered
      // group inv[g] of the same row from LDS (inv, the inverse of the order,
      // is built in LDS) and its block's scale (and zero point) from global
      // memory, and the wave stores the span's decoded values contiguously.
      // A wave issues all of its spans' loads of a unit before decoding any,
      // and the next unit's codes are loaded into registers while this one is
      // decoded.
      constexpr int WG = kBlockThreads / kWave;
      constexpr int CW = kStageMaxElems / CB / 16 / kBlockThreads;   // 16-byte code words per thread and unit
      constexpr int TB = 4;                                          // spans per batch
      int16_t* inv = lds_order + reorder_stage_offset(a.ro);
      uint4* codes_lds = reinterpret_cast<uint4*>(inv + reorder_stage_offset(a.ro));
      const int cols = a.ro.cols, ng = a.ro.ngroups;
      // identity first, so that an order that is not a permutation leaves no
      // entry unset (its output is unspecified, its accesses stay in the row)
      for (int i = (int)threadIdx.x; i < ng; i += kBlockThreads) inv[i] = (int16_t)i;
      __syncthreads();
      for (int i = (int)threadIdx.x; i < ng; i += kBlockThreads) inv[lds_order[i]] = (int16_t)i;
      const StageUnits su(a.n, cols, a.ro.stage_rows);
      uint4 next[CW];
      auto issue = [&](int64_t u) {   // past the last unit: an empty resource, zeros
        const rsrc_t r = make_rsrc32(a.codes + (u < su.count ? su.base(u) / CB : 0), su.elems(u) / CB);
#pragma unroll
        for (int j = 0; j < CW; ++j) next[j] = bload128<kNT>(r, 16 * ((int)threadIdx.x + j * kBlockThreads), 0);
      };
      issue(blockIdx.x);
      for (int64_t u = blockIdx.x; u < su.count; u += gridDim.x) {
        const int64_t ubase = su.base(u);
        const int uelems = su.elems(u);
#pragma unroll
        for (int j = 0; j < CW; ++j) {
          const int w = (int)threadIdx.x + j * kBlockThreads;
          if (w < uelems / CB / 16) codes_lds[w] = next[j];
        }
        __syncthreads();
        issue(u + gridDim.x);
        const rsrc_t rs = make_rsrc32(static_cast<const uint8_t*>(a.scale) + (ubase / B) * MB, (uelems / B) * MB);
        const rsrc_t rz = make_rsrc32(ASYM ? a.zero + ubase / B : a.codes, ASYM ? uelems / B : 0);
        const rsrc_t rout = make_rsrc32(static_cast<uint8_t*>(a.out) + ubase * OB, uelems * OB);
        const uint8_t* cb = reinterpret_cast<const uint8_t*>(codes_lds);
        // batches of four consecutive spans, batch b to wave b % 4, the
        // batch's loads first; a span past the unit's end reads the last span
        // again and its stores fall outside the output resource (dropped): no
        // branch, so the compiler keeps every load ahead of the arithmetic
        for (int bt = wave_in_group(); bt * TB * HALF < uelems; bt += WG) {
          LaneIn<FMT, B> in[TB];
#pragma unroll
          for (int i = 0; i < TB; ++i) {
            const int e0 = min((bt * TB + i) * HALF, uelems - HALF);   // span start inside the unit
            const int lrow = e0 / cols, col0 = e0 - lrow * cols;       // row inside the unit
            const int er = lrow * cols + 8 * inv[(col0 >> 3) + lane];  // the source group's first element
            in[i].q = make_uint4(0, 0, 0, 0);
            if constexpr (FMT == kINT4A) in[i].q.x = *reinterpret_cast<const uint32_t*>(cb + er / 2);
            else {
              const uint2 c = *reinterpret_cast<const uint2*>(cb + er);
              in[i].q.x = c.x;
              in[i].q.y = c.y;
            }
            in[i].z = 0;
            in[i].sh = 0;
            if constexpr (is_fp8(FMT)) {
              in[i].z = bload8(rs, er / B, 0);
            } else {
              in[i].s = __uint_as_float(bload32(rs, 4 * (er / B), 0));
              if constexpr (ASYM) in[i].z = bload8(rz, er / B, 0);
            }
          }
#pragma unroll
          for (int i = 0; i < TB; ++i) {
            if constexpr (is_fp8(FMT)) in[i].s = g * pow2f(-(int)(int8_t)(uint8_t)in[i].z);
            float d[V];
            dequant_lane<FMT, B, V>(in[i], d);
            uint4 w[NW];
            out_words(d, w);
            const int e0 = (bt * TB + i) * HALF;
#pragma unroll
            for (int q = 0; q < NW; ++q) bstore128<0>(w[q], rout, (e0 + lane * V) * OB + 16 * q, 0);
          }
        }
        __syncthreads();   // the unit's codes are read before the next unit's are written
      }
      return;
    }
  }
  for (int64_t t = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); t < ntiles; t += stride) {
    const int64_t base = t * kWaveElems;
    const int rt = t == ntiles - 1 ? (int)(a.n - base) : kWaveElems;   // a multiple of B
    const rsrc_t rout = make_rsrc32(static_cast<uint8_t*>(a.out) + base * OB, rt * OB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float d[V];
      decode(base, rt, h, d);
      // output resource and this lane's offset in it: the tile, or (reordered)
      // the row of this half's span, where group j goes back to group order[j]
      rsrc_t rdst = rout;
      int doff = lane * V * OB, dsoff = h * HALF * OB;
      if constexpr (REORD) {
        const int64_t e0 = base + h * HALF;
        const bool live = e0 < a.n;   // else: the empty half of a ragged last tile
        const SpanPos p = live ? span_pos(a.ro, e0) : SpanPos{0u, 0u};
        rdst = make_rsrc32(static_cast<uint8_t*>(a.out) + ((int64_t)p.row * a.ro.cols) * OB, live ? a.ro.cols * OB : 0);
        doff = live ? reordered_group(lds_order, p, lane) * kGroupElems * OB : 0;
        dsoff = 0;
      }
      uint4 w[NW];
      out_words(d, w);
#pragma unroll
      for (int q = 0; q < NW; ++q) bstore128<0>(w[q], rdst, doff + 16 * q, dsoff);
    }
  }
}

// Decompress N shards, sum in float32 in shard order, then optionally store
// the sum and/or re-quantize it (FP8: g' = g_0 + ... + g_{N-1}, clamped).
//
// Grid-stride over 1024-element wave tiles (launched with one tile per wave,
// so the loop runs once unless the grid is smaller). A wave walks a flat sequence
// of steps -- (tile, group of up to four shards), the groups of a tile in
// shard order -- with two register sets used alternately: the loads of the
// next step are issued before the current step is dequantized and added, so
// one step's loads are always in flight. All NMAX shard slots are read
// through buffer resources; slots r >= N get an empty resource, load zeros and
// add an exact +0 (acc is never -0), so the instruction stream is the same for
// every N <= NMAX. Steps past the last tile load nothing (their offsets lie
// outside every resource). A launch covers at most kReducePiece elements (the
// host splits larger tensors), so every byte offset fits 32 bits.
// Each shard's resources are rebased to the tile a step reads (scalar
// arithmetic), so every lane's offsets are the same for every tile and step:
// the codes, the block scales or exponents, and (asymmetric formats) the zero
// points, each clipped at the tensor's end.
template <int FMT, int B>
struct ShardRsrc {
  rsrc_t codes, meta, zero;
};

// Byte offsets of a lane's codes and block metadata inside its tile.
// FP8 exponents are read as the aligned dword that holds the lane's byte
// (byte loads let the compiler sink them past the scheduling barrier); a
// tile's first block index is a multiple of 8, so the rebased dwords stay
// aligned.
template <int FMT, int B>
struct LaneOffs {
  int code, meta, zero, sh;
  TACO_DEV explicit LaneOffs(int lane) {
    const int blk = lane * kLaneElems / B;
    code = FMT == kINT4A ? lane * (kLaneElems / 2) : lane * kLaneElems;
    meta = is_fp8(FMT) ? (blk & ~3) : 4 * blk;
    sh = is_fp8(FMT) ? 8 * (blk & 3) : 0;
    zero = blk;
  }
  // The offsets of the same lane inside the whole tensor, for tile t.
  TACO_DEV LaneOffs at_tile(int t) const {
    const unsigned e = (unsigned)t * kWaveElems, blk0 = e / B;
    LaneOffs r = *this;
    r.code += (int)(FMT == kINT4A ? e / 2 : e);
    r.meta += (int)(is_fp8(FMT) ? blk0 : 4 * blk0);
    r.zero += (int)blk0;
    return r;
  }
};

// n <= kReducePiece, and t is at most one grid stride past the last tile, so
// every size below is under 2^31. A slot r >= nshards, or a tile at or past
// the end, gets empty resources (its loads return zeros).
template <int FMT, int B>
TACO_DEV ShardRsrc<FMT, B> shard_rsrc(const ReduceArgs& a, int r, int n, int t) {
  constexpr bool ASYM = FMT == kINT4A || FMT == kINT8A;
  const unsigned e = (unsigned)t * kWaveElems;                             // the tile's first element
  const unsigned rem = (r < a.nshards && e < (unsigned)n) ? (unsigned)n - e : 0u;
  const unsigned blk0 = e / B, nbr = rem / B;
  const uint8_t* scale = static_cast<const uint8_t*>(a.in.scale[r]);
  ShardRsrc<FMT, B> s;
  s.codes = make_rsrc32(a.in.codes[r] + (FMT == kINT4A ? e / 2 : e), (int)(FMT == kINT4A ? rem / 2 : rem));
  if constexpr (is_fp8(FMT)) s.meta = make_rsrc32(scale + blk0, (int)((nbr + 3) & ~3u));
  else s.meta = make_rsrc32(scale + 4 * blk0, (int)(4 * nbr));
  s.zero = make_rsrc32(ASYM ? a.in.zero[r] + blk0 : a.in.codes[r], ASYM ? (int)nbr : 0);
  return s;
}

// One lane's codes and block metadata of one shard. FP8 leaves the exponent
// dword in z and its bit offset in sh: the scale is formed when the lane is
// added, so nothing here waits for the loads.
template <int FMT, int B>
TACO_DEV LaneIn<FMT, B> load_in_buf(const ShardRsrc<FMT, B>& s, const LaneOffs<FMT, B>& o) {
  LaneIn<FMT, B> r;
  if constexpr (FMT == kINT4A) {
    uint2 w = bload64<kNT>(s.codes, o.code, 0);
    r.q = make_uint4(w.x, w.y, 0, 0);
  } else {
    r.q = bload128<kNT>(s.codes, o.code, 0);
  }
  r.z = 0;
  r.sh = 0;
  r.s = 0.0f;
  if constexpr (is_fp8(FMT)) {
    r.z = bload32(s.meta, o.meta, 0);
    r.sh = o.sh;
  } else {
    r.s = __uint_as_float(bload32(s.meta, o.meta, 0));
    if constexpr (FMT == kINT4A || FMT == kINT8A) r.z = bload8(s.zero, o.zero, 0);
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

  // Issue the loads of shard group `grp` of tile t (FP8: the scale is formed
  // when the step is added).
  // With more than two groups the compiler would hoist every shard's
  // resources out of the loop and spill them; an opaque group index keeps
  // each step building only its own group's, rebased to the tile, so the
  // lane offsets need no per-step arithmetic (the instruction-bound
  // asymmetric inputs gain 5 %). With two groups the resources of all NMAX
  // shards cover the whole tensor and stay in scalar registers for the
  // whole loop, and a step adds the tile's offset to the lane's (two or three
  // adds): the loads then issue back to back, which the memory-bound FP8
  // reduce needs (rebuilding its resources per step measured 4-7 % slower).
  TACO_DEV void load(const ReduceArgs& a, int grp, int t, int n, const LaneOffs<FIN, BIN>& o) {
    if constexpr (NG > 2) {
      asm volatile("" : "+s"(grp));
#pragma unroll
      for (int u = 0; u < GRP; ++u)
        in[u] = load_in_buf<FIN, BIN>(shard_rsrc<FIN, BIN>(a, grp * GRP + u, n, t), o);
    } else {
      const LaneOffs<FIN, BIN> ot = o.at_tile(t);
#pragma unroll
      for (int u = 0; u < GRP; ++u)
        in[u] = load_in_buf<FIN, BIN>(shard_rsrc<FIN, BIN>(a, grp * GRP + u, n, 0), ot);
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
      if constexpr (FIN == kINT4A) {
        // the fast form when the whole wave qualifies (always, for shards the
        // compressor wrote); the first shard's values are the sum so far
        // (0 + d = d: the fast form never yields -0).
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!int4_fast_ok<BIN>(x)) == 0, 1)) {
          dequant_int4_fast<BIN>(x, d);
          if (grp == 0 && u == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = d[i];
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
          }
        } else {
          dequant_lane<FIN, BIN>(x, d);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            acc[i] = acc[i] + d[i];
            // keeps the compiler from merging the two branches' adds after
            // the branch, which would hold every step's values at once
            asm volatile("" : "+v"(acc[i]));
          }
        }
      } else {
        dequant_lane<FIN, BIN>(x, d);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = acc[i] + d[i];
      }
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
  // whole-tensor output resources (kept in scalar registers for the whole
  // loop; out-of-range lanes are dropped)
  const int nb_out = n / BOUT;
  const rsrc_t r_sum = make_rsrc32(a.sum, a.sum ? 4 * n : 0);
  const rsrc_t r_qc = make_rsrc32(a.rq_codes, rq ? n : 0);
  const rsrc_t r_qs = make_rsrc32(a.rq_scale, rq ? (is_fp8(FOUT) ? nb_out : 4 * nb_out) : 0);
  const rsrc_t r_qz = make_rsrc32(a.rq_zero, rq && FOUT == kINT8A ? nb_out : 0);

  // the finished sum of tile t: store it and/or re-quantize it
  auto finish = [&](int t, float* acc) {
    const unsigned e = (unsigned)t * kWaveElems;   // the tile's first element
    if (a.sum != nullptr) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bstore128(make_uint4(__float_as_uint(acc[4 * q]), __float_as_uint(acc[4 * q + 1]),
                             __float_as_uint(acc[4 * q + 2]), __float_as_uint(acc[4 * q + 3])),
                  r_sum, (int)(4 * e) + lane * (4 * kLaneElems) + 16 * q, 0);
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
      const int blk = (int)(e / BOUT) + lane * kLaneElems / BOUT;
      bstore128(q.q, r_qc, (int)e + lane * kLaneElems, 0);
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
  int t = (int)xcd_ordered_block() * (kBlockThreads / kWave) + wave_in_group();
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  RG buf[2];
  const LaneOffs<FIN, BIN> offs(lane);
  buf[0].load(a, 0, t, n, offs);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (is_fp8(FIN)) glane = *gp;   // lanes >= nshards: shard 0's g, read by no live step
  for (; t < ntiles; t += stride) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int tn = k + 1 < NG ? t : t + stride;   // tile and group of step k + 1
      const int gn = (k + 1) % NG;
      buf[(k + 1) & 1].load(a, gn, tn, n, offs);
      __builtin_amdgcn_sched_barrier(0);
      buf[k & 1].add_to(acc, k, glane);
    }
    finish(t, acc);
  }
}

// One hop of a quantized ring reduce-scatter: acc = (0 + dequant(incoming)) +
// local, one float32 rounding per add, then the FP32 sum and/or the partial sum
// quantized for the next hop. Grid-stride over 1024-element wave tiles, one
// tile per wave as launched, 16 consecutive values per lane (the two-half
// layout of k_quantize measured 8 % slower here: twice the code and scale
// instructions on the incoming and outgoing sides).
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
  return capped_grid((tiles + 3) / 4);
}

// One wave per tile and as many workgroups as that takes: the hardware keeps
// every CU at full occupancy as waves retire (5-8 % faster than a grid capped
// at 4 workgroups per CU on the INT8 and INT4 compress; two or four tiles per
// wave with all their loads issued first measured 2-7 % slower).
static dim3 quant_grid(const QuantArgs& a) { return grid_for(a.n); }

static size_t order_lds_bytes(const ReorderArgs& ro) { return ro.order ? ((size_t)ro.ngroups * 2 + 3) & ~size_t(3) : 0; }

// Staged reorder: the order and one unit of stage_rows rows of `elem_bytes`
// per element; the units of a tensor.
static size_t staged_lds_bytes(const ReorderArgs& ro, int elem_bytes) {
  return (size_t)reorder_stage_offset(ro) * 2 + (size_t)ro.stage_rows * ro.cols * elem_bytes;
}
static int64_t staged_units(int64_t n, const ReorderArgs& ro) { return (n / ro.cols + ro.stage_rows - 1) / ro.stage_rows; }

template <int FMT, int B>
static void launch_q(const QuantArgs& a, const QuantK& k, hipStream_t s) {
  dim3 grid = quant_grid(a), block(kBlockThreads);
  if constexpr (!is_fp8(FMT) || B == 128) {
    if (a.ro.order != nullptr) {   // bf16 input, no debug output (checked by the caller)
      QuantK ks = k;
      ks.ro.stage_rows = stage_rows_for(a.ro.cols, kWaveElems);
      ks.ro.staged = ks.ro.stage_rows > 0;
      if (ks.ro.staged) {
        auto* kern = k_quantize<FMT, B, false, false, true>;
        const size_t lds = staged_lds_bytes(ks.ro, 2);
        hipLaunchKernelGGL(kern, resident_grid(reinterpret_cast<const void*>(kern), lds, staged_units(a.n, ks.ro)),
                           block, lds, s, ks);
      } else
        hipLaunchKernelGGL((k_quantize<FMT, B, false, false, true>), grid, block, order_lds_bytes(a.ro), s, ks);
      return;
    }
  }
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
  if (a.ro.order != nullptr && (a.f32_in || a.dbg || (is_fp8(a.fmt) && a.block != 128))) return hipErrorInvalidValue;
  QuantK k{a.x, a.n, a.codes, a.scale, a.zero, a.g_hdr, a.g, a.g_from_ws ? 1 : 0,
           static_cast<Workspace*>(a.ws), a.dbg, a.ro};
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
  DequantK k{a.codes, a.scale, a.zero, a.g_hdr, a.n, a.out, a.ro};
  dim3 grid = grid_for(a.n), block(kBlockThreads);
  if constexpr (!is_fp8(FMT) || B == 128) {
    if (a.ro.order != nullptr) {
      // staged: the order, its inverse and one unit's codes in LDS
      k.ro.stage_rows = stage_rows_for(a.ro.cols, kSpanElems);
      k.ro.staged = k.ro.stage_rows > 0;
      const size_t lds = k.ro.staged ? (size_t)reorder_stage_offset(k.ro) * 4 +
                                           (size_t)k.ro.stage_rows * a.ro.cols / (FMT == kINT4A ? 2 : 1)
                                     : order_lds_bytes(a.ro);
      auto* kern = a.bf16_out ? k_dequantize<FMT, B, true, true> : k_dequantize<FMT, B, false, true>;
      if (k.ro.staged) grid = resident_grid(reinterpret_cast<const void*>(kern), lds, staged_units(a.n, k.ro));
      hipLaunchKernelGGL(kern, grid, block, lds, s, k);
      return;
    }
  }
  if (a.bf16_out) hipLaunchKernelGGL((k_dequantize<FMT, B, true>), grid, block, 0, s, k);
  else hipLaunchKernelGGL((k_dequantize<FMT, B, false>), grid, block, 0, s, k);
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.ro.order != nullptr && is_fp8(a.fmt) && a.block != 128) return hipErrorInvalidValue;
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

// Reduce grid: a workgroup per 4 * kReduceTilesPerWave tiles, dispatched by
// the hardware as CUs free up, which keeps every CU busy until the end. The
// asymmetric inputs, bound by instruction issue rather than memory, also run
// best this way (3-6 % faster than a persistent grid of 4 workgroups per CU,
// whose 16 waves per CU hid less latency than the 32 resident here).
template <int FIN, int BIN, int FOUT, int BOUT, int NMAX>
static void launch_r(const ReduceArgs& a, hipStream_t s) {
  const int64_t tiles = (a.n + kWaveElems - 1) / kWaveElems;
  const int64_t per_group = 4 * kReduceTilesPerWave;
  dim3 grid = capped_grid((tiles + per_group - 1) / per_group), block(kBlockThreads);
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
    for (int r = 0; r < a.nshards; ++r) {
      p.in.codes[r] = a.in.codes[r] + code_bytes(a.fin, e);
      p.in.scale[r] = static_cast<const uint8_t*>(a.in.scale[r]) + scale_bytes(a.fin, bi);
      p.in.zero[r] = a.in.zero[r] + bi;
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

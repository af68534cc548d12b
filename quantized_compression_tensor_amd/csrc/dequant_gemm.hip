// The consumer of a compressed activation: out[M, N] = decode(A)[M, K] * W^T,
// with the decode in the GEMM's prologue, so the decoded activation is never
// written to memory.
//
// Source: "Flash Communication: Reducing Tensor Parallelization Bottleneck for
// Fast Large Language Model Inference" (Pith review page) -- "What carries
// the argument" and Fig. 8: the quantized volume is dequantized fast on the
// receiving side and handed to the next computation. The A operand is a
// compressed buffer without the Hadamard transform (INT8 or INT4 asymmetric
// group 128, INT8 symmetric block 64, dual-scale FP8 with block 32, 64 or
// 128); each value is decoded in registers, between the global load and the
// LDS store of the A tile, to the bf16 number taco_decompress writes for it
// (the nearest-even bf16 of the float32 decoded value, itself the single
// rounding of the exact value). W is a bf16
// weight in the layout of a linear layer, [N, K] row-major, so both operands
// are contiguous along K.
//
// Tiling: a workgroup computes a BM x BN tile of `out` with WGM x WGN waves,
// each wave a (BM / WGM) x (BN / WGN) part as 32 x 32 tiles of the
// 32 x 32 x 16 bf16 MFMA (float32 accumulate): 256 x 256 with 8 waves when
// M and N allow it (each A value is then decoded N / 256 times), else
// 128 x 128 with 4 waves. K is walked in steps of 64 through two LDS
// buffers, one barrier per step. Each step is cut into four slices of 16:
// a slice's MFMAs are interleaved (scheduling barriers) with a quarter of the
// decode of the next step into the other buffer, and its MFMA operands are
// read from LDS one slice ahead. Global loads run two steps ahead (two
// register sets), through buffer resources over the workgroup's rows with
// the K offset as a scalar.
#include "device_common.h"
#include "taco_internal.h"

namespace taco {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

template <int BM_, int BN_, int WGM_, int WGN_>
struct GemmTiles {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WGM = WGM_, WGN = WGN_;
  static constexpr int kThreads = kWave * WGM * WGN;
  static constexpr int kLd = BK + 8;            // bf16 per LDS row; the 8 extra shift each row's
                                                // start by 16 bytes, so the 32 rows an MFMA
                                                // operand read touches start in distinct banks
  static constexpr int kTM = BM / WGM / 32;     // 32 x 32 MFMA tiles per wave along M
  static constexpr int kTN = BN / WGN / 32;     // ... along N
  static constexpr int kAChunks = BM * BK / 16 / kThreads;   // 16-element A chunks per thread
  static constexpr int kBChunks = BN * BK / 8 / kThreads;    // 8-element W chunks per thread
  static constexpr int kSlices = BK / 16;
  static constexpr int kLdsBytes = 2 * (BM + BN) * kLd * 2;
  static_assert(BM % (WGM * 32) == 0 && BN % (WGN * 32) == 0, "wave tiles of whole MFMA tiles");
  static_assert(kAChunks * 16 * kThreads == BM * BK && kBChunks * 8 * kThreads == BN * BK, "whole chunks");
  static_assert((2 * kAChunks) % kSlices == 0 && kBChunks % kSlices == 0, "decode pieces per slice");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};
using TilesLarge = GemmTiles<256, 256, 2, 4>;
using TilesSmall = GemmTiles<128, 128, 2, 2>;
constexpr int kGemmGroupM = 8;        // tile rows walked together (L2 reuse of W)
constexpr int kValuPerMfma = 3;       // decode instructions placed after each MFMA

// sched_group_barrier masks
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008;

// Two floats -> two bf16 in one dword (the hardware conversion, nearest-even).
TACO_DEV uint32_t pk_bf16(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// One step's loads of one thread: kAChunks chunks of 16 consecutive A codes
// of one row with the block metadata that covers them (every supported block
// holds whole chunks), and kBChunks chunks of 8 consecutive W values.
template <class TL>
struct StepRegs {
  u32x4 qa[TL::kAChunks];      // codes (INT4: .x, .y)
  uint32_t sa[TL::kAChunks];   // INT: scale bits; FP8: the block exponent byte
  uint32_t za[TL::kAChunks];   // zero point (asymmetric)
  u32x4 qb[TL::kBChunks];      // bf16 W values
};

// Per-thread offsets of its chunks inside the workgroup's tile rows (fixed
// for the whole K loop; a step adds a wave-uniform offset).
template <class TL>
struct ChunkOffsets {
  int a[TL::kAChunks], s[TL::kAChunks], z[TL::kAChunks], lds_a[TL::kAChunks];
  int b[TL::kBChunks], lds_b[TL::kBChunks];
};

// Elements 8 h ... 8 h + 7 of a chunk, decoded as taco_decompress forms them
// in float32 (each the single rounding of the exact value), then bf16.
template <int FMT>
TACO_DEV u32x4 decode_half(u32x4 q, float s, uint32_t z, int h, float neg_zero) {
  float d[8];
  if constexpr (FMT == kINT4A) {
    // element 2i in the low nibble of byte i, 2i + 1 in the high nibble
    const uint32_t w = h ? q.y : q.x;
    const float zf = (float)z;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      d[2 * b] = ((float)((w >> (8 * b)) & 0xFu) - zf) * s;
      d[2 * b + 1] = ((float)((w >> (8 * b + 4)) & 0xFu) - zf) * s;
    }
  } else {
    const uint32_t w[2] = {h ? q.z : q.x, h ? q.w : q.y};
    if constexpr (is_fp8(FMT)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) Fp8Code<FMT == kFP8E5>::unpack4(w[j], d + 4 * j);
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = d[i] * s;
    } else if constexpr (FMT == kINT8S) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) d[4 * j + b] = (float)(int)(int8_t)(uint8_t)(w[j] >> (8 * b)) * s;
    } else {
      // (q - z) * s in three exact steps: the bytes become the f16 numbers
      // 1024 + q (0x64 as their high byte), one packed f16 add subtracts
      // 1024 + z (all integers below 2048: exact), and an fma with the
      // caller's -0.0 as addend forms the single rounding of (q - z) * s in
      // float32 (x * s + (-0) is x * s for every x, signed zeros included),
      // reading the f16 operand directly
      const _Float16 nz = (_Float16)(-(float)(1024u + z));
      const h2 off = {nz, nz};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w[j], 0x04010400u)) + off;
        const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, w[j], 0x04030402u)) + off;
        d[4 * j] = __builtin_fmaf((float)lo.x, s, neg_zero);
        d[4 * j + 1] = __builtin_fmaf((float)lo.y, s, neg_zero);
        d[4 * j + 2] = __builtin_fmaf((float)hi.x, s, neg_zero);
        d[4 * j + 3] = __builtin_fmaf((float)hi.y, s, neg_zero);
      }
    }
  }
  return u32x4{pk_bf16(d[0], d[1]), pk_bf16(d[2], d[3]), pk_bf16(d[4], d[5]), pk_bf16(d[6], d[7])};
}

// Output tile of this workgroup: tiles are renumbered so that each XCD walks
// one contiguous range, and inside it groups of kGemmGroupM tile rows are
// walked column by column, so the workgroups resident on one XCD share both
// A rows and W rows through its L2.
template <class TL>
TACO_DEV void gemm_tile(const DGemmArgs& a, int64_t* tm, int64_t* tn) {
  const int64_t ntm = a.M / TL::BM, ntn = a.N / TL::BN;
  const int64_t t = xcd_ordered_block();
  const int64_t per_group = (int64_t)kGemmGroupM * ntn;
  const int64_t group = t / per_group, in_group = t % per_group;
  const int64_t first = group * kGemmGroupM;
  const int64_t rows = ntm - first < kGemmGroupM ? ntm - first : kGemmGroupM;
  *tm = first + in_group % rows;
  *tn = in_group / rows;
}

template <int FMT, int B, bool BF16OUT, class TL>
__global__ __launch_bounds__(TL::kThreads) void k_dequant_gemm(DGemmArgs a) {
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, LD = TL::kLd, TM = TL::kTM, TN = TL::kTN;
  constexpr int NT = TL::kThreads, CA = TL::kAChunks, CB = TL::kBChunks, KK = TL::kSlices;
  constexpr int AH = 2 * CA / KK, WB = CB / KK;    // A half-chunks and W chunks per slice
  constexpr int APR = BK / 16, BPR = BK / 8;       // chunks per tile row (A, W)
  constexpr int CPB = FMT == kINT4A ? 2 : 1;       // elements per code byte
  constexpr int MB = is_fp8(FMT) ? 1 : 4;          // metadata bytes per block
  constexpr bool ASYM = FMT == kINT4A || FMT == kINT8A;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LD];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid) / kWave;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  int64_t tm, tn;
  gemm_tile<TL>(a, &tm, &tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int K = (int)a.K, KB = K / B;   // K <= 2^20: every tile-relative offset fits 31 bits
  const float g = is_fp8(FMT) ? *a.g_hdr : 1.0f;

  // buffer resources over this workgroup's BM rows of A (codes, scales, zero
  // points) and BN rows of W
  const rsrc_t rA = make_rsrc32(a.codes + m0 * K / CPB, BM * K / CPB);
  const rsrc_t rS = make_rsrc32(static_cast<const uint8_t*>(a.scale) + m0 * KB * MB, BM * KB * MB);
  const rsrc_t rZ = make_rsrc32(ASYM ? a.zero + m0 * KB : a.codes, ASYM ? BM * KB : 0);
  const rsrc_t rW = make_rsrc32(a.w + n0 * K, BN * K * 2);
  ChunkOffsets<TL> off;
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT, row = c / APR, col = (c % APR) * 16;
    off.a[i] = (row * K + col) / CPB;
    off.z[i] = row * KB + col / B;   // a K step starts a block or lies inside one: col / B is its part
    off.s[i] = off.z[i] * MB;
    off.lds_a[i] = row * LD + col;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT, row = c / BPR, col = (c % BPR) * 8;
    off.b[i] = (row * K + col) * 2;
    off.lds_b[i] = row * LD + col;
  }
  // first element of K step `ks`, clamped to the last step: the look-ahead
  // past the end re-reads it and the result is never used
  const int ksteps = K / BK;
  auto step_k = [&](int ks) { return (ks < ksteps ? ks : ksteps - 1) * BK; };
  auto load_a = [&](StepRegs<TL>& r, int i, int k) {
    if constexpr (FMT == kINT4A) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rA, off.a[i], k / 2, 0);
      r.qa[i] = u32x4{v.x, v.y, 0u, 0u};
    } else {
      r.qa[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off.a[i], k, 0);
    }
    if constexpr (is_fp8(FMT)) r.sa[i] = __builtin_amdgcn_raw_buffer_load_b8(rS, off.s[i], k / B, 0);
    else r.sa[i] = __builtin_amdgcn_raw_buffer_load_b32(rS, off.s[i], 4 * (k / B), 0);
    if constexpr (ASYM) r.za[i] = __builtin_amdgcn_raw_buffer_load_b8(rZ, off.z[i], k / B, 0);
    else r.za[i] = 0u;
  };
  auto load_b = [&](StepRegs<TL>& r, int i, int k) {
    r.qb[i] = __builtin_amdgcn_raw_buffer_load_b128(rW, off.b[i], 2 * k, 0);
  };
  auto load = [&](StepRegs<TL>& r, int ks) {
    const int k = step_k(ks);
#pragma unroll
    for (int i = 0; i < CA; ++i) load_a(r, i, k);
#pragma unroll
    for (int i = 0; i < CB; ++i) load_b(r, i, k);
  };
  auto scale_of = [&](uint32_t sa) {
    return is_fp8(FMT) ? g * pow2f(-(int)(int8_t)(uint8_t)sa) : __uint_as_float(sa);
  };
  auto store_half = [&](const StepRegs<TL>& r, int i, int h, int buf) {
    const u32x4 v = decode_half<FMT>(r.qa[i], scale_of(r.sa[i]), r.za[i], h, a.neg_zero);
    *reinterpret_cast<u32x4*>(&As[buf][off.lds_a[i] + 8 * h]) = v;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // MFMA operands: lane l holds row (A) or column (B) l % 32 and the eight K
  // entries 8 * (l / 32) ... of the sixteen one MFMA takes; A and B use the
  // same K assignment, so the sum over K is the same whatever order the
  // instruction gives those entries
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int arow = wm * (BM / TL::WGM) + fr, brow = wn * (BN / TL::WGN) + fr;
  auto read_frags = [&](int buf, int kk, bf16x8* af, bf16x8* bf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(arow + i * 32) * LD + kk * 16 + fk]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(brow + j * 32) * LD + kk * 16 + fk]);
  };
  // One K step on LDS buffer `buf`: per slice, its MFMAs, a share of the
  // decode of `next` (the registers of step ks + 1) into the other buffer,
  // and the refill of each consumed chunk with the loads of step ks + 3.
  auto body = [&](int buf, StepRegs<TL>& next, int ks) {
    const int knext = step_k(ks + 3);
    bf16x8 fa[2][TM], fb[2][TN];
    read_frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KK) read_frags(buf, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int p = 0; p < AH; ++p) {
        const int hh = kk * AH + p, i = hh / 2, h = hh % 2;
        store_half(next, i, h, buf ^ 1);
        if (h == 1) load_a(next, i, knext);
      }
#pragma unroll
      for (int p = 0; p < WB; ++p) {
        const int i = kk * WB + p;
        *reinterpret_cast<u32x4*>(&Bs[buf ^ 1][off.lds_b[i]]) = next.qb[i];
        load_b(next, i, knext);
      }
#pragma unroll
      for (int m = 0; m < TM * TN; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  StepRegs<TL> r0, r1;
  load(r0, 0);
  load(r1, 1);
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    store_half(r0, i, 0, 0);
    store_half(r0, i, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(&Bs[0][off.lds_b[i]]) = r0.qb[i];
  load(r0, 2);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ks += 2) {   // ksteps is even (K is a multiple of 128)
    body(0, r1, ks);       // step ks: decode step ks + 1 (r1), refill r1 with step ks + 3
    __syncthreads();
    body(1, r0, ks + 1);   // step ks + 1: decode step ks + 2 (r0), refill r0 with step ks + 4
    __syncthreads();
  }

  // epilogue: accumulator e of lane l holds row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32 of its 32 x 32 tile
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t r = m0 + wm * (BM / TL::WGM) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t c = n0 + wn * (BN / TL::WGN) + j * 32 + (lane & 31);
        if constexpr (BF16OUT) static_cast<__bf16*>(a.out)[r * a.N + c] = (__bf16)acc[i][j][e];
        else static_cast<float*>(a.out)[r * a.N + c] = acc[i][j][e];
      }
}

template <int FMT, int B, class TL>
static void launch_tiles(const DGemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.M / TL::BM) * (a.N / TL::BN))), block(TL::kThreads);
  if (a.bf16_out) hipLaunchKernelGGL((k_dequant_gemm<FMT, B, true, TL>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_dequant_gemm<FMT, B, false, TL>), grid, block, 0, s, a);
}

template <int FMT, int B>
static void launch_dg(const DGemmArgs& a, hipStream_t s) {
  if (a.M % TilesLarge::BM == 0 && a.N % TilesLarge::BN == 0) launch_tiles<FMT, B, TilesLarge>(a, s);
  else launch_tiles<FMT, B, TilesSmall>(a, s);
}

hipError_t launch_dequant_gemm(const DGemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  switch (a.fmt) {
    case kFP8:
      if (a.block == 32) launch_dg<kFP8, 32>(a, s);
      else if (a.block == 64) launch_dg<kFP8, 64>(a, s);
      else launch_dg<kFP8, 128>(a, s);
      break;
    case kFP8E5:
      if (a.block == 32) launch_dg<kFP8E5, 32>(a, s);
      else if (a.block == 64) launch_dg<kFP8E5, 64>(a, s);
      else launch_dg<kFP8E5, 128>(a, s);
      break;
    case kINT8S: launch_dg<kINT8S, 64>(a, s); break;
    case kINT4A: launch_dg<kINT4A, 128>(a, s); break;
    case kINT8A: launch_dg<kINT8A, 128>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace taco

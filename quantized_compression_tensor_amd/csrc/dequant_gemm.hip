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
// (the single rounding of the exact decoded value, nearest-even). W is a bf16
// weight in the layout of a linear layer, [N, K] row-major, so both operands
// are contiguous along K.
//
// Tiling: a workgroup of four waves computes a 128 x 128 tile of `out`, each
// wave a 64 x 64 quarter as 2 x 2 tiles of the 32 x 32 x 16 bf16 MFMA (f32
// accumulate). The K dimension is walked in steps of 64 through two LDS
// buffers: the next step's global loads are issued before the current step's
// MFMAs, decoded and stored to the other buffer after them, one barrier per
// step. M, N and K are multiples of 128, so there are no partial tiles.
#include "device_common.h"
#include "taco_internal.h"

namespace taco {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 64;
constexpr int kGemmLd = kGemmBK + 8;   // bf16 per LDS row: 144 bytes, so the 32 rows an
                                        // MFMA operand read touches start in distinct banks
constexpr int kGemmGroupM = 8;          // tile rows walked together (L2 reuse of W)

// Two floats -> two bf16 in one dword (the hardware conversion, nearest-even).
TACO_DEV uint32_t pk_bf16(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// One thread's A run per K step: 32 consecutive codes of one row, with the
// block metadata that covers them (every supported block holds whole runs).
struct ARun {
  u32x4 q0, q1;    // codes: 32 bytes (INT4: q0 only)
  float s;         // INT: the block scale; FP8: g * 2^-k
  uint32_t z;      // zero point (asymmetric)
};

template <int FMT, int B>
TACO_DEV void load_a(const DGemmArgs& a, float g, int64_t row, int64_t k, ARun& r) {
  const int64_t e = row * a.K + k;   // first element of the run
  const int64_t blk = e / B;
  if constexpr (FMT == kINT4A) {
    r.q0 = *reinterpret_cast<const u32x4*>(a.codes + e / 2);
    r.q1 = u32x4{0u, 0u, 0u, 0u};
  } else {
    r.q0 = *reinterpret_cast<const u32x4*>(a.codes + e);
    r.q1 = *reinterpret_cast<const u32x4*>(a.codes + e + 16);
  }
  if constexpr (is_fp8(FMT)) {
    r.s = g * pow2f(-(int)static_cast<const int8_t*>(a.scale)[blk]);
  } else {
    r.s = static_cast<const float*>(a.scale)[blk];
  }
  r.z = (FMT == kINT4A || FMT == kINT8A) ? (uint32_t)a.zero[blk] : 0u;
}

// Decoded values as taco_decompress forms them in float32 (each the single
// rounding of the exact value), then bf16.
template <int FMT>
TACO_DEV void decode_a(const ARun& r, u32x4* out) {
  const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
  float d[32];
  if constexpr (is_fp8(FMT)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) Fp8Code<FMT == kFP8E5>::unpack4(w[j], d + 4 * j);
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = d[i] * r.s;
  } else if constexpr (FMT == kINT8S) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = (float)(int)(int8_t)(uint8_t)(w[j] >> (8 * b)) * r.s;
  } else if constexpr (FMT == kINT8A) {
    const float zf = (float)r.z;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) d[4 * j + b] = ((float)((w[j] >> (8 * b)) & 0xFFu) - zf) * r.s;
  } else {
    // element 2i in the low nibble of byte i, 2i + 1 in the high nibble
    const float zf = (float)r.z;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        d[8 * j + 2 * b] = ((float)((w[j] >> (8 * b)) & 0xFu) - zf) * r.s;
        d[8 * j + 2 * b + 1] = ((float)((w[j] >> (8 * b + 4)) & 0xFu) - zf) * r.s;
      }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
    out[v] = u32x4{pk_bf16(d[8 * v], d[8 * v + 1]), pk_bf16(d[8 * v + 2], d[8 * v + 3]),
                   pk_bf16(d[8 * v + 4], d[8 * v + 5]), pk_bf16(d[8 * v + 6], d[8 * v + 7])};
}

// Output tile of this workgroup: tiles are renumbered so that each XCD walks
// one contiguous range, and inside it groups of kGemmGroupM tile rows are
// walked column by column, so the workgroups resident on one XCD share both
// A rows and W rows through its L2.
TACO_DEV void gemm_tile(const DGemmArgs& a, int64_t* tm, int64_t* tn) {
  const int64_t ntm = a.M / kGemmBM, ntn = a.N / kGemmBN;
  const int64_t t = xcd_ordered_block();
  const int64_t per_group = (int64_t)kGemmGroupM * ntn;
  const int64_t group = t / per_group, in_group = t % per_group;
  const int64_t first = group * kGemmGroupM;
  const int64_t rows = ntm - first < kGemmGroupM ? ntm - first : kGemmGroupM;
  *tm = first + in_group % rows;
  *tn = in_group / rows;
}

template <int FMT, int B, bool BF16OUT>
__global__ __launch_bounds__(kBlockThreads) void k_dequant_gemm(DGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGemmBM * kGemmLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGemmBN * kGemmLd];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_in_group();
  const int wm = wave >> 1, wn = wave & 1;          // this wave's 64 x 64 quarter
  int64_t tm, tn;
  gemm_tile(a, &tm, &tn);
  const int64_t m0 = tm * kGemmBM, n0 = tn * kGemmBN;
  const int lr = tid >> 1, lk = (tid & 1) * 32;     // load slot: row, first column in the K step
  const float g = is_fp8(FMT) ? *a.g_hdr : 1.0f;
  const uint16_t* wrow = a.w + (n0 + lr) * a.K + lk;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  ARun ra;
  u32x4 rb0, rb1, rb2, rb3;
  auto load_step = [&](int64_t k) {
    load_a<FMT, B>(a, g, m0 + lr, k + lk, ra);
    const u32x4* p = reinterpret_cast<const u32x4*>(wrow + k);
    rb0 = p[0];
    rb1 = p[1];
    rb2 = p[2];
    rb3 = p[3];
  };
  auto store_step = [&](int buf) {
    u32x4 da[4];
    decode_a<FMT>(ra, da);
    u32x4* pa = reinterpret_cast<u32x4*>(&As[buf][lr * kGemmLd + lk]);
    u32x4* pb = reinterpret_cast<u32x4*>(&Bs[buf][lr * kGemmLd + lk]);
    pa[0] = da[0];
    pa[1] = da[1];
    pa[2] = da[2];
    pa[3] = da[3];
    pb[0] = rb0;
    pb[1] = rb1;
    pb[2] = rb2;
    pb[3] = rb3;
  };

  const int ksteps = (int)(a.K / kGemmBK);
  load_step(0);
  store_step(0);
  __syncthreads();
  // MFMA operands: lane l holds row (A) or column (B) l % 32 and the eight K
  // entries 8 * (l / 32) ... of the sixteen one MFMA takes; A and B use the
  // same K assignment, so the sum over K is the same whatever order the
  // instruction gives those entries
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < ksteps) load_step((int64_t)(ks + 1) * kGemmBK);
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 16) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + i * 32 + fr) * kGemmLd + kk + fk]);
        bf[i] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + i * 32 + fr) * kGemmLd + kk + fk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) store_step(cur ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator e of lane l holds row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32 of its 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t r = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t c = n0 + wn * 64 + j * 32 + (lane & 31);
        if constexpr (BF16OUT) static_cast<__bf16*>(a.out)[r * a.N + c] = (__bf16)acc[i][j][e];
        else static_cast<float*>(a.out)[r * a.N + c] = acc[i][j][e];
      }
}

template <int FMT, int B>
static void launch_dg(const DGemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.M / kGemmBM) * (a.N / kGemmBN))), block(kBlockThreads);
  if (a.bf16_out) hipLaunchKernelGGL((k_dequant_gemm<FMT, B, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_dequant_gemm<FMT, B, false>), grid, block, 0, s, a);
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

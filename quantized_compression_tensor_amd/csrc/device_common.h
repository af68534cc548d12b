// Device helpers shared by the gfx950 kernels of the compression library.
//
// Every floating-point step is written so that it performs exactly the float32
// operations (one round-to-nearest-even each) that the codec definitions call
// for; files are compiled with contraction off, IEEE mode and float32
// denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "taco_internal.h"
#include "taco.h"

#define TACO_DEV __device__ __forceinline__

namespace taco {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;

// Index of this wave in its workgroup, as a wave-uniform (scalar) value.
TACO_DEV int wave_in_group() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x) / kWave; }

// XCD-aware workgroup order. The dispatcher hands workgroup b to XCD b % 8,
// so consecutive workgroups land on different XCDs, each with its own L2; a
// 128-byte line of block metadata shared by neighbouring workgroups (one
// zero-point byte or FP8 exponent byte per block) is then fetched by several
// L2s. This renumbering gives each XCD one contiguous range of workgroup
// indices -- XCD x takes [x * q + min(x, r), ...) with q = grid / 8 and
// r = grid % 8, the first r XCDs one more -- a bijection of [0, grid), so any
// grid stays correct whatever the dispatcher actually does.
constexpr unsigned kXcds = 8;
TACO_DEV unsigned xcd_ordered_block() {
  const unsigned G = gridDim.x, b = blockIdx.x;
  const unsigned x = b % kXcds, l = b / kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + l;
}

// Blocks whose abs-max (symmetric) or range (asymmetric) is below this are
// stored as zero codes with a zero scale, so 127/A and qmax/r stay finite.
constexpr float kTiny = 0x1p-100f;

// ---------------------------------------------------------------- loads --
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is read once).
TACO_DEV uint4 ld16_nt(const void* p) {
  u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ----------------------------------------------------------- buffer ops --
// Raw buffer accesses through a 128-bit resource (base, byte size): a load
// outside [0, size) returns zeros and a store there is dropped, so ragged
// tails need no branches and every access is issued unconditionally (which
// also lets the compiler wait for exactly the loads it needs).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;   // gfx9-family raw buffer, 32-bit data format
constexpr int kNT = 2;                   // non-temporal cache policy (streamed once)

TACO_DEV rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nr = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, kRsrcFlags);
}
// The same for a size the caller knows lies in [0, 2^31).
TACO_DEV rsrc_t make_rsrc32(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcFlags);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int AUX = 0>
TACO_DEV uint4 bload128(rsrc_t r, int voff, int soff) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int AUX = 0>
TACO_DEV uint2 bload64(rsrc_t r, int voff, int soff) {
  u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
  return make_uint2(v.x, v.y);
}
TACO_DEV uint32_t bload32(rsrc_t r, int voff, int soff) { return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0); }
TACO_DEV uint32_t bload8(rsrc_t r, int voff, int soff) { return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0); }
// Stores of the codes and scales are streaming (non-temporal) by default: the
// compressed tensors are written once and consumed elsewhere, so they should
// not displace other data in the caches.
template <int AUX = kNT>
TACO_DEV void bstore128(uint4 v, rsrc_t r, int voff, int soff) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, soff, AUX);
}
TACO_DEV void bstore64(uint2 v, rsrc_t r, int voff, int soff) {
  u32x2 w = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, voff, soff, kNT);
}
TACO_DEV void bstore32(uint32_t v, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, kNT);
}
TACO_DEV void bstore8(uint32_t v, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, r, voff, soff, 0);
}

// ------------------------------------------------------------------ bf16 --
TACO_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
TACO_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16, nearest-even; NaN -> 0x7FC0.
TACO_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (f != f) ? 0x7FC0u : r;
}

// ------------------------------------------------------------------- E4M3 --
// Hardware OCP E4M3 conversions of gfx950 (nearest-even). Four floats ->
// one dword, element i in byte i.
TACO_DEV uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

TACO_DEV void e4m3_unpack4(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}

// ------------------------------------------------------------------- E5M2 --
// Hardware OCP E5M2 ("bf8") conversions of gfx950 (nearest-even), same
// packing as the E4M3 pair.
TACO_DEV uint32_t e5m2_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  return (uint32_t)w;
}

TACO_DEV void e5m2_unpack4(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}

// The two FP8 code formats of the dual-scale codec. kMax is the largest finite
// value, 1.75 * 2^kTop; the block exponent puts each block maximum in
// (kMax / 2, kMax].
template <bool E5>
struct Fp8Code {
  static constexpr float kMax = 448.0f;          // E4M3: 1.75 * 2^8
  static constexpr int kTop = 8;
  static TACO_DEV uint32_t pack4(float a, float b, float c, float d) { return e4m3_pack4(a, b, c, d); }
  static TACO_DEV void unpack4(uint32_t w, float* o) { e4m3_unpack4(w, o); }
};
template <>
struct Fp8Code<true> {
  static constexpr float kMax = 57344.0f;        // E5M2: 1.75 * 2^15
  static constexpr int kTop = 15;
  static TACO_DEV uint32_t pack4(float a, float b, float c, float d) { return e5m2_pack4(a, b, c, d); }
  static TACO_DEV void unpack4(uint32_t w, float* o) { e5m2_unpack4(w, o); }
};

// Saturate to +-kMax keeping NaN (only reached when a block exponent is
// clamped, i.e. the block maximum cannot be brought down to kMax).
template <bool E5>
TACO_DEV float sat_fp8(float v) {
  constexpr float M = Fp8Code<E5>::kMax;
  return (fabsf(v) > M) ? copysignf(M, v) : v;
}

// ------------------------------------------------------- scales, exponents --
// 2^k as a float for k in [-126, 127].
TACO_DEV float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Block exponent: largest k in [-64, 63] with m * 2^k <= kMax = 1.75 * 2^T
// (m >= 0), 0 for m == 0. From the float bits: with m = 1.f * 2^(e-127),
// 1.f <= 1.75 exactly when the stored mantissa is <= 0x600000, giving
// k = T + 127 - e or T + 126 - e (E4M3: 135 / 134; E5M2: 142 / 141); subnormal
// m clamps to 63 and infinity to -64.
template <bool E5>
TACO_DEV int block_exponent(float m) {
  constexpr int T = Fp8Code<E5>::kTop + 127;
  uint32_t b = __float_as_uint(m);
  int k = ((b & 0x7FFFFFu) <= 0x600000u ? T : T - 1) - (int)(b >> 23);
  k = k < -64 ? -64 : (k > 63 ? 63 : k);
  return b == 0 ? 0 : k;
}

// Data-driven tensor scale from an abs-max A (FP8 dual-scale).
template <bool E5>
TACO_DEV float tensor_scale_from_amax(float A) {
  if (A == 0.0f) return 1.0f;
  float g = A / Fp8Code<E5>::kMax;
  return fminf(fmaxf(g, kGMin), kGMax);
}

// Round to the nearest integer, ties to even, for |t| < 2^22: adding
// 1.5 * 2^23 lands in the binade whose spacing is 1, so the float add does
// the rounding; the result is read back from the bits.
TACO_DEV int rne_int(float t) {
  return (int)(__float_as_uint(t + 12582912.0f) - 0x4B400000u);
}

// ----------------------------------------------------------- lane exchange --
// DPP patterns inside a 16-lane row. Each is one hardware lane permutation:
//   X1 = lane ^ 1, X2 = lane ^ 2 (quad permutes), X7 = lane ^ 7 (half-row
//   mirror), X8 = lane ^ 8 (row rotate by 8).
#define TACO_DPP_X1 "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define TACO_DPP_X2 "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
#define TACO_DPP_X7 "row_half_mirror row_mask:0xf bank_mask:0xf"
#define TACO_DPP_X8 "row_ror:8 row_mask:0xf bank_mask:0xf"

// max / min over groups of G lanes (G = 1, 2, 4, 8, 16; groups aligned to G),
// one DPP op per step. The leading s_nop covers the hazards between a VALU or
// EXEC write and a DPP read; between chained steps one s_nop 1 suffices.
template <int G>
TACO_DEV float group_max(float a) {
  if constexpr (G >= 2) asm volatile("s_nop 4\n\tv_max_f32_dpp %0, %0, %0 " TACO_DPP_X1 : "+v"(a));
  if constexpr (G >= 4) asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " TACO_DPP_X2 : "+v"(a));
  if constexpr (G >= 8) asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " TACO_DPP_X7 : "+v"(a));
  if constexpr (G >= 16) asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " TACO_DPP_X8 : "+v"(a));
  return a;
}

template <int G>
TACO_DEV float group_min(float a) {
  if constexpr (G >= 2) asm volatile("s_nop 4\n\tv_min_f32_dpp %0, %0, %0 " TACO_DPP_X1 : "+v"(a));
  if constexpr (G >= 4) asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %0, %0 " TACO_DPP_X2 : "+v"(a));
  if constexpr (G >= 8) asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %0, %0 " TACO_DPP_X7 : "+v"(a));
  if constexpr (G >= 16) asm volatile("s_nop 1\n\tv_min_f32_dpp %0, %0, %0 " TACO_DPP_X8 : "+v"(a));
  return a;
}

// Max of 8 magnitudes (non-negative result).
TACO_DEV float absmax8(const float* v) {
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  float b = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  float c = fmaxf(fabsf(v[6]), fabsf(v[7]));
  return fmaxf(fmaxf(a, b), c);
}

// Whole-wave max of a non-negative float (result valid in every lane).
TACO_DEV float wave_max(float a) {
  a = group_max<16>(a);
  a = fmaxf(a, __shfl_xor(a, 16));
  a = fmaxf(a, __shfl_xor(a, 32));
  return a;
}

// ------------------------------------------------- channel-group reorder --
// Data-driven reshaping of the hidden dimension: the codec sees the channels
// in groups of 8, reordered group j being original group order[j] of the same
// row. Every access of a reordering kernel covers a 512-element span, which
// lies inside one row (cols is a multiple of 512), and each lane's 8 elements
// are one group, so a lane's 16-byte bf16 access just moves from group j to
// group order[j] of its row.
constexpr int kGroupElems = 8;
constexpr int kSpanElems = 512;
constexpr int kSpanShift = 9;

// The order is copied into LDS (int16) at the start of the workgroup, clamped
// into [0, ngroups) so that no access can leave its row whatever the caller
// passed; per-span lookups then wait on LDS only, never on the data loads in
// flight.
TACO_DEV void load_order_lds(const ReorderArgs& ro, int16_t* lds) {
  for (int i = (int)threadIdx.x; i < ro.ngroups; i += kBlockThreads) {
    int v = ro.order[i];
    v = v < 0 ? 0 : (v >= ro.ngroups ? ro.ngroups - 1 : v);
    lds[i] = (int16_t)v;
  }
  __syncthreads();
}

// Row of the span starting at flat element e (a multiple of 512) and the
// span's first column: row = floor(s / d) for the span index s = e / 512 and
// d = cols / 512 spans per row, as (s * ceil(2^38 / d)) >> 38, exact for
// s < 2^26 and d <= 256 (the error s * (ceil - exact) / 2^38 < 2^-12 stays
// below 1/d).
struct SpanPos {
  uint32_t row, col0;
};
TACO_DEV SpanPos span_pos(const ReorderArgs& ro, int64_t e) {
  const uint32_t s = (uint32_t)(e >> kSpanShift);
  const uint32_t row = (uint32_t)(((uint64_t)s * ro.magic) >> 38);
  return SpanPos{row, (s - row * ro.spans_per_row) * (uint32_t)kSpanElems};
}

// Source (compress) or destination (decode) group of a lane whose group in the
// reordered span is `col0 / 8 + lane_group`.
TACO_DEV int reordered_group(const int16_t* lds, const SpanPos& p, int lane_group) {
  return lds[(p.col0 >> 3) + lane_group];
}

// Units of whole rows staged through LDS. A workgroup walks units
// u = blockIdx.x, blockIdx.x + gridDim.x, ...; unit u starts at element
// u * rows * cols and holds rows * cols elements (at most kStageMaxElems), the
// last one possibly fewer.
struct StageUnits {
  int64_t n, per, count;
  TACO_DEV StageUnits(int64_t n_, int cols, int rows)
      : n(n_), per((int64_t)rows * cols), count((n_ / cols + rows - 1) / rows) {}
  TACO_DEV int64_t base(int64_t u) const { return u * per; }
  TACO_DEV int elems(int64_t u) const { return u >= count ? 0 : (int)(n - u * per < per ? n - u * per : per); }
};
static_assert(8 * 8 * kBlockThreads == kStageMaxElems, "a staged bf16 unit is eight 16-byte words per thread");

// The loads of bf16 unit u into registers, eight 16-byte words per thread;
// past the last unit, or past its end, zeros from the resource.
TACO_DEV void stage_issue(const uint16_t* x, const StageUnits& su, int64_t u, uint4* next) {
  const rsrc_t r = make_rsrc32(x + (u < su.count ? su.base(u) : 0), su.elems(u) * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) next[j] = bload128<kNT>(r, 16 * ((int)threadIdx.x + j * kBlockThreads), 0);
}
// The unit's words from registers into LDS (its first elems / 8 words).
TACO_DEV void stage_commit(const uint4* next, uint4* lds, int elems) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = (int)threadIdx.x + j * kBlockThreads;
    if (w < elems / 8) lds[w] = next[j];
  }
}
// A decoded unit (n16 16-byte words) from LDS to global memory, eight words per
// thread at once.
TACO_DEV void stage_drain(const uint4* lds, rsrc_t dst, int n16) {
  for (int i0 = (int)threadIdx.x; i0 < n16; i0 += 8 * kBlockThreads) {
    uint4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = i0 + j * kBlockThreads < n16 ? lds[i0 + j * kBlockThreads] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (i0 + j * kBlockThreads < n16) bstore128<0>(t[j], dst, 16 * (i0 + j * kBlockThreads), 0);
  }
}

// ------------------------------------------------------------- workspace --
// Abs-max history of an FP8 tensor scale, in caller-owned memory that is
// zero-filled once. Calls on one workspace are ordered (one stream), and any
// call may run any grid.
//
// Call index. The workspace has 64 ticket counters; workgroup b adds to
// counter b % 64, and the members of each counter add shares that total
// exactly 2^24 per call (2^24 / members each, the first member the
// remainder; with fewer than 64 workgroups some take several counters). A counter therefore holds t * 2^24 when call t
// starts, and every workgroup's ticket (the value before its add) gives the
// same t = ticket >> 24, whatever the grid.
//
// Banks. Three banks of 32 record lines each; call t
//   * reads the previous call's maxima from bank (t + 2) % 3,
//   * folds each wave's or workgroup's maximum into bank t % 3 (atomic max,
//     not awaited),
//   * zeroes bank (t + 1) % 3 for the next call (first wave of workgroup 0).
// No bank is read and written by the same call, and the kernel boundary orders
// calls, so there is no fence, no spin and no "last workgroup" chain. Every
// counter and record line is a 128-byte line of its own. Only the first wave of
// a workgroup takes the ticket and reads the history; it hands t % 3 (and the
// tensor scale) to the others through LDS.
constexpr int kTicketGroups = 64;
constexpr int kAccLines = 32;
constexpr int kLineWords = 32;
constexpr int kShareShift = 24;
static_assert(kAccLines <= kWave, "one lane per record line");

struct WsLine {
  uint32_t amax;                                 // float bits
  uint32_t pad[kLineWords - 1];
};
struct WsCounter {
  unsigned long long v;
  uint32_t pad[kLineWords - 2];
};
struct Workspace {
  uint32_t pad0[kLineWords];
  WsCounter cnt[kTicketGroups];
  WsLine bank[3][kAccLines];
};
static_assert(sizeof(Workspace) <= TACO_WORKSPACE_BYTES, "workspace size");

#define TACO_AT_MAX(p, v) __hip_atomic_fetch_max((p), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
#define TACO_AT_ADD(p, v) __hip_atomic_fetch_add((p), (v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)

// This workgroup's ticket (first wave, all lanes; lane 0 issues the add and
// holds the result). The caller issues its data loads next and reads the
// result only when it needs the call index. With fewer than 64 workgroups,
// workgroup b also adds the whole 2^24 to every counter b + k * grid < 64
// (k >= 1, lane k, not awaited), so every counter still advances by exactly
// 2^24 per call.
TACO_DEV unsigned long long ws_ticket(Workspace* ws) {
  const uint32_t G = kTicketGroups;
  const uint32_t g = blockIdx.x % G;
  const uint32_t members = (gridDim.x - g + G - 1) / G;
  const unsigned long long total = 1ull << kShareShift;
  unsigned long long share = total / members;
  if (blockIdx.x < G) share = total - (unsigned long long)(members - 1) * share;
  const uint32_t lane = threadIdx.x & (kWave - 1);
  unsigned long long t = 0;
  if (lane == 0) t = TACO_AT_ADD(&ws->cnt[g].v, share);
  if (gridDim.x < G && lane > 0) {
    const uint32_t j = g + lane * gridDim.x;
    if (j < G) (void)TACO_AT_ADD(&ws->cnt[j].v, total);
  }
  return t;
}
// The call index mod 3 from lane 0's ticket (wave-uniform).
TACO_DEV uint32_t ws_bank_of(unsigned long long ticket) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)ticket);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(ticket >> 32));
  return (uint32_t)(((((unsigned long long)hi) << 32 | lo) >> kShareShift) % 3ull);
}

// History read before the call index is known: record line `lane` of every
// bank (used where no bank is written yet when the read is issued).
TACO_DEV uint3 ws_history_all(const Workspace* ws) {
  const int lane = threadIdx.x & (kWave - 1);
  uint3 h = make_uint3(0, 0, 0);
  if (lane < kAccLines) h = make_uint3(ws->bank[0][lane].amax, ws->bank[1][lane].amax, ws->bank[2][lane].amax);
  return h;
}
// The previous call's abs-max (wave-uniform) from ws_history_all's lanes.
TACO_DEV float ws_prev_from(uint3 h, uint32_t e) {
  const uint32_t pb = e == 0 ? 2u : e - 1u;
  const float v = __uint_as_float(pb == 0 ? h.x : (pb == 1 ? h.y : h.z));
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_max(v))));
}
// The previous call's abs-max read once the call index is known.
TACO_DEV float ws_prev_amax(const Workspace* ws, uint32_t e) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t pb = e == 0 ? 2u : e - 1u;
  float v = 0.0f;
  if (lane < kAccLines) v = __uint_as_float(ws->bank[pb][lane].amax);
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_max(v))));
}
// Zero the next call's bank (first wave of workgroup 0, all lanes).
TACO_DEV void ws_clear_next(Workspace* ws, uint32_t e) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t nb = e == 2 ? 0u : e + 1u;
  if (lane < kAccLines) ws->bank[nb][lane].amax = 0u;
}

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not
// make every wave wait for its outstanding global loads and stores first.
TACO_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Fold this wave's max (any value per lane) into its record line of bank e
// (one atomic per wave, no barrier). Every lane of the wave calls it.
TACO_DEV void ws_record_wave(Workspace* ws, uint32_t e, float lane_max) {
  const float m = wave_max(lane_max);
  const uint32_t line = (blockIdx.x * (kBlockThreads / kWave) + wave_in_group()) % kAccLines;
  if ((threadIdx.x & (kWave - 1)) == 0) TACO_AT_MAX(&ws->bank[e][line].amax, __float_as_uint(m));
}

// Fold the workgroup's max (any value per lane) into its record line of bank
// e: every thread of the workgroup calls it; one atomic per workgroup. `lds`
// holds one float per wave.
TACO_DEV void ws_record_group(Workspace* ws, uint32_t e, float lane_max, float* lds) {
  const float m = wave_max(lane_max);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_in_group();
  if (lane == 0) lds[wave] = m;
  lds_barrier();
  if (wave == 0 && lane == 0) {
    float g = lds[0];
#pragma unroll
    for (int w = 1; w < kBlockThreads / kWave; ++w) g = fmaxf(g, lds[w]);
    TACO_AT_MAX(&ws->bank[e][blockIdx.x % kAccLines].amax, __float_as_uint(g));
  }
}

}  // namespace taco

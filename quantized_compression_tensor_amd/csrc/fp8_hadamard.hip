// TACO FP8 path with the block Hadamard transform: fused compress, the
// abs-max pre-pass for the data-driven tensor scale, and the consumer-side
// decode.
//
// Source: "TACO: Efficient Communication Compression of Intermediate Tensors
// for Scalable Tensor-Parallel LLM Training" (Pith review page) -- Fig. 7
// (adaptive rescaling, ASH transform, dual-scale quantization), Fig. 9 (one
// fused operator instead of a chain of kernels), abstract (the fused operator
// cuts memory traffic and launches). The transform is the unnormalised
// Sylvester Walsh-Hadamard matrix on B contiguous elements along the hidden
// dimension, butterflies of half-width 1, 2, ..., B/2 in that order; the
// dual scale is a float32 tensor scale g times a per-block power of two 2^-k.
//
// Wave layout. A wave holds 512 consecutive elements, 8 per lane (one 16-byte
// bf16 load). A block of B elements sits in G = B/8 consecutive lanes. Inside
// a lane the 8 elements differ in index bits 0-2, so the first three
// butterfly stages are plain register arithmetic. Index bits 3-6 select the
// lane's 8-element chunk; lane j of a group holds chunk
//     c(j) = j ^ (bit2(j) ? 3 : 0),
// which makes flipping chunk bit 0, 1, 2, 3 the lane permutations j^1, j^2,
// j^7, j^8 -- each a single DPP pattern (quad permute, quad permute, half-row
// mirror, row rotate by 8). The memory access stays one contiguous 1 KiB
// span per wave.
//
// Sign tracking. A cross-lane butterfly needs a+b in one lane and a-b in its
// partner. Each lane instead computes own + s * partner with one DPP-fed
// fused multiply-add (s = +-1, so the product is exact and the single
// rounding equals that of a+b or a-b); the upper lane then holds -(a-b). The
// sign a lane carries after all stages is the parity of its chunk index, and
// is folded into the scale that follows. Nonzero results are bit-identical
// to the plain butterflies; an exact zero may carry either sign and is
// normalised to +0 by the final fused multiply-add with a +0 addend.
#include "device_common.h"
#include "taco_internal.h"

namespace taco {

constexpr int kTileElems = 512;   // per wave

template <int LOGB>
struct HadGeom {
  static constexpr int B = 1 << LOGB;
  static constexpr int G = B / 8;            // lanes per block
  static constexpr int BPT = kTileElems / B; // blocks per wave tile
  static constexpr int STAGES = LOGB - 3;    // cross-lane stages
};

// Chunk index of this lane inside its block.
template <int G>
TACO_DEV int lane_chunk(int lane) {
  int j = lane & (G - 1);
  if constexpr (G >= 8) j ^= ((j >> 2) & 1) * 3;
  return j;
}

TACO_DEV float sgn_bit(int c, int bit) { return ((c >> bit) & 1) ? -1.0f : 1.0f; }

// Butterflies of half-width 1, 2, 4 on the lane's 8 registers.
TACO_DEV void fwht_in_lane(float* v) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

#define TACO_FMAC8(S, DPP)                                   \
  "v_fmac_f32_dpp %0, %0, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %1, %1, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %2, %2, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %3, %3, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %4, %4, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %5, %5, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %6, %6, " S " " DPP "\n\t"                 \
  "v_fmac_f32_dpp %7, %7, " S " " DPP "\n\t"

// Cross-lane butterfly stages (chunk bits 0 .. STAGES-1). Eight independent
// registers per stage keep every DPP read at least seven instructions after
// the write it depends on; the leading s_nop covers the code before.
template <int STAGES>
TACO_DEV void fwht_cross_lane(float* v, float s0, float s1, float s2, float s3) {
  if constexpr (STAGES == 1) {
    asm volatile("s_nop 4\n\t" TACO_FMAC8("%8", TACO_DPP_X1)
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "v"(s0));
  } else if constexpr (STAGES == 2) {
    asm volatile("s_nop 4\n\t" TACO_FMAC8("%8", TACO_DPP_X1) TACO_FMAC8("%9", TACO_DPP_X2)
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "v"(s0), "v"(s1));
  } else if constexpr (STAGES == 3) {
    asm volatile("s_nop 4\n\t" TACO_FMAC8("%8", TACO_DPP_X1) TACO_FMAC8("%9", TACO_DPP_X2)
                     TACO_FMAC8("%10", TACO_DPP_X7)
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "v"(s0), "v"(s1), "v"(s2));
  } else {
    static_assert(STAGES == 4, "block of 16 to 128");
    asm volatile("s_nop 4\n\t" TACO_FMAC8("%8", TACO_DPP_X1) TACO_FMAC8("%9", TACO_DPP_X2)
                     TACO_FMAC8("%10", TACO_DPP_X7) TACO_FMAC8("%11", TACO_DPP_X8)
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "v"(s0), "v"(s1), "v"(s2), "v"(s3));
  }
}

// Lane constants of the transform: per-stage signs and the final parity sign.
template <int LOGB>
struct LaneSigns {
  float s0, s1, s2, s3, parity;
  int elem_off;  // element offset of this lane's chunk inside the wave tile
  TACO_DEV explicit LaneSigns(int lane) {
    using Gm = HadGeom<LOGB>;
    const int c = lane_chunk<Gm::G>(lane);
    s0 = sgn_bit(c, 0); s1 = sgn_bit(c, 1); s2 = sgn_bit(c, 2); s3 = sgn_bit(c, 3);
    parity = (__builtin_popcount(c) & 1) ? -1.0f : 1.0f;
    elem_off = ((lane & ~(Gm::G - 1)) | c) * 8;
  }
};

TACO_DEV void widen8(uint4 w, float* v) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// ------------------------------------------------------------ compress --
//
// One pass: load bf16, transform, block abs-max, exponent, scale, E4M3
// encode, store codes and exponents. With GFROM_WS the tensor scale comes from
// the abs-max the workspace recorded (the pre-pass of this call, or the
// previous call: delayed scaling); otherwise from the argument. With a
// workspace the kernel also records this tensor's abs-max for the next call.
//
// Work unit: a chunk of T consecutive wave tiles (T * 512 elements). For
// large tensors the launch gives every wave one chunk, and the hardware keeps
// every CU at full occupancy as waves retire: 13 % faster on a 32768 x 5120
// tensor than a persistent grid of 4 workgroups per CU whose waves walk many
// chunks. The kernel takes any grid: a wave walks chunks with a stride of the
// whole grid, loading the chunk after next while it transforms the current one
// (two register sets, used alternately).
// All accesses go through buffer resources rebased per chunk, so the ragged
// last chunk reads zeros and drops its out-of-range stores, and the look-ahead
// past the last chunk loads nothing.
// Chunk length in wave tiles: kChunkTiles, or kSmallChunkTiles for tensors of
// fewer than 2^16 large chunks (there the arithmetic left after the last loads
// land bounds the launch, and it scales with the chunk).
constexpr int kChunkTiles = 4;
constexpr int kSmallChunkTiles = 2;

template <int LOGB, int T>
struct HadChunk {
  using Gm = HadGeom<LOGB>;
  static constexpr int64_t ELEMS = (int64_t)T * kTileElems;

  static TACO_DEV void load(const uint16_t* x, int64_t c, int64_t elems, int elem_off, uint4* raw) {
    const rsrc_t r = make_rsrc(x + c * ELEMS, (elems - c * ELEMS) * 2);
#pragma unroll
    for (int i = 0; i < T; ++i) raw[i] = bload128<kNT>(r, elem_off * 2, i * kTileElems * 2);
  }
};

// The chunk's loads with the input's channel groups reordered: tile i of the
// chunk is one 512-element span of a row, and the lane whose 8 elements are
// group j of that span loads group order[j] of the same row instead. Tiles at
// or past the end load nothing (an empty resource returns zeros).
template <int LOGB, int T, bool REORD>
TACO_DEV void load_chunk(const uint16_t* x, int64_t c, int64_t elems, int elem_off, const ReorderArgs& ro,
                         const int16_t* lds_order, uint4* raw) {
  if constexpr (!REORD) {
    HadChunk<LOGB, T>::load(x, c, elems, elem_off, raw);
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) {
      // spans at or past the end (the look-ahead of the last chunks) read an
      // empty resource and look nothing up: their span index may lie beyond
      // the range where span_pos is exact
      const int64_t e0 = c * HadChunk<LOGB, T>::ELEMS + (int64_t)i * kTileElems;
      const bool live = e0 < elems;
      const SpanPos p = live ? span_pos(ro, e0) : SpanPos{0u, 0u};
      const int src = live ? reordered_group(lds_order, p, elem_off / kGroupElems) : 0;
      const rsrc_t r = make_rsrc32(x + (int64_t)p.row * ro.cols, live ? ro.cols * 2 : 0);
      raw[i] = bload128<kNT>(r, src * kGroupElems * 2, 0);
    }
  }
}

// The transform of one tile and its block abs-max (independent of the tensor
// scale).
template <int LOGB>
TACO_DEV float had_transform_tile(uint4 raw, const LaneSigns<LOGB>& ls, float* v) {
  using Gm = HadGeom<LOGB>;
  widen8(raw, v);
  fwht_in_lane(v);
  fwht_cross_lane<Gm::STAGES>(v, ls.s0, ls.s1, ls.s2, ls.s3);
  return group_max<Gm::G>(absmax8(v));
}

// Scale, encode and store tile i of chunk c from its transformed values v and
// block abs-max M.
template <int LOGB, int T, bool E5, bool DEBUG>
TACO_DEV void had_encode_tile(float* v, float M, int i, int64_t c, int64_t elems, const LaneSigns<LOGB>& ls, int row,
                              float inv_g, rsrc_t rc, rsrc_t rk, float* dbg) {
  using Gm = HadGeom<LOGB>;
  using F = Fp8Code<E5>;
  const float m = M * inv_g;
  const int k = block_exponent<E5>(m);
  const float cs = inv_g * pow2f(k) * ls.parity;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fmaf(v[e], cs, 0.0f);
  if (__builtin_expect(m * pow2f(k) > F::kMax, 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sat_fp8<E5>(v[e]);
  }
  uint2 q;
  q.x = F::pack4(v[0], v[1], v[2], v[3]);
  q.y = F::pack4(v[4], v[5], v[6], v[7]);
  bstore64(q, rc, ls.elem_off, i * kTileElems);
  // every lane of the block writes the same exponent byte
  bstore8((uint32_t)k, rk, row, i * Gm::BPT);
  if constexpr (DEBUG) {
    constexpr int64_t E = HadChunk<LOGB, T>::ELEMS;
    const rsrc_t rd = make_rsrc(dbg + c * E, (elems - c * E) * 4);
    bstore128(make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                         __float_as_uint(v[3])), rd, ls.elem_off * 4, i * kTileElems * 4);
    bstore128(make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                         __float_as_uint(v[7])), rd, ls.elem_off * 4 + 16, i * kTileElems * 4);
  }
}

template <int LOGB, int T>
struct ChunkOut {
  rsrc_t rc, rk;
  TACO_DEV ChunkOut(uint8_t* codes, int8_t* kexp, int64_t c, int64_t elems) {
    constexpr int64_t E = HadChunk<LOGB, T>::ELEMS;
    const int64_t rem = elems - c * E;
    rc = make_rsrc(codes + c * E, rem);
    rk = make_rsrc(kexp + (c * E >> LOGB), rem >> LOGB);
  }
};

// Transform, scale, encode and store one chunk.
template <int LOGB, int T, bool E5, bool DEBUG>
TACO_DEV void had_compress_chunk(const uint4* raw, int64_t c, int64_t elems, const LaneSigns<LOGB>& ls, int row,
                                 float inv_g, uint8_t* codes, int8_t* kexp, float* dbg, float& run_max) {
  const ChunkOut<LOGB, T> o(codes, kexp, c, elems);
#pragma unroll
  for (int i = 0; i < T; ++i) {
    float v[8];
    const float M = had_transform_tile<LOGB>(raw[i], ls, v);
    run_max = fmaxf(run_max, M);
    had_encode_tile<LOGB, T, E5, DEBUG>(v, M, i, c, elems, ls, row, inv_g, o.rc, o.rk, dbg);
  }
}

template <int LOGB, int T, bool E5, bool GFROM_WS, bool DEBUG, bool PERSIST, bool REORD>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_had_compress(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, int8_t* __restrict__ kexp,
    float* __restrict__ g_hdr, int64_t nblocks, float g_arg, Workspace* __restrict__ ws,
    float* __restrict__ dbg, ReorderArgs ro) {
  using Gm = HadGeom<LOGB>;
  using CH = HadChunk<LOGB, T>;
  static_assert(!(REORD && PERSIST), "the reordering compress does not run the persistent grid");
  __shared__ uint32_t lds_e;
  __shared__ float lds_g;
  __shared__ float lds_m[kBlockThreads / kWave];
  extern __shared__ __attribute__((aligned(16))) int16_t lds_order[];
  if constexpr (REORD) load_order_lds(ro, lds_order);
  const int lane = threadIdx.x & (kWave - 1);
  const LaneSigns<LOGB> ls(lane);
  const int row = lane / Gm::G;
  bool staged = false;   // rows staged through LDS (reordered input, rows up to 16384 columns)
  if constexpr (REORD) staged = ro.staged;

  const int64_t elems = nblocks << LOGB;
  const int64_t nchunks = (elems + CH::ELEMS - 1) / CH::ELEMS;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  int64_t c = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group();

  // With a workspace the first wave requests its ticket (and, on the
  // persistent grid, the history of all three banks) before every wave loads
  // its first two chunks. Loads complete in issue order, so waiting for the
  // ticket never waits for the chunks, and the barrier that hands the bank
  // index and tensor scale to the other waves orders LDS only. On the
  // one-chunk-per-wave grid the history is read after the ticket, from the
  // previous call's bank alone: the bank being recorded is never read while
  // other workgroups write it.
  const bool wave0 = wave_in_group() == 0;
  unsigned long long tk = 0;
  uint3 hist = make_uint3(0, 0, 0);
  if (ws != nullptr && wave0) {
    tk = ws_ticket(ws);
    if (PERSIST && GFROM_WS) hist = ws_history_all(ws);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 ra[T], rb[T];
  if (!staged) {
    load_chunk<LOGB, T, REORD>(x, c, elems, ls.elem_off, ro, lds_order, ra);
    load_chunk<LOGB, T, REORD>(x, c + stride, elems, ls.elem_off, ro, lds_order, rb);
  }
  __builtin_amdgcn_sched_barrier(0);
  // On the persistent grid the first chunk is transformed while the ticket
  // returns; only its scaling and encoding wait for the tensor scale.
  float v0[T][8], M0[T];
  float run_max = 0.0f;
  float g = g_arg;
  uint32_t e = 0;
  if (ws != nullptr) {
    if constexpr (PERSIST) {
#pragma unroll
      for (int i = 0; i < T; ++i) {
        M0[i] = had_transform_tile<LOGB>(ra[i], ls, v0[i]);
        run_max = fmaxf(run_max, M0[i]);
      }
    }
    if (wave0) {
      const uint32_t ee = ws_bank_of(tk);
      float gg = g_arg;
      if constexpr (GFROM_WS) gg = tensor_scale_from_amax<E5>(PERSIST ? ws_prev_from(hist, ee) : ws_prev_amax(ws, ee));
      if (blockIdx.x == 0) ws_clear_next(ws, ee);
      if (lane == 0) { lds_e = ee; lds_g = gg; }
    }
    lds_barrier();
    e = lds_e;
    if constexpr (GFROM_WS) g = lds_g;
  }
  const float inv_g = 1.0f / g;
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_hdr = g;

  if constexpr (REORD) {
    if (staged) {
      // units of stage_rows whole rows (at most kStageMaxElems elements):
      // loaded into LDS contiguously, then the lane that holds group j of a
      // span takes group order[j] of the span's row from LDS; the waves take
      // the unit's tiles in turn, four at a time. The next unit's loads are
      // issued into registers before this unit's tiles are encoded, so they
      // are in flight during the arithmetic.
      constexpr int NW = kBlockThreads / kWave;
      uint16_t* rows_lds = reinterpret_cast<uint16_t*>(lds_order) + reorder_stage_offset(ro);
      const int cols = ro.cols;
      const StageUnits su(elems, cols, ro.stage_rows);
      uint4 next[8];
      stage_issue(x, su, blockIdx.x, next);
      for (int64_t u = blockIdx.x; u < su.count; u += gridDim.x) {
        const int64_t ubase = su.base(u);
        const int uelems = su.elems(u);
        const int utiles = uelems / kTileElems;   // cols is a multiple of the tile
        stage_commit(next, reinterpret_cast<uint4*>(rows_lds), uelems);
        __syncthreads();
        stage_issue(x, su, u + gridDim.x, next);
        for (int lt0 = wave_in_group(); lt0 < utiles; lt0 += 4 * NW) {
          uint4 raw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lt = lt0 + i * NW;
            const int e0 = lt * kTileElems;   // span start inside the unit
            const int lrow = e0 / cols, col0 = e0 - lrow * cols;   // row inside the unit
            raw[i] = make_uint4(0, 0, 0, 0);
            if (lt < utiles) {
              const int src = lds_order[(col0 >> 3) + ls.elem_off / kGroupElems];
              raw[i] = *reinterpret_cast<const uint4*>(rows_lds + lrow * cols + src * kGroupElems);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (lt0 + i * NW < utiles)
              had_compress_chunk<LOGB, 1, E5, DEBUG>(raw + i, ubase / kTileElems + lt0 + i * NW, elems, ls, row,
                                                     inv_g, codes, kexp, dbg, run_max);
        }
        __syncthreads();   // the unit's LDS rows are read before the next unit's are written
      }
      if (ws != nullptr) ws_record_group(ws, e, run_max, lds_m);
      return;
    }
  }

  if (c < nchunks) {
    // first chunk (ra), then the chunks alternate between rb and ra
    if (PERSIST && ws != nullptr) {
      const ChunkOut<LOGB, T> o(codes, kexp, c, elems);
#pragma unroll
      for (int i = 0; i < T; ++i) had_encode_tile<LOGB, T, E5, DEBUG>(v0[i], M0[i], i, c, elems, ls, row, inv_g, o.rc, o.rk, dbg);
    } else {
      had_compress_chunk<LOGB, T, E5, DEBUG>(ra, c, elems, ls, row, inv_g, codes, kexp, dbg, run_max);
    }
    load_chunk<LOGB, T, REORD>(x, c + 2 * stride, elems, ls.elem_off, ro, lds_order, ra);
    c += stride;
    while (c < nchunks) {
      had_compress_chunk<LOGB, T, E5, DEBUG>(rb, c, elems, ls, row, inv_g, codes, kexp, dbg, run_max);
      load_chunk<LOGB, T, REORD>(x, c + 2 * stride, elems, ls.elem_off, ro, lds_order, rb);
      c += stride;
      if (c >= nchunks) break;
      had_compress_chunk<LOGB, T, E5, DEBUG>(ra, c, elems, ls, row, inv_g, codes, kexp, dbg, run_max);
      load_chunk<LOGB, T, REORD>(x, c + 2 * stride, elems, ls.elem_off, ro, lds_order, ra);
      c += stride;
    }
  }
  // records: per wave on the persistent grid (no closing barrier; 0.3 us
  // faster on 4096 x 4096), per workgroup on the one-chunk-per-wave grid
  // (a quarter of the atomics for the many short-lived workgroups)
  if (ws != nullptr) {
    if constexpr (PERSIST) ws_record_wave(ws, e, run_max);
    else ws_record_group(ws, e, run_max, lds_m);
  }
}

// Abs-max of the transformed tensor, recorded in the workspace.
template <int LOGB, bool REORD>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_had_amax(const uint16_t* __restrict__ x, int64_t nblocks,
                                                                Workspace* __restrict__ ws, ReorderArgs ro) {
  using Gm = HadGeom<LOGB>;
  using CH = HadChunk<LOGB, kChunkTiles>;
  extern __shared__ __attribute__((aligned(16))) int16_t lds_order[];
  if constexpr (REORD) load_order_lds(ro, lds_order);
  const int lane = threadIdx.x & (kWave - 1);
  const LaneSigns<LOGB> ls(lane);
  const int64_t elems = nblocks << LOGB;
  const int64_t nchunks = (elems + CH::ELEMS - 1) / CH::ELEMS;
  const int64_t stride = (int64_t)gridDim.x * (kBlockThreads / kWave);
  float run_max = 0.0f;
  bool staged = false;
  if constexpr (REORD) staged = ro.staged;
  if (staged) {
    // units of whole rows through LDS as in the staged compress (the next
    // unit's loads in registers while this one is transformed)
    constexpr int NW = kBlockThreads / kWave;
    const uint16_t* rows_lds = reinterpret_cast<const uint16_t*>(lds_order) + reorder_stage_offset(ro);
    const int cols = ro.cols;
    const StageUnits su(elems, cols, ro.stage_rows);
    uint4 next[8];
    stage_issue(x, su, blockIdx.x, next);
    for (int64_t u = blockIdx.x; u < su.count; u += gridDim.x) {
      const int utiles = su.elems(u) / kTileElems;
      stage_commit(next, reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(lds_order) + reorder_stage_offset(ro)),
                   su.elems(u));
      __syncthreads();
      stage_issue(x, su, u + gridDim.x, next);
      for (int lt = wave_in_group(); lt < utiles; lt += NW) {
        const int e0 = lt * kTileElems;   // span start inside the unit
        const int lrow = e0 / cols, col0 = e0 - lrow * cols;   // row inside the unit
        const int src = lds_order[(col0 >> 3) + ls.elem_off / kGroupElems];
        float v[8];
        widen8(*reinterpret_cast<const uint4*>(rows_lds + lrow * cols + src * kGroupElems), v);
        fwht_in_lane(v);
        fwht_cross_lane<Gm::STAGES>(v, ls.s0, ls.s1, ls.s2, ls.s3);
        run_max = fmaxf(run_max, absmax8(v));
      }
      __syncthreads();   // the unit's LDS rows are read before the next unit's are written
    }
  }
  for (int64_t c = (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_group(); !staged && c < nchunks;
       c += stride) {
    uint4 raw[kChunkTiles];
    load_chunk<LOGB, kChunkTiles, REORD>(x, c, elems, ls.elem_off, ro, lds_order, raw);
#pragma unroll
    for (int i = 0; i < kChunkTiles; ++i) {
      float v[8];
      widen8(raw[i], v);
      fwht_in_lane(v);
      fwht_cross_lane<Gm::STAGES>(v, ls.s0, ls.s1, ls.s2, ls.s3);
      run_max = fmaxf(run_max, absmax8(v));
    }
  }
  __shared__ float lds_m[kBlockThreads / kWave];
  __shared__ uint32_t lds_e;
  if (wave_in_group() == 0) {
    const uint32_t e = ws_bank_of(ws_ticket(ws));
    if (blockIdx.x == 0) ws_clear_next(ws, e);
    if ((threadIdx.x & (kWave - 1)) == 0) lds_e = e;
  }
  lds_barrier();
  ws_record_group(ws, lds_e, run_max, lds_m);
}

// --------------------------------------------------------------- decode --
//
// One wave tile of the decode: the lane's eight codes times g * 2^-k, the
// inverse transform (the forward one, which is its own inverse up to 2^-LOGB),
// then 2^-LOGB and the lane's sign.
template <bool E5, int LOGB>
TACO_DEV void decode_tile(uint2 raw, float d, float outscale, const LaneSigns<LOGB>& ls, float* v) {
  Fp8Code<E5>::unpack4(raw.x, v);
  Fp8Code<E5>::unpack4(raw.y, v + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = v[e] * d;
  fwht_in_lane(v);
  fwht_cross_lane<HadGeom<LOGB>::STAGES>(v, ls.s0, ls.s1, ls.s2, ls.s3);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fmaf(v[e], outscale, 0.0f);
}

// Consumer side: dequantize (dec(q) * g * 2^-k, the combined scale is exact),
// inverse transform (the same butterflies; H H = B I) and the 2^-log2(B)
// factor, then float32 or bf16 output. T wave tiles per wave as launched; a
// smaller grid walks them with a stride of the grid.
template <int LOGB, bool E5, bool BF16OUT, int T, bool REORD>
__global__ __launch_bounds__(kBlockThreads) void k_fp8_had_decode(
    const uint8_t* __restrict__ codes, const int8_t* __restrict__ kexp, const float* __restrict__ g_hdr,
    int64_t nblocks, void* __restrict__ out, ReorderArgs ro) {
  using Gm = HadGeom<LOGB>;
  extern __shared__ __attribute__((aligned(16))) int16_t lds_order[];
  if constexpr (REORD) load_order_lds(ro, lds_order);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const LaneSigns<LOGB> ls(lane);
  const int row = lane / Gm::G;
  const float g = *g_hdr;
  const float outscale = pow2f(-LOGB) * ls.parity;
  const int64_t ntiles = ((nblocks << LOGB) + kTileElems - 1) / kTileElems;
  if constexpr (REORD) {
    if (ro.staged) {
      // units of stage_rows whole rows (at most kStageMaxElems elements, 32
      // tiles): wave w decodes tiles w, w + 4, ... of the unit and each lane
      // writes its decoded group j to group order[j] of the span's row in LDS;
      // then the unit is stored contiguously. The next unit's codes and block
      // exponents are loaded before this unit is decoded, so they are in
      // flight during the arithmetic and the store.
      constexpr int OB = BF16OUT ? 2 : 4;
      constexpr int NW = kBlockThreads / kWave;
      constexpr int TW = kStageMaxElems / kTileElems / NW;   // tiles per wave and unit, at most
      uint8_t* rows_lds = reinterpret_cast<uint8_t*>(lds_order) + 2 * reorder_stage_offset(ro);
      const int cols = ro.cols;
      const StageUnits su(nblocks << LOGB, cols, ro.stage_rows);
      uint2 nraw[TW];
      int nk[TW];
      auto issue = [&](int64_t u) {   // past the last unit, or past its end: zeros
        const int64_t tb = u < su.count ? su.base(u) / kTileElems : 0;
        const int ut = su.elems(u) / kTileElems;
        const rsrc_t rc = make_rsrc32(codes + tb * kTileElems, ut * kTileElems);
        const rsrc_t rk = make_rsrc32(kexp + tb * Gm::BPT, ut * Gm::BPT);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const int lt = wave + i * NW;
          nraw[i] = bload64<kNT>(rc, lt * kTileElems + ls.elem_off, 0);
          nk[i] = (int)(int8_t)(uint8_t)bload8(rk, lt * Gm::BPT + row, 0);
        }
      };
      issue(blockIdx.x);
      for (int64_t u = blockIdx.x; u < su.count; u += gridDim.x) {
        const int uelems = su.elems(u);
        const int utiles = uelems / kTileElems;   // cols is a multiple of the tile
        uint2 raw[TW];
        int kk[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          raw[i] = nraw[i];
          kk[i] = nk[i];
        }
        issue(u + gridDim.x);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const int lt = wave + i * NW;
          if (lt < utiles) {
            float v[8];
            decode_tile<E5>(raw[i], g * pow2f(-kk[i]), outscale, ls, v);
            const int e0 = lt * kTileElems;   // span start inside the unit
            const int lrow = e0 / cols, col0 = e0 - lrow * cols;   // row inside the unit
            const int dst = lds_order[(col0 >> 3) + ls.elem_off / kGroupElems];
            uint8_t* p = rows_lds + ((int64_t)lrow * cols + dst * kGroupElems) * OB;
            if constexpr (BF16OUT) {
              *reinterpret_cast<uint4*>(p) = make_uint4(
                  f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16), f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16),
                  f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16), f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16));
            } else {
              reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
              reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
          }
        }
        __syncthreads();
        stage_drain(reinterpret_cast<const uint4*>(rows_lds),
                    make_rsrc32(static_cast<uint8_t*>(out) + su.base(u) * OB, uelems * OB), uelems * OB / 16);
        __syncthreads();   // the unit is stored before the next unit's decode writes LDS
      }
      return;
    }
  }
  for (int64_t tile0 = ((int64_t)blockIdx.x * 4 + wave) * T; tile0 < ntiles; tile0 += (int64_t)gridDim.x * 4 * T) {
  uint2 raw[T];
  int kk[T];
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int64_t blk = (tile0 + i) * Gm::BPT + row;
    raw[i] = make_uint2(0, 0);
    kk[i] = 0;
    if (blk < nblocks) {
      raw[i] = *reinterpret_cast<const uint2*>(codes + (tile0 + i) * kTileElems + ls.elem_off);
      kk[i] = kexp[blk];
    }
  }
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const int64_t blk = (tile0 + i) * Gm::BPT + row;
    float v[8];
    decode_tile<E5>(raw[i], g * pow2f(-kk[i]), outscale, ls, v);
    if (blk < nblocks) {
      // reordered: group j of this span goes back to group order[j] of its row
      int64_t eoff = (tile0 + i) * kTileElems + ls.elem_off;
      if constexpr (REORD) {
        const SpanPos p = span_pos(ro, (tile0 + i) * kTileElems);
        eoff = (int64_t)p.row * ro.cols + (int64_t)reordered_group(lds_order, p, ls.elem_off / kGroupElems) * kGroupElems;
      }
      if constexpr (BF16OUT) {
        uint4 o;
        o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
        o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
        o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
        o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + eoff) = o;
      } else {
        float4* d4 = reinterpret_cast<float4*>(static_cast<float*>(out) + eoff);
        d4[0] = make_float4(v[0], v[1], v[2], v[3]);
        d4[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
  }
}

// ------------------------------------------------------------ launchers --

static int64_t had_groups(int logb, int64_t nblocks, int T) {
  const int64_t elems = nblocks << logb;
  const int64_t tiles = (elems + kTileElems - 1) / kTileElems;
  return (tiles + 4 * T - 1) / (4 * T);
}

// Dynamic LDS of the reordering kernels: the order as int16.
static size_t order_lds_bytes(const ReorderArgs& ro) { return ro.order ? ((size_t)ro.ngroups * 2 + 3) & ~size_t(3) : 0; }

// walk_units > 0: the grid is every resident workgroup, at most walk_units
// (a kernel that prefetches its next unit), instead of `grid`.
template <int LOGB, int T, bool E5, bool DEBUG, bool PERSIST, bool REORD = false>
static void launch_compress_t(const FP8HadArgs& a, dim3 grid, hipStream_t s, const ReorderArgs& ro,
                              size_t lds = 0, int64_t walk_units = 0) {
  dim3 block(kBlockThreads);
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* ws = static_cast<Workspace*>(a.ws);
  auto* kern = a.g_from_ws ? k_fp8_had_compress<LOGB, T, E5, true, DEBUG, PERSIST, REORD>
                           : k_fp8_had_compress<LOGB, T, E5, false, DEBUG, PERSIST, REORD>;
  if (walk_units > 0) grid = resident_grid(reinterpret_cast<const void*>(kern), lds, walk_units);
  hipLaunchKernelGGL(kern, grid, block, lds, s, x, a.codes, a.kexp, a.g_hdr, a.nblocks, a.g, ws, a.dbg, ro);
}

// Grid. Tensors of fewer than 2^16 large chunks take the small chunks on a
// persistent grid of kPersistentGroupsPerCU workgroups per CU (each wave walks
// a few chunks; the workspace history is read up front and the first chunk is
// transformed while the ticket returns). Larger tensors give every wave one
// large chunk (the uncapped grid described above).
template <int LOGB, bool E5>
static hipError_t launch_compress_fmt(const FP8HadArgs& a, hipStream_t s) {
  const int64_t elems = a.nblocks << LOGB;
  if (elems == 0) return hipSuccess;
  const int64_t chunks = (elems + kChunkTiles * kTileElems - 1) / (kChunkTiles * kTileElems);
  const bool small = !a.dbg && chunks < (int64_t(1) << 16);
  dim3 block(kBlockThreads);
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* ws = static_cast<Workspace*>(a.ws);
  const dim3 big_grid = capped_grid(had_groups(LOGB, a.nblocks, kChunkTiles));
  if (a.ro.order != nullptr) {
    // reordered input (block 128 only): never the persistent small-tensor grid
    if constexpr (LOGB == 7) {
      if (a.dbg) return hipErrorInvalidValue;
      // rows staged through LDS in units of whole rows (the abs-max pre-pass
      // too), else gathered
      ReorderArgs ro = a.ro;
      ro.stage_rows = stage_rows_for(ro.cols, kTileElems);
      ro.staged = ro.stage_rows > 0;
      if (ro.staged) {
        const int64_t units = (elems / ro.cols + ro.stage_rows - 1) / ro.stage_rows;
        const size_t lds = (size_t)reorder_stage_offset(ro) * 2 + (size_t)ro.stage_rows * ro.cols * 2;
        if (a.auto_prepass) {
          auto* amax = k_fp8_had_amax<LOGB, true>;
          hipLaunchKernelGGL(amax, resident_grid(reinterpret_cast<const void*>(amax), lds, units), block, lds, s, x,
                             a.nblocks, ws, ro);
        }
        launch_compress_t<LOGB, kChunkTiles, E5, false, false, true>(a, dim3(1), s, ro, lds, units);
      } else {
        if (a.auto_prepass)
          hipLaunchKernelGGL((k_fp8_had_amax<LOGB, true>), big_grid, block, order_lds_bytes(a.ro), s, x, a.nblocks,
                             ws, ro);
        launch_compress_t<LOGB, kChunkTiles, E5, false, false, true>(a, big_grid, s, ro, order_lds_bytes(a.ro));
      }
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (a.auto_prepass)
    hipLaunchKernelGGL((k_fp8_had_amax<LOGB, false>), big_grid, block, 0, s, x, a.nblocks, ws, a.ro);
  if (small) {
    const int64_t need = had_groups(LOGB, a.nblocks, kSmallChunkTiles);
    const int64_t cap = (int64_t)device_cu_count() * kPersistentGroupsPerCU;
    launch_compress_t<LOGB, kSmallChunkTiles, E5, false, true>(a, capped_grid(need < cap ? need : cap), s, a.ro);
  } else {
    if (a.dbg) launch_compress_t<LOGB, kChunkTiles, E5, true, false>(a, big_grid, s, a.ro);   // test hook: the large chunks
    else launch_compress_t<LOGB, kChunkTiles, E5, false, false>(a, big_grid, s, a.ro);
  }
  return hipGetLastError();
}

template <int LOGB>
static hipError_t launch_compress_logb(const FP8HadArgs& a, hipStream_t s) {
  return a.e5 ? launch_compress_fmt<LOGB, true>(a, s) : launch_compress_fmt<LOGB, false>(a, s);
}

hipError_t launch_fp8_had_compress(const FP8HadArgs& a, hipStream_t s) {
  switch (a.logb) {
    case 4: return launch_compress_logb<4>(a, s);
    case 5: return launch_compress_logb<5>(a, s);
    case 6: return launch_compress_logb<6>(a, s);
    case 7: return launch_compress_logb<7>(a, s);
  }
  return hipErrorInvalidValue;
}

// walk_units > 0: the grid is every resident workgroup, at most walk_units.
template <int LOGB, bool E5, bool REORD>
static void launch_decode_fmt(const FP8HadDecodeArgs& a, dim3 grid, hipStream_t s, const ReorderArgs& ro,
                              size_t lds, int64_t walk_units = 0) {
  constexpr int T = 2;
  dim3 block(kBlockThreads);
  auto* kern = a.bf16_out ? k_fp8_had_decode<LOGB, E5, true, T, REORD> : k_fp8_had_decode<LOGB, E5, false, T, REORD>;
  if (walk_units > 0) grid = resident_grid(reinterpret_cast<const void*>(kern), lds, walk_units);
  hipLaunchKernelGGL(kern, grid, block, lds, s, a.codes, a.kexp, a.g_hdr, a.nblocks, a.out, ro);
}

template <int LOGB>
static hipError_t launch_decode_logb(const FP8HadDecodeArgs& a, hipStream_t s) {
  const int64_t groups = had_groups(LOGB, a.nblocks, 2);
  if (groups == 0) return hipSuccess;
  const dim3 grid = capped_grid(groups);
  if (a.ro.order != nullptr) {
    if constexpr (LOGB == 7) {
      // rows staged through LDS in units of whole rows, else scattered
      ReorderArgs ro = a.ro;
      const int ob = a.bf16_out ? 2 : 4;
      ro.stage_rows = stage_rows_for(ro.cols, kTileElems);
      ro.staged = ro.stage_rows > 0;
      size_t lds = order_lds_bytes(ro);
      int64_t units = 0;
      if (ro.staged) {
        units = ((a.nblocks << LOGB) / ro.cols + ro.stage_rows - 1) / ro.stage_rows;
        lds = (size_t)reorder_stage_offset(ro) * 2 + (size_t)ro.stage_rows * ro.cols * ob;
      }
      if (a.e5) launch_decode_fmt<LOGB, true, true>(a, grid, s, ro, lds, units);
      else launch_decode_fmt<LOGB, false, true>(a, grid, s, ro, lds, units);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (a.e5) launch_decode_fmt<LOGB, true, false>(a, grid, s, a.ro, 0);
  else launch_decode_fmt<LOGB, false, false>(a, grid, s, a.ro, 0);
  return hipGetLastError();
}

hipError_t launch_fp8_had_decode(const FP8HadDecodeArgs& a, hipStream_t s) {
  switch (a.logb) {
    case 4: return launch_decode_logb<4>(a, s);
    case 5: return launch_decode_logb<5>(a, s);
    case 6: return launch_decode_logb<6>(a, s);
    case 7: return launch_decode_logb<7>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace taco

// Host-side interface between the C ABI (taco_abi.hip) and the kernel files.
// Argument structs carry plain device pointers and sizes that the ABI layer
// has already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taco {

enum Format : int { kFP8 = 1, kINT8S = 2, kINT4A = 3, kINT8A = 4, kFP8E5 = 5 };

// The dual-scale FP8 formats (E4M3 and E5M2 codes).
constexpr bool is_fp8(int f) { return f == kFP8 || f == kFP8E5; }

// Range of the per-tensor scale g (FP8 dual-scale): both g * 2^-k and
// (1/g) * 2^k stay normal float32 numbers for every block exponent k in
// [-64, 63], so the combined per-block scales are exact.
constexpr float kGMin = 0x1p-60f;
constexpr float kGMax = 0x1p60f;

// Data-driven reorder of the hidden channels in groups of 8 (null order: none).
struct ReorderArgs {
  const int32_t* order;     // device int32 [ngroups]: reordered group j = original group order[j]
  int ngroups;              // cols / 8
  int cols;                 // a multiple of 512
  uint32_t spans_per_row;   // cols / 512 (at most 256)
  uint64_t magic;           // ceil(2^38 / spans_per_row)
  bool staged;              // rows staged through LDS (set per launch, stage_rows_for)
  int stage_rows;           // rows per staged unit
};
constexpr int kReorderMaxCols = 131072;
constexpr int kReorderColsMultiple = 512;
// Largest unit of whole rows the reorder kernels stage through LDS (rows at
// most this wide; wider rows are gathered from global memory group by group).
// A staging workgroup holds the next unit's loads in registers: 16384 bf16
// elements are eight 16-byte words per thread of 256, 16384 FP8 codes eight
// 512-element tiles per wave.
constexpr int kStageMaxElems = 16384;
// Rows per staged unit whose elements are a multiple of `align` (the kernel's
// tile; 0: not staged): the fewest rows that hold at least 8192 elements
// (about two 1024-element tiles per wave of a workgroup; larger units hold more
// LDS per workgroup and fewer workgroups fit on a CU) within kStageMaxElems;
// else the fewest that fit.
inline int stage_rows_for(int64_t cols, int align) {
  if (cols <= 0 || cols > kStageMaxElems) return 0;
  int first = 0;
  for (int r = 1; r * cols <= kStageMaxElems; ++r) {
    if ((r * cols) % align != 0) continue;
    if (r * cols >= 8192) return r;
    if (first == 0) first = r;
  }
  return first;
}
// LDS of the staged reorder kernels: the order (int16, rounded up to 16
// bytes) and then the staged rows; the offset of the rows in int16 units.
__host__ __device__ inline int reorder_stage_offset(const ReorderArgs& ro) { return (ro.ngroups + 7) & ~7; }
inline ReorderArgs make_reorder(const int32_t* order, int64_t cols) {
  ReorderArgs r{};
  r.order = order;
  if (order != nullptr) {
    r.ngroups = (int)(cols / 8);
    r.cols = (int)cols;
    r.spans_per_row = (uint32_t)(cols / 512);
    r.magic = ((uint64_t(1) << 38) + r.spans_per_row - 1) / r.spans_per_row;

  }
  return r;
}

// FP8 dual-scale with the Hadamard transform, bf16 input.
struct FP8HadArgs {
  const void* x;        // bf16 [nblocks << logb]
  uint8_t* codes;
  int8_t* kexp;
  float* g_hdr;
  int64_t nblocks;
  int logb;
  bool e5;              // E5M2 codes (else E4M3)
  float g;              // used when !g_from_ws
  bool g_from_ws;       // tensor scale from the workspace's recorded abs-max
  bool auto_prepass;    // run the abs-max pass first (data-driven g of this tensor)
  void* ws;             // Workspace* or null
  float* dbg;           // pre-rounding values or null
  ReorderArgs ro;       // channel-group reorder of the input (order null: none)
};

struct FP8HadDecodeArgs {
  const uint8_t* codes;
  const int8_t* kexp;
  const float* g_hdr;
  int64_t nblocks;
  int logb;
  bool e5;              // E5M2 codes (else E4M3)
  bool bf16_out;
  void* out;
  ReorderArgs ro;       // restore the original channel order on output (order null: none)
};

// Quantization without a transform (INT8 symmetric, asymmetric INT4/INT8,
// and FP8 dual-scale with hadamard off or on already-transformed float32).
struct QuantArgs {
  int fmt;
  int block;
  bool f32_in;          // input float32 (else bf16)
  const void* x;
  int64_t n;            // elements, a multiple of block
  uint8_t* codes;
  void* scale;          // FP8: int8 k; others: float s
  uint8_t* zero;        // asymmetric only
  float* g_hdr;         // FP8 only
  float g;
  bool g_from_ws;
  bool auto_prepass;
  void* ws;
  float* dbg;
  ReorderArgs ro;       // channel-group reorder of a bf16 input (order null: none)
};

struct DequantArgs {
  int fmt;
  int block;
  const uint8_t* codes;
  const void* scale;
  const uint8_t* zero;
  const float* g_hdr;
  int64_t n;
  bool bf16_out;
  void* out;
  ReorderArgs ro;       // restore the original channel order on output (order null: none)
};

// Decode fused into the consumer's GEMM: out[M, N] = decode(A)[M, K] * W^T.
struct DGemmArgs {
  int fmt;
  int block;
  const uint8_t* codes;   // A's codes, [M, K] in the compressed layout
  const void* scale;
  const uint8_t* zero;
  const float* g_hdr;
  const uint16_t* w;      // bf16 [N, K] row-major
  int64_t M, N, K;        // multiples of 128
  bool bf16_out;
  void* out;              // [M, N] row-major, float32 or bf16
  float neg_zero;         // -0.0f (an addend the compiler cannot fold away)
};

constexpr int kMaxShards = 16;

struct ShardPtrs {
  const uint8_t* codes[kMaxShards];
  const void* scale[kMaxShards];
  const uint8_t* zero[kMaxShards];
  const float* g[kMaxShards];
};

struct ReduceArgs {
  int fin, fout;
  int bin, bout;        // block sizes
  int nshards;
  int64_t n;
  ShardPtrs in;
  float* sum;           // nullable
  uint8_t* rq_codes;    // nullable (no requantization)
  void* rq_scale;
  uint8_t* rq_zero;
  float* rq_g_hdr;
  bool write_g;         // this launch writes the requantized tensor scale
};

struct HopArgs {
  int fin, fout;
  int bin, bout;
  int64_t n;
  const uint8_t* codes;   // incoming shard (nullptr: first hop)
  const void* scale;
  const uint8_t* zero;
  const uint16_t* local;  // bf16
  float* sum;             // nullable
  uint8_t* rq_codes;      // nullable
  void* rq_scale;
  uint8_t* rq_zero;
};

// Largest number of elements one reduce launch covers (keeps every buffer
// offset, including the float32 sum's, below 2^31 bytes).
constexpr int64_t kReducePiece = int64_t(1) << 28;
static_assert(4 * kReducePiece < (int64_t(1) << 31), "a piece's float32 sum must be addressable with 32-bit offsets");

// Compute units of the current device (queried once per device).
int device_cu_count();

// Workgroup cap of the calling host thread (taco_set_launch_limit; 0 = none)
// and a grid of `groups` workgroups under it. Every kernel it is applied to
// walks its work with a stride of the whole grid, so any grid gives the same
// results.
int launch_limit();
inline dim3 capped_grid(int64_t groups) {
  const int lim = launch_limit();
  return dim3((unsigned)(lim > 0 && groups > lim ? lim : groups));
}
// Workgroups of `kernel` (256 threads, `lds` bytes of dynamic LDS) that fit on
// one CU at once (the runtime's occupancy figure, cached per device, kernel and
// LDS size; 1 if it cannot be had).
int resident_groups(const void* kernel, size_t lds);
// Grid of a kernel that walks `units` units with a stride of the grid and
// keeps the next unit's loads in flight: every workgroup resident at once (one
// pass over the device, so no workgroup waits for another to end), at most
// `units`, under the launch limit.
inline dim3 resident_grid(const void* kernel, size_t lds, int64_t units) {
  const int64_t full = (int64_t)device_cu_count() * resident_groups(kernel, lds);
  return capped_grid(units < full ? units : full);
}
// Workgroups per CU (4 waves each) of the persistent FP8 compress of small
// tensors.
#ifndef TACO_GROUPS_PER_CU
#define TACO_GROUPS_PER_CU 4
#endif
constexpr int kPersistentGroupsPerCU = TACO_GROUPS_PER_CU;
static_assert(kPersistentGroupsPerCU > 0, "persistent kernels need at least one workgroup per CU");
// Tiles per wave of the reduce (one workgroup per 4 * this many).
#ifndef TACO_REDUCE_TILES_PER_WAVE
#define TACO_REDUCE_TILES_PER_WAVE 1
#endif
constexpr int kReduceTilesPerWave = TACO_REDUCE_TILES_PER_WAVE;
static_assert(kReduceTilesPerWave > 0, "tiles per wave");

hipError_t launch_fp8_had_compress(const FP8HadArgs& a, hipStream_t s);
hipError_t launch_fp8_had_decode(const FP8HadDecodeArgs& a, hipStream_t s);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_ring_hop(const HopArgs& a, hipStream_t s);
hipError_t launch_fp8_encode(bool e5, const float* x, uint8_t* out, int64_t n, hipStream_t s);
hipError_t launch_dequant_gemm(const DGemmArgs& a, hipStream_t s);
hipError_t launch_chunk_order(const void* stats, int64_t rows, int64_t cols, int32_t* order, hipStream_t s);

}  // namespace taco

// The order of the data-driven reshaping: rank the hidden dimension's groups
// of 8 channels by their largest magnitude over a statistics tensor.
//
// Source: "TACO: Efficient Communication Compression of Intermediate Tensors
// for Scalable Tensor-Parallel LLM Training" (Pith review page) -- abstract
// and "What carries the argument": the tensor is reshaped adaptively, from
// the data, before the Adaptive Scale-Hadamard Transform; the page leaves the
// rule open. Here the groups are ranked largest magnitude first, equal
// magnitudes by group index, so that the blocks of the reordered tensor hold
// channels of similar magnitude.
//
// Four launches on the caller's stream, with the output array as the only
// memory: it first holds each group's abs-max (float bits, as unsigned
// integers they order like the non-negative floats they are; the abs-max of
// bf16 values has zero low 16 bits), then the abs-max with each group's rank in
// the low 16 bits, then the order.
#include "device_common.h"
#include "taco_internal.h"

namespace taco {

constexpr int kRankThreads = 1024;   // the scatter's workgroup
constexpr int kStatRows = 64;   // rows per workgroup of the statistics pass

__global__ __launch_bounds__(kBlockThreads) void k_zero_u32(uint32_t* p, int n) {
  const int i = (int)(blockIdx.x * kBlockThreads + threadIdx.x);
  if (i < n) p[i] = 0u;
}

// Workgroup (s, b): span s of every row (64 groups, one per lane) over the
// row blocks b, b + gridDim.y, ... of 64 rows, the four waves taking every
// fourth row; one atomic max per group and workgroup. |x| is formed on the
// bits; NaN counts as infinity.
__global__ __launch_bounds__(kBlockThreads) void k_group_absmax(const uint16_t* __restrict__ x, int64_t rows,
                                                                int cols, uint32_t* __restrict__ gmax) {
  __shared__ uint32_t part[kBlockThreads / kWave][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_in_group();
  const int group = (int)blockIdx.x * kWave + lane;
  uint32_t m = 0u;
  for (int64_t r0 = (int64_t)blockIdx.y * kStatRows; r0 < rows; r0 += (int64_t)gridDim.y * kStatRows) {
    for (int64_t r = r0 + wave; r < rows && r < r0 + kStatRows; r += kBlockThreads / kWave) {
      const uint4 w = ld16_nt(x + r * cols + (int64_t)group * kGroupElems);
      const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (h[i] << 16) & 0x7FFFFFFFu, hi = h[i] & 0x7FFF0000u;
        m = max(m, max(lo, hi));
      }
    }
  }
  m = min(m, 0x7F800000u);   // NaN -> infinity
  part[wave][lane] = m;
  __syncthreads();
  if (wave == 0) {
    uint32_t v = part[0][lane];
#pragma unroll
    for (int w = 1; w < kBlockThreads / kWave; ++w) v = max(v, part[w][lane]);
    __hip_atomic_fetch_max(&gmax[group], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Group j's rank is #{i : a_i > a_j} + #{i < j : a_i = a_j}. Workgroup
// (bj, bi) counts, for each group j of tile bj, the groups i of tile bi that
// precede it and adds the count into the low 16 bits of j's entry (ranks are
// below 2^14). Every read masks those bits off, so tiles running at the same
// time see the same abs-maxima.
constexpr int kRankTile = 256;
constexpr uint32_t kValueBits = 0xFFFF0000u;
__global__ __launch_bounds__(kRankTile) void k_rank_tiles(uint32_t* __restrict__ buf, int ngroups) {
  __shared__ __attribute__((aligned(16))) uint32_t ai[kRankTile];
  const int i0 = (int)blockIdx.y * kRankTile, j = (int)blockIdx.x * kRankTile + (int)threadIdx.x;
  const int ni = ngroups - i0 < kRankTile ? ngroups - i0 : kRankTile;
  if ((int)threadIdx.x < ni) ai[threadIdx.x] = buf[i0 + threadIdx.x] & kValueBits;
  __syncthreads();
  if (j >= ngroups) return;
  const uint32_t aj = buf[j] & kValueBits;
  // ni is a multiple of 64 (cols is a multiple of 512): four entries per LDS
  // read, several reads in flight
  uint32_t cnt = 0;
#pragma unroll 4
  for (int t = 0; t < ni; t += 4) {
    const uint4 q = *reinterpret_cast<const uint4*>(&ai[t]);
    const int i = i0 + t;
    cnt += (q.x > aj) || (q.x == aj && i < j);
    cnt += (q.y > aj) || (q.y == aj && i + 1 < j);
    cnt += (q.z > aj) || (q.z == aj && i + 2 < j);
    cnt += (q.w > aj) || (q.w == aj && i + 3 < j);
  }
  if (cnt != 0) __hip_atomic_fetch_add(&buf[j], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup: read every group's rank into LDS, then write order[rank] = j
// into the same array (every read happens before the barrier).
__global__ __launch_bounds__(kRankThreads) void k_scatter_order(uint32_t* __restrict__ buf, int ngroups) {
  extern __shared__ uint32_t rank[];
  for (int i = (int)threadIdx.x; i < ngroups; i += kRankThreads) rank[i] = buf[i] & ~kValueBits;
  __syncthreads();
  for (int j = (int)threadIdx.x; j < ngroups; j += kRankThreads) buf[rank[j]] = (uint32_t)j;
}

hipError_t launch_chunk_order(const void* stats, int64_t rows, int64_t cols, int32_t* order, hipStream_t s) {
  const int ngroups = (int)(cols / kGroupElems);
  auto* buf = reinterpret_cast<uint32_t*>(order);
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((ngroups + kBlockThreads - 1) / kBlockThreads)),
                     dim3(kBlockThreads), 0, s, buf, ngroups);
  if (rows > 0) {
    const int64_t blocks = (rows + kStatRows - 1) / kStatRows;
    const dim3 grid((unsigned)(cols / kSpanElems), (unsigned)(blocks < 4096 ? blocks : 4096));
    hipLaunchKernelGGL(k_group_absmax, grid, dim3(kBlockThreads), 0, s, static_cast<const uint16_t*>(stats), rows,
                       (int)cols, buf);
  }
  const unsigned tiles = (unsigned)((ngroups + kRankTile - 1) / kRankTile);
  hipLaunchKernelGGL(k_rank_tiles, dim3(tiles, tiles), dim3(kRankTile), 0, s, buf, ngroups);
  hipLaunchKernelGGL(k_scatter_order, dim3(1), dim3(kRankThreads), (size_t)ngroups * 4, s, buf, ngroups);
  return hipGetLastError();
}

}  // namespace taco

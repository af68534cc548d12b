/*
 * taco.h -- C ABI of the MI355X (gfx950) library that compresses and
 * decompresses tensor-parallel activations.
 *
 * What it computes, by source (Pith review pages, cited by title and the
 * section or figure on them):
 *
 *  [TACO]      "TACO: Efficient Communication Compression of Intermediate
 *              Tensors for Scalable Tensor-Parallel LLM Training": Fig. 7
 *              (adaptive rescaling -> ASH transform -> dual-scale FP8
 *              quantization), Fig. 9 (one fused compression operator), Fig. 3
 *              (E4M3), Fig. 6 / Eq. (3) (FP8 rounding error bound).
 *  [EQuARX]    "EQuARX: Efficient Quantized AllReduce in XLA for Distributed
 *              Machine Learning Acceleration": "What carries the argument"
 *              (dynamic block-wise symmetric int8, one FP32 scale per 64
 *              entries, dequantize to FP32 before adding; the quantized
 *              ring reduce-scatter hop).
 *  [FlashComm] "Flash Communication: Reducing Tensor Parallelization
 *              Bottleneck for Fast Large Language Model Inference": "What
 *              carries the argument" (asymmetric group-128 INT4/INT8, local sum
 *              of all chunks, INT8 re-quantization for the gather), Algorithm 1
 *              (dequantize from codes, zero point and scale).
 *
 * Conventions shared by every entry point
 *  - Tensors are row-major [rows, cols]; blocks (groups) are `block`
 *    contiguous elements along cols, so cols must be a multiple of block. The
 *    tensor is treated as n / block independent blocks (n = rows * cols).
 *  - Device pointers are HIP device memory owned by the caller, 16-byte
 *    aligned; the library allocates nothing and keeps no pointer after a
 *    call returns. Inputs are never written; outputs must not overlap inputs.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    the caller synchronizes. All validation happens before anything is
 *    enqueued; a call that returns an error has enqueued nothing.
 *  - Host state: per-device caches filled on first use (the CU count, the
 *    occupancy the reordering kernels size their grids by, the address of
 *    the scratch array of taco_compress_noalloc), each under an atomic or a
 *    lock, and the calling thread's launch cap (taco_set_launch_limit).
 *    Calls from several host threads are safe; calls that share a workspace
 *    or the scratch array must be ordered on the device by the caller.
 *  - rows == 0 is valid and enqueues nothing; rows * cols above 2^35 is
 *    TACO_ERR_INVALID_ARG.
 *  - Return value: TACO_OK or a negative TACO_ERR_* code
 *    (taco_status_string names it).
 *  - Values are finite: for blocks whose inputs or intermediate results are
 *    not finite the codes of that block are unspecified (no crash, other
 *    blocks unaffected; with the data-driven FP8 tensor scale the whole
 *    tensor is affected).
 */
#ifndef TACO_H_
#define TACO_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define TACO_OK 0
#define TACO_ERR_INVALID_ARG (-1) /* null pointer, bad size, n out of [1,16], bad tensor_scale */
#define TACO_ERR_SHAPE (-2)       /* cols not a multiple of block, or block not allowed for the format */
#define TACO_ERR_FORMAT (-3)      /* unknown format, hadamard on a non-FP8 format, pair not allowed */
#define TACO_ERR_ALIGN (-4)       /* a device pointer not 16-byte aligned */
#define TACO_ERR_WORKSPACE (-5)   /* workspace missing or too small where one is required */
#define TACO_ERR_HIP (-6)         /* a kernel launch failed (hipGetLastError) */

/* ---- formats ------------------------------------------------------------
 * TACO_FMT_FP8_DUAL  [TACO] E4M3 codes with a float32 tensor scale g and a
 *                    per-block power-of-two exponent k (value = dec(q) * 2^-k * g);
 *                    block 16, 32, 64 or 128; hadamard = 1 applies the
 *                    unnormalised Sylvester Walsh-Hadamard transform to every
 *                    block before quantizing (the ASH transform).
 * TACO_FMT_INT8_SYM  [EQuARX] int8 in [-127, 127], float32 scale s = absmax / 127
 *                    per block of 64 (value = q * s).
 * TACO_FMT_INT4_ASYM [FlashComm] 4-bit codes, two per byte (element 2j in the
 *                    low nibble), float32 scale s and uint8 zero point z per
 *                    group of 128 (value = (q - z) * s). Compression writes
 *                    z in [0, 15]; buffers read back must keep z <= 15
 *                    (larger zero points give unspecified values).
 * TACO_FMT_INT8_ASYM [FlashComm] the same at 8 bits (gather stage).
 * TACO_FMT_FP8E5_DUAL the TACO dual-scale scheme with E5M2 codes instead of
 *                    E4M3 ([TACO] Fig. 3 sets E5M2 beside E4M3; bit layout of
 *                    "FP8 Formats for Deep Learning", in TACO's reference list):
 *                    the block exponent k brings each block maximum into
 *                    (28672, 57344], AUTO g = abs-max / 57344; block, hadamard,
 *                    layout, workspace and scale modes as TACO_FMT_FP8_DUAL.
 */
#define TACO_FMT_FP8_DUAL 1
#define TACO_FMT_INT8_SYM 2
#define TACO_FMT_INT4_ASYM 3
#define TACO_FMT_INT8_ASYM 4
#define TACO_FMT_FP8E5_DUAL 5

typedef struct taco_codec {
  int32_t format;   /* TACO_FMT_* */
  int32_t block;    /* elements per block / group along cols */
  int32_t hadamard; /* FP8 only: 1 = block Walsh-Hadamard transform */
  int32_t reserved; /* must be 0 */
} taco_codec;

/* Byte layout of one compressed tensor: one caller-allocated buffer of
 * total_bytes, regions at 256-byte aligned offsets:
 *   codes   n bytes (INT4: n / 2)
 *   scale   FP8: int8 k[n / block]; others: float32 s[n / block]
 *   aux     asymmetric formats: uint8 z[n / block]; others: empty
 *   tensor  FP8: float32 g (16 bytes reserved); others: empty           */
typedef struct taco_layout_t {
  int64_t codes_off, codes_bytes;
  int64_t scale_off, scale_bytes;
  int64_t aux_off, aux_bytes;
  int64_t tensor_off, tensor_bytes;
  int64_t total_bytes;
} taco_layout_t;

/* tensor_scale values for taco_compress / taco_requantize (FP8 formats only):
 *   > 0   use this g; it must lie in [2^-60, 2^60]
 *   AUTO  g from this tensor: an abs-max pass over the transformed values
 *         first, g = absmax / 448 (E5M2: / 57344; 1 for an all-zero tensor),
 *         clamped to [2^-60, 2^60]. Needs a workspace.
 *   DELAYED  g from the abs-max the workspace recorded in its previous call
 *         (1 if none): one pass; the history lives in the caller's workspace.
 * Every FP8 call given a workspace records its own abs-max there.          */
#define TACO_SCALE_AUTO 0.0f
#define TACO_SCALE_DELAYED (-1.0f)
#define TACO_MAX_SHARDS 16
#define TACO_WORKSPACE_BYTES 32768

/* Layout of a compressed [rows, cols] tensor. Host only. */
int taco_layout(taco_codec c, int64_t rows, int64_t cols, taco_layout_t* out);

/* total_bytes of taco_layout, or a negative status. Host only. */
int64_t taco_compressed_bytes(taco_codec c, int64_t rows, int64_t cols);

/* Workspace size the FP8 scale modes need (TACO_WORKSPACE_BYTES; 0 for the
 * other formats). The workspace is caller-owned device memory, zero-filled
 * once before its first use; every call leaves it in a reusable state and
 * carries the abs-max history for TACO_SCALE_DELAYED. Calls sharing one
 * workspace must be ordered (same stream). Host only. */
size_t taco_workspace_bytes(taco_codec c, int64_t rows, int64_t cols);

/* Compress one bf16 shard: [TACO] Fig. 7 / Fig. 9 (transform, tensor scale,
 * block exponent and E4M3 codes in one pass), [EQuARX] block-wise INT8,
 * [FlashComm] group-128 asymmetric INT4/INT8.
 *   x_bf16   device, bf16 [rows, cols]
 *   out      device, taco_compressed_bytes(c, rows, cols) bytes (see layout)
 *   tensor_scale, workspace, ws_bytes: FP8 only (see above); ignored otherwise */
int taco_compress(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale, void* out,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* taco_compress for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and outputs, with the FP8 tensor-scale workspace taken
 * from a TACO_WORKSPACE_BYTES (32 KiB) array that the library holds in each
 * GPU's memory until the process ends, instead of a workspace argument. The
 * call allocates nothing and calls no allocating routine. The array is the
 * same size for every tensor, so no size is too large for it (the 2^35
 * element limit of every entry point applies).
 *   - Every call on one GPU shares that GPU's array: TACO_SCALE_DELAYED takes
 *     the abs-max recorded by the previous FP8 call on that GPU (any stream,
 *     any caller), and every FP8 call records its own. Calls that overlap on
 *     one GPU (concurrent streams or host threads) race on it: order them.
 *   - The first call on a device clears the array with a fill kernel on
 *     `stream`, ordered before its own work; a graph that captured that first
 *     call clears it again on every replay.
 *   - Non-FP8 formats use no workspace; this call then equals taco_compress.
 * Errors as taco_compress; TACO_ERR_HIP also when the array's device address
 * cannot be obtained. */
int taco_compress_noalloc(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale,
                          void* out, hipStream_t stream);

/* taco_compress that also writes, for every element, the float32 value handed
 * to the final rounding step (FP8: the scaled value encoded to E4M3; INT:
 * value * (1/scale) before rounding) to `prequant` (device, n floats). */
int taco_compress_debug(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale, void* out,
                        void* workspace, size_t ws_bytes, float* prequant, hipStream_t stream);

/* Decompress-reduce: dequantize each of n shards to float32 and add them in
 * shard order, acc = ((0 + x_0) + x_1) + ..., one float32 rounding per add
 * ([EQuARX]: dequantize to FP32 before adding; [FlashComm]: local sum of the
 * chunks). Then, optionally,
 *   sum_fp32     device float32 [rows, cols] receives acc (nullable)
 *   requant_out  device buffer in c_out's layout receives acc re-quantized for
 *                the gather stage (nullable): FP8 -> FP8 (same code format) with tensor scale
 *                g' = g_0 + ... + g_{n-1} and no second transform (the
 *                transform is linear and shared by all shards); INT8_SYM ->
 *                INT8_SYM; INT4_ASYM -> INT8_ASYM; INT8_ASYM -> INT8_ASYM. FP8
 *                pairs need equal block and hadamard.
 * At least one output must be given.
 *   shards   host array of n device pointers, each a buffer in c_in's layout
 *   n        1 .. TACO_MAX_SHARDS                                            */
int taco_decompress_reduce(taco_codec c_in, const void* const* shards, int32_t n, int64_t rows, int64_t cols,
                           float* sum_fp32, taco_codec c_out, void* requant_out, hipStream_t stream);

/* One hop of a quantized ring reduce-scatter ([EQuARX] "What carries the
 * argument": a received shard is dequantized to FP32 before the receiver adds
 * its own contribution, and the partial sum is quantized again for the next
 * hop; the full-loop ring takes N - 1 hops):
 *   acc = (0 + dequant(incoming)) + local, one float32 rounding per add,
 * then, optionally,
 *   sum_fp32     device float32 [rows, cols] receives acc (nullable)
 *   requant_out  device buffer in c_out's layout receives acc quantized for
 *                the next hop (nullable)
 * At least one output must be given.
 *   incoming     device buffer in c_in's layout, or NULL for the first hop
 *                (acc = 0 + local; c_in must still be a valid codec)
 *   local_bf16   device bf16 [rows, cols], this rank's contribution
 * Pairs: INT8_SYM -> INT8_SYM, INT4_ASYM -> INT8_ASYM, INT8_ASYM -> INT8_ASYM.
 * The FP8 codec is not a ring codec (its shards live in the Hadamard domain
 * and its gather scale would need the local tensor's abs-max):
 * TACO_ERR_FORMAT. */
int taco_ring_hop(taco_codec c_in, const void* incoming, const void* local_bf16, int64_t rows, int64_t cols,
                  float* sum_fp32, taco_codec c_out, void* requant_out, hipStream_t stream);

/* Quantize a caller-supplied float32 tensor with c_out: the gather-stage
 * re-quantization on its own ([FlashComm] "What carries the argument": the
 * locally summed partial results are quantized again, to INT8, before the
 * All-Gather; [EQuARX] "What carries the argument": the partial sum is
 * quantized again before it is sent on; [TACO] Fig. 7: dual-scale FP8
 * quantization of values already in the transformed domain). FP8 takes the
 * values as already transformed (no transform is applied); tensor_scale /
 * workspace as for taco_compress. */
int taco_requantize(taco_codec c_out, const float* x_fp32, int64_t rows, int64_t cols, float tensor_scale, void* out,
                    void* workspace, size_t ws_bytes, hipStream_t stream);

/* Consumer-side decode of one compressed tensor to float32 (out_dtype 0) or
 * bf16 (out_dtype 1, nearest-even): dequantize ([FlashComm] Algorithm 1:
 * dequantization from codes, zero point and scale; [EQuARX] "What carries the
 * argument": q * s) and, for FP8 with hadamard, undo the ASH transform of
 * [TACO] Fig. 7 (x = H y * 2^-log2(block), since H H = block * I). */
int taco_decompress(taco_codec c, const void* in, int64_t rows, int64_t cols, void* out, int32_t out_dtype,
                    hipStream_t stream);

/* Test hooks: the device's E4M3 / E5M2 encoder (the one every FP8 kernel of
 * that format uses) on n float32 values; codes are 1 byte each. Same argument
 * rules as above. */
int taco_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);
int taco_e5m2_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);

/* ---- data-driven reshaping ------------------------------------------------
 * [TACO] abstract and "What carries the argument": the tensor is reshaped
 * adaptively, from the data, before the ASH transform (the rule is not given).
 * Here: the hidden channels are taken in groups of 8 consecutive channels and
 * the codec sees the groups in an order computed from a statistics tensor
 * (e.g. an earlier step's activation; every rank must use the same order):
 * largest magnitude first, equal magnitudes by group index, so that each
 * block holds channels of similar magnitude. `order` is a device int32 array
 * of cols / 8 entries, reordered group j being original group order[j] of the
 * same row; it must be a permutation of [0, cols / 8) (other values are
 * clamped into range: no fault and no access outside the row or the output,
 * but unspecified codes and decoded values). Shapes: cols a multiple
 * of 512 and at most 131072, FP8 block 128 (TACO_ERR_SHAPE otherwise).
 * Compressed buffers, decompress-reduce, requantize and the ring hop work on
 * the reordered tensor unchanged; taco_decompress_reordered restores the
 * original channel order. */

/* The order of the groups of a statistics tensor (device bf16 [rows, cols];
 * rows may be 0: identity order) into `order` (device int32 [cols / 8]).
 * Four launches on `stream`; `order` is their only memory. */
int taco_chunk_order(const void* stats_bf16, int64_t rows, int64_t cols, int32_t* order, hipStream_t stream);

/* taco_compress of the reordered tensor: column 8 j + i of the tensor the
 * codec sees is column 8 order[j] + i of x_bf16 (same row). Arguments and
 * errors as taco_compress, plus `order` (device, 16-byte aligned). */
int taco_compress_reordered(taco_codec c, const void* x_bf16, int64_t rows, int64_t cols, float tensor_scale,
                            void* out, void* workspace, size_t ws_bytes, const int32_t* order, hipStream_t stream);

/* taco_decompress of a buffer holding a reordered tensor, writing each
 * decoded group j to original group order[j] of its row. */
int taco_decompress_reordered(taco_codec c, const void* in, int64_t rows, int64_t cols, void* out, int32_t out_dtype,
                              const int32_t* order, hipStream_t stream);

/* ---- decode fused into the consumer -----------------------------------
 * [FlashComm] "What carries the argument" and Fig. 8: the quantized volume is
 * dequantized on the receiving side and handed to the next computation. This
 * is that computation for a linear layer, with the decode in its prologue:
 *   out[M, N] = decode(A)[M, K] * W^T,
 * where decode(A) is the bf16 tensor taco_decompress(c, a, M, K, ., 1, .)
 * writes (each value the nearest-even bf16 of its float32 decoded value,
 * which is the single rounding of the exact one; for a NaN the sign and
 * payload may differ), W is bf16 [N, K] row-major (the
 * weight layout of a linear layer), and the products are summed in float32
 * on the matrix cores. The decoded activation is never written to memory.
 *   c          a compressed format without the Hadamard transform: INT8_SYM,
 *              INT4_ASYM, INT8_ASYM, or FP8_DUAL / FP8E5_DUAL with hadamard 0
 *              and block 32, 64 or 128 (hadamard 1 or block 16:
 *              TACO_ERR_FORMAT / TACO_ERR_SHAPE)
 *   a          device buffer in the compressed layout of an [M, K] tensor
 *   M, N, K    multiples of 128 and K at most 2^20 (else TACO_ERR_SHAPE),
 *              K >= 128, N >= 128 (256 x 256 output tiles when M and N are
 *              multiples of 256, else 128 x 128);
 *              M may be 0 (nothing enqueued); M * K, N * K and M * N at most
 *              2^35 (else TACO_ERR_INVALID_ARG)
 *   w          device bf16 [N, K]
 *   out        device [M, N], float32 (out_dtype 0) or bf16 (1, nearest-even);
 *              must overlap neither a nor w
 * One launch on `stream`; the launch cap does not apply (one workgroup per
 * 128 x 128 output tile). */
int taco_decompress_gemm(taco_codec c, const void* a, int64_t M, int64_t K, const void* w_bf16, int64_t N, void* out,
                         int32_t out_dtype, hipStream_t stream);

/* Cap on the workgroups of every later launch made by the calling host
 * thread (0 = no cap, the default): lets the codec share the GPU with a
 * concurrent kernel, e.g. the GEMM that produces the next activation on
 * another stream ([TACO] abstract: the compression operator is built so that
 * it overlaps with other work). Each kernel walks its tiles with a stride of
 * its grid, so the results are the same under any cap; only the speed and the
 * share of the GPU change. Applies to taco_compress, taco_compress_noalloc,
 * taco_compress_debug, taco_compress_reordered, taco_requantize,
 * taco_decompress_reduce, taco_ring_hop, taco_decompress and
 * taco_decompress_reordered; not to taco_chunk_order or the encoder test
 * hooks.
 *   max_workgroups  >= 0 (256 threads each); negative is TACO_ERR_INVALID_ARG
 *   previous        nullable; receives the cap that was in force
 * Host only; the setting is per host thread. */
int taco_set_launch_limit(int32_t max_workgroups, int32_t* previous);

/* Name of a status code. Host only; never returns NULL. */
const char* taco_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TACO_H_ */

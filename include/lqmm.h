/*
 * lqmm.h -- C interface of liblqmm, block-quantized weight matrix multiply for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the hot path of local LLM inference described in
 * "Resumo Tecnico: Llamas na Web" (summary of the LlamaWeb paper), section
 * "Design de Shader Consciente de Quantizacao": for the decode mat-vec the
 * llama.cpp weight blocks are dequantized directly in registers; for the
 * prefill matmul the blocks are loaded, dequantized into shared memory (LDS
 * here) and reused. The plain tiled fp32 matmul is the one printed in
 * "Compute Shaders con WebGPU para Inferencia ML", section "El Nucleo:
 * Multiplicacion de Matrices en WGSL".
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *   owned by the caller. The library never allocates, frees or synchronizes.
 * - Every matrix is dense, row-major and contiguous; fp16 values are raw
 *   IEEE binary16 bits (uint16_t).
 * - Every pointer must be 16-byte aligned (LQMM_ERR_ALIGN otherwise).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). A call
 *   only validates its arguments and enqueues kernels on that stream; it
 *   returns before the GPU work finishes. Device-side faults surface at the
 *   caller's next synchronization.
 * - All argument checks run on the host before any HIP call, so invalid
 *   arguments are reported without touching the GPU and with nothing
 *   enqueued. Sizes are int64_t; sizes <= 0 are LQMM_ERR_SHAPE (an empty
 *   problem is not a call to make). Outputs must not overlap inputs.
 * - Calls are thread-safe and re-entrant: the only library state is set up
 *   once per device under std::call_once (the device's properties, and each
 *   kernel's LDS limit on its first launch there).
 * - NaN and Inf inputs propagate; no value is checked.
 *
 * Weight block layouts (llama.cpp / GGUF style). The pages name the formats
 * (legacy Q4_0/Q8_0 and the K-quants) and describe them as flat buffers of
 * packed integers with the dequantization chosen at compile time; the byte
 * layout below is the llama.cpp one:
 *   Q4_0: 32 weights in 18 bytes: [d: fp16][qs: 16 bytes]. Weight j (j < 16)
 *         is the low nibble of qs[j], weight j+16 its high nibble;
 *         w = d * (q - 8) with q in 0..15.
 *   Q8_0: 32 weights in 34 bytes: [d: fp16][q: 32 x int8]; w = d * q.
 *   Q4_K: 256 weights in 144 bytes: [d: fp16][dmin: fp16][scales: 12 bytes]
 *         [qs: 128 bytes]. Sub-block s (weights 32s..32s+31) has a 6-bit
 *         scale sc_s and a 6-bit min m_s packed in `scales`:
 *           s < 4 : sc_s = scales[s] & 63,  m_s = scales[s+4] & 63
 *           s >= 4: sc_s = (scales[s+4] & 15) | ((scales[s-4] >> 6) << 4)
 *                   m_s  = (scales[s+4] >> 4) | ((scales[s]   >> 6) << 4)
 *         Weight l of sub-block s has q = the low (even s) or high (odd s)
 *         nibble of qs[32*(s/2) + l]; w = d * sc_s * q - dmin * m_s.
 * A quantized weight matrix W has N rows (output features) of K weights
 * (input features); row n is stored as K/32 (Q4_0, Q8_0) or K/256 (Q4_K)
 * consecutive blocks, and rows follow each other with no padding. fp16
 * scales are used as stored, subnormals included.
 *
 * Precision
 * ---------
 * Accumulation is fp32 everywhere. The quantized GEMVs round each activation
 * x to fp16 (round to nearest even, no scaling) before the dot products:
 * |x| must stay below 65504 (larger values become infinite), and in the
 * fp16 normal range, 2^-14 <= |x| < 65504, x contributes a relative rounding
 * error of at most 2^-11 per element; smaller |x| are rounded to fp16
 * subnormals, an absolute error of at most 2^-25 per element. For one or two
 * activation rows per pass the dequantized weights are exact (the block
 * scales are applied in fp32). From three rows up the GEMVs run on the fp16
 * matrix cores and round each dequantized weight to fp16: Q4_0 once
 * (d*(q-8)); Q4_K rounds d*sc and dmin*m to fp16 once per sub-block and then
 * each weight once (one fused multiply-add).
 * The Q8_0 GEMM rounds each dequantized weight d*q to fp16 (one rounding)
 * and the output to fp16. The fp32 GEMM uses fp32 matrix-core products with
 * fp32 accumulation.
 */
#ifndef LQMM_H
#define LQMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LQMM_OK = 0,
  LQMM_ERR_NULL = 1,      /* a required pointer is NULL */
  LQMM_ERR_SHAPE = 2,     /* a size is <= 0, not a block multiple, or too large */
  LQMM_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  LQMM_ERR_WORKSPACE = 4, /* the call needs a workspace (split-K partial sums) and got none or too small a one */
  LQMM_ERR_DEVICE = 5,    /* no usable HIP device, or it is not a gfx950 GPU */
  LQMM_ERR_LAUNCH = 6     /* a kernel launch failed (hipGetLastError) */
} lqmm_status;

/* Largest size accepted for any dimension (elements). */
#define LQMM_MAX_DIM ((int64_t)1 << 31)
/* lqmm_gemm_q8_0_f16 needs K < LQMM_GEMM_MAX_K (LQMM_ERR_SHAPE otherwise). */
#define LQMM_GEMM_MAX_K ((int64_t)1 << 22)

/*
 * Dense fp32 GEMM: C[M x N] = A[M x K] * B[K x N], all fp32 row-major.
 * The tiled matmul of "Compute Shaders con WebGPU para Inferencia ML",
 * "El Nucleo: Multiplicacion de Matrices en WGSL": any M, N, K >= 1, ragged
 * edges handled by zero padding, C overwritten (no alpha/beta).
 */
lqmm_status lqmm_sgemm(const float *A, const float *B, float *C,
                       int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Q4_0 GEMV (decode): y[b][n] = sum_k W[n][k] * x[b][k] for b < batch.
 * W: N x (K/32) Q4_0 blocks (N*K/32*18 bytes); x: batch x K fp32;
 * y: batch x N fp32 (overwritten). K % 32 == 0; any batch >= 1 (the batch
 * rows share each weight load: up to 2 rows per pass on the vector ALUs, up
 * to 16 per pass on the matrix cores, which take over from 3 rows).
 * Dequantization happens in registers ("Llamas na Web", "Design de Shader
 * Consciente de Quantizacao", mat-vec case).
 * workspace/workspace_bytes: device memory for split-K plans, which split a
 * row's K range over several workgroups (on different CUs) and add their
 * partial sums in a fixed order (results do not depend on timing). At least
 * lqmm_gemv_workspace_bytes(N, K, batch) bytes, 16-byte aligned, owned by
 * the caller, zero-filled once before its first use: every completed call
 * leaves the bytes it used (arrival counters and partial sums) zero again. Calls that may run at the same
 * time (other streams, other threads) must not share a workspace. NULL (or
 * too few bytes) is valid: the planner then uses no split-K plan, except
 * when a tuning override forces one (LQMM_ERR_WORKSPACE).
 */
lqmm_status lqmm_gemv_q4_0(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * lqmm_gemv_q4_0 for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments (without the workspace) and same
 * results as lqmm_gemv_q4_0 given a workspace. Its split-K plans use a
 * static device array of LQMM_NOALLOC_SCRATCH_BYTES instead, one per GPU,
 * held until the process ends; the call itself allocates and frees nothing.
 * Before each split-K launch it zeroes the plan's arrival counters with a
 * kernel on `stream`. Every call on a GPU shares that GPU's array, so calls
 * that may overlap on one GPU (other streams, other threads) race: order
 * them. A split-K plan needing more scratch than the array holds (possible
 * only when a tuning override forces one) returns LQMM_ERR_WORKSPACE.
 */
#define LQMM_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
lqmm_status lqmm_gemv_q4_0_noalloc(const void *W, const float *x, float *y,
                                   int64_t N, int64_t K, int64_t batch, void *stream);

/*
 * Q8_0 x fp16 GEMM (prefill): Y[m][n] = sum_k X[m][k] * W[n][k], i.e.
 * Y = X * W^T. W: N x (K/32) Q8_0 blocks; X: M x K fp16; Y: M x N fp16
 * (fp32 accumulation, rounded to nearest even at the end). K % 32 == 0 and
 * K < LQMM_GEMM_MAX_K.
 * The raw weight blocks of each output tile are loaded into LDS and each
 * weight is dequantized once per workgroup, in registers, into the fp16
 * matrix-core operand that every row of the M tile reuses ("Llamas na Web",
 * "Design de Shader Consciente de Quantizacao", matmul case: blocks loaded
 * into shared memory, dequantized and reused). When K % 64 == 32 a second
 * kernel writes dequantized fp16 tiles to LDS instead.
 */
lqmm_status lqmm_gemm_q8_0_f16(const void *W, const uint16_t *X, uint16_t *Y,
                               int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Q4_K GEMV (decode): y[b][n] = sum_k W[n][k] * x[b][k].
 * W: N x (K/256) Q4_K super-blocks (N*K/256*144 bytes); x: batch x K fp32;
 * y: batch x N fp32. K % 256 == 0; any batch >= 1. Arguments as for
 * lqmm_gemv_q4_0.
 */
lqmm_status lqmm_gemv_q4_k(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * The other format x phase pairs and more block formats. "Llamas na Web",
 * "Design de Shader Consciente de Quantizacao" applies both kernel styles to
 * every quantization format (mat-vec: dequantize in registers; matmul:
 * dequantize into shared memory and reuse) and adds a format by adding its
 * dequantization routine.
 *
 * Decode GEMVs y[b][n] = sum_k W[n][k] * x[b][k]; arguments, layouts,
 * workspace and precision as for lqmm_gemv_q4_0 (x rounded to fp16, block
 * scales applied in fp32, fp32 accumulation; every activation row on the
 * vector ALUs, in passes of up to four rows). Split-K plans, for rows longer
 * than one wave's slice (2048 weights of Q8_0 or the int4 layout, 4096 when
 * N is at least four times the CU count; 8192 of Q6_K or Q2_K; 2048 of
 * q1_0, 4096 when N is at least four times the CU count), need the
 * workspace (LQMM_ERR_WORKSPACE without it).
 *   lqmm_gemv_q8_0: W is N x (K/32) Q8_0 blocks (34 bytes), K % 32 == 0.
 *   lqmm_gemv_q6_k: W is N x (K/256) Q6_K super-blocks (210 bytes), K % 256 ==
 *     0. Super-block: [ql 128][qh 64][scales 16 x int8][d fp16];
 *     w = d * scales[k/16] * (q - 32), q = 6 bits: weight k = 128h + 32j + l
 *     (h < 2, j < 4, l < 32) has low 4 bits from the low (j < 2) or high
 *     (j >= 2) nibble of ql[64h + 32(j%2) + l], high 2 bits from bits
 *     2j..2j+1 of qh[32h + l].
 *   lqmm_gemv_q2_k: W is N x (K/256) Q2_K super-blocks (84 bytes), K % 256 ==
 *     0. Super-block: [scales 16][qs 64][d fp16][dmin fp16]; scales[g] =
 *     sc | m << 4 for weights 16g..16g+15; w = d * sc * q - dmin * m, q =
 *     bits 2j..2j+1 of qs[32h + l] for weight k = 128h + 32j + l.
 *   lqmm_gemv_q1_0: the 1-bit format "Llamas na Web" names under
 *     "Extensibilidade" (q1_0; the page gives no bytes), read as the _0
 *     family at one bit per weight: W is N x (K/32) blocks of 6 bytes,
 *     [d fp16][4 bytes of code bits]; the bit c of weight j is bit j % 8 of
 *     code byte j / 8; w = d * (2c - 1). K % 32 == 0.
 *   lqmm_gemv_i4g32: the int4 layout of "Compute Shaders con WebGPU para
 *     Inferencia ML", "Yendo a Cuantizado: Matmul INT4" (GPTQ/AWQ style):
 *     Wq holds N*K/8 32-bit words, weight (n, k) being nibble (n*K + k) % 8
 *     (bits 4i..4i+3) of word (n*K + k) / 8, a two's-complement code s in
 *     -8..7; scales and zeros are fp32 arrays of N x K/32 (per row and group
 *     of 32 along K); w = (s - zero) * scale. K % 32 == 0. (The page writes
 *     result[row * N + col] with row = weight row; y here is batch x N like
 *     every GEMV of this library.)
 */
lqmm_status lqmm_gemv_q8_0(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);
lqmm_status lqmm_gemv_q6_k(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);
lqmm_status lqmm_gemv_q2_k(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);
lqmm_status lqmm_gemv_q1_0(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);
lqmm_status lqmm_gemv_i4g32(const uint32_t *Wq, const float *scales,
                            const float *zeros, const float *x, float *y,
                            int64_t N, int64_t K, int64_t batch,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefill GEMMs Y = X * W^T over Q4_0 (K % 32 == 0) and Q4_K (K % 256 == 0)
 * weights: X is M x K fp16, Y is M x N fp16, fp32 accumulation, K <
 * LQMM_GEMM_MAX_K. Each step's blocks are dequantized to fp16 into LDS
 * tiles reused by the whole M tile: each weight rounded once to fp16 (Q4_0
 * d*(q-8); Q4_K d*sc*q - dmin*m formed in fp32). Output rounded to nearest
 * even.
 */
lqmm_status lqmm_gemm_q4_0_f16(const void *W, const uint16_t *X, uint16_t *Y,
                               int64_t M, int64_t N, int64_t K, void *stream);
lqmm_status lqmm_gemm_q4_k_f16(const void *W, const uint16_t *X, uint16_t *Y,
                               int64_t M, int64_t N, int64_t K, void *stream);

/* Workspace the GEMV calls of these sizes can use, in bytes (0 = none):
 * enough for every GEMV entry point on any device. */
size_t lqmm_gemv_workspace_bytes(int64_t N, int64_t K, int64_t batch);

/* Static, human-readable name of a status code. Takes any int (a status
 * code read back from elsewhere may hold any value); values that are not an
 * lqmm_status give a static "unknown status" string. */
const char *lqmm_status_string(int s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lqmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LQMM_H */

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
 * - Calls are thread-safe; the only library state is per-device properties
 *   cached on first use.
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
 * Accumulation is fp32 everywhere. The quantized GEMVs round the activations
 * x to fp16 (round to nearest even) before the dot products, so |x| must stay
 * below 65504 and x contributes a relative rounding error of at most 2^-11
 * per element. For one or two activation rows per pass the dequantized
 * weights are exact (the block scales are applied in fp32). From three rows
 * up the GEMVs run on the fp16 matrix cores and round each dequantized
 * weight to fp16: Q4_0 once (d*(q-8)); Q4_K rounds d*sc and dmin*m to fp16
 * once per sub-block and then each weight once (one fused multiply-add).
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
  LQMM_ERR_WORKSPACE = 4, /* reserved: workspace argument inconsistent */
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
 * workspace/workspace_bytes: optional device scratch; pass NULL/0. The
 * current kernels need none (lqmm_gemv_workspace_bytes returns 0).
 */
lqmm_status lqmm_gemv_q4_0(const void *W, const float *x, float *y,
                           int64_t N, int64_t K, int64_t batch,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Q8_0 x fp16 GEMM (prefill): Y[m][n] = sum_k X[m][k] * W[n][k], i.e.
 * Y = X * W^T. W: N x (K/32) Q8_0 blocks; X: M x K fp16; Y: M x N fp16
 * (fp32 accumulation, rounded to nearest even at the end). K % 32 == 0 and
 * K < LQMM_GEMM_MAX_K.
 * Weight blocks are dequantized to fp16 into LDS and reused by every row
 * of the M tile ("Llamas na Web", "Design de Shader Consciente de
 * Quantizacao", matmul case).
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

/* Workspace the GEMV calls can use for these sizes, in bytes (0 = none). */
size_t lqmm_gemv_workspace_bytes(int64_t N, int64_t K, int64_t batch);

/* Static, human-readable name of a status code. */
const char *lqmm_status_string(lqmm_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lqmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LQMM_H */

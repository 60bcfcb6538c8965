/*
 * lqmm oracle: plain, slow, double-precision CPU reference for the
 * block-quantized matmul hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg use it. It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes (the plain definition, in IEEE double):
 *   1. decode every fp16 field from its raw bits;
 *   2. dequantize every weight to a real number with the block format's
 *      value formula;
 *   3. multiply the dense dequantized matrix with the activations.
 * The method being checked is the quantization-aware matmul of
 * "Resumo Tecnico: Llamas na Web", section "Design de Shader Consciente de
 * Quantizacao": quantized blocks are dequantized (in registers for the decode
 * mat-vec, in shared memory for the prefill matmul) and multiplied. Whatever
 * order a kernel dequantizes and accumulates in, the exact result is this
 * dequantize-then-multiply product, which the oracle computes with only
 * summation rounding (relative error about K * 2^-53).
 *
 * The fp32 tiled GEMM follows "Compute Shaders con WebGPU para Inferencia ML",
 * section "El Nucleo: Multiplicacion de Matrices en WGSL": C = A * B on
 * row-major M x K and K x N matrices, any M, N, K; its zero-padded edge tiles
 * add nothing, so the plain triple sum is the definition.
 *
 * Block byte layouts (llama.cpp / GGUF style; the pages name these formats but
 * do not print their bytes, so this reading is stated here once):
 *   Q4_0, 18 bytes per 32 weights: bytes 0-1 fp16 d (little endian),
 *     bytes 2-17 qs[16]; weight j (0<=j<16) is the low nibble of qs[j],
 *     weight j+16 the high nibble; w = d * (q - 8), q in 0..15.
 *   Q8_0, 34 bytes per 32 weights: bytes 0-1 fp16 d, bytes 2-33 int8 q[32]
 *     (two's complement); w = d * q.
 *   Q4_K, 144 bytes per 256 weights: bytes 0-1 fp16 d, 2-3 fp16 dmin,
 *     4-15 scales[12], 16-143 qs[128]. Sub-block s (weights 32s..32s+31) has a
 *     6-bit scale sc_s and 6-bit min m_s:
 *       s < 4 : sc_s = scales[s] & 63,  m_s = scales[s+4] & 63
 *       s >= 4: sc_s = (scales[s+4] & 15) | ((scales[s-4] >> 6) << 4)
 *               m_s  = (scales[s+4] >> 4) | ((scales[s]   >> 6) << 4)
 *     weight l of sub-block s has q = nibble of qs[32*(s/2) + l], low nibble
 *     for even s, high nibble for odd s; w = d * sc_s * q - dmin * m_s.
 * Further llama.cpp K-quant super-blocks of 256 weights (the pages name the
 * K-quants and q2_k among the formats; this byte reading is stated once here):
 *   Q6_K, 210 bytes: ql[128] (low 4 bits of q), qh[64] (high 2 bits),
 *     int8 scales[16] (one per 16 weights), fp16 d at bytes 208-209;
 *     w = d * scales[k/16] * (q - 32), q in 0..63. Weight k = 128h + 32j + l
 *     (h < 2, j < 4, l < 32) takes its low bits from the low (j < 2) or
 *     high (j >= 2) nibble of ql[64h + l + 32*(j % 2)] and its high bits
 *     from bits 2j..2j+1 of qh[32h + l].
 *   Q2_K, 84 bytes: scales[16] (low nibble: scale sc, high nibble: min m,
 *     one pair per 16 weights), qs[64], fp16 d at bytes 80-81, fp16 dmin at
 *     bytes 82-83; w = d * sc[k/16] * q - dmin * m[k/16], q in 0..3. Weight
 *     k = 128h + 32j + l takes bits 2j..2j+1 of qs[32h + l].
 * q1_0, the 1-bit format "Resumo Tecnico: Llamas na Web" names under
 * "Extensibilidade" without giving its bytes; read as the _0 family at one
 * bit per weight: 6 bytes per 32 weights, bytes 0-1 fp16 d, bytes 2-5 the
 * 32 code bits, weight j's bit c = bit (j % 8) of byte 2 + j / 8 (least
 * significant bit first); w = d * (2c - 1), i.e. -d or +d.
 * A weight matrix of N output rows and K inputs stores row n as K/32 (or
 * K/256) consecutive blocks; rows are consecutive with no padding.
 *
 * The int4 layout of "Compute Shaders con WebGPU para Inferencia ML",
 * section "Yendo a Cuantizado: Matmul INT4" (GPTQ/AWQ style): weight (n, k)
 * is nibble (n*K + k) % 8 (bits 4*i..4*i+3) of 32-bit word (n*K + k) / 8,
 * read as a two's-complement value s in -8..7; scales and zeros are fp32
 * arrays of N x K/32 (one per row and group of 32 along K); w = (s - zero)
 * * scale. (The page's listing does not declare the scales and zeros
 * buffers; fp32 is the reading its f32 arithmetic supports.)
 *
 * Test hooks: LQMM_ORACLE_MUTANT selects a deliberately wrong variant of one
 * step. It is 0 in every normal build and is only set by the test that checks
 * that the pins catch such mistakes.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef LQMM_ORACLE_MUTANT
#define LQMM_ORACLE_MUTANT 0
#endif

#define QK 32    /* weights per Q4_0 / Q8_0 block */
#define QKK 256  /* weights per Q4_K super-block */

/* IEEE 754 binary16 -> double, from the format's definition: sign bit,
 * 5-bit biased exponent (bias 15), 10-bit fraction; exponent 0 encodes zero
 * and subnormals (fraction * 2^-24), exponent 31 encodes inf / NaN. */
double lqmm_oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
#if LQMM_ORACLE_MUTANT == 7
    v = ldexp((double)(1024 + f), -25); /* subnormal treated as normal */
#else
    v = ldexp((double)f, -24);
#endif
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
#if LQMM_ORACLE_MUTANT == 8
    v = ldexp((double)(1024 + f), e - 24); /* exponent bias off by one */
#else
    v = ldexp((double)(1024 + f), e - 25);
#endif
  }
  return sign ? -v : v;
}

/* Element-wise decode of n fp16 bit patterns. */
void lqmm_oracle_f16_array_to_f64(const uint16_t *h, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = lqmm_oracle_f16_to_f64(h[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Dequantize one Q4_0 block (18 bytes) into 32 doubles: w = d * (q - 8). */
static void deq_q4_0_block(const uint8_t *blk, double *w) {
  double d = lqmm_oracle_f16_to_f64(rd16(blk));
  const uint8_t *qs = blk + 2;
  for (int j = 0; j < 16; ++j) {
    int lo = qs[j] & 15, hi = qs[j] >> 4;
#if LQMM_ORACLE_MUTANT == 1
    /* sequential nibble order (weight 2j low, 2j+1 high) */
    w[2 * j] = d * (lo - 8);
    w[2 * j + 1] = d * (hi - 8);
#elif LQMM_ORACLE_MUTANT == 2
    w[j] = d * lo; /* offset 8 dropped */
    w[j + 16] = d * hi;
#else
    w[j] = d * (lo - 8);
    w[j + 16] = d * (hi - 8);
#endif
  }
}

/* Dequantize one Q8_0 block (34 bytes) into 32 doubles: w = d * q. */
static void deq_q8_0_block(const uint8_t *blk, double *w) {
  double d = lqmm_oracle_f16_to_f64(rd16(blk));
  for (int j = 0; j < QK; ++j) {
#if LQMM_ORACLE_MUTANT == 6
    int q = blk[2 + j]; /* read as unsigned */
#else
    int q = (int8_t)blk[2 + j];
#endif
    w[j] = d * q;
  }
}

/* The 6-bit scale and min of sub-block s of a Q4_K super-block. */
static void q4_k_scale_min(const uint8_t *scales, int s, int *sc, int *m) {
  if (s < 4) {
    *sc = scales[s] & 63;
    *m = scales[s + 4] & 63;
  } else {
#if LQMM_ORACLE_MUTANT == 3
    *sc = scales[s + 4] & 15; /* high two bits of sc dropped */
#else
    *sc = (scales[s + 4] & 15) | ((scales[s - 4] >> 6) << 4);
#endif
    *m = (scales[s + 4] >> 4) | ((scales[s] >> 6) << 4);
  }
}

/* Dequantize one Q4_K super-block (144 bytes) into 256 doubles:
 * w = d * sc_s * q - dmin * m_s. */
static void deq_q4_k_block(const uint8_t *blk, double *w) {
  double d = lqmm_oracle_f16_to_f64(rd16(blk));
  double dmin = lqmm_oracle_f16_to_f64(rd16(blk + 2));
  const uint8_t *scales = blk + 4;
  const uint8_t *qs = blk + 16;
  for (int s = 0; s < 8; ++s) {
    int sc, m;
    q4_k_scale_min(scales, s, &sc, &m);
    for (int l = 0; l < 32; ++l) {
      uint8_t byte = qs[32 * (s / 2) + l];
#if LQMM_ORACLE_MUTANT == 5
      int q = (s % 2 == 0) ? (byte >> 4) : (byte & 15); /* halves swapped */
#else
      int q = (s % 2 == 0) ? (byte & 15) : (byte >> 4);
#endif
#if LQMM_ORACLE_MUTANT == 4
      w[32 * s + l] = d * sc * q + dmin * m; /* min term sign flipped */
#else
      w[32 * s + l] = d * sc * q - dmin * m;
#endif
    }
  }
}

/* Dequantize one Q6_K super-block (210 bytes) into 256 doubles:
 * w = d * scales[k/16] * (q - 32). */
static void deq_q6_k_block(const uint8_t *blk, double *w) {
  const uint8_t *ql = blk, *qh = blk + 128;
  const int8_t *sc = (const int8_t *)(blk + 192);
  double d = lqmm_oracle_f16_to_f64(rd16(blk + 208));
  for (int k = 0; k < 256; ++k) {
    int h = k / 128, j = (k % 128) / 32, l = k % 32;
    uint8_t lb = ql[64 * h + l + 32 * (j % 2)];
#if LQMM_ORACLE_MUTANT == 12
    int lo = j < 2 ? (lb >> 4) : (lb & 15); /* nibble halves swapped */
#else
    int lo = j < 2 ? (lb & 15) : (lb >> 4);
#endif
#if LQMM_ORACLE_MUTANT == 11
    int hi = (qh[32 * h + l] >> j) & 3; /* high bits at the wrong shift */
#else
    int hi = (qh[32 * h + l] >> (2 * j)) & 3;
#endif
    int q = lo | (hi << 4);
    w[k] = d * sc[k / 16] * (q - 32);
  }
}

/* Dequantize one Q2_K super-block (84 bytes) into 256 doubles:
 * w = d * sc * q - dmin * m with (sc, m) the nibbles of scales[k/16]. */
static void deq_q2_k_block(const uint8_t *blk, double *w) {
  const uint8_t *scales = blk, *qs = blk + 16;
  double d = lqmm_oracle_f16_to_f64(rd16(blk + 80));
  double dmin = lqmm_oracle_f16_to_f64(rd16(blk + 82));
  for (int k = 0; k < 256; ++k) {
    int h = k / 128, j = (k % 128) / 32, l = k % 32;
    int q = (qs[32 * h + l] >> (2 * j)) & 3;
#if LQMM_ORACLE_MUTANT == 13
    int m = scales[k / 16] & 15, sc = scales[k / 16] >> 4; /* scale and min swapped */
#else
    int sc = scales[k / 16] & 15, m = scales[k / 16] >> 4;
#endif
    w[k] = d * sc * q - dmin * m;
  }
}

/* Dequantize one q1_0 block (6 bytes) into 32 doubles: w = d * (2c - 1). */
static void deq_q1_0_block(const uint8_t *blk, double *w) {
  double d = lqmm_oracle_f16_to_f64(rd16(blk));
  for (int j = 0; j < QK; ++j) {
#if LQMM_ORACLE_MUTANT == 17
    int c = (blk[2 + j / 8] >> (7 - j % 8)) & 1; /* most significant bit first */
#else
    int c = (blk[2 + j / 8] >> (j % 8)) & 1;
#endif
#if LQMM_ORACLE_MUTANT == 18
    w[j] = d * c; /* codes read as 0 / +d instead of -d / +d */
#else
    w[j] = d * (2 * c - 1);
#endif
  }
}

/* ---- dense dequantization of whole rows (exposed for the pins) ---- */

void lqmm_oracle_dequant_q4_0(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q4_0_block(W + (n * nb + b) * 18, out + n * K + b * QK);
}

void lqmm_oracle_dequant_q1_0(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q1_0_block(W + (n * nb + b) * 6, out + n * K + b * QK);
}

void lqmm_oracle_dequant_q8_0(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q8_0_block(W + (n * nb + b) * 34, out + n * K + b * QK);
}

void lqmm_oracle_dequant_q4_k(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QKK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q4_k_block(W + (n * nb + b) * 144, out + n * K + b * QKK);
}

void lqmm_oracle_dequant_q6_k(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QKK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q6_k_block(W + (n * nb + b) * 210, out + n * K + b * QKK);
}

void lqmm_oracle_dequant_q2_k(const uint8_t *W, int64_t N, int64_t K, double *out) {
  int64_t nb = K / QKK;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nb; ++b)
      deq_q2_k_block(W + (n * nb + b) * 84, out + n * K + b * QKK);
}

/* The int4 group-32 layout ("Yendo a Cuantizado: Matmul INT4"): row n of
 * N x K, w = (s - zero) * scale with s the sign-extended nibble. */
static void deq_i4g32_row(const uint32_t *Wq, const float *scales, const float *zeros,
                          int64_t n, int64_t K, double *w) {
  for (int64_t k = 0; k < K; ++k) {
    int64_t idx = n * K + k;
#if LQMM_ORACLE_MUTANT == 16
    int nib = (int)((Wq[idx / 8] >> (4 * (7 - idx % 8))) & 15u); /* nibble order reversed */
#else
    int nib = (int)((Wq[idx / 8] >> (4 * (idx % 8))) & 15u);
#endif
#if LQMM_ORACLE_MUTANT == 14
    int sv = nib; /* not sign-extended */
#else
    int sv = nib >= 8 ? nib - 16 : nib;
#endif
    double scale = scales[n * (K / QK) + k / QK];
    double zero = zeros[n * (K / QK) + k / QK];
#if LQMM_ORACLE_MUTANT == 15
    w[k] = (sv + zero) * scale; /* zero point added */
#else
    w[k] = (sv - zero) * scale;
#endif
  }
}

void lqmm_oracle_dequant_i4g32(const uint32_t *Wq, const float *scales, const float *zeros,
                               int64_t N, int64_t K, double *out) {
  for (int64_t n = 0; n < N; ++n) deq_i4g32_row(Wq, scales, zeros, n, K, out + n * K);
}

/* ---- GEMV: y[b][n] = sum_k W[n][k] * x[b][k] ----
 * Weight-matrix times activation for decode (one or a few tokens), the
 * mat-vec case of "Llamas na Web", "Design de Shader Consciente de
 * Quantizacao". x is batch x K fp32 row-major; y is batch x N double.
 * rows/nrows select the output rows to compute (rows == NULL: all N, and
 * nrows is ignored); y is then batch x nrows in the order given. */
typedef void (*deq_row_fn)(const uint8_t *W, int64_t n, int64_t K, double *w);

static void row_q4_0(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QK;
  for (int64_t b = 0; b < nb; ++b) deq_q4_0_block(W + (n * nb + b) * 18, w + b * QK);
}
static void row_q8_0(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QK;
  for (int64_t b = 0; b < nb; ++b) deq_q8_0_block(W + (n * nb + b) * 34, w + b * QK);
}
static void row_q4_k(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QKK;
  for (int64_t b = 0; b < nb; ++b) deq_q4_k_block(W + (n * nb + b) * 144, w + b * QKK);
}
static void row_q6_k(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QKK;
  for (int64_t b = 0; b < nb; ++b) deq_q6_k_block(W + (n * nb + b) * 210, w + b * QKK);
}
static void row_q1_0(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QK;
  for (int64_t b = 0; b < nb; ++b) deq_q1_0_block(W + (n * nb + b) * 6, w + b * QK);
}
static void row_q2_k(const uint8_t *W, int64_t n, int64_t K, double *w) {
  int64_t nb = K / QKK;
  for (int64_t b = 0; b < nb; ++b) deq_q2_k_block(W + (n * nb + b) * 84, w + b * QKK);
}

/* The int4 layout's three arrays, for gemv_generic's row decoder. */
typedef struct {
  const uint32_t *Wq;
  const float *scales, *zeros;
} i4g32_arrays;

static void gemv_generic_ex(deq_row_fn deq, const uint8_t *W, const i4g32_arrays *i4,
                            const float *x, double *y, int64_t N, int64_t K, int64_t batch,
                            const int64_t *rows, int64_t nrows) {
  int64_t R = rows ? nrows : N;
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
      int64_t n = rows ? rows[i] : i;
      if (i4)
        deq_i4g32_row(i4->Wq, i4->scales, i4->zeros, n, K, w);
      else
        deq(W, n, K, w);
      for (int64_t b = 0; b < batch; ++b) {
        const float *xb = x + b * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += w[k] * (double)xb[k];
        y[b * R + i] = acc;
      }
    }
    free(w);
  }
}

static void gemv_generic(deq_row_fn deq, const uint8_t *W, const float *x, double *y,
                         int64_t N, int64_t K, int64_t batch, const int64_t *rows,
                         int64_t nrows) {
  gemv_generic_ex(deq, W, NULL, x, y, N, K, batch, rows, nrows);
}

void lqmm_oracle_gemv_q4_0(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q4_0, W, x, y, N, K, batch, rows, nrows);
}

void lqmm_oracle_gemv_q4_k(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q4_k, W, x, y, N, K, batch, rows, nrows);
}

/* Decode mat-vec over Q8_0, Q6_K and Q2_K rows: the same definition with the
 * other block formats (every format takes both kernel styles in "Llamas na
 * Web", "Design de Shader Consciente de Quantizacao"). */
void lqmm_oracle_gemv_q8_0(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q8_0, W, x, y, N, K, batch, rows, nrows);
}

void lqmm_oracle_gemv_q6_k(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q6_k, W, x, y, N, K, batch, rows, nrows);
}

void lqmm_oracle_gemv_q1_0(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q1_0, W, x, y, N, K, batch, rows, nrows);
}

void lqmm_oracle_gemv_q2_k(const uint8_t *W, const float *x, double *y, int64_t N,
                           int64_t K, int64_t batch, const int64_t *rows, int64_t nrows) {
  gemv_generic(row_q2_k, W, x, y, N, K, batch, rows, nrows);
}

/* The int4 matmul of "Yendo a Cuantizado: Matmul INT4": sum over k of
 * input * (s - zero) * scale, for every weight row and activation row. The
 * page writes result[row * N + col] with row = weight row and col = input
 * vector; here y[b][n] (activation-major), the same numbers. */
void lqmm_oracle_gemv_i4g32(const uint32_t *Wq, const float *scales, const float *zeros,
                            const float *x, double *y, int64_t N, int64_t K, int64_t batch,
                            const int64_t *rows, int64_t nrows) {
  i4g32_arrays a = {Wq, scales, zeros};
  gemv_generic_ex(NULL, NULL, &a, x, y, N, K, batch, rows, nrows);
}

/* ---- quantized x fp16 GEMM: Y[m][n] = sum_k X[m][k] * W[n][k] ----
 * The prefill matmul of "Llamas na Web", "Design de Shader Consciente de
 * Quantizacao" (blocks loaded, dequantized and reused). X is M x K raw fp16
 * bits, row-major; Y is M x N double (the unrounded product). cols/ncols
 * select output columns n (cols == NULL: all N); Y is then M x ncols. */
static void gemm_generic(deq_row_fn deq, const uint8_t *W, const uint16_t *X, double *Y,
                         int64_t M, int64_t N, int64_t K, const int64_t *cols, int64_t ncols) {
  int64_t C = cols ? ncols : N;
  double *Xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
  for (int64_t i = 0; i < M * K; ++i) Xd[i] = lqmm_oracle_f16_to_f64(X[i]);
#pragma omp parallel
  {
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int64_t j = 0; j < C; ++j) {
      int64_t n = cols ? cols[j] : j;
      deq(W, n, K, w);
      for (int64_t m = 0; m < M; ++m) {
        const double *xm = Xd + m * K;
        double acc = 0.0;
#if LQMM_ORACLE_MUTANT == 10
        for (int64_t k = 0; k < K; ++k) acc += xm[k] * w[(k * 7) % K]; /* k index scrambled */
#else
        for (int64_t k = 0; k < K; ++k) acc += xm[k] * w[k];
#endif
        Y[m * C + j] = acc;
      }
    }
    free(w);
  }
  free(Xd);
}

void lqmm_oracle_gemm_q8_0_f16(const uint8_t *W, const uint16_t *X, double *Y, int64_t M,
                               int64_t N, int64_t K, const int64_t *cols, int64_t ncols) {
  gemm_generic(row_q8_0, W, X, Y, M, N, K, cols, ncols);
}

/* The prefill matmul over Q4_0 and Q4_K weights. */
void lqmm_oracle_gemm_q4_0_f16(const uint8_t *W, const uint16_t *X, double *Y, int64_t M,
                               int64_t N, int64_t K, const int64_t *cols, int64_t ncols) {
  gemm_generic(row_q4_0, W, X, Y, M, N, K, cols, ncols);
}

void lqmm_oracle_gemm_q4_k_f16(const uint8_t *W, const uint16_t *X, double *Y, int64_t M,
                               int64_t N, int64_t K, const int64_t *cols, int64_t ncols) {
  gemm_generic(row_q4_k, W, X, Y, M, N, K, cols, ncols);
}

/* ---- fp32 GEMM: C[i][j] = sum_k A[i][k] * B[k][j] ----
 * "Compute Shaders con WebGPU para Inferencia ML", "El Nucleo: Multiplicacion
 * de Matrices en WGSL". A is M x K, B is K x N, both fp32 row-major; C is
 * M x N double. rows/nrows select output rows i (rows == NULL: all M). */
void lqmm_oracle_sgemm(const float *A, const float *B, double *C, int64_t M, int64_t N,
                       int64_t K, const int64_t *rows, int64_t nrows) {
  int64_t R = rows ? nrows : M;
  /* column j of B, gathered once so the inner sum walks contiguous memory */
  double *Bt = (double *)malloc(sizeof(double) * (size_t)(N * K));
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j)
#if LQMM_ORACLE_MUTANT == 9
      Bt[j * K + k] = (double)B[(j % K) * N + (k % N)]; /* B read transposed */
#else
      Bt[j * K + k] = (double)B[k * N + j];
#endif
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    int64_t i = rows ? rows[r] : r;
    const float *a = A + i * K;
    for (int64_t j = 0; j < N; ++j) {
      const double *b = Bt + j * K;
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (double)a[k] * b[k];
      C[r * N + j] = acc;
    }
  }
  free(Bt);
}

/* Threads the OpenMP loops above use. */
int lqmm_oracle_threads(void) { return omp_get_max_threads(); }

/* Set the threads of the loops above (n >= 1); used to time the oracle on
   one core as well as on all of them. */
void lqmm_oracle_set_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
}

/* Mutant id this library was built with (0 = the real oracle). */
int lqmm_oracle_mutant(void) { return LQMM_ORACLE_MUTANT; }

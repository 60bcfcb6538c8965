/* Host sanitizer run of the CPU oracle (test infrastructure).
 *
 * Built with gcc -fsanitize=address,undefined together with
 * oracle/lqmm_oracle.c; calls every exported oracle function on ragged shapes
 * with buffers of exactly the documented sizes (so that a read or write one
 * element past a buffer is reported), with and without row / column subsets,
 * and checks that every output is finite. Any sanitizer report, or a
 * non-finite output, ends the program with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double lqmm_oracle_f16_to_f64(uint16_t h);
void lqmm_oracle_f16_array_to_f64(const uint16_t *h, double *out, int64_t n);
void lqmm_oracle_dequant_q4_0(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_q8_0(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_q4_k(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_q6_k(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_q2_k(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_q1_0(const uint8_t *W, int64_t N, int64_t K, double *out);
void lqmm_oracle_dequant_i4g32(const uint32_t *Wq, const float *scales, const float *zeros,
                               int64_t N, int64_t K, double *out);
typedef void (*gemv_fn)(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                        const int64_t *, int64_t);
void lqmm_oracle_gemv_q4_0(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_q4_k(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_q8_0(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_q6_k(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_q2_k(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_q1_0(const uint8_t *, const float *, double *, int64_t, int64_t, int64_t,
                           const int64_t *, int64_t);
void lqmm_oracle_gemv_i4g32(const uint32_t *Wq, const float *scales, const float *zeros,
                            const float *x, double *y, int64_t N, int64_t K, int64_t batch,
                            const int64_t *rows, int64_t nrows);
typedef void (*gemm_fn)(const uint8_t *, const uint16_t *, double *, int64_t, int64_t, int64_t,
                        const int64_t *, int64_t);
void lqmm_oracle_gemm_q8_0_f16(const uint8_t *, const uint16_t *, double *, int64_t, int64_t,
                               int64_t, const int64_t *, int64_t);
void lqmm_oracle_gemm_q4_0_f16(const uint8_t *, const uint16_t *, double *, int64_t, int64_t,
                               int64_t, const int64_t *, int64_t);
void lqmm_oracle_gemm_q4_k_f16(const uint8_t *, const uint16_t *, double *, int64_t, int64_t,
                               int64_t, const int64_t *, int64_t);
void lqmm_oracle_sgemm(const float *A, const float *B, double *C, int64_t M, int64_t N,
                       int64_t K, const int64_t *rows, int64_t nrows);
void lqmm_oracle_set_threads(int n);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float next_f(void) { return (float)(next_u32() % 2001) / 1000.0f - 1.0f; }

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static int failures = 0;
static void check_finite(const char *what, const double *v, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(v[i])) {
      fprintf(stderr, "%s: non-finite output at %lld\n", what, (long long)i);
      ++failures;
      return;
    }
}

/* Block-quantized rows with random codes and small normal fp16 scale fields
 * at the given byte offsets of each block (every other byte random). */
static uint8_t *make_blocks(int64_t nblocks, int bytes, const int *f16_offsets, int nf16) {
  uint8_t *W = (uint8_t *)xmalloc((size_t)(nblocks * bytes));
  for (int64_t i = 0; i < nblocks * bytes; ++i) W[i] = (uint8_t)next_u32();
  for (int64_t b = 0; b < nblocks; ++b)
    for (int j = 0; j < nf16; ++j) {
      uint16_t h = (uint16_t)(0x2000 + next_u32() % 0x1000); /* 2^-7 .. 2^-6 range */
      memcpy(W + b * bytes + f16_offsets[j], &h, 2);
    }
  return W;
}

struct fmt {
  const char *name;
  int blk, bytes;
  int f16_off[2], nf16;
  gemv_fn gemv;
  gemm_fn gemm;
  void (*dequant)(const uint8_t *, int64_t, int64_t, double *);
};

static void run_format(const struct fmt *f, int64_t N, int64_t K, int64_t batch) {
  const int64_t nb = N * (K / f->blk);
  uint8_t *W = make_blocks(nb, f->bytes, f->f16_off, f->nf16);
  double *deq = (double *)xmalloc(sizeof(double) * (size_t)(N * K));
  f->dequant(W, N, K, deq);
  check_finite(f->name, deq, N * K);
  float *x = (float *)xmalloc(sizeof(float) * (size_t)(batch * K));
  for (int64_t i = 0; i < batch * K; ++i) x[i] = next_f();
  double *y = (double *)xmalloc(sizeof(double) * (size_t)(batch * N));
  f->gemv(W, x, y, N, K, batch, NULL, 0);
  check_finite(f->name, y, batch * N);
  int64_t rows[2] = {N - 1, 0};
  double *ys = (double *)xmalloc(sizeof(double) * (size_t)(batch * 2));
  f->gemv(W, x, ys, N, K, batch, rows, 2);
  check_finite(f->name, ys, batch * 2);
  for (int64_t b = 0; b < batch; ++b)
    if (ys[b * 2] != y[b * N + N - 1] || ys[b * 2 + 1] != y[b * N]) {
      fprintf(stderr, "%s: row subset differs from the full product\n", f->name);
      ++failures;
    }
  if (f->gemm) {
    const int64_t M = 3;
    uint16_t *X = (uint16_t *)xmalloc(2 * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; ++i) X[i] = (uint16_t)(0x3000 + next_u32() % 0x0800);
    double *Y = (double *)xmalloc(sizeof(double) * (size_t)(M * N));
    f->gemm(W, X, Y, M, N, K, NULL, 0);
    check_finite(f->name, Y, M * N);
    int64_t cols[1] = {N - 1};
    double *Yc = (double *)xmalloc(sizeof(double) * (size_t)M);
    f->gemm(W, X, Yc, M, N, K, cols, 1);
    for (int64_t m = 0; m < M; ++m)
      if (Yc[m] != Y[m * N + N - 1]) {
        fprintf(stderr, "%s: column subset differs from the full product\n", f->name);
        ++failures;
      }
    free(X);
    free(Y);
    free(Yc);
  }
  free(W);
  free(deq);
  free(x);
  free(y);
  free(ys);
}

int main(void) {
  lqmm_oracle_set_threads(2);
  const struct fmt fmts[] = {
      {"q4_0", 32, 18, {0, 0}, 1, lqmm_oracle_gemv_q4_0, lqmm_oracle_gemm_q4_0_f16,
       lqmm_oracle_dequant_q4_0},
      {"q8_0", 32, 34, {0, 0}, 1, lqmm_oracle_gemv_q8_0, lqmm_oracle_gemm_q8_0_f16,
       lqmm_oracle_dequant_q8_0},
      {"q4_k", 256, 144, {0, 2}, 2, lqmm_oracle_gemv_q4_k, lqmm_oracle_gemm_q4_k_f16,
       lqmm_oracle_dequant_q4_k},
      {"q6_k", 256, 210, {208, 208}, 1, lqmm_oracle_gemv_q6_k, NULL, lqmm_oracle_dequant_q6_k},
      {"q2_k", 256, 84, {80, 82}, 2, lqmm_oracle_gemv_q2_k, NULL, lqmm_oracle_dequant_q2_k},
      {"q1_0", 32, 6, {0, 0}, 1, lqmm_oracle_gemv_q1_0, NULL, lqmm_oracle_dequant_q1_0},
  };
  const int64_t shapes[][3] = {{1, 1, 1}, {3, 2, 2}, {7, 3, 5}};  /* N, blocks per row, batch */
  for (size_t i = 0; i < sizeof(fmts) / sizeof(fmts[0]); ++i)
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
      run_format(&fmts[i], shapes[s][0], shapes[s][1] * fmts[i].blk, shapes[s][2]);

  /* int4 group-32: 8 codes per uint32, scales and zeros per 32 weights */
  {
    const int64_t N = 5, K = 96, batch = 3;
    uint32_t *Wq = (uint32_t *)xmalloc(4 * (size_t)(N * K / 8));
    for (int64_t i = 0; i < N * K / 8; ++i) Wq[i] = next_u32();
    float *sc = (float *)xmalloc(4 * (size_t)(N * K / 32));
    float *z = (float *)xmalloc(4 * (size_t)(N * K / 32));
    for (int64_t i = 0; i < N * K / 32; ++i) {
      sc[i] = next_f();
      z[i] = next_f();
    }
    double *deq = (double *)xmalloc(sizeof(double) * (size_t)(N * K));
    lqmm_oracle_dequant_i4g32(Wq, sc, z, N, K, deq);
    check_finite("i4g32", deq, N * K);
    float *x = (float *)xmalloc(4 * (size_t)(batch * K));
    for (int64_t i = 0; i < batch * K; ++i) x[i] = next_f();
    double *y = (double *)xmalloc(sizeof(double) * (size_t)(batch * N));
    lqmm_oracle_gemv_i4g32(Wq, sc, z, x, y, N, K, batch, NULL, 0);
    check_finite("i4g32", y, batch * N);
    int64_t rows[1] = {N - 1};
    double *ys = (double *)xmalloc(sizeof(double) * (size_t)batch);
    lqmm_oracle_gemv_i4g32(Wq, sc, z, x, ys, N, K, batch, rows, 1);
    for (int64_t b = 0; b < batch; ++b)
      if (ys[b] != y[b * N + N - 1]) {
        fprintf(stderr, "i4g32: row subset differs from the full product\n");
        ++failures;
      }
    free(Wq);
    free(sc);
    free(z);
    free(deq);
    free(x);
    free(y);
    free(ys);
  }

  /* fp32 GEMM, full and with a row subset; fp16 decoding of every bit pattern */
  {
    const int64_t M = 5, N = 7, K = 3;
    float *A = (float *)xmalloc(4 * (size_t)(M * K)), *B = (float *)xmalloc(4 * (size_t)(K * N));
    for (int64_t i = 0; i < M * K; ++i) A[i] = next_f();
    for (int64_t i = 0; i < K * N; ++i) B[i] = next_f();
    double *C = (double *)xmalloc(sizeof(double) * (size_t)(M * N));
    lqmm_oracle_sgemm(A, B, C, M, N, K, NULL, 0);
    check_finite("sgemm", C, M * N);
    int64_t rows[2] = {M - 1, 1};
    double *Cr = (double *)xmalloc(sizeof(double) * 2 * (size_t)N);
    lqmm_oracle_sgemm(A, B, Cr, M, N, K, rows, 2);
    for (int64_t j = 0; j < N; ++j)
      if (Cr[j] != C[(M - 1) * N + j] || Cr[N + j] != C[N + j]) {
        fprintf(stderr, "sgemm: row subset differs from the full product\n");
        ++failures;
      }
    uint16_t *h = (uint16_t *)xmalloc(2 * 65536);
    double *hd = (double *)xmalloc(sizeof(double) * 65536);
    for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
    lqmm_oracle_f16_array_to_f64(h, hd, 65536);
    for (int i = 0; i < 65536; ++i) {
      const double v = lqmm_oracle_f16_to_f64((uint16_t)i);
      if (!(v == hd[i] || (isnan(v) && isnan(hd[i])))) {
        fprintf(stderr, "f16 decode: array and scalar forms differ at 0x%04x\n", i);
        ++failures;
        break;
      }
    }
    free(A);
    free(B);
    free(C);
    free(Cr);
    free(h);
    free(hd);
  }
  if (failures) return 1;
  printf("oracle sanitizer run: ok\n");
  return 0;
}

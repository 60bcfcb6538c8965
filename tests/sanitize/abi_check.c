/* Host sanitizer run of the C ABI's host code (test infrastructure).
 *
 * Linked against objects of the library whose host code is built with
 * -fsanitize=address,undefined. Calls every entry point with arguments the
 * boundary rejects (NULL pointers, sizes <= 0 or past LQMM_MAX_DIM or not a
 * block multiple, pointers off 16-byte alignment, short workspaces) and checks
 * the documented status; queries workspace sizes over a range of shapes and
 * status strings of every status. None of these calls reaches a device.
 * With the argument "nodevice" (no GPU visible) it also makes well-formed
 * calls, which must fail with LQMM_ERR_DEVICE and launch nothing; the host
 * pointers passed then are never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lqmm.h"

static int failures = 0;
#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    lqmm_status got_ = (call);                                                         \
    if (got_ != (want)) {                                                              \
      fprintf(stderr, "line %d: %s -> %d (%s), expected %d\n", __LINE__, #call, got_,  \
              lqmm_status_string(got_), (want));                                       \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

typedef lqmm_status (*gemv_ws_fn)(const void *, const float *, float *, int64_t, int64_t,
                                  int64_t, void *, size_t, void *);
typedef lqmm_status (*gemm_fn)(const void *, const uint16_t *, uint16_t *, int64_t, int64_t,
                               int64_t, void *);

int main(int argc, char **argv) {
  const int nodevice = argc > 1 && strcmp(argv[1], "nodevice") == 0;
  /* 16-byte aligned host buffers standing in for device pointers */
  void *buf = aligned_alloc(256, 4096);
  memset(buf, 0, 4096);
  const float *xf = (const float *)buf;
  float *yf = (float *)buf;
  uint8_t *mis = (uint8_t *)buf + 4; /* 4-byte aligned only */
  const int64_t big = LQMM_MAX_DIM + 1;

  if (lqmm_version() <= 0) {
    fprintf(stderr, "lqmm_version() <= 0\n");
    ++failures;
  }
  for (int s = -1; s <= 8; ++s) {
    const char *str = lqmm_status_string(s);
    if (!str || !*str) {
      fprintf(stderr, "empty status string for %d\n", s);
      ++failures;
    }
  }
  /* workspace queries: any shape, including rejected ones, returns a size */
  const int64_t dims[] = {-1, 0, 1, 31, 32, 256, 4096, 8192, 28672, (int64_t)1 << 20, big};
  for (size_t i = 0; i < sizeof(dims) / sizeof(dims[0]); ++i)
    for (size_t j = 0; j < sizeof(dims) / sizeof(dims[0]); ++j)
      for (int64_t b = -1; b <= 20; b += 7) {
        const size_t ws = lqmm_gemv_workspace_bytes(dims[i], dims[j], b);
        if (ws > ((size_t)1 << 40)) {
          fprintf(stderr, "workspace size %zu for N=%lld K=%lld batch=%lld\n", ws,
                  (long long)dims[i], (long long)dims[j], (long long)b);
          ++failures;
        }
      }

  /* GEMVs with a workspace argument: (function, weights per block) */
  const struct {
    gemv_ws_fn fn;
    int64_t blk;
  } gemvs[] = {{lqmm_gemv_q4_0, 32}, {lqmm_gemv_q4_k, 256}, {lqmm_gemv_q8_0, 32},
               {lqmm_gemv_q6_k, 256}, {lqmm_gemv_q2_k, 256}, {lqmm_gemv_q1_0, 32}};
  for (size_t i = 0; i < sizeof(gemvs) / sizeof(gemvs[0]); ++i) {
    gemv_ws_fn f = gemvs[i].fn;
    const int64_t K = gemvs[i].blk;
    EXPECT(f(NULL, xf, yf, 1, K, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, NULL, yf, 1, K, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, xf, NULL, 1, K, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, xf, yf, 0, K, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, xf, yf, 1, 0, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, xf, yf, 1, K, 0, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, xf, yf, -5, K, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, xf, yf, big, K, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, xf, yf, 1, K + 16, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(mis, xf, yf, 1, K, 1, NULL, 0, NULL), LQMM_ERR_ALIGN);
    EXPECT(f(buf, (const float *)mis, yf, 1, K, 1, NULL, 0, NULL), LQMM_ERR_ALIGN);
    EXPECT(f(buf, xf, (float *)mis, 1, K, 1, NULL, 0, NULL), LQMM_ERR_ALIGN);
    EXPECT(f(buf, xf, yf, 1, K, 1, mis, 256, NULL), LQMM_ERR_ALIGN);
    if (nodevice) EXPECT(f(buf, xf, yf, 3, K, 2, NULL, 0, NULL), LQMM_ERR_DEVICE);
  }
  /* int4 group-32 */
  {
    const uint32_t *wq = (const uint32_t *)buf;
    EXPECT(lqmm_gemv_i4g32(NULL, xf, xf, xf, yf, 1, 32, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(lqmm_gemv_i4g32(wq, NULL, xf, xf, yf, 1, 32, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(lqmm_gemv_i4g32(wq, xf, NULL, xf, yf, 1, 32, 1, NULL, 0, NULL), LQMM_ERR_NULL);
    EXPECT(lqmm_gemv_i4g32(wq, xf, xf, xf, yf, 1, 48, 1, NULL, 0, NULL), LQMM_ERR_SHAPE);
    EXPECT(lqmm_gemv_i4g32(wq, (const float *)mis, xf, xf, yf, 1, 32, 1, NULL, 0, NULL),
           LQMM_ERR_ALIGN);
    if (nodevice)
      EXPECT(lqmm_gemv_i4g32(wq, xf, xf, xf, yf, 2, 64, 1, NULL, 0, NULL), LQMM_ERR_DEVICE);
  }
  /* allocation-free Q4_0 GEMV */
  EXPECT(lqmm_gemv_q4_0_noalloc(NULL, xf, yf, 1, 32, 1, NULL), LQMM_ERR_NULL);
  EXPECT(lqmm_gemv_q4_0_noalloc(buf, xf, yf, 1, 33, 1, NULL), LQMM_ERR_SHAPE);
  EXPECT(lqmm_gemv_q4_0_noalloc(mis, xf, yf, 1, 32, 1, NULL), LQMM_ERR_ALIGN);
  if (nodevice) EXPECT(lqmm_gemv_q4_0_noalloc(buf, xf, yf, 1, 32, 1, NULL), LQMM_ERR_DEVICE);

  /* GEMMs over fp16 activations: (function, weights per block) */
  const uint16_t *X = (const uint16_t *)buf;
  uint16_t *Y = (uint16_t *)buf;
  const struct {
    gemm_fn fn;
    int64_t blk;
  } gemms[] = {{lqmm_gemm_q8_0_f16, 32}, {lqmm_gemm_q4_0_f16, 32}, {lqmm_gemm_q4_k_f16, 256}};
  for (size_t i = 0; i < sizeof(gemms) / sizeof(gemms[0]); ++i) {
    gemm_fn f = gemms[i].fn;
    const int64_t K = gemms[i].blk;
    EXPECT(f(NULL, X, Y, 1, 1, K, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, NULL, Y, 1, 1, K, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, X, NULL, 1, 1, K, NULL), LQMM_ERR_NULL);
    EXPECT(f(buf, X, Y, 0, 1, K, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, X, Y, 1, 0, K, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, X, Y, 1, 1, K / 2, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(buf, X, Y, big, 1, K, NULL), LQMM_ERR_SHAPE);
    EXPECT(f(mis, X, Y, 1, 1, K, NULL), LQMM_ERR_ALIGN);
    EXPECT(f(buf, (const uint16_t *)mis, Y, 1, 1, K, NULL), LQMM_ERR_ALIGN);
    if (nodevice) EXPECT(f(buf, X, Y, 2, 3, K, NULL), LQMM_ERR_DEVICE);
  }
  EXPECT(lqmm_gemm_q8_0_f16(buf, X, Y, 1, 1, LQMM_GEMM_MAX_K, NULL), LQMM_ERR_SHAPE);

  /* fp32 GEMM */
  EXPECT(lqmm_sgemm(NULL, xf, yf, 1, 1, 1, NULL), LQMM_ERR_NULL);
  EXPECT(lqmm_sgemm(xf, xf, yf, 1, 0, 1, NULL), LQMM_ERR_SHAPE);
  EXPECT(lqmm_sgemm(xf, xf, yf, 1, 1, big, NULL), LQMM_ERR_SHAPE);
  EXPECT(lqmm_sgemm(xf, (const float *)mis, yf, 1, 1, 1, NULL), LQMM_ERR_ALIGN);
  if (nodevice) EXPECT(lqmm_sgemm(xf, xf, yf, 2, 2, 2, NULL), LQMM_ERR_DEVICE);

  free(buf);
  if (failures) return 1;
  printf("abi sanitizer run: ok (%s)\n", nodevice ? "with device-less calls" : "rejections only");
  return 0;
}

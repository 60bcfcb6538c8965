// Instances of the small-problem GEMV kernel (gemv_small.hpp) for the Q4_0
// and Q4_K formats, the split-K counter clear, and the dispatch over all
// formats (the others' instances are in gemv_small_more.hip, which compiles
// in parallel).
#include "gemv_small.hpp"

namespace lqmm {
namespace {

// Zero n ints (the split-K arrival counters) with a plain kernel, so that a
// graph capturing the call records a kernel node, not a memset node.
__global__ void __launch_bounds__(256) clear_ints_kernel(int *__restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

}  // namespace

hipError_t gemv_small_clear_counters(int *counters, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int grid = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(clear_ints_kernel, dim3(grid), dim3(256), 0, stream, counters, n);
  return hipGetLastError();
}

size_t gemv_small_max_lds() { return kMaxSmallLds; }

size_t gemv_small_lds_bytes(GemvFormat f, int batch, int nus) {
  if (batch == 3) batch = 4;  // batch 3 runs on the 4-row instance
  switch (f) {
    case GemvFormat::Q4_0: return small_lds<FmtQ4_0>(batch, nus);
    case GemvFormat::Q4_0x2: return small_lds<FmtQ4_0x2>(batch, nus);
    case GemvFormat::Q4_K: return small_lds<FmtQ4_K>(batch, nus);
    default: return gemv_small_lds_bytes_more(f, batch, nus);
  }
}

hipError_t gemv_small_launch(const SmallGemvPlan &pl, const uint8_t *W, const float *x, float *y,
                             float *part, int *cnt, hipStream_t stream) {
  if (pl.slices > 1 && (!part || !cnt)) return hipErrorInvalidValue;
  switch (pl.f) {
    case GemvFormat::Q4_0: return launch_small_fmt<FmtQ4_0>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::Q4_0x2: return launch_small_fmt<FmtQ4_0x2>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::Q4_K: return launch_small_fmt<FmtQ4_K>(pl, W, x, y, part, cnt, stream);
    default: return gemv_small_launch_more(pl, W, x, y, part, cnt, stream);
  }
}

}  // namespace lqmm

// Instances of the small-problem GEMV kernel (gemv_small.hpp) for the further
// block formats of gemv_formats.hpp: Q8_0, q1_0, Q6_K, Q2_K and the int4
// group-32 layout.
#include "gemv_formats.hpp"
#include "gemv_small.hpp"

namespace lqmm {

size_t gemv_small_lds_bytes_more(GemvFormat f, int batch, int nus) {
  switch (f) {
    case GemvFormat::Q8_0: return small_lds<FmtQ8_0>(batch, nus);
    case GemvFormat::Q1_0: return small_lds<FmtQ1_0>(batch, nus);
    case GemvFormat::Q6_K: return small_lds<FmtQ6_K>(batch, nus);
    case GemvFormat::Q2_K: return small_lds<FmtQ2_K>(batch, nus);
    case GemvFormat::I4G32: return small_lds<FmtI4G32>(batch, nus);
    default: return (size_t)1 << 30;
  }
}

hipError_t gemv_small_launch_more(const SmallGemvPlan &pl, const uint8_t *W, const float *x,
                                  float *y, float *part, int *cnt, hipStream_t stream) {
  switch (pl.f) {
    case GemvFormat::Q8_0: return launch_small_fmt<FmtQ8_0>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::Q1_0: return launch_small_fmt<FmtQ1_0>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::Q6_K: return launch_small_fmt<FmtQ6_K>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::Q2_K: return launch_small_fmt<FmtQ2_K>(pl, W, x, y, part, cnt, stream);
    case GemvFormat::I4G32: return launch_small_fmt<FmtI4G32>(pl, W, x, y, part, cnt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lqmm

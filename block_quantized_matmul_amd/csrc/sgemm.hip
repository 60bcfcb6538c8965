// Dense fp32 GEMM C = A * B (row-major) on the gfx950 fp32 matrix cores.
//
// Semantics are those of the tiled matmul in "Compute Shaders con WebGPU para
// Inferencia ML", section "El Nucleo: Multiplicacion de Matrices en WGSL":
// shared-memory tiles, zero padding at ragged edges, two barriers around each
// tile's use, guarded stores. The page's 16x16 scalar tiles are replaced by a
// CDNA4 design:
// * 128x128 output tile per 1024-thread workgroup, sixteen waves of 32x32
//   (four per SIMD, so that the latency of one wave's LDS reads is covered
//   by the others' MFMAs), each wave a 2x2 grid of v_mfma_f32_16x16x4_f32
//   accumulators (fp32 products, fp32 accumulation). Measured: 152 -> 144 us
//   at 2048^3 against eight waves of 64x32; the matrix cores alone (no LDS
//   reads) take 115 us, so the remaining gap is LDS read latency;
// * K advances 64 (BK) at a time through two LDS buffers: the next tile's global
//   loads are issued before the current tile's MFMAs, and one barrier per step
//   separates reuse of a buffer;
// * A is kept k-contiguous in LDS so one ds_read_b128 supplies four MFMA
//   steps: MFMA s of a 16-wide k group takes, in lane group g, the k index
//   4g + s (a permutation of the sum's terms; B is read with the same one).
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kKQ = BK / 4;  // float4 groups per A row
constexpr int LDA = BK + 4;  // As row stride (floats)
constexpr int LDB = BN + 4;  // Bs row stride (floats)
constexpr int kThreads = 1024;
constexpr int kLoads = BM * BK / 4 / kThreads;  // float4 loads per thread per tile (A, and B)
static_assert(BM * BK == BK * BN && BM * BK % (4 * kThreads) == 0, "");

template <bool VEC>
__device__ __forceinline__ float4_t load4_a(const float *__restrict__ A, int64_t M, int64_t K,
                                            int64_t gm, int64_t gk) {
  if (VEC) {
    if (gm < M && gk < K) return *reinterpret_cast<const float4_t *>(A + gm * K + gk);
    return float4_t{0, 0, 0, 0};
  }
  float4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (gm < M && gk + e < K) ? A[gm * K + gk + e] : 0.0f;
  return v;
}

template <bool VEC>
__device__ __forceinline__ float4_t load4_b(const float *__restrict__ B, int64_t K, int64_t N,
                                            int64_t gk, int64_t gn) {
  if (VEC) {
    if (gk < K && gn < N) return *reinterpret_cast<const float4_t *>(B + gk * N + gn);
    return float4_t{0, 0, 0, 0};
  }
  float4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (gk < K && gn + e < N) ? B[gk * N + gn + e] : 0.0f;
  return v;
}

// VEC: K % 4 == 0 and N % 4 == 0, so every float4 is either fully inside or
// fully outside the matrix and 16-byte aligned.
template <bool VEC>
__global__ void __launch_bounds__(kThreads)
sgemm_kernel(const float *__restrict__ A, const float *__restrict__ B, float *__restrict__ C,
             int64_t M, int64_t N, int64_t K, int tiles_n) {
  __shared__ __attribute__((aligned(16))) float As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

  const int tid = threadIdx.x;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;  // 4 x 4 waves of 32 x 32
  const int li = lane & 15, lg = lane >> 4;

  float4_t ra[kLoads], rb[kLoads];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      int idx = tid + kThreads * it;
      int row = idx / kKQ, kq = idx % kKQ;
      ra[it] = load4_a<VEC>(A, M, K, m0 + row, k0 + 4 * kq);
    }
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      int idx = tid + kThreads * it;
      int k = idx >> 5, jq = idx & 31;
      rb[it] = load4_b<VEC>(B, K, N, k0 + k, n0 + 4 * jq);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      int idx = tid + kThreads * it;
      int row = idx / kKQ, kq = idx % kKQ;
      *reinterpret_cast<float4_t *>(&As[buf][row * LDA + 4 * kq]) = ra[it];
    }
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      int idx = tid + kThreads * it;
      int k = idx >> 5, jq = idx & 31;
      *reinterpret_cast<float4_t *>(&Bs[buf][k * LDB + 4 * jq]) = rb[it];
    }
  };

  float4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float4_t{0, 0, 0, 0};

  const int64_t nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      float4_t a[2];
      float b[2][4];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
        a[ti] = *reinterpret_cast<const float4_t *>(
            &As[cur][(wm * 32 + ti * 16 + li) * LDA + kk * 16 + 4 * lg]);
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b[tj][s] = Bs[cur][(kk * 16 + 4 * lg + s) * LDB + wn * 32 + tj * 16 + li];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int tj = 0; tj < 2; ++tj)
            acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[ti][s], b[tj][s], acc[ti][tj],
                                                                0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // D layout of a 16x16 MFMA tile: lane holds rows 4*lg + v, column li.
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int64_t col = n0 + wn * 32 + tj * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = m0 + wm * 32 + ti * 16 + 4 * lg + v;
        if (row < M && col < N) C[row * N + col] = acc[ti][tj][v];
      }
    }
}

}  // namespace

hipError_t sgemm_launch(const float *A, const float *B, float *C, int64_t M, int64_t N,
                        int64_t K, int num_cus, hipStream_t stream) {
  (void)num_cus;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = (K % 4 == 0) && (N % 4 == 0);
  if (vec)
    hipLaunchKernelGGL(sgemm_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, A,
                       B, C, M, N, K, (int)tiles_n);
  else
    hipLaunchKernelGGL(sgemm_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, A,
                       B, C, M, N, K, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace lqmm

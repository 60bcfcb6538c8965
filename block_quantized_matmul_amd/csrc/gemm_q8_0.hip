// Q8_0 x fp16 GEMM for prefill: Y[m][n] = sum_k X[m][k] * W[n][k], fp32
// accumulation, fp16 output, on the gfx950 fp16 matrix cores.
//
// This is the matmul case of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao": quantized blocks are loaded,
// dequantized into shared memory and reused by the whole M tile. Here the
// shared memory is the CU's LDS and the reuse feeds
// v_mfma_f32_16x16x32_f16:
// * 128x128 output tile per 256-thread workgroup (four waves of 64x64, 4x4
//   MFMA tiles each); K advances 64 (two Q8_0 blocks) per step through two
//   LDS buffers, the next step's global loads in flight during the MFMAs;
// * each thread fetches one raw 34-byte block (fp16 d + 32 int8) and
//   dequantizes it in registers: q ^ 0x80 placed in the mantissa of 1024.0
//   with v_perm_b32 gives the exact fp16 value 1152 + q, one packed subtract
//   gives q, one packed multiply gives fp16(d*q) (a single rounding); the 32
//   fp16 weights go to LDS as four 16-byte stores;
// * both operands sit k-contiguous in LDS, so each MFMA operand is one
//   ds_read_b128; X rows and W rows use the same k order, which is all the
//   dot product needs.
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halves per LDS row (144 bytes)
constexpr int kThreads = 256;

struct RawQ8 {
  u32x4 q0, q1;  // 32 int8 codes
  uint32_t d;    // fp16 bits
};

__device__ __forceinline__ void dequant_q8_0(const RawQ8 &r, u32x4 (&out)[4]) {
  const half2_t d2 = as_half2((r.d & 0xFFFF) * 0x10001u);
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t u = w[i] ^ 0x80808080u;
    half2_t lo = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
    half2_t hi = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
    lo = (lo - bias) * d2;
    hi = (hi - bias) * d2;
    out[i >> 1][(i & 1) * 2 + 0] = as_u32(lo);
    out[i >> 1][(i & 1) * 2 + 1] = as_u32(hi);
  }
}

__global__ void __launch_bounds__(kThreads)
gemm_q8_0_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ X,
                 uint16_t *__restrict__ Y, int64_t M, int64_t N, int64_t K, int tiles_n) {
  __shared__ __attribute__((aligned(16))) half_t Xs[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) half_t Ws[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x;
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
  // L2. Renumber so that consecutive logical tiles (the M tiles that share
  // one weight N tile) run on the same XCD and share its L2.
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t ntiles = tiles_m * tiles_n;
  int64_t tile = blockIdx.x;
  if (ntiles % 8 == 0) tile = (tile % 8) * (ntiles / 8) + tile / 8;
  const int tm = (int)(tile % tiles_m);
  const int tn = (int)(tile / tiles_m);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t nb = K / 32;
  const int64_t row_bytes = nb * 34;

  u32x4 rx[4];
  RawQ8 rw;
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int idx = tid + kThreads * it;
      int row = idx >> 3, c = idx & 7;
      int64_t gm = m0 + row, gk = k0 + 8 * c;
      rx[it] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4 *>(X + gm * K + gk)
                                  : u32x4{0, 0, 0, 0};
    }
    {
      int row = tid >> 1, blk = tid & 1;
      int64_t gn = n0 + row, kb = k0 / 32 + blk;
      if (gn < N && kb < nb) {
        const uint8_t *p = W + gn * row_bytes + kb * 34;
        rw.d = load_u16(p);
        rw.q0 = load_u32x4_unaligned(p + 2);
        rw.q1 = load_u32x4_unaligned(p + 18);
      } else {
        rw.d = 0;
        rw.q0 = u32x4{0, 0, 0, 0};
        rw.q1 = rw.q0;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int idx = tid + kThreads * it;
      int row = idx >> 3, c = idx & 7;
      *reinterpret_cast<u32x4 *>(&Xs[buf][row * LDS_STRIDE + 8 * c]) = rx[it];
    }
    {
      int row = tid >> 1, blk = tid & 1;
      u32x4 out[4];
      dequant_q8_0(rw, out);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4 *>(&Ws[buf][row * LDS_STRIDE + 32 * blk + 8 * j]) = out[j];
    }
  };

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0, 0, 0, 0};

  const int64_t nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      half8_t a[4], b[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        a[ti] = *reinterpret_cast<const half8_t *>(
            &Xs[cur][(wm * 64 + ti * 16 + li) * LDS_STRIDE + kk * 32 + 8 * lg]);
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
        b[tj] = *reinterpret_cast<const half8_t *>(
            &Ws[cur][(wn * 64 + tj * 16 + li) * LDS_STRIDE + kk * 32 + 8 * lg]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj)
          acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ti], b[tj], acc[ti][tj], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int64_t col = n0 + wn * 64 + tj * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = m0 + wm * 64 + ti * 16 + 4 * lg + v;
        if (row < M && col < N)
          Y[row * N + col] = __builtin_bit_cast(uint16_t, (half_t)acc[ti][tj][v]);
      }
    }
}

}  // namespace

hipError_t gemm_q8_0_launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M,
                            int64_t N, int64_t K, int num_cus, hipStream_t stream) {
  (void)num_cus;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_q8_0_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, W, X, Y,
                     M, N, K, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace lqmm

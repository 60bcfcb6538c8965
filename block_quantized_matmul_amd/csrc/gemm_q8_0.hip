// Q8_0 x fp16 GEMM for prefill: Y[m][n] = sum_k X[m][k] * W[n][k], fp32
// accumulation, fp16 output, on the gfx950 fp16 matrix cores.
//
// This is the matmul case of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao": quantized blocks are loaded,
// dequantized into shared memory and reused by the whole M tile. Here the
// shared memory is the CU's LDS and the reuse feeds
// v_mfma_f32_32x32x16_f16:
// * 128x128 output tile per 256-thread workgroup (four waves of 64x64, 2x2
//   tiles of v_mfma_f32_32x32x16_f16 each); K advances 64 (two Q8_0 blocks)
//   per step through two LDS buffers, the global loads of the step after
//   next in flight during the MFMAs;
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
  // d arrives zero-extended; taking its low half needs no instruction, and
  // the packed multiplies broadcast it with op_sel.
  const half_t dh = __builtin_bit_cast(half_t, (uint16_t)r.d);
  const half2_t d2 = {dh, dh};
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

// Raw global data of one K step for one thread: four 16-byte pieces of the X
// tile and one Q8_0 block of the W tile.
struct RawStep {
  u32x4 x[4];
  RawQ8 w;
};

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
  const uint32_t Ku = (uint32_t)K;
  const uint32_t row_bytes = Ku / 32 * 34;
  const int nk = (int)((K + BK - 1) / BK);
  const bool ragged = K % BK != 0;  // the last step holds one block, not two

  // The tile's X rows and W rows through buffer resources that end at the
  // last row of the tensor: loads of rows past M or N return zeros (their
  // results are never stored). Offsets are 32-bit (the host keeps
  // BM * K * 2 < 2^32). Nothing is computed from loaded data before it is
  // written to LDS, so the loads of two steps stay in flight together.
  const int64_t xrows = M - m0 < BM ? M - m0 : BM;
  const int64_t wrows = N - n0 < BN ? N - n0 : BN;
  const rsrc_t xr = make_rsrc(X + m0 * K, (uint32_t)(xrows * K * 2));
  const rsrc_t wr = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)(wrows * row_bytes));
  uint32_t xoff[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + kThreads * it;
    xoff[it] = ((uint32_t)(idx >> 3) * Ku + 8 * (idx & 7)) * 2;
  }
  const int wblk = tid & 1;
  const uint32_t woff = (uint32_t)(tid >> 1) * row_bytes + 34 * wblk;

  auto load_step = [&](RawStep &r, int kt) {
#pragma unroll
    for (int it = 0; it < 4; ++it) r.x[it] = buf_load_b128(xr, xoff[it] + kt * (BK * 2));
    const uint32_t wo = woff + kt * 68;
    r.w.d = buf_load_u16(wr, wo);
    r.w.q0 = buf_load_b128(wr, wo + 2);
    r.w.q1 = buf_load_b128(wr, wo + 18);
  };
  auto store_step = [&](int buf, RawStep &r, int kt) {
    // Keep the scheduler from hoisting work on the loaded values into the
    // MFMA section, where it would wait for loads still in flight.
    __builtin_amdgcn_sched_barrier(0);
    if (ragged && kt == nk - 1) {
      // Only the first block of this step lies inside K: zero the X pieces
      // and the W block past it (they were read from the next row).
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (8 * ((tid + kThreads * it) & 7) >= 32) r.x[it] = u32x4{0, 0, 0, 0};
      if (wblk) r.w.d = 0;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + kThreads * it;
      *reinterpret_cast<u32x4 *>(&Xs[buf][(idx >> 3) * LDS_STRIDE + 8 * (idx & 7)]) = r.x[it];
    }
    u32x4 out[4];
    dequant_q8_0(r.w, out);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4 *>(&Ws[buf][(tid >> 1) * LDS_STRIDE + 32 * wblk + 8 * j]) = out[j];
    __builtin_amdgcn_sched_barrier(0);
  };

  // Each wave owns a 64 x 64 block as 2 x 2 tiles of v_mfma_f32_32x32x16_f16:
  // lane l supplies row (or column) l % 32 and the 8 k values 8 * (l / 32)
  // .. +7 of each operand, and holds D[8 * (v / 4) + 4 * (l / 32) + v % 4]
  // [l % 32] for v = 0..15.
  const int l32 = lane & 31, lh = lane >> 5;
  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      half8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const half8_t *>(
            &Xs[buf][(wm * 64 + i * 32 + l32) * LDS_STRIDE + kk * 16 + 8 * lh]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const half8_t *>(
            &Ws[buf][(wn * 64 + j * 32 + l32) * LDS_STRIDE + kk * 16 + 8 * lh]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Software pipeline: the global loads of step kt + 2 are issued before the
  // MFMAs of step kt, and step kt + 1 (loaded one step earlier) is written
  // to the other LDS buffer after them, so every load has two steps of
  // matrix work to arrive. Steps past the end are loaded from clamped
  // addresses and never used.
  RawStep ra, rb;
  load_step(ra, 0);
  load_step(rb, nk > 1 ? 1 : 0);
  store_step(0, ra, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    load_step(ra, kt + 2);
    compute(0);
    store_step(1, rb, kt + 1);
    __syncthreads();
    load_step(rb, kt + 3 < nk ? kt + 3 : kt + 2);
    compute(1);
    store_step(0, ra, kt + 2);
    __syncthreads();
  }
  compute(0);
  if (kt + 1 < nk) {
    store_step(1, rb, kt + 1);
    __syncthreads();
    compute(1);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        if (row < M && col < N)
          Y[row * N + col] = __builtin_bit_cast(uint16_t, (half_t)acc[i][j][v]);
      }
    }
}

}  // namespace

hipError_t gemm_q8_0_launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M,
                            int64_t N, int64_t K, int num_cus, hipStream_t stream) {
  (void)num_cus;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff || (int64_t)BM * K * 2 >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_q8_0_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, W, X, Y,
                     M, N, K, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace lqmm

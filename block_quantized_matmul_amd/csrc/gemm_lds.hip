// Quantized x fp16 GEMM with the weights dequantized into LDS: Y[m][n] =
// sum_k X[m][k] * W[n][k], fp32 accumulation on the f16 matrix cores, fp16
// output, for any block format with a trait below (Q8_0, Q4_0, Q4_K).
//
// This is the matmul case of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao", as the page states it: the
// blocks of each K step are loaded, dequantized into shared memory (LDS) and
// reused by every row of the M tile; the format only changes the load and
// dequantization routine.
//
// * 128 x 128 output tile per 256-thread workgroup; four waves, each a 64 x
//   64 block of 2 x 2 v_mfma_f32_32x32x16_f16 tiles.
// * K advances 64 per step. Thread t loads, for weight row t / 2 of the tile,
//   the 32 weights 32 * (t % 2) .. +31 of the step (one Q8_0 or Q4_0 block,
//   or one Q4_K sub-block with its super-block header), and four 16-byte
//   pieces of the X tile; it dequantizes its 32 weights to fp16, one
//   rounding per weight (Q8_0 d*q, Q4_0 d*(q-8), Q4_K d*sc*q - dmin*m
//   formed in fp32), and writes them, in k order, into the W tile in LDS
//   next to the X tile.
// * Two LDS buffers; the global loads of step kt + 2 are in flight during the
//   MFMAs of step kt, and step kt + 1 is written to the other buffer after
//   them.
// * Ragged K (K % 64 == 32, formats with 32-weight blocks): the last step holds
//   one block; its second half is zeroed.
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halves per LDS row (144 bytes)
constexpr int kThreads = 256;

// Two bytes b0, b1 of dword v (byte selector sel) as the 16-bit lanes
// (b0, b1); nibble masks and a magic exponent then give exact fp16 values.
__device__ __forceinline__ uint32_t byte_pair(uint32_t v, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, v, sel);
}
constexpr uint32_t kSel01 = 0x0C010C00u;  // bytes 0, 1 -> 16-bit lanes 0, 1
constexpr uint32_t kSel23 = 0x0C030C02u;  // bytes 2, 3

// ---- Q8_0: 34-byte blocks; a thread's 32 weights are one block -----------------
struct GemmQ8_0 {
  static constexpr int kBlock = 32;  // weights per block (ragged K allowed)
  static __host__ __device__ int64_t row_bytes(int64_t K) { return K / 32 * 34; }
  struct Raw {
    u32x4 q0, q1;
    uint32_t d;
  };
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t row_off, int kt, int h) {
    const uint32_t o = row_off + (uint32_t)(2 * kt + h) * 34u;
    Raw w;
    w.d = buf_load_u16(r, o);
    w.q0 = buf_load_b128(r, o + 2);
    w.q1 = buf_load_b128(r, o + 18);
    return w;
  }
  static __device__ __forceinline__ void zero(Raw &w) { w.d = 0; }
  // q ^ 0x80 in the mantissa of 1024.0 is exactly 1152 + q; then (-1152, *d).
  static __device__ __forceinline__ void dequant(const Raw &r, int /*h*/, u32x4 (&out)[4]) {
    const half_t dh = __builtin_bit_cast(half_t, (uint16_t)r.d);
    const half2_t d2 = {dh, dh};
    const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
    const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t u = w[i] ^ 0x80808080u;
      half2_t lo = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
      half2_t hi = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
      lo = (lo - bias) * d2;
      hi = (hi - bias) * d2;
      out[i >> 1][(i & 1) * 2 + 0] = as_u32(lo);
      out[i >> 1][(i & 1) * 2 + 1] = as_u32(hi);
    }
  }
};

// ---- Q4_0: 18-byte blocks; weight j < 16 is the low nibble of qs[j], weight
// j + 16 its high nibble. A byte pair (b, b+1) of qs gives the fp16 pairs
// (1024 + lo_b, 1024 + lo_b+1) (weights b, b+1) and (64 + hi_b, 64 + hi_b+1)
// (weights 16 + b, 17 + b); then (-1032 or -72, *d): d * (q - 8), one rounding.
struct GemmQ4_0 {
  static constexpr int kBlock = 32;
  static __host__ __device__ int64_t row_bytes(int64_t K) { return K / 32 * 18; }
  struct Raw {
    u32x4 q;
    uint32_t d;
  };
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t row_off, int kt, int h) {
    const uint32_t o = row_off + (uint32_t)(2 * kt + h) * 18u;
    Raw w;
    w.d = buf_load_u16(r, o);
    w.q = buf_load_b128(r, o + 2);
    return w;
  }
  static __device__ __forceinline__ void zero(Raw &w) { w.d = 0; }
  static __device__ __forceinline__ void dequant(const Raw &r, int /*h*/, u32x4 (&out)[4]) {
    const half_t dh = __builtin_bit_cast(half_t, (uint16_t)r.d);
    const half2_t d2 = {dh, dh};
    const half2_t blo = {(half_t)-1032.0f, (half_t)-1032.0f};
    const half2_t bhi = {(half_t)-72.0f, (half_t)-72.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // byte pair 2i, 2i + 1 of qs
      const uint32_t pr = byte_pair(r.q[i >> 1], (i & 1) ? kSel23 : kSel01);
      const half2_t lo = as_half2((pr & 0x000F000Fu) | 0x64006400u);
      const half2_t hi = as_half2((pr & 0x00F000F0u) | 0x54005400u);
      out[i >> 2][i & 3] = as_u32((lo + blo) * d2);        // weights 2i, 2i + 1
      out[2 + (i >> 2)][i & 3] = as_u32((hi + bhi) * d2);  // weights 16 + 2i, 17 + 2i
    }
  }
};

// ---- Q4_K: 144-byte super-blocks of 256 weights; a step (64 weights) is the
// sub-block pair j = kt % 4 of super-block kt / 4, and thread half h takes
// sub-block s = 2j + h: the low (h = 0) or high (h = 1) nibbles of qs[32j ..
// 32j + 31], in k order, with its 6-bit scale and min from the header.
struct GemmQ4_K {
  static constexpr int kBlock = 256;
  static __host__ __device__ int64_t row_bytes(int64_t K) { return K / 256 * 144; }
  struct Raw {
    u32x4 hdr;  // d | dmin << 16, scales[0..3], scales[4..7], scales[8..11]
    u32x4 q0, q1;
    int kt;
  };
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t row_off, int kt, int /*h*/) {
    const uint32_t o = row_off + (uint32_t)(kt >> 2) * 144u;
    const uint32_t qo = o + 16 + 32 * (uint32_t)(kt & 3);
    Raw w;
    w.hdr = buf_load_b128(r, o);
    w.q0 = buf_load_b128(r, qo);
    w.q1 = buf_load_b128(r, qo + 16);
    w.kt = kt;
    return w;
  }
  static __device__ __forceinline__ void zero(Raw &w) { w.hdr.x = 0; }
  static __device__ __forceinline__ uint32_t sbyte(const u32x4 &hdr, int i) {  // scales[i]
    return (hdr[1 + (i >> 2)] >> (8 * (i & 3))) & 0xFFu;
  }
  static __device__ __forceinline__ void dequant(const Raw &r, int h, u32x4 (&out)[4]) {
    const int s = 2 * (r.kt & 3) + h;
    uint32_t sc, m;
    if (s < 4) {
      sc = sbyte(r.hdr, s) & 63u;
      m = sbyte(r.hdr, s + 4) & 63u;
    } else {
      sc = (sbyte(r.hdr, s + 4) & 15u) | ((sbyte(r.hdr, s - 4) >> 6) << 4);
      m = (sbyte(r.hdr, s + 4) >> 4) | ((sbyte(r.hdr, s) >> 6) << 4);
    }
    // d*sc and dmin*m are exact in fp32 (11 x 6 significant bits), and so is
    // d*sc*q - dmin*m up to one fp32 rounding: each weight is rounded to fp16
    // once, like the other formats' weights.
    const float dsc = f16_bits_to_f32(r.hdr.x & 0xFFFFu) * (float)sc;
    const float dmm = f16_bits_to_f32(r.hdr.x >> 16) * (float)m;
    const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // weights 4i .. 4i + 3 of the sub-block
      const uint32_t v = (h ? w[i] >> 4 : w[i]) & 0x0F0F0F0Fu;
      float f[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) f[b] = __builtin_fmaf((float)((v >> (8 * b)) & 0xFFu), dsc, -dmm);
      out[i >> 1][(i & 1) * 2 + 0] = pack_half2(f[0], f[1]);
      out[i >> 1][(i & 1) * 2 + 1] = pack_half2(f[2], f[3]);
    }
  }
};

// Raw global data of one K step for one thread: four 16-byte pieces of the X
// tile and its 32 weights' raw bytes.
template <class F>
struct RawStep {
  u32x4 x[4];
  typename F::Raw w;
};

template <class F>
__global__ void __launch_bounds__(kThreads)
gemm_lds_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ X,
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
  const uint32_t Ku = (uint32_t)K;
  const uint32_t row_bytes = (uint32_t)F::row_bytes(K);
  const int nk = (int)((K + BK - 1) / BK);
  const bool ragged = K % BK != 0;  // the last step holds one 32-weight block

  // The tile's X rows and W rows through buffer resources that end at the
  // last row of the tensor: loads of rows past M or N return zeros (their
  // results are never stored). Offsets are 32-bit (the host keeps
  // BM * K * 2 and BN * row_bytes below 2^31). Nothing is computed from
  // loaded data before it is written to LDS, so the loads of two steps stay
  // in flight together.
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
  const int wh = tid & 1;  // which 32 weights of the step
  const uint32_t wrow_off = (uint32_t)(tid >> 1) * row_bytes;

  auto load_step = [&](RawStep<F> &r, int kt) {
#pragma unroll
    for (int it = 0; it < 4; ++it) r.x[it] = buf_load_b128(xr, xoff[it] + kt * (BK * 2));
    r.w = F::load(wr, wrow_off, kt, wh);
  };
  auto store_step = [&](int buf, RawStep<F> &r, int kt) {
    // Keep the scheduler from hoisting work on the loaded values into the
    // MFMA section, where it would wait for loads still in flight.
    __builtin_amdgcn_sched_barrier(0);
    if (ragged && kt == nk - 1) {
      // Only the first 32 weights of this step lie inside K: zero the X
      // pieces and the weights past it (they were read from the next row).
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (8 * ((tid + kThreads * it) & 7) >= 32) r.x[it] = u32x4{0, 0, 0, 0};
      if (wh) F::zero(r.w);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + kThreads * it;
      *reinterpret_cast<u32x4 *>(&Xs[buf][(idx >> 3) * LDS_STRIDE + 8 * (idx & 7)]) = r.x[it];
    }
    u32x4 out[4];
    F::dequant(r.w, wh, out);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4 *>(&Ws[buf][(tid >> 1) * LDS_STRIDE + 32 * wh + 8 * j]) = out[j];
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
  RawStep<F> ra, rb;
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

template <class F>
hipError_t launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M, int64_t N,
                  int64_t K, hipStream_t stream) {
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  // 32-bit buffer offsets within a tile (the resource sizes included).
  if (tiles > 0x7fffffff || (int64_t)BM * K * 2 >= ((int64_t)1 << 31) ||
      (int64_t)BN * F::row_bytes(K) >= ((int64_t)1 << 31) || K % F::kBlock != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_lds_kernel<F>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, W, X, Y,
                     M, N, K, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_lds_launch(GemmFormat f, const uint8_t *W, const uint16_t *X, uint16_t *Y,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (f) {
    case GemmFormat::Q8_0: return launch<GemmQ8_0>(W, X, Y, M, N, K, stream);
    case GemmFormat::Q4_0: return launch<GemmQ4_0>(W, X, Y, M, N, K, stream);
    case GemmFormat::Q4_K: return launch<GemmQ4_K>(W, X, Y, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lqmm

// Dequantize-in-register GEMV for llama.cpp Q4_0 and Q4_K weight blocks on
// gfx950: y[b][n] = sum_k W[n][k] * x[b][k] for a few activation rows b.
//
// This is the decode mat-vec of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao": weight blocks are never
// expanded in memory; each lane unpacks its block's nibbles in registers and
// multiplies them with the activations. The quantization format is a
// compile-time trait (the page's "dequantization chosen at compile time").
//
// Design for CDNA4:
// * A workgroup (512 threads) first stages its activations in LDS as fp16,
//   in the exact pair order the nibble unpacker produces (below), together
//   with per-unit sums of the staged values. It then walks rows with a grid
//   stride; every wave reads weights straight from HBM into registers.
// * A "unit" is the run of weights one lane handles per row: one Q4_0 block
//   (32 weights, 18 bytes) or a quarter of a Q4_K super-block (64 weights:
//   the 16-byte header plus 32 bytes of nibbles). Consecutive lanes take
//   consecutive units, so each wave-wide load covers one contiguous span.
//   LPR lanes share a row (LPR = units per row rounded up to a power of two,
//   at most 64) and their partial sums are combined with DPP.
// * Nibble unpacking uses the fp16 exponent trick: OR-ing a nibble into the
//   mantissa of 1024.0 (0x6400) gives the exact fp16 value 1024 + q (low
//   nibble) or 1024 + 16q (high nibble) with one v_and_or_b32 per pair. The
//   bias terms are removed with the staged sums, and high-nibble pairs are
//   matched with activations pre-scaled by 1/16. Two fp16 products are
//   accumulated in fp32 by v_dot2_f32_f16; the block scales are applied in
//   fp32 once per unit.
// * Each lane handles R rows per unit so an activation word read from LDS is
//   used R times.
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int kGemvThreads = 512;
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024.0, 1024.0)

// Unpack one 32-bit word of nibbles (bytes e = 0..3, each holding a "lo"
// nibble and a "hi" nibble) into four fp16 pairs:
//   P0 = (1024+lo0, 1024+lo2)      P1 = (1024+16hi0, 1024+16hi2)
//   P2 = (1024+lo1, 1024+lo3)      P3 = (1024+16hi1, 1024+16hi3)
struct Nibbles {
  half2_t p0, p1, p2, p3;
};
__device__ __forceinline__ Nibbles unpack_word(uint32_t v) {
  uint32_t v8 = v >> 8;
  Nibbles n;
  n.p0 = as_half2((v & 0x000F000Fu) | kMagic);
  n.p1 = as_half2((v & 0x00F000F0u) | kMagic);
  n.p2 = as_half2((v8 & 0x000F000Fu) | kMagic);
  n.p3 = as_half2((v8 & 0x00F000F0u) | kMagic);
  return n;
}

// ---- Q4_0: unit = one block of 32 weights ----------------------------------
// Word t (t = 0..3) of the block's qs holds lo positions 4t..4t+3 and hi
// positions 16+4t..16+4t+3. The staged sums hold, per unit and batch row,
// -(1032*S_lo + 1152*S_hi) where S_lo is the sum of the staged lo values and
// S_hi the sum of the staged (x/16) hi values; then
//   sum_j (q_j - 8) x_j = staged + sum of the dot products.
struct FmtQ4_0 {
  static constexpr int kUnitWeights = 32;
  static constexpr int kWords = 4;
  static constexpr int kSums = 1;
  struct Raw {
    u32x4 q;
    uint32_t d;
  };
  static __device__ __forceinline__ Raw load(const uint8_t *row, int64_t unit) {
    const uint8_t *p = row + unit * 18;
    Raw r;
    r.q = load_u32x4_unaligned(p + 2);
    r.d = load_u16(p);
    return r;
  }
  static __device__ __forceinline__ Raw zero() {
    Raw r;
    r.q = u32x4{0, 0, 0, 0};
    r.d = 0;
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, float slo, float shi) {
    sums[idx] = -(1032.0f * slo + 1152.0f * shi);
  }

  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs,
                                                 const float *sums, int u, int nu,
                                                 float (&acc)[R][B]) {
    float s[R][B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float c = sums[b * nu + u];
#pragma unroll
      for (int r = 0; r < R; ++r) s[r][b] = c;
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * nu + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Nibbles n = unpack_word(raw[r].q[t]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float a = s[r][b];
          a = dot2(n.p0, as_half2(X[b].x), a);
          a = dot2(n.p1, as_half2(X[b].y), a);
          a = dot2(n.p2, as_half2(X[b].z), a);
          a = dot2(n.p3, as_half2(X[b].w), a);
          s[r][b] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float d = f16_bits_to_f32(raw[r].d);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d, s[r][b], acc[r][b]);
    }
  }
};

// ---- Q4_K: unit = a quarter super-block (sub-blocks 2i and 2i+1) -----------
// Lane unit u of a row is sub-block pair i = u % 4 of super-block u / 4.
// Word t (t = 0..7) of the pair's 32 qs bytes holds sub-block 2i weights
// 4t..4t+3 (low nibbles, "lo") and sub-block 2i+1 weights 4t..4t+3 (high
// nibbles, "hi"). The staged sums are (-1024*S_lo, -1024*S_hi) per unit and
// batch row, which remove the 1024 bias of each dot product; they also give
// the activation sums needed by the dmin * m term.
struct FmtQ4_K {
  static constexpr int kUnitWeights = 64;
  static constexpr int kWords = 8;
  static constexpr int kSums = 2;
  struct Raw {
    u32x4 h;   // d | dmin << 16, scales[0..3], scales[4..7], scales[8..11]
    u32x4 q0;  // qs words 0..3 of the pair
    u32x4 q1;  // qs words 4..7
  };
  static __device__ __forceinline__ Raw load(const uint8_t *row, int64_t unit) {
    const uint8_t *sb = row + (unit >> 2) * 144;
    const uint8_t *qs = sb + 16 + (unit & 3) * 32;
    Raw r;
    r.h = *reinterpret_cast<const u32x4 *>(sb);
    r.q0 = *reinterpret_cast<const u32x4 *>(qs);
    r.q1 = *reinterpret_cast<const u32x4 *>(qs + 16);
    return r;
  }
  static __device__ __forceinline__ Raw zero() {
    Raw r;
    r.h = u32x4{0, 0, 0, 0};
    r.q0 = r.h;
    r.q1 = r.h;
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, float slo, float shi) {
    sums[2 * idx] = -1024.0f * slo;
    sums[2 * idx + 1] = -1024.0f * shi;
  }

  // 6-bit scale and min of sub-block s from the scale words h1, h2, h3.
  static __device__ __forceinline__ void scale_min(const u32x4 &h, int s, uint32_t &sc,
                                                   uint32_t &m) {
    uint32_t sh = (s & 3) * 8;
    uint32_t b1 = (h.y >> sh) & 0xFF, b2 = (h.z >> sh) & 0xFF, b3 = (h.w >> sh) & 0xFF;
    uint32_t sc_lo = b1 & 63, m_lo = b2 & 63;
    uint32_t sc_hi = (b3 & 15) | ((b1 >> 6) << 4);
    uint32_t m_hi = (b3 >> 4) | ((b2 >> 6) << 4);
    sc = s < 4 ? sc_lo : sc_hi;
    m = s < 4 ? m_lo : m_hi;
  }

  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs,
                                                 const float *sums, int u, int nu,
                                                 float (&acc)[R][B]) {
    float slo[R][B], shi[R][B], nsl[B], nsh[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      nsl[b] = sums[2 * (b * nu + u)];
      nsh[b] = sums[2 * (b * nu + u) + 1];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        slo[r][b] = nsl[b];
        shi[r][b] = nsh[b];
      }
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * nu + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t w = t < 4 ? raw[r].q0[t & 3] : raw[r].q1[t & 3];
        Nibbles n = unpack_word(w);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float lo = slo[r][b], hi = shi[r][b];
          lo = dot2(n.p0, as_half2(X[b].x), lo);
          hi = dot2(n.p1, as_half2(X[b].y), hi);
          lo = dot2(n.p2, as_half2(X[b].z), lo);
          hi = dot2(n.p3, as_half2(X[b].w), hi);
          slo[r][b] = lo;
          shi[r][b] = hi;
        }
      }
    }
    const int pair = u & 3;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float d = f16_bits_to_f32(raw[r].h.x & 0xFFFF);
      float dmin = f16_bits_to_f32(raw[r].h.x >> 16);
      uint32_t sc0, m0, sc1, m1;
      scale_min(raw[r].h, 2 * pair, sc0, m0);
      scale_min(raw[r].h, 2 * pair + 1, sc1, m1);
      float dsc0 = d * (float)sc0, dsc1 = d * (float)sc1;
      // -dmin*m*S = dmin*m*(-1024*S)/1024; the hi sum is of x/16 values.
      float dm0 = dmin * (float)m0 * (1.0f / 1024.0f);
      float dm1 = dmin * (float)m1 * (1.0f / 64.0f);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float a = acc[r][b];
        a = __builtin_fmaf(dsc0, slo[r][b], a);
        a = __builtin_fmaf(dsc1, shi[r][b], a);
        a = __builtin_fmaf(dm0, nsl[b], a);
        a = __builtin_fmaf(dm1, nsh[b], a);
        acc[r][b] = a;
      }
    }
  }
};

// ---- the kernel -------------------------------------------------------------
// x rows: x + b*ldx, covering units [unit0, unit0 + nu) of every weight row.
// accumulate != 0: y += result (used when K is split over several launches).
template <class F, int B, int R>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int64_t unit0, int nu,
            const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
            int64_t N, int lpr_log2, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);
  float *sums = reinterpret_cast<float *>(smem + (size_t)B * F::kWords * nu * 16);

  const int tid = threadIdx.x;

  // 1. stage activations: item (b, u, t) -> 8 fp16 values in unpack order.
  {
    constexpr int T = F::kWords;
    constexpr int HALF = F::kUnitWeights / 2;
    const int nitems = B * nu * T;
    for (int i = tid; i < nitems; i += kGemvThreads) {
      const int t = i % T;
      const int bu = i / T;
      const int u = bu % nu;
      const int b = bu / nu;
      const float *base = x + b * ldx + (int64_t)u * F::kUnitWeights + 4 * t;
      float4_t lo = *reinterpret_cast<const float4_t *>(base);
      float4_t hi = *reinterpret_cast<const float4_t *>(base + HALF) * 0.0625f;
      half_t l0 = (half_t)lo.x, l1 = (half_t)lo.y, l2 = (half_t)lo.z, l3 = (half_t)lo.w;
      half_t h0 = (half_t)hi.x, h1 = (half_t)hi.y, h2 = (half_t)hi.z, h3 = (half_t)hi.w;
      u32x4 word;
      word.x = as_u32(half2_t{l0, l2});
      word.y = as_u32(half2_t{h0, h2});
      word.z = as_u32(half2_t{l1, l3});
      word.w = as_u32(half2_t{h1, h3});
      xs[(b * T + t) * nu + u] = word;
      float slo = ((float)l0 + (float)l1) + ((float)l2 + (float)l3);
      float shi = ((float)h0 + (float)h1) + ((float)h2 + (float)h3);
      slo = group_sum(slo, T);
      shi = group_sum(shi, T);
      if (t == T - 1) F::stage_sums(sums, b * nu + u, slo, shi);
    }
  }
  __syncthreads();

  // 2. rows.
  const int lane = tid & (kWave - 1);
  const int lpr = 1 << lpr_log2;
  const int slot = lane >> lpr_log2;
  const int p = lane & (lpr - 1);
  const int slots = kWave >> lpr_log2;
  const int64_t rows_per_iter = (int64_t)slots * R;
  const int64_t wave = (int64_t)blockIdx.x * (kGemvThreads / kWave) + (tid / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * (kGemvThreads / kWave);

  for (int64_t rowbase = wave * rows_per_iter; rowbase < N; rowbase += nwaves * rows_per_iter) {
    const int64_t row0 = rowbase + (int64_t)slot * R;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

    for (int u = p; u < nu; u += lpr) {
      typename F::Raw raw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        raw[r] = row < N ? F::load(W + row * row_bytes, unit0 + u) : F::zero();
      }
      F::template compute<B, R>(raw, xs, sums, u, nu, acc);
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = group_sum(acc[r][b], lpr);

    if (p == lpr - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        if (row < N) {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            float v = acc[r][b];
            if (accumulate) v += y[b * ldy + row];
            y[b * ldy + row] = v;
          }
        }
      }
    }
  }
}

template <class F, int B, int R>
hipError_t launch_one(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                      hipStream_t stream) {
  auto kern = gemv_kernel<F, B, R>;
  static bool attr_done = false;  // benign race: setting the attribute twice is harmless
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxGemvLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.unit0, pl.nu, x, pl.ldx, y, pl.ldy, pl.N, pl.lpr_log2,
                     pl.accumulate);
  return hipGetLastError();
}

template <class F, int B>
hipError_t launch_r(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                    hipStream_t s) {
  switch (pl.rows_per_lane) {
    case 1: return launch_one<F, B, 1>(pl, W, x, y, s);
    case 2: return launch_one<F, B, 2>(pl, W, x, y, s);
    default: return launch_one<F, B, 4>(pl, W, x, y, s);
  }
}

template <class F>
hipError_t launch_b(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                    hipStream_t s) {
  switch (pl.batch) {
    case 1: return launch_r<F, 1>(pl, W, x, y, s);
    case 2: return launch_r<F, 2>(pl, W, x, y, s);
    case 3: return launch_r<F, 3>(pl, W, x, y, s);
    case 4: return launch_r<F, 4>(pl, W, x, y, s);
    case 5: return launch_r<F, 5>(pl, W, x, y, s);
    case 6: return launch_r<F, 6>(pl, W, x, y, s);
    case 7: return launch_r<F, 7>(pl, W, x, y, s);
    default: return launch_r<F, 8>(pl, W, x, y, s);
  }
}

}  // namespace

size_t gemv_lds_bytes(GemvFormat f, int batch, int nu) {
  if (f == GemvFormat::Q4_0)
    return (size_t)batch * nu * (FmtQ4_0::kWords * 16 + FmtQ4_0::kSums * 4);
  return (size_t)batch * nu * (FmtQ4_K::kWords * 16 + FmtQ4_K::kSums * 4);
}

int gemv_unit_weights(GemvFormat f) {
  return f == GemvFormat::Q4_0 ? FmtQ4_0::kUnitWeights : FmtQ4_K::kUnitWeights;
}

int gemv_threads() { return kGemvThreads; }

hipError_t gemv_launch(GemvFormat f, const GemvPlan &pl, const uint8_t *W, const float *x,
                       float *y, hipStream_t stream) {
  if (f == GemvFormat::Q4_0) return launch_b<FmtQ4_0>(pl, W, x, y, stream);
  return launch_b<FmtQ4_K>(pl, W, x, y, stream);
}

}  // namespace lqmm

// More block formats for the dot2 GEMV (gfx950): Q8_0, the 1-bit q1_0, the
// K-quants Q6_K and Q2_K, and the int4 group-32 layout of the pages' int4
// matmul. Each is a
// trait in the shape of those in gemv_common.hpp (units, staged activation
// words, staged sums, dot2 arithmetic), so the small-problem kernel takes it
// unchanged: "Resumo Tecnico: Llamas na Web", section "Design de Shader
// Consciente de Quantizacao", adds a format by adding its dequantization
// routine, without rewriting the matmul core.
//
// Every trait turns codes into exact fp16 values c + bias (bias 1024 or 64,
// by the exponent trick), multiplies them with fp16 activations in fp32
// (v_dot2_f32_f16), removes bias * sum(x) with staged activation sums, and
// applies its block scales in fp32 once per group.
#pragma once

#include "gemv_common.hpp"

namespace lqmm {
namespace {

constexpr uint32_t kMagicBytes = 0x64646464u;  // bytes 0x64: fp16 high byte of 1024.0

// Eight code bytes (dwords a: c0..c3, b: c4..c7, each c < 256) as the fp16
// pairs (1024+c0, 1024+c2), (1024+c4, 1024+c6), (1024+c1, 1024+c3),
// (1024+c5, 1024+c7): the pairing of pack_xword's activation word.
__device__ __forceinline__ Nibbles bytes_to_halves(uint32_t a, uint32_t b) {
  Nibbles n;
  n.p0 = as_half2(__builtin_amdgcn_perm(kMagicBytes, a, 0x04020400u));
  n.p1 = as_half2(__builtin_amdgcn_perm(kMagicBytes, b, 0x04020400u));
  n.p2 = as_half2(__builtin_amdgcn_perm(kMagicBytes, a, 0x04030401u));
  n.p3 = as_half2(__builtin_amdgcn_perm(kMagicBytes, b, 0x04030401u));
  return n;
}

__device__ __forceinline__ float dot_word(const Nibbles &n, const u32x4 &X, float a) {
  a = dot2(n.p0, as_half2(X.x), a);
  a = dot2(n.p1, as_half2(X.y), a);
  a = dot2(n.p2, as_half2(X.z), a);
  a = dot2(n.p3, as_half2(X.w), a);
  return a;
}

// ---- Q8_0: unit = one block (32 weights, 34 bytes) ---------------------------
// [d fp16][q 32 x int8] at byte 34 u (2-byte aligned: a 2-byte and two
// unaligned 16-byte loads). Code byte q ^ 0x80 = q + 128 in the mantissa of
// 1024.0 is exactly 1152 + q. Word t holds weights 8t..8t+7 (code dwords
// 2t, 2t+1); the staged sum is -1152 * sum(x) over the block.
struct FmtQ8_0 {
  static constexpr int kUnitWeights = 32;
  static constexpr int kWords = 4;
  static constexpr int kSums = 1;
  static constexpr int kSumWords = 4;
  static __device__ __forceinline__ int x_lo(int t) { return 8 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 8 * t + 4; }
  struct Raw {
    u32x4 q0, q1;  // the 32 codes
    uint32_t d;
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) { return unit * 34; }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *p = row + unit * 34u;
    Raw r;
    r.d = load_u16(p);
    r.q0 = load_u32x4_unaligned(p + 2);
    r.q1 = load_u32x4_unaligned(p + 18);
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int /*g*/, float slo,
                                                    float shi) {
    sums[idx] = -1152.0f * (slo + shi);
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks & /*k*/, float (&acc)[R][B]) {
    float s[R][B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float c = sums[b * nu + u];
#pragma unroll
      for (int r = 0; r < R; ++r) s[r][b] = c;
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4 &q = t < 2 ? raw[r].q0 : raw[r].q1;
        const int i = 2 * (t & 1);
        const Nibbles n = bytes_to_halves(q[i] ^ 0x80808080u, q[i + 1] ^ 0x80808080u);
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b] = dot_word(n, X[b], s[r][b]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d = valid ? f16_bits_to_f32(raw[r].d) : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d, s[r][b], acc[r][b]);
    }
  }
};

// ---- q1_0: unit = one block (32 weights, 6 bytes) ---------------------------
// [d fp16][32 code bits, least significant bit first] at byte 6 u (2-byte
// aligned: a 2-byte and an unaligned 4-byte load). Word t holds weights
// 8t..8t+7, the bits of code byte t: spread as v = b | b << 14, bit pairs
// (0, 2), (4, 6), (1, 3), (5, 7) sit at bits 0 and 16 of v, v >> 4, v >> 1
// and v >> 5, and one v_and_or_b32 with 0x00010001 puts each pair into the
// mantissas of fp16 (1024.0, 1024.0): exactly (1024 + c, 1024 + c'). The
// dot products give sum (1024 + c) x; since w = d (2c - 1),
// sum w x = 2d (dot - 1024.5 S), so the staged sum is -1024.5 * S and the
// scale 2d is applied in fp32.
struct FmtQ1_0 {
  static constexpr int kUnitWeights = 32;
  static constexpr int kWords = 4;
  static constexpr int kSums = 1;
  static constexpr int kSumWords = 4;
  static __device__ __forceinline__ int x_lo(int t) { return 8 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 8 * t + 4; }
  struct Raw {
    uint32_t bits;
    uint32_t d;
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) { return unit * 6; }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *p = row + unit * 6u;
    Raw r;
    r.d = load_u16(p);
    __builtin_memcpy(&r.bits, p + 2, 4);
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int /*g*/, float slo,
                                                    float shi) {
    sums[idx] = -1024.5f * (slo + shi);
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks &k, float (&acc)[R][B]) {
    const uint32_t pair_mask = 0x00010001u;
    float s[R][B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float c = sums[b * nu + u];
#pragma unroll
      for (int r = 0; r < R; ++r) s[r][b] = c;
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t byte = (raw[r].bits >> (8 * t)) & 0xFFu;
        const uint32_t v = byte | (byte << 14);
        Nibbles n;
        n.p0 = as_half2(and_or(v, pair_mask, k.magic));
        n.p1 = as_half2(and_or(v >> 4, pair_mask, k.magic));
        n.p2 = as_half2(and_or(v >> 1, pair_mask, k.magic));
        n.p3 = as_half2(and_or(v >> 5, pair_mask, k.magic));
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b] = dot_word(n, X[b], s[r][b]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d2 = valid ? 2.0f * f16_bits_to_f32(raw[r].d) : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d2, s[r][b], acc[r][b]);
    }
  }
};

// ---- Q6_K: unit = half a super-block (128 weights) -------------------------
// Super-block (210 bytes, 2-byte aligned): [ql 128][qh 64][scales 16 x
// int8][d]. Half h (unit parity) reads ql[64h..64h+63], qh[32h..32h+31] and
// scales[8h..8h+7]. Weight i = 32j + l of the half (j < 4, l < 32) has low
// bits from the low (j < 2) or high (j >= 2) nibble of ql[64h + 32(j%2) + l]
// and high bits 2j..2j+1 of qh[32h + l]; its scale is scales[8h + i/16].
// Word t (weights 8t..8t+7: j = t/4, l = 8(t%4) + 0..7) builds the 6-bit
// codes bytewise, then the fp16 values 1024 + q. Group g (weights 16g..16g+15,
// words 2g and 2g+1) has the staged sum -1056 * sum(x), removing 1024 + 32.
struct FmtQ6_K {
  static constexpr int kUnitWeights = 128;
  static constexpr int kWords = 16;
  static constexpr int kSums = 8;
  static constexpr int kSumWords = 2;
  static __device__ __forceinline__ int x_lo(int t) { return 8 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 8 * t + 4; }
  struct Raw {
    u32x4 ql[4];
    u32x4 qh[2];
    uint32_t sc0, sc1;  // scales[8h .. 8h+7]
    uint32_t d;
  };
  // Units come in pairs per super-block; a slice starts on an even unit.
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) {
    return (unit >> 1) * 210;
  }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *sb = row + (unit >> 1) * 210u;
    const uint32_t h = unit & 1u;
    Raw r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.ql[i] = load_u32x4_unaligned(sb + 64 * h + 16 * i);
#pragma unroll
    for (int i = 0; i < 2; ++i) r.qh[i] = load_u32x4_unaligned(sb + 128 + 32 * h + 16 * i);
    __builtin_memcpy(&r.sc0, sb + 192 + 8 * h, 4);
    __builtin_memcpy(&r.sc1, sb + 196 + 8 * h, 4);
    r.d = load_u16(sb + 208);
    return r;
  }
  static __device__ __forceinline__ uint32_t ql_dw(const Raw &r, int i) { return r.ql[i >> 2][i & 3]; }
  static __device__ __forceinline__ uint32_t qh_dw(const Raw &r, int i) { return r.qh[i >> 2][i & 3]; }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int g, float slo,
                                                    float shi) {
    sums[kSums * idx + g] = -1056.0f * (slo + shi);
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks & /*k*/, float (&acc)[R][B]) {
    float s[R][B][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float c = sums[kSums * (b * nu + u) + g];
#pragma unroll
        for (int r = 0; r < R; ++r) s[r][b][g] = c;
      }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      const int j = t >> 2, q4 = t & 3;
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int li = (j & 1) * 8 + 2 * q4;  // ql dword of bytes 32(j%2) + 8 q4
        const int ns = j >= 2 ? 4 : 0;
        const uint32_t ha = (qh_dw(raw[r], 2 * q4) >> (2 * j)) & 0x03030303u;
        const uint32_t hb = (qh_dw(raw[r], 2 * q4 + 1) >> (2 * j)) & 0x03030303u;
        const uint32_t qa = ((ql_dw(raw[r], li) >> ns) & 0x0F0F0F0Fu) | (ha << 4);
        const uint32_t qb = ((ql_dw(raw[r], li + 1) >> ns) & 0x0F0F0F0Fu) | (hb << 4);
        const Nibbles n = bytes_to_halves(qa, qb);
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b][t >> 1] = dot_word(n, X[b], s[r][b][t >> 1]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d = valid ? f16_bits_to_f32(raw[r].d) : 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t w = g < 4 ? raw[r].sc0 : raw[r].sc1;
        const float dg = d * (float)(int8_t)(w >> (8 * (g & 3)));
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(dg, s[r][b][g], acc[r][b]);
      }
    }
  }
};

// ---- Q2_K: unit = half a super-block (128 weights) -------------------------
// Super-block (84 bytes, 4-byte aligned): [scales 16][qs 64][d][dmin]. Half h
// reads qs[32h..32h+31] and scales[8h..8h+7]; weight i = 32j + l of the half
// is bits 2j..2j+1 of qs[32h + l]; group g (16 weights) has scale sc = low
// nibble and min m = high nibble of scales[8h + g]. The staged sum is the
// plain sum of the group's activations S: y += d sc (dot - 1024 S) - dmin m S.
struct FmtQ2_K {
  static constexpr int kUnitWeights = 128;
  static constexpr int kWords = 16;
  static constexpr int kSums = 8;
  static constexpr int kSumWords = 2;
  static __device__ __forceinline__ int x_lo(int t) { return 8 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 8 * t + 4; }
  struct Raw {
    u32x4 q[2];
    uint32_t sc0, sc1;
    uint32_t dd;  // d | dmin << 16
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) {
    return (unit >> 1) * 84;
  }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *sb = row + (unit >> 1) * 84u;
    const uint32_t h = unit & 1u;
    Raw r;
    r.q[0] = load_u32x4_unaligned(sb + 16 + 32 * h);
    r.q[1] = load_u32x4_unaligned(sb + 32 + 32 * h);
    __builtin_memcpy(&r.sc0, sb + 8 * h, 4);
    __builtin_memcpy(&r.sc1, sb + 4 + 8 * h, 4);
    __builtin_memcpy(&r.dd, sb + 80, 4);
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int g, float slo,
                                                    float shi) {
    sums[kSums * idx + g] = slo + shi;
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks & /*k*/, float (&acc)[R][B]) {
    float s[R][B][8];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float c = -1024.0f * sums[kSums * (b * nu + u) + g];
#pragma unroll
        for (int r = 0; r < R; ++r) s[r][b][g] = c;
      }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      const int j = t >> 2, q4 = t & 3;
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t qa = (raw[r].q[q4 >> 1][2 * (q4 & 1)] >> (2 * j)) & 0x03030303u;
        const uint32_t qb = (raw[r].q[q4 >> 1][2 * (q4 & 1) + 1] >> (2 * j)) & 0x03030303u;
        const Nibbles n = bytes_to_halves(qa, qb);
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b][t >> 1] = dot_word(n, X[b], s[r][b][t >> 1]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d = valid ? f16_bits_to_f32(raw[r].dd & 0xFFFFu) : 0.0f;
      const float dmin = valid ? f16_bits_to_f32(raw[r].dd >> 16) : 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t w = ((g < 4 ? raw[r].sc0 : raw[r].sc1) >> (8 * (g & 3))) & 0xFFu;
        const float dsc = d * (float)(w & 15u), dmm = dmin * (float)(w >> 4);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float S = sums[kSums * (b * nu + u) + g];
          acc[r][b] = __builtin_fmaf(dsc, s[r][b][g], __builtin_fmaf(-dmm, S, acc[r][b]));
        }
      }
    }
  }
};

// ---- int4 group-32: unit = one group (32 weights) ----------------------------
// The layout of "Compute Shaders con WebGPU para Inferencia ML", "Yendo a
// Cuantizado: Matmul INT4": 16 bytes of codes at byte 16 u of the row (eight
// sequential 4-bit codes per 32-bit word, two's complement), and the group's
// fp32 scale and zero point from separate arrays (GemvAux a, b). Code
// nibble ^ 8 is s + 8 in 0..15; unpack_word gives 1024 + s + 8 for the
// nibbles in bits 0-3 of a byte and 64 + s + 8 for those in bits 4-7,
// paired as (w0,w4), (w1,w5), (w2,w6), (w3,w7) (kAcrossPairs). Staged sums per
// group: -(1032 S_lo + 72 S_hi) and S = S_lo + S_hi;
// y += scale * (dot + staged - zero * S).
struct FmtI4G32 {
  static constexpr int kUnitWeights = 32;
  static constexpr int kWords = 4;
  static constexpr int kSums = 2;
  static constexpr int kSumWords = 4;
  static constexpr bool kAcrossPairs = true;
  static constexpr bool kAux = true;
  static __device__ __forceinline__ int x_lo(int t) { return 8 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 8 * t + 4; }
  struct Raw {
    u32x4 q;
    float scale, zero;
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) { return unit * 16; }
  static __device__ __forceinline__ Raw load_aux(const uint8_t *row, uint32_t unit, int64_t n,
                                                 int u0, const GemvAux &aux) {
    Raw r;
    r.q = *reinterpret_cast<const u32x4 *>(row + unit * 16u);
    const int64_t g = n * aux.groups_per_row + u0 + (int64_t)unit;
    r.scale = aux.a[g];
    r.zero = aux.b[g];
    return r;
  }
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int /*g*/, float slo,
                                                    float shi) {
    sums[2 * idx] = -(1032.0f * slo + 72.0f * shi);
    sums[2 * idx + 1] = slo + shi;
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks &k, float (&acc)[R][B]) {
    float s[R][B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float c = sums[2 * (b * nu + u)];
#pragma unroll
      for (int r = 0; r < R; ++r) s[r][b] = c;
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const Nibbles n = unpack_word(raw[r].q[t] ^ 0x88888888u, k);
#pragma unroll
        for (int b = 0; b < B; ++b) s[r][b] = dot_word(n, X[b], s[r][b]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = valid ? raw[r].scale : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float S = sums[2 * (b * nu + u) + 1];
        acc[r][b] = __builtin_fmaf(sc, __builtin_fmaf(-raw[r].zero, S, s[r][b]), acc[r][b]);
      }
    }
  }
};

}  // namespace
}  // namespace lqmm

// Block-format traits and activation staging shared by the GEMV kernels
// (gfx950). Each translation unit that includes this header gets its own
// copy (anonymous namespace); nothing here is part of the C ABI.
//
// A "unit" is the run of weights one lane takes from one weight row: one
// Q4_0 block (32 weights, 18 bytes), two consecutive Q4_0 blocks (64 weights,
// 36 bytes) or a quarter of a Q4_K super-block (64 weights: the 16-byte header
// plus 32 bytes of nibbles). The traits load units, unpack their nibbles in
// registers and multiply them with activations staged in LDS as fp16 words in
// unpack order ("Resumo Tecnico: Llamas na Web", section "Design de Shader
// Consciente de Quantizacao": the mat-vec dequantizes in registers; the
// dequantization is chosen at compile time).
#pragma once

#include <type_traits>

#include "lqmm_device.hpp"

namespace lqmm {
namespace {

constexpr uint32_t kMagic = 0x64006400u;    // fp16 pair (1024.0, 1024.0): low nibbles
constexpr uint32_t kMagicHi = 0x54005400u;  // fp16 pair (64.0, 64.0): high nibbles

// Unpack one 32-bit word of nibbles (bytes e = 0..3, each holding a "lo"
// nibble and a "hi" nibble) into four fp16 pairs, all exact:
//   p0 = (1024+lo0, 1024+lo2)      p1 = (64+hi0, 64+hi2)
//   p2 = (1024+lo1, 1024+lo3)      p3 = (64+hi1, 64+hi3)
// The staged activation word uses the same order: (x_lo0, x_lo2),
// (x_hi0, x_hi2), (x_lo1, x_lo3), (x_hi1, x_hi3).
struct Nibbles {
  half2_t p0, p1, p2, p3;
};

// (a & m) | o as one v_and_or_b32. Written out because the VOP3 encoding
// cannot take the two 32-bit literal masks, and with them inline the compiler
// splits every pair into a v_and_b32 and a v_or_b32; here the masks live in
// VGPRs (see UnpackMasks).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// The unpack constants, materialized once per kernel in VGPRs.
struct UnpackMasks {
  uint32_t lo, hi, magic, magic_hi;
  __device__ __forceinline__ UnpackMasks()
      : lo(0x000F000Fu), hi(0x00F000F0u), magic(kMagic), magic_hi(kMagicHi) {
    asm volatile("" : "+v"(lo), "+v"(hi), "+v"(magic), "+v"(magic_hi));
  }
};

__device__ __forceinline__ Nibbles unpack_word(uint32_t v, const UnpackMasks &k) {
  uint32_t v8 = v >> 8;
  Nibbles n;
  n.p0 = as_half2(and_or(v, k.lo, k.magic));
  n.p1 = as_half2(and_or(v, k.hi, k.magic_hi));
  n.p2 = as_half2(and_or(v8, k.lo, k.magic));
  n.p3 = as_half2(and_or(v8, k.hi, k.magic_hi));
  return n;
}

__device__ __forceinline__ half2_t h2(float v) { return half2_t{(half_t)v, (half_t)v}; }
__device__ __forceinline__ half2_t pk_fma(half2_t a, half2_t b, half2_t c) {
  return __builtin_elementwise_fma(a, b, c);
}

// ---- Q4_0: unit = one block of 32 weights ----------------------------------
// Word t (t = 0..3) of the block's qs holds lo positions 4t..4t+3 and hi
// positions 16+4t..16+4t+3.
struct FmtQ4_0 {
  static constexpr int kUnitWeights = 32;
  static constexpr int kWords = 4;
  static constexpr int kSums = 1;
  static constexpr int kSumWords = 4;  // words per staged activation sum
  // Activations of word t: lo values at x_lo(t) .. +3, hi values 16 later.
  static __device__ __forceinline__ int x_lo(int t) { return 4 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 16 + 4 * t; }
  struct Raw {
    u32x4 q;
    uint32_t d;
  };
  struct Prep {
    half2_t d2;
  };
  // Byte offset of unit `unit` (a multiple of 4 for Q4_K) in a row.
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) { return unit * 18; }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *p = row + unit * 18u;
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
  static __device__ __forceinline__ uint32_t word(const Raw &r, int t) { return r.q[t]; }

  // VALU mode. Staged sum per (unit, batch row): -(1032*S_lo + 72*S_hi) with
  // S_lo the sum of the staged lo activations and S_hi of the hi ones, so
  // that sum_j (q_j - 8) x_j = staged + the dot products (which multiply
  // 1024 + q and 64 + q).
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int /*g*/, float slo,
                                                    float shi) {
    sums[idx] = -(1032.0f * slo + 72.0f * shi);
  }
  // u must index a staged unit; `valid` = 0 makes the unit contribute 0.
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks &k, float (&acc)[R][B]) {
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
      for (int b = 0; b < B; ++b) X[b] = xs[(b * kWords + t) * xstride + u];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Nibbles n = unpack_word(raw[r].q[t], k);
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
      float d = valid ? f16_bits_to_f32(raw[r].d) : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d, s[r][b], acc[r][b]);
    }
  }

  // MFMA mode: fp16 weights d*(q-8) of word t (exact q-8, one rounding);
  // valid == false yields zero weights.
  static __device__ __forceinline__ Prep prep(const Raw &r, int /*pair*/, bool valid) {
    Prep p;
    p.d2 = as_half2(valid ? (r.d & 0xFFFFu) * 0x10001u : 0u);
    return p;
  }
  static __device__ __forceinline__ u32x4 dequant(const Raw &r, const Prep &p, int t,
                                                 const UnpackMasks &k) {
    Nibbles n = unpack_word(r.q[t], k);
    const half2_t lo_bias = h2(-1032.0f), hi_bias = h2(-72.0f);
    u32x4 w;
    w.x = as_u32((n.p0 + lo_bias) * p.d2);
    w.y = as_u32((n.p1 + hi_bias) * p.d2);
    w.z = as_u32((n.p2 + lo_bias) * p.d2);
    w.w = as_u32((n.p3 + hi_bias) * p.d2);
    return w;
  }
  // U consecutive units starting at `unit`, each clamped to `last`.
  template <int U>
  static __device__ __forceinline__ void load_units(const uint8_t *row, uint32_t unit,
                                                    uint32_t last, Raw (&out)[U]) {
#pragma unroll
    for (int j = 0; j < U; ++j) out[j] = load(row, unit + j <= last ? unit + j : last);
  }
};

// ---- Q4_K: unit = a quarter super-block (sub-blocks 2i and 2i+1) -----------
// Lane unit u of a row is sub-block pair i = u % 4 of super-block u / 4.
// Word t (t = 0..7) of the pair's 32 qs bytes holds sub-block 2i weights
// 4t..4t+3 (low nibbles, "lo") and sub-block 2i+1 weights 4t..4t+3 (high
// nibbles, "hi").
struct FmtQ4_K {
  static constexpr int kUnitWeights = 64;
  static constexpr int kWords = 8;
  static constexpr int kSums = 2;
  static constexpr int kSumWords = 8;
  // Activations of word t: sub-block 2i at x_lo(t) .. +3, sub-block 2i + 1
  // 32 later.
  static __device__ __forceinline__ int x_lo(int t) { return 4 * t; }
  static __device__ __forceinline__ int x_hi(int t) { return 32 + 4 * t; }
  struct Raw {
    u32x4 h;   // d | dmin << 16, scales[0..3], scales[4..7], scales[8..11]
    u32x4 q0;  // qs words 0..3 of the pair
    u32x4 q1;  // qs words 4..7
  };
  struct Prep {
    half2_t dsc_lo, dmm_lo, dsc_hi, dmm_hi;
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) {
    return (unit >> 2) * 144;
  }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *sb = row + (unit >> 2) * 144u;
    const uint8_t *qs = sb + 16 + (unit & 3u) * 32u;
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
  static __device__ __forceinline__ uint32_t word(const Raw &r, int t) {
    return t < 4 ? r.q0[t & 3] : r.q1[t & 3];
  }

  // 6-bit scales and mins of sub-blocks 2 * pair and 2 * pair + 1 from the
  // scale words h.y, h.z, h.w, as 16-bit lanes (sub-block 2 * pair low).
  // Their fields are bytes j and j + 1 (j = 2 * (pair & 1)) of the three
  // words: 6-bit fields of words 1 and 2 for sub-blocks 0..3, 4 + 2 bits of
  // word 3 and of word 1 (scale) or 2 (min) for 4..7. One byte permute per
  // word moves both bytes to the low byte of a 16-bit lane.
  static __device__ __forceinline__ void scale_min_pair(const u32x4 &h, int pair, uint32_t &sc,
                                                        uint32_t &m) {
    const uint32_t sel = 0x0C010C00u + (uint32_t)(pair & 1) * 0x00020002u;
    const uint32_t b1 = __builtin_amdgcn_perm(h.y, h.y, sel);
    const uint32_t b2 = __builtin_amdgcn_perm(h.z, h.z, sel);
    const uint32_t b3 = __builtin_amdgcn_perm(h.w, h.w, sel);
    const uint32_t sc_hi = (b3 & 0x000F000Fu) | ((b1 >> 2) & 0x00300030u);
    const uint32_t m_hi = ((b3 >> 4) & 0x000F000Fu) | ((b2 >> 2) & 0x00300030u);
    sc = pair < 2 ? b1 & 0x003F003Fu : sc_hi;
    m = pair < 2 ? b2 & 0x003F003Fu : m_hi;
  }

  // Unit uc of a chunk of whole super-blocks copied to LDS at `slot`.
  static __device__ __forceinline__ Raw read_stream_unit(const u32x4 *slot, int uc) {
    const u32x4 *sbp = slot + (uc >> 2) * 9;
    Raw r;
    r.h = sbp[0];
    r.q0 = sbp[1 + 2 * (uc & 3)];
    r.q1 = sbp[2 + 2 * (uc & 3)];
    return r;
  }
  // VALU mode. Staged sums per (unit, batch row): (-1024*S_lo, -64*S_hi),
  // which remove the 1024 and 64 biases of the dot products and give the
  // activation sums the dmin * m term needs.
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int /*g*/, float slo,
                                                    float shi) {
    sums[2 * idx] = -1024.0f * slo;
    sums[2 * idx + 1] = -64.0f * shi;
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks &k, float (&acc)[R][B]) {
    compute_with<B, R>(
        raw, [&](int b, int t) { return xs[(b * kWords + t) * xstride + u]; },
        [&](int b, int h) { return sums[2 * (b * nu + u) + h]; }, u, valid, k, acc);
  }
  // The same with the unit's staged words and sums taken from xword(b, t)
  // and sum(b, h) (h = 0: lo, 1: hi), wherever the caller keeps them.
  template <int B, int R, class XW, class SW>
  static __device__ __forceinline__ void compute_with(const Raw (&raw)[R], XW xword, SW sum, int u,
                                                      bool valid, const UnpackMasks &k,
                                                      float (&acc)[R][B]) {
    float slo[R][B], shi[R][B], nsl[B], nsh[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      nsl[b] = sum(b, 0);
      nsh[b] = sum(b, 1);
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
      for (int b = 0; b < B; ++b) X[b] = xword(b, t);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Nibbles n = unpack_word(word(raw[r], t), k);
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
      float d = valid ? f16_bits_to_f32(raw[r].h.x & 0xFFFF) : 0.0f;
      float dmin = valid ? f16_bits_to_f32(raw[r].h.x >> 16) : 0.0f;
      uint32_t sc, m;
      scale_min_pair(raw[r].h, pair, sc, m);
      const uint32_t sc0 = sc & 0xFF, sc1 = sc >> 16, m0 = m & 0xFF, m1 = m >> 16;
      float dsc0 = d * (float)sc0, dsc1 = d * (float)sc1;
      // -dmin*m*S = dmin*m*(-1024*S)/1024 (lo) = dmin*m*(-64*S)/64 (hi).
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

  // MFMA mode: fp16 weights d*sc*q - dmin*m with d*sc and dmin*m each
  // rounded to fp16 once per sub-block, then one fused rounding per weight;
  // valid == false yields zero weights.
  // Both sub-blocks are decoded at once as 16-bit lanes (sub-block 2*pair
  // low, 2*pair + 1 high): their scale and min fields are bytes j and j + 1
  // (j = 2*(pair & 1)) of the three scale words, 6-bit fields in words 1 and
  // 2 for sub-blocks 0..3, 4 + 2 bits from words 3 and 1 (or 2) for 4..7.
  // 1024 + v is exact in fp16, so v comes back exactly; the packed fp16
  // products d*sc and dmin*m are the exact products rounded once, as above.
  static __device__ __forceinline__ Prep prep(const Raw &r, int pair, bool valid) {
    const uint32_t sel = (pair & 1) ? 0x0C030C02u : 0x0C010C00u;  // bytes j, j+1 -> 16-bit lanes
    const uint32_t y = __builtin_amdgcn_perm(0u, r.h.y, sel);
    const uint32_t z = __builtin_amdgcn_perm(0u, r.h.z, sel);
    const uint32_t w = __builtin_amdgcn_perm(0u, r.h.w, sel);
    const bool first = pair < 2;
    const uint32_t m6 = first ? 0x003F003Fu : 0u, m2 = first ? 0u : 0x00300030u,
                   m4 = first ? 0u : 0x000F000Fu;
    const uint32_t sc = (y & m6) | ((y >> 2) & m2) | (w & m4);
    const uint32_t mn = (z & m6) | ((z >> 2) & m2) | ((w >> 4) & m4);
    const half2_t scv = as_half2(sc | kMagic) + h2(-1024.0f);
    const half2_t mnv = as_half2(mn | kMagic) + h2(-1024.0f);
    const uint32_t dd = valid ? r.h.x : 0u;
    const half2_t d2 = as_half2(__builtin_amdgcn_perm(dd, dd, 0x01000100u));   // d, d
    const half2_t dm2 = as_half2(__builtin_amdgcn_perm(dd, dd, 0x03020302u));  // dmin, dmin
    const half2_t dsc = scv * d2;
    const half2_t dmm = -(mnv * dm2);
    Prep p;
    p.dsc_lo = dsc.xx;
    p.dsc_hi = dsc.yy;
    p.dmm_lo = dmm.xx;
    p.dmm_hi = dmm.yy;
    return p;
  }
  static __device__ __forceinline__ u32x4 dequant(const Raw &r, const Prep &p, int t,
                                                 const UnpackMasks &k) {
    Nibbles n = unpack_word(word(r, t), k);
    const half2_t lo_bias = h2(-1024.0f), hi_bias = h2(-64.0f);
    u32x4 w;
    w.x = as_u32(pk_fma(n.p0 + lo_bias, p.dsc_lo, p.dmm_lo));
    w.y = as_u32(pk_fma(n.p1 + hi_bias, p.dsc_hi, p.dmm_hi));
    w.z = as_u32(pk_fma(n.p2 + lo_bias, p.dsc_lo, p.dmm_lo));
    w.w = as_u32(pk_fma(n.p3 + hi_bias, p.dsc_hi, p.dmm_hi));
    return w;
  }
  // U consecutive units starting at `unit`; four units starting at a
  // super-block boundary share one header load.
  // A row holds a multiple of 4 units (last + 1 is a multiple of 4). For
  // U == 4 the run is one whole super-block: its start is clamped to the
  // last super-block, so every load stays inside the row.
  template <int U>
  static __device__ __forceinline__ void load_units(const uint8_t *row, uint32_t unit,
                                                    uint32_t last, Raw (&out)[U]) {
    if (U == 4) {
      const uint32_t sbi = (unit >> 2) <= (last >> 2) ? (unit >> 2) : (last >> 2);
      const uint8_t *sb = row + sbi * 144u;
      const u32x4 h = *reinterpret_cast<const u32x4 *>(sb);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        out[j].h = h;
        out[j].q0 = *reinterpret_cast<const u32x4 *>(sb + 16 + 32 * j);
        out[j].q1 = *reinterpret_cast<const u32x4 *>(sb + 32 + 32 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < U; ++j) out[j] = load(row, unit + j <= last ? unit + j : last);
    }
  }
};

// ---- Q4_0 in VALU mode: unit = two consecutive blocks ----------------------
// 64 weights in 36 bytes at byte 36 u of the row: 4-byte aligned, loaded as
// 16 + 16 + 4 bytes. A lane that takes one 18-byte block per load issues a
// 2-byte-aligned 16-byte load and a 2-byte load per block; that pattern
// streamed at about 3.3 TB/s where aligned 16-byte loads (and this one) reach
// 4.5 TB/s (27 MiB, cold). Words 0..3 are block 0's qs (2 bytes into the
// unit, realigned with v_alignbyte_b32), words 4..7 block 1's (aligned).
// Each block keeps its own scale and its own staged activation sum.
struct FmtQ4_0x2 {
  static constexpr int kUnitWeights = 64;
  static constexpr int kWords = 8;
  static constexpr int kSums = 2;
  static constexpr int kSumWords = 4;
  static __device__ __forceinline__ int x_lo(int t) { return 32 * (t >> 2) + 4 * (t & 3); }
  static __device__ __forceinline__ int x_hi(int t) { return 16 + x_lo(t); }
  struct Raw {
    u32x4 a, b;  // bytes 0..15, 16..31
    uint32_t c;  // bytes 32..35
  };
  static __host__ __device__ __forceinline__ int64_t unit_offset(int64_t unit) { return unit * 36; }
  // Unit uc of a chunk of whole units copied to LDS at `slot` (36 bytes,
  // 4-byte aligned: read as dwords).
  static __device__ __forceinline__ Raw read_stream_unit(const u32x4 *slot, int uc) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(slot) + 9 * uc;
    Raw r;
    r.a = u32x4{w[0], w[1], w[2], w[3]};
    r.b = u32x4{w[4], w[5], w[6], w[7]};
    r.c = w[8];
    return r;
  }
  static __device__ __forceinline__ Raw load(const uint8_t *row, uint32_t unit) {
    const uint8_t *p = row + unit * 36u;
    Raw r;
    r.a = load_u32x4_unaligned(p);
    r.b = load_u32x4_unaligned(p + 16);
    __builtin_memcpy(&r.c, p + 32, 4);
    return r;
  }
  static __device__ __forceinline__ uint32_t word(const Raw &r, int t) {
    switch (t) {
      case 0: return __builtin_amdgcn_alignbyte(r.a.y, r.a.x, 2);
      case 1: return __builtin_amdgcn_alignbyte(r.a.z, r.a.y, 2);
      case 2: return __builtin_amdgcn_alignbyte(r.a.w, r.a.z, 2);
      case 3: return __builtin_amdgcn_alignbyte(r.b.x, r.a.w, 2);
      case 4: return r.b.y;
      case 5: return r.b.z;
      case 6: return r.b.w;
      default: return r.c;
    }
  }
  // Staged sum per (unit, batch row, block g): as for one Q4_0 block.
  static __device__ __forceinline__ void stage_sums(float *sums, int idx, int g, float slo,
                                                    float shi) {
    sums[2 * idx + g] = -(1032.0f * slo + 72.0f * shi);
  }
  template <int B, int R>
  static __device__ __forceinline__ void compute(const Raw (&raw)[R], const u32x4 *xs, int xstride,
                                                 const float *sums, int u, int nu, bool valid,
                                                 const UnpackMasks &k, float (&acc)[R][B]) {
    compute_with<B, R>(
        raw, [&](int b, int t) { return xs[(b * kWords + t) * xstride + u]; },
        [&](int b, int h) { return sums[2 * (b * nu + u) + h]; }, u, valid, k, acc);
  }
  // The same with the unit's staged words and sums taken from xword(b, t)
  // and sum(b, h) (h: block of the unit), wherever the caller keeps them.
  template <int B, int R, class XW, class SW>
  static __device__ __forceinline__ void compute_with(const Raw (&raw)[R], XW xword, SW sum,
                                                      int /*u*/, bool valid, const UnpackMasks &k,
                                                      float (&acc)[R][B]) {
    float s[R][B][2];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float c0 = sum(b, 0), c1 = sum(b, 1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s[r][b][0] = c0;
        s[r][b][1] = c1;
      }
    }
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      u32x4 X[B];
#pragma unroll
      for (int b = 0; b < B; ++b) X[b] = xword(b, t);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Nibbles n = unpack_word(word(raw[r], t), k);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float a = s[r][b][t >> 2];
          a = dot2(n.p0, as_half2(X[b].x), a);
          a = dot2(n.p1, as_half2(X[b].y), a);
          a = dot2(n.p2, as_half2(X[b].z), a);
          a = dot2(n.p3, as_half2(X[b].w), a);
          s[r][b][t >> 2] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d0 = valid ? f16_bits_to_f32(raw[r].a.x) : 0.0f;
      const float d1 = valid ? f16_bits_to_f32(raw[r].b.x >> 16) : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b)
        acc[r][b] = __builtin_fmaf(d1, s[r][b][1], __builtin_fmaf(d0, s[r][b][0], acc[r][b]));
    }
  }
};

// ---- super-chunk readers of the matrix-core kernels ---------------------------
// Both formats pack 256 weights of a row into 144 bytes (a super-chunk): one
// Q4_K super-block or eight Q4_0 blocks. A lane in group q = l / 16 reads its
// units of a super-chunk staged in LDS (16-byte pieces).
// Q4_K: unit = sub-block pair (64 weights); 4 units per super-chunk, one per
// lane group.
struct CoalQ4_K {
  using F = FmtQ4_K;
  static constexpr int kUnitsPerSC = 4;
  static constexpr int kLaneUnits = 1;
  // Unit j of lane group q in the super-chunk at `sc` (16-byte pieces).
  static __device__ __forceinline__ F::Raw read(const u32x4 *sc, int q, int /*j*/) {
    F::Raw r;
    r.h = sc[0];
    r.q0 = sc[1 + 2 * q];
    r.q1 = sc[2 + 2 * q];
    return r;
  }
};

// Q4_0: unit = one block (32 weights, 18 bytes at byte 18 * b of the
// super-chunk); 8 units per super-chunk, blocks 2q and 2q + 1 for lane group
// q. Their 36 bytes start 4-byte aligned; the even block's codes start 2
// bytes into a dword and are realigned with v_alignbyte_b32.
struct CoalQ4_0 {
  using F = FmtQ4_0;
  static constexpr int kUnitsPerSC = 8;
  static constexpr int kLaneUnits = 2;
  static __device__ __forceinline__ F::Raw read(const u32x4 *sc, int q, int j) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(sc) + 9 * q;
    F::Raw r;
    if (j == 0) {
      const uint32_t d0 = w[0], d1 = w[1], d2 = w[2], d3 = w[3], d4 = w[4];
      r.d = d0 & 0xFFFFu;
      r.q = u32x4{__builtin_amdgcn_alignbyte(d1, d0, 2), __builtin_amdgcn_alignbyte(d2, d1, 2),
                  __builtin_amdgcn_alignbyte(d3, d2, 2), __builtin_amdgcn_alignbyte(d4, d3, 2)};
    } else {
      r.d = w[4] >> 16;
      r.q = u32x4{w[5], w[6], w[7], w[8]};
    }
    return r;
  }
};

// ---- activation staging ------------------------------------------------------
// Word (b, u, t) holds the 8 activations of word t of unit u for batch row b,
// in unpack order, each rounded to fp16 (no scaling: both nibble halves
// unpack to exact small integers plus a bias).
struct XWord {
  float4_t lo, hi;
};
template <class F>
__device__ __forceinline__ XWord load_xword(const float *__restrict__ x, int64_t ldx, int b, int u,
                                            int t) {
  const float *base = x + b * ldx + (int64_t)u * F::kUnitWeights;
  return XWord{*reinterpret_cast<const float4_t *>(base + F::x_lo(t)),
               *reinterpret_cast<const float4_t *>(base + F::x_hi(t))};
}
// Formats may declare kAcrossPairs = true: their weight words unpack to the
// pairs (w0,w4), (w1,w5), (w2,w6), (w3,w7) of eight consecutive weights, and
// the activations are paired the same way (see pack_xword_for). Formats may
// also declare kAux = true: their units carry per-group values from
// separate arrays (GemvAux), loaded by F::load_aux.
template <class F, class = void>
struct across_pairs : std::false_type {};
template <class F>
struct across_pairs<F, std::void_t<decltype(F::kAcrossPairs)>>
    : std::integral_constant<bool, F::kAcrossPairs> {};
template <class F, class = void>
struct has_aux : std::false_type {};
template <class F>
struct has_aux<F, std::void_t<decltype(F::kAux)>> : std::integral_constant<bool, F::kAux> {};

// Separate per-group arrays of a weight format (the int4 layout's fp32
// scales and zero points): group g of row n at a[n * groups_per_row + g].
struct GemvAux {
  const float *a;
  const float *b;
  int64_t groups_per_row;
};

__device__ __forceinline__ u32x4 pack_xword(const XWord &w) {
  const float4_t hi = w.hi;
  u32x4 word;
  word.x = pack_half2(w.lo.x, w.lo.z);
  word.y = pack_half2(hi.x, hi.z);
  word.z = pack_half2(w.lo.y, w.lo.w);
  word.w = pack_half2(hi.y, hi.w);
  return word;
}

// The activation word of a format: pack_xword's pairing, or for formats with
// kAcrossPairs (lo = x0..x3, hi = x4..x7) the pairs (x0,x4), (x1,x5),
// (x2,x6), (x3,x7). Either way word_sums' "lo" halves (x and z) go with the
// words' low-nibble weights and its "hi" halves (y and w) with the high ones.
template <class F>
__device__ __forceinline__ u32x4 pack_xword_for(const XWord &w) {
  if constexpr (across_pairs<F>::value) {
    u32x4 word;
    word.x = pack_half2(w.lo.x, w.hi.x);
    word.y = pack_half2(w.lo.y, w.hi.y);
    word.z = pack_half2(w.lo.z, w.hi.z);
    word.w = pack_half2(w.lo.w, w.hi.w);
    return word;
  } else {
    return pack_xword(w);
  }
}

// Load unit `unit` of a row slice: the format's own load, or for formats with
// separate per-group arrays its load_aux (row index and the slice's first
// unit locate the groups).
template <class F>
__device__ __forceinline__ typename F::Raw load_unit(const uint8_t *rowp, uint32_t unit, int64_t row,
                                                     int u0, const GemvAux &aux) {
  if constexpr (has_aux<F>::value)
    return F::load_aux(rowp, unit, row, u0, aux);
  else
    return F::load(rowp, unit);
}

// Staged words are grouped by word index t: word t of every (row, unit) pair
// lies in a block of `stride` slots. LDS has 32 banks (8 slots of 16 bytes),
// and the stride is padded to 8/T modulo 8 slots (T words per unit), so that
// the eight lanes that stage the words of one or two (row, unit) pairs write
// to distinct banks.
template <class F>
__host__ __device__ __forceinline__ int staged_stride(int n) {
  return ((n + 7) & ~7) + 8 / F::kWords;
}

// Stage the words of batch rows 0..nb-1 and units 0..nu-1 into xs, word
// (b, u, t) at slot(b, u, t). Threads take the words in (t, b, u) order, t
// fastest, so T neighbouring lanes read the contiguous activations of one
// (row, unit) pair and the global loads are coalesced. Each thread keeps
// kBatch words' loads in flight (clamped indices, so the loads are
// unconditional and the compiler waits once per batch, not once per word).
template <class F, int kThreads, int kBatch, class Slot>
__device__ __forceinline__ void stage_words(u32x4 *xs, int nb, int nu, const float *__restrict__ x,
                                            int64_t ldx, Slot slot) {
  constexpr int T = F::kWords;
  const int total = nb * nu * T;
  for (int base = threadIdx.x; base < total; base += kBatch * kThreads) {
    XWord w[kBatch];
    int dst[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * kThreads;
      const int ic = i < total ? i : total - 1;
      const int t = ic % T, r = ic / T;
      const int b = r % nb, u = r / nb;
      w[k] = load_xword<F>(x, ldx, b, u, t);
      dst[k] = i < total ? slot(b, u, t) : -1;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (dst[k] >= 0) xs[dst[k]] = pack_xword_for<F>(w[k]);
  }
}

// Sum of the lo (x, z halves) and hi (y, w halves) values of a staged word.
__device__ __forceinline__ void word_sums(const u32x4 &w, float &slo, float &shi) {
  half2_t a = as_half2(w.x), b = as_half2(w.y), c = as_half2(w.z), d = as_half2(w.w);
  slo += ((float)a.x + (float)a.y) + ((float)c.x + (float)c.y);
  shi += ((float)b.x + (float)b.y) + ((float)d.x + (float)d.y);
}

}  // namespace
}  // namespace lqmm

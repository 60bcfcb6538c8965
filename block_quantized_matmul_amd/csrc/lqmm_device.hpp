// Device-side helpers shared by the lqmm kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lqmm {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp16 bits (low 16 bits of `bits`) -> fp32, subnormals kept.
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)bits);
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Two fp32 values -> packed fp16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  half2_t h = {(half_t)a, (half_t)b};
  return as_u32(h);
}

// fp32 += a.x*b.x + a.y*b.y with fp16 inputs (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Unaligned-safe loads (the hardware runs in unaligned access mode; the
// compiler emits one global_load for each).
__device__ __forceinline__ u32x4 load_u32x4_unaligned(const uint8_t *p) {
  u32x4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}
__device__ __forceinline__ uint32_t load_u16(const uint8_t *p) {
  uint16_t v;
  __builtin_memcpy(&v, p, 2);
  return v;
}

// ---- buffer loads -----------------------------------------------------------
// A raw buffer resource covers [base, base + nbytes); a load whose offset
// (the VGPR offset plus the immediate; the SGPR offset is not checked) lies
// past nbytes returns zeros without touching memory. Word 3 selects 32-bit
// untyped access on gfx9-family GPUs.
// base and nbytes must be the same in every lane; they are read from the
// first active lane, so that the resource lives in scalar registers (a
// resource the compiler cannot prove uniform makes it loop over lanes).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(hi << 32 | lo), 0,
                                           __builtin_amdgcn_readfirstlane((int)nbytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// ---- cross-lane sums with DPP -------------------------------------------
// dpp<CTRL, ROW_MASK>(v): v read from the lane selected by CTRL; rows that
// ROW_MASK disables read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// Sum of v over aligned groups of `n` lanes (n a power of two, 1..64).
// For n <= 16 every lane of the group receives the sum; for n == 32 lanes
// 16..31 of each half-wave hold it; for n == 64 lanes 48..63 hold it. In all
// cases lane (group_start + n - 1) holds the group sum.
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n > 1) v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
  if (n > 2) v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
  if (n > 4) v += dpp<0x141>(v);        // row_half_mirror
  if (n > 8) v += dpp<0x140>(v);        // row_mirror
  if (n > 16) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (n > 32) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

}  // namespace lqmm

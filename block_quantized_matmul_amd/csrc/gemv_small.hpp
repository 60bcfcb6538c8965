// Latency-bound GEMV for small problems: y[b][n] = sum_k W[n][k] * x[b][k]
// for one or two activation rows (up to four when forced for tests), when the whole weight matrix is a few MB
// (a 4096 x 4096 Q4_0 layer is 9.4 MB: 1.2 us at the HBM peak, less than
// two round trips to memory).
//
// The decode mat-vec of "Resumo Tecnico: Llamas na Web", section "Design de
// Shader Consciente de Quantizacao" (blocks dequantized in registers), with
// the block-format traits and dot2 arithmetic of the other GEMV kernels. The
// difference is the schedule, built so the kernel waits on memory once:
// * every lane requests all of its weight units (one to four, all of its
//   rows' share) before anything else, then its share of the activation
//   staging: one round trip to memory for the whole workgroup;
// * one workgroup per (row block, K slice); a workgroup of NW waves covers
//   NW * 64 / LPR rows (LPR lanes per row). The planner takes the widest
//   workgroups that still leave a quarter of the CUs one: each workgroup
//   stages its x slice once, so wider ones move less from L2, and latency,
//   not the CUs' load bandwidth, bounds these problems (4096 x 4096: 256
//   sixteen-wave workgroups; 1024 x 1024: 64 four-wave ones);
// * split-K across workgroups: with S > 1 slices, each workgroup stages only
//   its slice of x and writes its partial sums to a caller-provided workspace;
//   the last workgroup of a row block to arrive (an agent-scope arrival
//   counter per row block) adds the S partials in slice order 0..S-1, so the
//   result does not depend on arrival order, writes y, and zeroes the
//   partials it read and the counter, so that the workspace is all zero
//   again when the call completes. All workspace traffic is agent-scope
//   atomic loads and stores (coherent across XCDs without fences).
#pragma once

#include "gemv_common.hpp"
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

// Dynamic LDS limit: the whole LDS but room for the kernel's static word.
constexpr int kMaxSmallLds = kMaxLds - 1024;

// B: activation rows the instance computes; nb <= B of them are real (the
// others read stale LDS and store nothing).
template <class F, int B, int U, int NW, int XB>
__global__ void __launch_bounds__(NW * kWave)
gemv_small_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int nu, int nus, int S,
                  const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                  int64_t N, int nb, int lpr_log2, float *__restrict__ part, int *__restrict__ cnt,
                  GemvAux aux) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int last_arrival;
  constexpr int T = F::kWords;
  constexpr int kThreads = NW * kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int s = (int)(blockIdx.x % (unsigned)S);   // K slice
  const int rb = (int)(blockIdx.x / (unsigned)S);  // row block
  const int lpr = 1 << lpr_log2;
  const int slot = lane >> lpr_log2, p = lane & (lpr - 1);
  const int rows_per_wave = kWave >> lpr_log2;
  const int rows_per_wg = NW * rows_per_wave;
  const int64_t row = (int64_t)rb * rows_per_wg + wave * rows_per_wave + slot;
  const int u0 = s * nus;                           // first unit of the slice
  const int nuss = nu - u0 < nus ? nu - u0 : nus;   // units in this slice (>= 1)

  // 1. All weight loads of this lane: unit j * LPR + p of the slice, j < U
  //    (clamped addresses, so the loads are unconditional; clamped units and
  //    rows past N are computed but contribute or store nothing).
  typename F::Raw raw[U];
  {
    const int64_t rc = row < N ? row : N - 1;
    const uint8_t *rowp = W + rc * row_bytes + F::unit_offset(u0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = j * lpr + p;
      raw[j] = load_unit<F>(rowp, (uint32_t)(u < nuss ? u : nuss - 1), rc, u0, aux);
    }
  }

  // 2. Stage the slice's activations (fp16 words in unpack order), then the
  //    per-(row, unit) sums that remove the unpack biases.
  const int NS = staged_stride<F>(nuss);
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);
  float *sums = reinterpret_cast<float *>(smem + (size_t)B * T * NS * 16);
  stage_words<F, kThreads, XB>(xs, nb, nuss, x + (int64_t)u0 * F::kUnitWeights, ldx,
                               [&](int b, int u, int t) { return (b * T + t) * NS + u; });
  __syncthreads();
  for (int i = tid; i < nb * nuss; i += kThreads) {
    const int u = i % nuss, b = i / nuss;
#pragma unroll
    for (int g = 0; g < T / F::kSumWords; ++g) {
      float slo = 0.0f, shi = 0.0f;
#pragma unroll
      for (int t = g * F::kSumWords; t < (g + 1) * F::kSumWords; ++t)
        word_sums(xs[(b * T + t) * NS + u], slo, shi);
      F::stage_sums(sums, i, g, slo, shi);
    }
  }
  __syncthreads();

  // 3. Dot products, then the sum over the LPR lanes of each row.
  const UnpackMasks kmask;
  float acc[1][B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[0][b] = 0.0f;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int u = j * lpr + p;
    const typename F::Raw one[1] = {raw[j]};
    F::template compute<B, 1>(one, xs, NS, sums, u < nuss ? u : nuss - 1, nuss, u < nuss, kmask,
                              acc);
  }
#pragma unroll
  for (int b = 0; b < B; ++b) acc[0][b] = group_sum(acc[0][b], lpr);
  const bool owner = p == lpr - 1 && row < N;

  if (S == 1) {
    if (owner) {
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (b < nb) y[b * ldy + row] = acc[0][b];
    }
    return;
  }

  // 4. Split-K: partial sums of slice s at part[(s * B + b) * N + row].
  //    Every access to the workspace is an agent-scope atomic: its stores
  //    are written through to the device's point of coherence and its loads
  //    read from there, so they are coherent across the XCDs without a
  //    device-scope fence (which on this GPU writes back and invalidates the
  //    XCD's L2: measured, a 5 us call took 117 us with one per wave). The
  //    order is kept by waits: each thread waits for its partial stores to
  //    complete before the barrier that precedes the workgroup's arrival;
  //    the last arrival reads the partials only after its arrival returned.
  if (owner) {
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (b < nb)
        __hip_atomic_store(part + ((int64_t)s * B + b) * N + row, acc[0][b], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): the stores have completed
  __syncthreads();
  if (tid == 0)
    last_arrival =
        __hip_atomic_fetch_add(cnt + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last_arrival) return;
  // The last arrival adds the S partials of each of its rows in slice order,
  // then zeroes them and the counter: every call leaves the workspace it
  // used all zero, so the next call may lay out its counters and partials
  // differently (other sizes, other slices). No other workgroup of this
  // call touches them again, and the next call is ordered after this kernel
  // by its stream.
  const int64_t r0 = (int64_t)rb * rows_per_wg;
  for (int i = tid; i < nb * rows_per_wg; i += kThreads) {
    const int b = i / rows_per_wg;
    const int64_t r = r0 + i % rows_per_wg;
    if (r < N) {
      float v = 0.0f;
      for (int s2 = 0; s2 < S; ++s2) {
        float *pp = part + ((int64_t)s2 * B + b) * N + r;
        v += __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pp, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      y[b * ldy + r] = v;
    }
  }
  if (tid == 0) __hip_atomic_store(cnt + rb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class F, int B, int U, int NW>
hipError_t launch_small(const SmallGemvPlan &pl, const uint8_t *W, const float *x, float *y,
                        float *part, int *cnt, hipStream_t stream) {
  // Activation words per thread: all of them in one batch of loads when
  // they fit (at most B * U * T / NW words per thread), so that the staging
  // waits on memory once.
  constexpr int kWords = B * U * F::kWords / NW;
  constexpr int XB = kWords <= 1 ? 1 : kWords <= 2 ? 2 : kWords <= 4 ? 4 : 8;
  auto kern = gemv_small_kernel<F, B, U, NW, XB>;
  const hipError_t e = ensure_max_lds<gemv_small_kernel<F, B, U, NW, XB>>(kMaxSmallLds);
  if (e != hipSuccess) return e;
  const GemvAux aux{pl.aux_a, pl.aux_b, pl.aux_groups};
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(NW * kWave), pl.lds_bytes, stream, W, pl.row_bytes,
                     pl.nu, pl.nus, pl.slices, x, pl.ldx, y, pl.ldy, pl.N, pl.batch, pl.lpr_log2,
                     part, cnt, aux);
  return hipGetLastError();
}

// Workgroups of 1, 2 or 4 waves for every shape; 8 and 16 waves (fewer
// workgroups, each staging x once for more rows) for one or two activation
// rows.
template <class F, int B, int U>
hipError_t launch_small_nw(const SmallGemvPlan &pl, const uint8_t *W, const float *x, float *y,
                           float *part, int *cnt, hipStream_t s) {
  switch (pl.waves) {
    case 1: return launch_small<F, B, U, 1>(pl, W, x, y, part, cnt, s);
    case 2: return launch_small<F, B, U, 2>(pl, W, x, y, part, cnt, s);
    case 4: return launch_small<F, B, U, 4>(pl, W, x, y, part, cnt, s);
    default: break;
  }
  if constexpr (B <= 2) {
    if (pl.waves == 8) return launch_small<F, B, U, 8>(pl, W, x, y, part, cnt, s);
    if (pl.waves == 16) return launch_small<F, B, U, 16>(pl, W, x, y, part, cnt, s);
  }
  return hipErrorInvalidValue;
}

template <class F, int B>
hipError_t launch_small_u(const SmallGemvPlan &pl, const uint8_t *W, const float *x, float *y,
                          float *part, int *cnt, hipStream_t s) {
  switch (pl.units_per_lane) {
    case 1: return launch_small_nw<F, B, 1>(pl, W, x, y, part, cnt, s);
    case 2: return launch_small_nw<F, B, 2>(pl, W, x, y, part, cnt, s);
    default: return hipErrorInvalidValue;
  }
}

template <class F>
hipError_t launch_small_fmt(const SmallGemvPlan &pl, const uint8_t *W, const float *x, float *y,
                            float *part, int *cnt, hipStream_t s) {
  // instances for 1, 2 and 4 activation rows; three run on the 4-row one
  switch (pl.batch) {
    case 1: return launch_small_u<F, 1>(pl, W, x, y, part, cnt, s);
    case 2: return launch_small_u<F, 2>(pl, W, x, y, part, cnt, s);
    case 3:
    case 4: return launch_small_u<F, 4>(pl, W, x, y, part, cnt, s);
    default: return hipErrorInvalidValue;
  }
}

template <class F>
size_t small_lds(int batch, int nus) {
  return (size_t)batch * F::kWords * staged_stride<F>(nus) * 16 +
         (size_t)batch * nus * F::kSums * 4;
}

}  // namespace
}  // namespace lqmm

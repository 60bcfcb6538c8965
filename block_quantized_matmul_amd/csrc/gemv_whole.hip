// Matrix-core GEMV for layers of a few tiles per CU: the workgroup's whole
// weight share is requested at once (gfx950).
//
// "Resumo Tecnico: Llamas na Web", section "Design de Shader Consciente de
// Quantizacao": the decode mat-vec dequantizes the weight blocks in
// registers. At three or more activation rows the products run on the matrix
// cores (v_mfma_f32_16x16x32_f16) with the tiles, B-operand layout and
// in-workgroup k-slices of gemv.hip's coalesced kernel. That kernel streams
// each wave's chunks through a ring two deep, so a layer of 2-3 tiles per CU
// waits for several memory round trips, and its activation loads queue
// behind the first chunks (loads return in order). Here, when the whole share
// fits the LDS:
// 1. every thread issues its loads of x (all of it; one batch of at most
//    kWholeWords words per thread);
// 2. every wave requests all of its chunks (MAXT tiles x CPS super-chunks,
//    16 rows x 144 bytes each) into its own LDS slots with buffer-to-LDS
//    loads: two of 16 bytes per lane and one of 4 bytes per lane for the
//    chunk's last 256 bytes, so a slot holds exactly the chunk;
// 3. the x words are converted to fp16 and staged in LDS (the waits cover
//    the x loads only: they were issued first);
// 4. tile by tile, each wave waits until its chunks of that tile have landed,
//    computes them, and the KS waves of the tile add their partial sums
//    through LDS (two alternating areas, one barrier per tile).
// So the whole launch waits for one memory round trip, with the later tiles'
// loads landing while the first tiles are computed. Tiles past the matrix
// and super-chunks past the row are requested from an empty buffer range
// (zeros, no memory traffic), so the number of loads per wave, and the
// load-counter waits, are the same in every wave.

#include "gemv_common.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int kWholeWaves = 8;
constexpr int kWholeThreads = kWholeWaves * kWave;
constexpr int kWholeChunk = 16 * 144;  // 16 rows x one super-chunk
constexpr int kWholeLoads = 3;         // load instructions per chunk
static_assert(kWholeChunk == 2 * kWave * 16 + kWave * 4, "two 16-byte and one 4-byte load");
constexpr size_t kWholeRed = (size_t)2 * kWholeWaves * kWave * 16;
constexpr int kWholeWords = 8;  // activation words per thread (all loaded at once)

template <class C>
size_t whole_lds_bytes(int cps, int maxt, int nu, int nb) {
  using F = typename C::F;
  return (size_t)kWholeWaves * maxt * cps * kWholeChunk + kWholeRed +
         (size_t)F::kWords * staged_stride<F>(nu * nb) * 16;
}

template <class C, int CPS, int KS, int MAXT>
__global__ void __launch_bounds__(kWholeThreads)
gemv_whole_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int nsc,
                  const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                  int64_t N, int nb) {
  using F = typename C::F;
  constexpr int NW = kWholeWaves;
  constexpr int T = F::kWords;
  constexpr int LU = C::kLaneUnits;
  constexpr int UPS = C::kUnitsPerSC;
  constexpr int kTeams = NW / KS;
  constexpr int PR = 9;            // 16-byte pieces of one row's super-chunk
  constexpr int NI = MAXT * CPS;   // chunks per wave
  static_assert((NI - 1) * kWholeLoads <= 63, "load counter range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float4_t *const red = reinterpret_cast<float4_t *>(smem + (size_t)NW * NI * kWholeChunk);
  u32x4 *const xs = reinterpret_cast<u32x4 *>(smem + (size_t)NW * NI * kWholeChunk + kWholeRed);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int team = wave / KS, slice = wave % KS;
  const int lane = tid & (kWave - 1);
  const int n = lane & 15;
  const int q = lane >> 4;
  const int ngroups = (int)((N + 15) / 16);
  const int nu = nsc * UPS;  // units per row
  const int sc0 = slice * CPS;
  const int group_stride = gridDim.x * kTeams;
  const int g0 = blockIdx.x * kTeams + team;  // this wave's first tile
  uint8_t *const slots = smem + (size_t)wave * NI * kWholeChunk;

  // 1. x words: word (b, u, t) of all nb rows and nu units, t fastest, so T
  //    neighbouring lanes read one contiguous run of a row.
  const int TS = staged_stride<F>(nu * nb);
  const int total = nb * nu * T;
  XWord xw[kWholeWords];
  int xdst[kWholeWords];
#pragma unroll
  for (int k = 0; k < kWholeWords; ++k) {
    const int i = tid + k * kWholeThreads;
    const int ic = i < total ? i : total - 1;
    const int t = ic % T, r = ic / T;
    const int b = r % nb, u = r / nb;
    xw[k] = load_xword<F>(x, ldx, b, u, t);
    xdst[k] = i < total ? t * TS + u * nb + b : -1;
  }

  // 2. every chunk of this wave: tile g0 + it * group_stride, super-chunk
  //    sc0 + c, into slot it * CPS + c
  {
    uint32_t off[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pc = k * kWave + lane;
      off[k] = (uint32_t)(pc / PR) * (uint32_t)row_bytes + (uint32_t)(pc % PR) * 16;
    }
    const int pct = 2 * kWave + (lane >> 2);
    const uint32_t off_tail =
        (uint32_t)(pct / PR) * (uint32_t)row_bytes + (uint32_t)(pct % PR) * 16 + (lane & 3) * 4;
#pragma unroll
    for (int it = 0; it < MAXT; ++it) {
      const int g = g0 + it * group_stride;
      const int gc = g < ngroups ? g : ngroups - 1;
      // 32-bit, wave-uniform (gc < ceil(N / 16), N <= 2^31): scalar compares
      const uint32_t r0 = (uint32_t)gc * 16u, left = (uint32_t)N - r0;
      const int64_t rows = left < 16u ? left : 16u;
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        const bool live = g < ngroups && sc0 + c < nsc;
        const rsrc_t rs = make_rsrc(W + (int64_t)r0 * row_bytes, live ? (uint32_t)(rows * row_bytes) : 0u);
        const int sc = sc0 + c < nsc ? sc0 + c : nsc - 1;
        uint8_t *dst = slots + (it * CPS + c) * kWholeChunk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (int)off[0], sc * 144, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + kWave * 16, 16, (int)off[1], sc * 144,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 2 * kWave * 16, 4, (int)off_tail,
                                                 sc * 144, 0, 0);
      }
    }
  }

  // 3. stage x (these writes wait for the x loads only, which were issued
  //    before the chunk requests)
#pragma unroll
  for (int k = 0; k < kWholeWords; ++k)
    if (xdst[k] >= 0) xs[xdst[k]] = pack_xword(xw[k]);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // 4. tile by tile
  const UnpackMasks kmask;
  const int xb = n < nb ? n : 0;  // rows >= nb are computed but never stored
#pragma unroll
  for (int it = 0; it < MAXT; ++it) {
    // this wave's chunks of tile it have landed (the later tiles' may not)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((MAXT - 1 - it) * CPS * kWholeLoads) : "memory");
    float4_t acc = float4_t{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      if (sc0 + c >= nsc) continue;  // the same in every lane of the wave
      const u32x4 *wbuf = reinterpret_cast<const u32x4 *>(slots + (it * CPS + c) * kWholeChunk);
      u32x4 xa[LU][T];
      typename F::Raw rw[LU];
#pragma unroll
      for (int j = 0; j < LU; ++j) {
        const int u = (sc0 + c) * UPS + q * LU + j;
        const u32x4 *xrow = xs + u * nb + xb;
#pragma unroll
        for (int t = 0; t < T; ++t) xa[j][t] = xrow[t * TS];
        rw[j] = C::read(wbuf + n * PR, q, j);
      }
#pragma unroll
      for (int j = 0; j < LU; ++j) {
        const typename F::Prep pr = F::prep(rw[j], q, true);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const half8_t a = __builtin_bit_cast(half8_t, xa[j][t]);
          const half8_t wv = __builtin_bit_cast(half8_t, F::dequant(rw[j], pr, t, kmask));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wv, acc, 0, 0, 0);
        }
      }
    }
    if (KS > 1) {
      red[((it & 1) * NW + wave) * kWave + lane] = acc;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (slice == 0) {
#pragma unroll
        for (int s2 = 1; s2 < KS; ++s2) acc += red[((it & 1) * NW + wave + s2) * kWave + lane];
      }
    }
    const int g = g0 + it * group_stride;
    if (slice == 0 && g < ngroups) {
      const int64_t row = (int64_t)g * 16 + n;
      if (row < N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int b = 4 * q + v;
          if (b < nb) y[b * ldy + row] = acc[v];
        }
      }
    }
  }
  // no buffer-to-LDS load may be left in flight when the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class C, int CPS, int KS, int MAXT>
hipError_t launch_whole(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                        hipStream_t s) {
  const hipError_t e = ensure_max_lds<gemv_whole_kernel<C, CPS, KS, MAXT>>(kMaxLds);
  if (e != hipSuccess) return e;
  const int nsc = (int)(pl.row_bytes / 144);
  const size_t lds = whole_lds_bytes<C>(CPS, MAXT, nsc * C::kUnitsPerSC, pl.batch);
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_whole_kernel<C, CPS, KS, MAXT>), dim3(pl.grid), dim3(kWholeThreads), lds,
                     s, W, pl.row_bytes, nsc, x, pl.ldx, y, pl.ldy, pl.N, pl.batch);
  return hipGetLastError();
}

template <class C, int CPS, int KS>
hipError_t launch_whole_t(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                          hipStream_t s) {
  switch (pl.depth) {
    case 1: return launch_whole<C, CPS, KS, 1>(pl, W, x, y, s);
    case 2: return launch_whole<C, CPS, KS, 2>(pl, W, x, y, s);
    case 3: return launch_whole<C, CPS, KS, 3>(pl, W, x, y, s);
    default: return hipErrorInvalidValue;
  }
}

template <class C>
hipError_t launch_whole_fmt(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                            hipStream_t s) {
  if (pl.cps == 1 && pl.ksplit == 8) return launch_whole_t<C, 1, 8>(pl, W, x, y, s);
  if (pl.cps == 2 && pl.ksplit == 8) return launch_whole_t<C, 2, 8>(pl, W, x, y, s);
  if (pl.cps == 2 && pl.ksplit == 4) return launch_whole_t<C, 2, 4>(pl, W, x, y, s);
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemv_whole_lds_bytes(GemvFormat f, int cps, int maxt, int nu, int nb) {
  return f == GemvFormat::Q4_K ? whole_lds_bytes<CoalQ4_K>(cps, maxt, nu, nb)
                               : whole_lds_bytes<CoalQ4_0>(cps, maxt, nu, nb);
}

int gemv_whole_max_words() { return kWholeWords * kWholeThreads; }
int gemv_whole_waves() { return kWholeWaves; }

hipError_t gemv_whole_launch(GemvFormat f, const GemvPlan &pl, const uint8_t *W, const float *x,
                             float *y, hipStream_t stream) {
  if (pl.row_bytes % 144 != 0 || pl.row_bytes <= 0 || pl.batch < 1 || pl.batch > 16 ||
      pl.grid < 1 || pl.ksplit * pl.cps * 144 < pl.row_bytes)
    return hipErrorInvalidValue;
  if (f == GemvFormat::Q4_K) return launch_whole_fmt<CoalQ4_K>(pl, W, x, y, stream);
  if (f == GemvFormat::Q4_0) return launch_whole_fmt<CoalQ4_0>(pl, W, x, y, stream);
  return hipErrorInvalidValue;
}

}  // namespace lqmm

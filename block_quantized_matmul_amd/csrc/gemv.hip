// Dequantize-in-register GEMV for llama.cpp Q4_0 and Q4_K weight blocks on
// gfx950: y[b][n] = sum_k W[n][k] * x[b][k] for a few activation rows b.
//
// This is the decode mat-vec of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao": weight blocks are never
// expanded in memory; each lane unpacks its block's nibbles in registers and
// multiplies them with the activations. The quantization format is a
// compile-time trait (the page's "dequantization chosen at compile time").
//
// Common structure (both modes):
// * A "unit" is the run of weights one lane takes from one weight row: one
//   Q4_0 block (32 weights, 18 bytes) or a quarter of a Q4_K super-block (64
//   weights: the 16-byte header plus 32 bytes of nibbles).
// * A workgroup (512 threads) stages the activations in LDS as fp16, then its
//   waves stream weight rows with a grid stride. Each wave walks "groups" of
//   rows in "chunks" of U units per lane through two register buffers: the
//   next chunk loads while the current one is computed. The first chunk is
//   requested before the activations are staged.
// * Nibbles become fp16 with the exponent trick, one v_and_or_b32 per pair of
//   weights: a low nibble (bits 0-3 of a 16-bit half) OR-ed into the mantissa
//   of 1024.0 (0x6400, mantissa step 1) gives exactly 1024 + q; a high nibble
//   (bits 4-7, mantissa value 16q) OR-ed into the mantissa of 64.0 (0x5400,
//   mantissa step 1/16) gives exactly 64 + q. The activations therefore stay
//   unscaled on both halves.
//
// VALU mode (batch 1..8, used for 1..2): consecutive lanes take consecutive
// units of the same row(s) (LPR lanes per row), the activation pairs are
// multiplied with v_dot2_f32_f16 into fp32, the 1024 biases are removed with
// staged activation sums, block scales are applied in fp32 once per unit and
// the LPR lane partials are summed with DPP.
//
// MFMA mode (batch up to 16 per launch, used from 3 up): a wave covers 16
// weight rows at once. Lane l takes row l % 16 and unit offset l / 16, which
// is exactly the B-operand layout of v_mfma_f32_16x16x32_f16 (column = weight
// row, 8 k values per lane); the nibbles of each 32-bit word are dequantized
// to fp16 weights in registers (one rounding per weight) and fed to the MFMA
// with the staged activations (row = batch row) as the A operand. The matrix
// core does the k reduction, so the per-weight VALU cost no longer grows with
// the batch.
#include <type_traits>

#include "gemv_common.hpp"
#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int kGemvThreads = 512;
constexpr int kWavesPerWg = kGemvThreads / kWave;
constexpr int kCoalrRing = 6;  // chunk slots per wave of gemv_coalr_kernel

// ---- VALU-mode kernel -----------------------------------------------------
// x rows: x + b*ldx, covering units [unit0, unit0 + nu) of every weight row.
// accumulate != 0: y += result (used when K is split over several launches).
// A group is the slots*R rows one wave covers at once (slots = 64/LPR row
// slots, R rows per lane).
// FULL: all 64 lanes share each row (lpr_log2 == 6), so the rows a wave reads
// are wave-uniform and their addresses live in scalar registers.
template <class F, int B, int R, int U, bool FULL>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int64_t unit0, int nu,
            const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
            int64_t N, int lpr_log2_arg, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int T = F::kWords;
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);  // slot (b*T + t)*NS + u
  const int NS = staged_stride<F>(nu);
  float *sums = reinterpret_cast<float *>(smem + (size_t)B * T * NS * 16);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int lpr_log2 = FULL ? 6 : lpr_log2_arg;
  const int lpr = 1 << lpr_log2;
  const int slot = FULL ? 0 : lane >> lpr_log2;
  const int p = lane & (lpr - 1);
  const int slots = kWave >> lpr_log2;
  const int64_t rows_per_group = (int64_t)slots * R;
  const int64_t ngroups = (N + rows_per_group - 1) / rows_per_group;
  const int units_per_chunk = lpr * U;
  const int nchunks = (nu + units_per_chunk - 1) / units_per_chunk;
  const int64_t wave_stride = (int64_t)gridDim.x * kWavesPerWg;

  // Loads are issued unconditionally from clamped (always valid) addresses:
  // a conditional load would make the compiler wait for every outstanding
  // load before using the current chunk, which serializes the prefetch.
  // Rows past N are computed but never stored; units past nu are skipped.
  typename F::Raw buf0[R][U], buf1[R][U];
  auto load = [&](typename F::Raw (&dst)[R][U], int64_t g, int c) {
    const int64_t row0 = g * rows_per_group + (int64_t)slot * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r < N ? row0 + r : N - 1;
      const uint8_t *rowp = W + row * row_bytes + F::unit_offset(unit0);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        int u = c * units_per_chunk + j * lpr + p;
        u = u < nu ? u : nu - 1;
        dst[r][j] = F::load(rowp, (uint32_t)u);
      }
    }
  };

  int64_t g = (int64_t)blockIdx.x * kWavesPerWg + __builtin_amdgcn_readfirstlane(tid / kWave);
  int c = 0;
  load(buf0, g < ngroups ? g : ngroups - 1, 0);

  // Stage the words, then the per-(b, u) sums.
  // (one or two words per thread at batch 1 and 2: no batching)
  stage_words<F, kGemvThreads, 1>(xs, B, nu, x, ldx,
                                  [&](int b, int u, int t) { return (b * T + t) * NS + u; });
  __syncthreads();
  for (int i = tid; i < B * nu; i += kGemvThreads) {
    const int u = i % nu, b = i / nu;
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

  const UnpackMasks kmask;
  float acc[R][B];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

  // Compute chunk (g, c) from src while the next chunk loads into dst.
  auto stage = [&](typename F::Raw (&src)[R][U], typename F::Raw (&dst)[R][U]) -> bool {
    int64_t g2 = g;
    int c2 = c + 1;
    if (c2 == nchunks) {
      c2 = 0;
      g2 += wave_stride;
    }
    // past the last group: reload the current chunk (an L2 hit) so the
    // load stays unconditional
    load(dst, g2 < ngroups ? g2 : g, g2 < ngroups ? c2 : c);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = c * units_per_chunk + j * lpr + p;
      typename F::Raw one[R];
#pragma unroll
      for (int r = 0; r < R; ++r) one[r] = src[r][j];
      F::template compute<B, R>(one, xs, NS, sums, u < nu ? u : nu - 1, nu, u < nu, kmask, acc);
    }
    if (c == nchunks - 1) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = group_sum(acc[r][b], lpr);
      if (p == lpr - 1) {
        const int64_t row0 = g * rows_per_group + (int64_t)slot * R;
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
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    }
    g = g2;
    c = c2;
    return g < ngroups;
  };

  if (g < ngroups) {
    while (stage(buf0, buf1) && stage(buf1, buf0)) {
    }
  }
}

// ---- MFMA-mode kernel -----------------------------------------------------
// nb (1..16) batch rows. A "tile" is 16 weight rows. The KS waves of a
// k-split team share R tiles: wave slice s takes units [s*nus, (s+1)*nus) of
// every row (nus = units per slice), and the team's partial sums meet in LDS.
// Within a slice, lane l takes weight row l % 16 of each tile and, in chunk c,
// the U consecutive units c*4U + (l/16)*U + j (j < U), so every row is read in
// runs of 4U units. The lane's activations (A operand) are those of batch row
// l % 16 for the same unit; lanes with l % 16 >= nb feed zeros. The result
// D[4*(l/16) + v][l % 16] is batch row 4*(l/16) + v of weight row l % 16.
// The 8/KS teams of a workgroup walk tile groups with a grid stride; every
// wave of the workgroup runs the same number of iterations, so the team
// reduction can use workgroup barriers.
template <class F, int R, int U, int KS, int NW>
__global__ void __launch_bounds__(NW * kWave)
gemv_mfma_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int64_t unit0, int nu,
                 const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                 int64_t N, int nb, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int T = F::kWords;
  constexpr int kThreads = NW * kWave;
  constexpr int kTeams = NW / KS;
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);  // slot t*TS + u*nb + b
  const int TS = staged_stride<F>(nu * nb);
  float4_t *red = reinterpret_cast<float4_t *>(smem + (size_t)T * TS * 16);

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int team = wave / KS, slice = wave % KS;
  const int lane = tid & (kWave - 1);
  const int n = lane & 15;   // weight row within a tile; batch row of the A operand
  const int q = lane >> 4;   // k group of the MFMA operands
  const int64_t rows_per_group = 16 * R;
  const int64_t ngroups = (N + rows_per_group - 1) / rows_per_group;
  const int units_per_chunk = 4 * U;
  // Units per slice, a whole number of chunks; every slice runs the same
  // number of chunks (units past the end feed zero activations).
  const int nus = (((nu + KS - 1) / KS) + units_per_chunk - 1) / units_per_chunk * units_per_chunk;
  const int ubeg = slice * nus;
  const int uend = ubeg + nus < nu ? ubeg + nus : nu;
  const int nchunks = nus / units_per_chunk;
  const int64_t group_stride = (int64_t)gridDim.x * kTeams;

  // First unit of the run lane group q loads in chunk c: the nominal start,
  // moved back so that the run ends at nu when it would run past it (never
  // below 0; shorter rows are handled by the per-unit clamp in load_units).
  auto run_start = [&](int c) -> int {
    const int u = ubeg + c * units_per_chunk + q * U;
    if (u + U <= nu) return u;
    return nu - U > 0 ? nu - U : 0;
  };

  // Unconditional loads from clamped addresses (see the VALU kernel).
  typename F::Raw buf0[R][U], buf1[R][U];
  auto load = [&](typename F::Raw (&dst)[R][U], int64_t gg, int c) {
    const int64_t gc = gg < ngroups ? gg : ngroups - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t row = gc * rows_per_group + 16 * r + n;
      row = row < N ? row : N - 1;
      const uint8_t *rowp = W + row * row_bytes + F::unit_offset(unit0);
      // The U units of a lane are consecutive: the run is moved back to end
      // at nu, and each unit is also clamped for rows shorter than a run.
      F::template load_units<U>(rowp, (uint32_t)run_start(c), (uint32_t)(nu - 1), dst[r]);
    }
  };

  // All waves of the workgroup walk the same sequence of group steps; a
  // team whose group is past the end computes on clamped data and stores
  // nothing.
  int64_t gb = (int64_t)blockIdx.x * kTeams;  // first group of this workgroup
  int c = 0;
  load(buf0, gb + team, 0);

  stage_words<F, kThreads, 4>(xs, nb, nu, x, ldx,
                              [&](int b, int u, int t) { return t * TS + u * nb + b; });
  __syncthreads();

  const UnpackMasks kmask;
  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0, 0, 0, 0};

  auto stage = [&](typename F::Raw (&src)[R][U], typename F::Raw (&dst)[R][U]) -> bool {
    int64_t gb2 = gb;
    int c2 = c + 1;
    if (c2 == nchunks) {
      c2 = 0;
      gb2 += group_stride;
    }
    load(dst, (gb2 < ngroups ? gb2 : gb) + team, gb2 < ngroups ? c2 : c);
    // The loader clamped the run to [nu - U, nu); recover which units were
    // actually loaded so the activations match, and zero the weights of
    // units outside this slice.
    const int ufirst = ubeg + c * units_per_chunk + q * U;
    const int uload = run_start(c);
    const int xb = n < nb ? n : 0;  // rows >= nb are computed but never stored
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = uload + j;
      const bool valid = u >= ufirst && u < uend;
      const int ux = u < nu ? u : nu - 1;  // the unit load_units fetched
      const u32x4 *xrow = xs + (int64_t)ux * nb + xb;
      typename F::Prep pr[R];
#pragma unroll
      for (int r = 0; r < R; ++r) pr[r] = F::prep(src[r][j], ux & 3, valid);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const half8_t a = __builtin_bit_cast(half8_t, xrow[t * TS]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const half8_t wv = __builtin_bit_cast(half8_t, F::dequant(src[r][j], pr[r], t, kmask));
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wv, acc[r], 0, 0, 0);
        }
      }
    }
    if (c == nchunks - 1) {
      // team reduction in LDS, stored by the slice-0 wave
      if (KS > 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) red[(wave * R + r) * kWave + lane] = acc[r];
        __syncthreads();
        if (slice == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s2 = 1; s2 < KS; ++s2) acc[r] += red[((wave + s2) * R + r) * kWave + lane];
        }
      }
      const int64_t g = gb + team;
      if (slice == 0 && g < ngroups) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t row = g * rows_per_group + 16 * r + n;
          if (row < N) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int b = 4 * q + v;
              if (b < nb) {
                float val = acc[r][v];
                if (accumulate) val += y[b * ldy + row];
                y[b * ldy + row] = val;
              }
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = float4_t{0, 0, 0, 0};
      if (KS > 1) __syncthreads();
    }
    gb = gb2;
    c = c2;
    return gb < ngroups;
  };

  if (gb < ngroups) {
    while (stage(buf0, buf1) && stage(buf1, buf0)) {
    }
  }
}

// ---- MFMA mode with coalesced loads (Q4_K and Q4_0) ---------------------------
// Both formats pack 256 weights of a row into 144 bytes: one Q4_K super-block
// or eight Q4_0 blocks (a "super-chunk", 16-byte aligned in every row whose
// byte length is a multiple of 16). A chunk is U super-chunks of each of the
// 16 rows of a tile. It is fetched with coalesced 16-byte buffer loads
// (piece p of the chunk goes to lane p % 64 of load p / 64, so consecutive
// lanes read consecutive bytes of a row), written to a wave-private LDS
// buffer and read back in the MFMA B-operand layout: lane l takes row l % 16
// and 64 weights of each super-chunk (lane group q = l / 16 takes Q4_K
// sub-block pair q, or Q4_0 blocks 2q and 2q + 1). The MFMA-layout loads of
// gemv_mfma_kernel touch 16 rows per instruction and keep the address unit
// stalled; these touch one to four rows.
//
// Load addresses: every lane's byte offset within the 16-row tile is fixed
// (row * row_bytes + piece * 16, in a VGPR); the tile base goes in the
// buffer resource and the chunk offset in the scalar offset. The resource
// ends at the last row of the matrix, so rows past N read zeros; unused
// piece slots get an offset past the resource and read zeros too.
// D chunks are in flight per wave through a ring of D register buffers.

template <class C, int U, int KS, int D>
__global__ void __launch_bounds__(kGemvThreads)
gemv_coal_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int64_t unit0, int nu,
                 const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                 int64_t N, int nb, int accumulate) {
  using F = typename C::F;
  constexpr int NW = kWavesPerWg;
  constexpr int T = F::kWords;
  constexpr int kTeams = NW / KS;
  constexpr int PR = 9 * U;           // 16-byte pieces per row per chunk
  constexpr int NP = 16 * PR;         // pieces per chunk
  constexpr int NI = (NP + 63) / 64;  // loads per lane per chunk
  constexpr int UPC = U * C::kUnitsPerSC;  // units per chunk
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);  // slot t*TS + u*nb + b
  const int TS = staged_stride<F>(nu * nb);
  // Per-wave weight staging areas; the k-split reduction reuses them.
  u32x4 *wbase = reinterpret_cast<u32x4 *>(smem + (size_t)T * TS * 16);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int team = wave / KS, slice = wave % KS;
  const int lane = tid & (kWave - 1);
  const int n = lane & 15;
  const int q = lane >> 4;
  u32x4 *wbuf = wbase + wave * NI * kWave;
  auto red = [&](int w) { return reinterpret_cast<float4_t *>(wbase + w * NI * kWave) + lane; };
  const int ngroups = (int)((N + 15) / 16);
  // Units per slice, a whole number of chunks; every slice runs the same
  // number of chunks (units past the end of its range are zeroed).
  const int nus = (((nu + KS - 1) / KS) + UPC - 1) / UPC * UPC;
  const int ubeg = slice * nus;
  const int uend = ubeg + nus < nu ? ubeg + nus : nu;
  const int nchunks = nus / UPC;
  const int group_stride = gridDim.x * kTeams;
  const uint32_t unit0_bytes = (uint32_t)(unit0 / C::kUnitsPerSC * 144);

  // First unit of chunk c, moved back so that the chunk ends inside the row
  // (nu is a multiple of kUnitsPerSC, so the start stays on a super-chunk).
  auto chunk_start = [&](int c) -> int {
    const int u = ubeg + c * UPC;
    return u + UPC <= nu ? u : nu - UPC;
  };

  uint32_t off[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int pc = k * kWave + lane;
    off[k] = pc < NP ? (uint32_t)(pc / PR) * (uint32_t)row_bytes + (uint32_t)(pc % PR) * 16
                     : 0x80000000u;
  }

  // Chunk c of tile g (clamped to the last tile) into dst.
  auto load = [&](u32x4 (&dst)[NI], int g, int c) {
    const int gc = g < ngroups ? g : ngroups - 1;
    // 32-bit, wave-uniform (gc < ceil(N / 16), N <= 2^31): scalar compares
    const uint32_t r0 = (uint32_t)gc * 16u, left = (uint32_t)N - r0;
    const int64_t rows = left < 16u ? left : 16u;
    const rsrc_t rs = make_rsrc(W + (int64_t)r0 * row_bytes + unit0_bytes,
                                (uint32_t)(rows * row_bytes - unit0_bytes));
    const int soff = chunk_start(c) / C::kUnitsPerSC * 144;
#pragma unroll
    for (int k = 0; k < NI; ++k)
      dst[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[k], soff, 0));
  };

  // Items of this wave: chunk c of tile g, c running fastest; g starts at
  // blockIdx.x * kTeams + team and steps by group_stride. Every wave of the
  // workgroup runs the same number of items (the workgroup loops while its
  // first team's tile is in range), so the barriers of the reduction match.
  u32x4 bufs[D][NI];
  int pg = blockIdx.x * kTeams, pc = 0;  // next item to prefetch (tile of team 0)
  auto advance = [&](int &g, int &c) {
    if (++c == nchunks) {
      c = 0;
      g += group_stride;
    }
  };
#pragma unroll
  for (int k = 0; k < D; ++k) {
    load(bufs[k], pg + team, pc);
    advance(pg, pc);
  }

  stage_words<F, kGemvThreads, 4>(xs, nb, nu, x, ldx,
                                  [&](int b, int u, int t) { return t * TS + u * nb + b; });
  __syncthreads();

  const UnpackMasks kmask;
  float4_t acc = float4_t{0, 0, 0, 0};
  const int xb = n < nb ? n : 0;  // rows >= nb are computed but never stored
  int cg = blockIdx.x * kTeams, cc = 0;  // item being consumed

  // Consume buffer `src` (item (cg, cc)), then refill it with the item D
  // places later.
  auto stage = [&](u32x4 (&src)[NI]) {
    // Wave-private transpose through LDS; one wave's LDS operations complete
    // in order, so the reads below see these writes.
#pragma unroll
    for (int k = 0; k < NI; ++k) wbuf[k * kWave + lane] = src[k];
    load(src, pg + team, pc);
    advance(pg, pc);
    const int nominal = ubeg + cc * UPC;
    const int ustart = chunk_start(cc);
    // All LDS reads of the chunk (activations, then the lane's weight units)
    // are issued together, so the wave waits for LDS once per chunk rather
    // than before every MFMA.
    constexpr int LU = U * C::kLaneUnits;
    u32x4 xa[LU][T];
    typename F::Raw rw[LU];
#pragma unroll
    for (int s = 0; s < U; ++s)
#pragma unroll
      for (int j = 0; j < C::kLaneUnits; ++j) {
        const int u = ustart + s * C::kUnitsPerSC + q * C::kLaneUnits + j;
        const u32x4 *xrow = xs + u * nb + xb;
#pragma unroll
        for (int t = 0; t < T; ++t) xa[s * C::kLaneUnits + j][t] = xrow[t * TS];
      }
#pragma unroll
    for (int s = 0; s < U; ++s)
#pragma unroll
      for (int j = 0; j < C::kLaneUnits; ++j)
        rw[s * C::kLaneUnits + j] = C::read(wbuf + n * PR + 9 * s, q, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < U; ++s) {
#pragma unroll
      for (int j = 0; j < C::kLaneUnits; ++j) {
        const int ul = s * C::kUnitsPerSC + q * C::kLaneUnits + j;  // unit within the chunk
        const int u = ustart + ul;
        const bool valid = u >= nominal && u < uend;
        const typename F::Raw &r = rw[s * C::kLaneUnits + j];
        const typename F::Prep pr = F::prep(r, q, valid);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const half8_t a = __builtin_bit_cast(half8_t, xa[s * C::kLaneUnits + j][t]);
          const half8_t wv = __builtin_bit_cast(half8_t, F::dequant(r, pr, t, kmask));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wv, acc, 0, 0, 0);
        }
      }
    }
    if (cc == nchunks - 1) {
      // The wave's own staging area is free once its chunk is computed (one
      // wave's LDS operations complete in order); the closing barrier keeps
      // the next chunk's staging writes behind the slice-0 wave's reads.
      if (KS > 1) {
        *red(wave) = acc;
        __syncthreads();
        if (slice == 0) {
#pragma unroll
          for (int s2 = 1; s2 < KS; ++s2) acc += *red(wave + s2);
        }
      }
      const int g = cg + team;
      if (slice == 0 && g < ngroups) {
        const int64_t row = (int64_t)g * 16 + n;
        if (row < N) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int b = 4 * q + v;
            if (b < nb) {
              float val = acc[v];
              if (accumulate) val += y[b * ldy + row];
              y[b * ldy + row] = val;
            }
          }
        }
      }
      acc = float4_t{0, 0, 0, 0};
      if (KS > 1) __syncthreads();
    }
    advance(cg, cc);
  };

  // Whole rounds of D stages, then the remainder: a loop without an early
  // exit between the stages lets the compiler's load-counter waits keep the
  // other buffers' loads in flight (with an exit between them it drained
  // every load once per round).
  const int gfirst = blockIdx.x * kTeams;
  const int n_items = (ngroups - gfirst + group_stride - 1) / group_stride * nchunks;
  int it = 0;
  for (; it + D <= n_items; it += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) stage(bufs[k]);
  }
#pragma unroll
  for (int k = 0; k < D - 1; ++k)
    if (it + k < n_items) stage(bufs[k]);
}

// ---- MFMA mode, coalesced loads, activations in registers ---------------------
// The tiles, k-slices, chunk loads and B-operand layout of gemv_coal_kernel
// (one super-chunk per chunk), for launches whose k-slice spans at most CPS
// <= 4 super-chunks. A wave's slice is the same for every tile it visits, so
// it loads the fp16 A operands of its slice into registers once (32 VGPRs per
// super-chunk; lanes whose batch row n >= nb hold zeros). LDS then holds only
// a ring of DR chunk slots per wave, filled by buffer-to-LDS loads up to DR
// chunks ahead of the one being computed (no register round trip, no LDS
// write instructions), and a k-split reduction area that alternates between
// tiles, so that each tile needs one barrier.
//
// Order per chunk i: chunk i's slot was read into registers during chunk
// i-1's arithmetic (so the LDS latency is hidden). The wave waits for those
// reads, refills the slot with chunk i+DR, waits until chunk i+1 has landed,
// issues the reads of chunk i+1, and then computes chunk i.
// Waits: the compiler does not see the LDS data the buffer-to-LDS loads
// write, so the wave waits for them explicitly. After the refill, the loads
// of chunks i+2 .. i+DR (NI each) may stay in flight; loads return in order.
// Stores to y issued after them are not counted, which can only make the
// wait longer, never too short. A slot is refilled only after the wave's
// reads of it have completed. Chunks past the end of the wave's work are
// requested from an empty buffer range: they return zeros, touch no memory,
// and keep the count of loads in flight constant.
template <class C, int CPS, int KS, int DR>
__global__ void __launch_bounds__(kGemvThreads)
gemv_coalr_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int64_t unit0, int nu,
                  const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                  int64_t N, int nb, int accumulate) {
  using F = typename C::F;
  constexpr int NW = kWavesPerWg;
  constexpr int T = F::kWords;
  constexpr int LU = C::kLaneUnits;
  constexpr int kTeams = NW / KS;
  constexpr int PR = 9;                // 16-byte pieces of one row's super-chunk
  constexpr int NP = 16 * PR;          // pieces per chunk
  constexpr int NI = (NP + 63) / 64;   // loads per lane per chunk
  constexpr int kSlot = NI * kWave * 16;
  static_assert((DR - 1) * NI <= 63, "load counter range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int team = wave / KS, slice = wave % KS;
  const int lane = tid & (kWave - 1);
  const int n = lane & 15;
  const int q = lane >> 4;
  uint8_t *const ring = smem + wave * (DR * kSlot);
  float4_t *const red = reinterpret_cast<float4_t *>(smem + NW * DR * kSlot);  // [2][NW][kWave]
  const int ngroups = (int)((N + 15) / 16);
  const int nsc = nu / C::kUnitsPerSC;  // super-chunks per row in this launch
  const int sc0 = slice * CPS;          // first super-chunk of this wave's slice
  const int group_stride = gridDim.x * kTeams;
  const int gfirst = blockIdx.x * kTeams;
  // Tiles per wave: the same for every wave of the workgroup (counted from
  // team 0's first tile), so the reduction barriers match.
  const int n_tiles = gfirst < ngroups ? (ngroups - gfirst + group_stride - 1) / group_stride : 0;
  const uint32_t unit0_bytes = (uint32_t)(unit0 / C::kUnitsPerSC * 144);

  uint32_t off[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int pc = k * kWave + lane;
    off[k] = pc < NP ? (uint32_t)(pc / PR) * (uint32_t)row_bytes + (uint32_t)(pc % PR) * 16
                     : 0x80000000u;
  }

  // Request chunk (item) `it` of this wave into ring slot `slot`: tile
  // gfirst + team + (it / CPS) * group_stride, super-chunk sc0 + it % CPS
  // (clamped into the row; such chunks are zeroed at compute time).
  int ig = gfirst + team, ic = 0, issued = 0;
  const int n_items = n_tiles * CPS;
  auto issue = [&](int slot) {
    const bool live = issued < n_items;
    const int gc = ig < ngroups ? ig : ngroups - 1;
    // 32-bit, wave-uniform (gc < ceil(N / 16), N <= 2^31): scalar compares
    const uint32_t r0 = (uint32_t)gc * 16u, left = (uint32_t)N - r0;
    const int64_t rows = left < 16u ? left : 16u;
    const rsrc_t rs = make_rsrc(W + (int64_t)r0 * row_bytes + unit0_bytes,
                                live ? (uint32_t)(rows * row_bytes - unit0_bytes) : 0u);
    const int sc = sc0 + ic < nsc ? sc0 + ic : nsc - 1;
#pragma unroll
    for (int k = 0; k < NI; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ring + slot * kSlot + k * (kWave * 16), 16,
                                               (int)off[k], sc * 144, 0, 0);
    ++issued;
    if (++ic == CPS) {
      ic = 0;
      ig += group_stride;
    }
  };
  // A operands of the slice (super-chunk c, lane unit j, word t). Loaded in
  // the A-operand layout straight from memory, every 16-byte load would touch
  // one cache line per lane; instead the wave stages its slice as fp16 words
  // in its own ring area with coalesced loads (word (b, u, t) at slot
  // t * TS + u * nb + b, as the LDS-staged kernels lay it out), reads its
  // operands back, and only then requests its first chunks into that area.
  // (Chunks requested earlier into free slots made the staging loads wait
  // for them: loads return in order.) Units past the row end stage zeros;
  // lanes n >= nb take zeros.
  constexpr int nus = CPS * C::kUnitsPerSC;  // units of the slice
  u32x4 xr[CPS][LU * T];
  {
    u32x4 *const xs = reinterpret_cast<u32x4 *>(ring);
    const int TS = staged_stride<F>(nus * nb);
    const int ubase = slice * nus;
    const int total = nb * nus * T;
    // words in flight per lane: a batch past `total` loads clamped
    // duplicates, so small slices want small batches (measured: 4 is as
    // fast as 8 at eight activation rows and faster at four)
    constexpr int kXB = 4;
    for (int base = lane; base < total; base += kXB * kWave) {
      XWord w[kXB];
      int dst[kXB];
      bool zero[kXB];
#pragma unroll
      for (int k = 0; k < kXB; ++k) {
        const int i = base + k * kWave;
        const int ic = i < total ? i : total - 1;
        const int t = ic % T, r = ic / T;
        const int b = r % nb, u = r / nb;
        const int ua = ubase + u < nu ? ubase + u : nu - 1;
        w[k] = load_xword<F>(x, ldx, b, ua, t);
        dst[k] = i < total ? t * TS + u * nb + b : -1;
        zero[k] = ubase + u >= nu;
      }
#pragma unroll
      for (int k = 0; k < kXB; ++k)
        if (dst[k] >= 0) xs[dst[k]] = zero[k] ? u32x4{0, 0, 0, 0} : pack_xword(w[k]);
    }
    const int xn = n < nb ? n : 0;
#pragma unroll
    for (int c = 0; c < CPS; ++c)
#pragma unroll
      for (int j = 0; j < LU; ++j)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const u32x4 v = xs[t * TS + (c * C::kUnitsPerSC + q * LU + j) * nb + xn];
          xr[c][j * T + t] = n < nb ? v : u32x4{0, 0, 0, 0};
        }
    // the chunk requests below overwrite the staged words
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  int slot = 0;  // ring slot of the next item to compute
#pragma unroll
  for (int k = 0; k < DR; ++k) issue(k);

  const UnpackMasks kmask;
  float4_t acc = float4_t{0, 0, 0, 0};
  int par = 0;
  int cg = gfirst + team;  // tile being computed
  // chunk 0's reads (the last of the DR requests may stay in flight)
  typename F::Raw nx[LU];
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DR - 1) * NI) : "memory");
#pragma unroll
  for (int j = 0; j < LU; ++j)
    nx[j] = C::read(reinterpret_cast<const u32x4 *>(ring) + n * PR, q, j);
  for (int tt = 0; tt < n_tiles; ++tt) {
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      // keep the previous chunk's work ahead of this chunk's waits
      __builtin_amdgcn_sched_barrier(0);
      typename F::Raw rw[LU];
#pragma unroll
      for (int j = 0; j < LU; ++j) rw[j] = nx[j];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(slot);
      slot = slot + 1 == DR ? 0 : slot + 1;
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DR - 1) * NI) : "memory");
      {
        // past the wave's last chunk this reads a slot of zeros: harmless
        const u32x4 *wbuf = reinterpret_cast<const u32x4 *>(ring + slot * kSlot);
#pragma unroll
        for (int j = 0; j < LU; ++j) nx[j] = C::read(wbuf + n * PR, q, j);
      }
      const bool valid = sc0 + c < nsc;
#pragma unroll
      for (int j = 0; j < LU; ++j) {
        const typename F::Prep pr = F::prep(rw[j], q, valid);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const half8_t a = __builtin_bit_cast(half8_t, xr[c][j * T + t]);
          const half8_t wv = __builtin_bit_cast(half8_t, F::dequant(rw[j], pr, t, kmask));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wv, acc, 0, 0, 0);
        }
      }
    }
    if (KS > 1) {
      red[(par * NW + wave) * kWave + lane] = acc;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (slice == 0) {
#pragma unroll
        for (int s2 = 1; s2 < KS; ++s2) acc += red[(par * NW + wave + s2) * kWave + lane];
      }
      par ^= 1;
    }
    if (slice == 0 && cg < ngroups) {
      const int64_t row = (int64_t)cg * 16 + n;
      if (row < N) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int b = 4 * q + v;
          if (b < nb) {
            float val = acc[v];
            if (accumulate) val += y[b * ldy + row];
            y[b * ldy + row] = val;
          }
        }
      }
    }
    acc = float4_t{0, 0, 0, 0};
    cg += group_stride;
  }
  // no buffer-to-LDS load may be left in flight when the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---- VALU mode, weight rows streamed through LDS ------------------------------
// Batch-1 GEMV (Q4_K with K <= 8192, or Q4_0 taken two blocks per unit with
// K <= 4096) whose weights reach each wave as contiguous chunks: a chunk (64
// units of one row, 2304 bytes: 16 Q4_K super-blocks or 128 Q4_0 blocks) is
// copied into a wave-private LDS ring slot by buffer-to-LDS loads of 64 x 16
// consecutive bytes, with non-temporal hints (every byte is read once), up
// to DR chunks ahead. Lane l then reads unit l of the chunk from the slot
// (for Q4_K the super-block header and the unit's two 16-byte quant pieces)
// and uses the dot2 arithmetic of gemv_kernel. Every load instruction covers
// 1 KB of one row; gemv_kernel's unit-shaped loads put lanes 32 bytes apart
// and, for Q4_K, read each header line from four lanes, which rules out
// non-temporal loads.
// Lane l always takes units l, l + 64, ... of a row (chunk c holds units
// 64c .. 64c + 63), so after the workgroup has staged x it keeps the staged
// words and sums of its first unit in registers: for rows of up to 4096
// weights the LDS then serves only the weight chunks. Sixteen waves per
// workgroup, one workgroup per CU; waves take whole rows, row r by wave
// r mod (waves in the grid). The first chunks are requested before the
// staging (the ring does not overlap the staged activations). Per chunk the
// wave waits until that chunk has landed, reads its unit from the slot,
// refills the slot with the chunk DR ahead and only then computes, so that
// DR chunks are in flight during the arithmetic. (Reading the next chunk's
// unit during the current chunk's arithmetic hid that LDS read but had the
// wave wait for the next chunk before computing the current one, with one
// chunk in flight meanwhile: Q4_K 28672 x 8192 batch 1 26.0 us against
// 25.1 us, batch 2 31.7 against 30.9 us, same process.)
// Waits: as in gemv_coalr_kernel (loads return in order; a slot is refilled
// only after the wave's reads of it are complete; chunks past the wave's
// work come from an empty buffer range).
constexpr int kStreamWaves = 16;
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kStreamUnitBytes = 36;                // a Q4_K quarter super-block or two Q4_0 blocks
constexpr int kStreamChunk = kWave * kStreamUnitBytes;  // a chunk: 64 units, 2304 bytes
constexpr int kStreamLoads = (kStreamChunk + kWave * 16 - 1) / (kWave * 16);  // 3
// A ring slot holds whole loads (3 KB): the last load's lanes past the chunk
// fall outside the buffer range, read zeros without memory traffic and write
// them into the slot's padding. With no lane-masked load, the compiler's
// load-counter waits for the staged activations no longer cover chunk loads
// (Q4_K 28672 x 8192 batch 1: 26.5 -> 25.7 us, shuffled A/B).
constexpr int kStreamSlot = kStreamLoads * kWave * 16;
constexpr int kStreamMaxUPL = 2;                   // chunks (units per lane) per row: K <= 8192
constexpr int kStreamDepth = 2;  // ring slots per wave (measured: faster than 3 at every shape tried)
// Activation rows per launch. Measured on Q4_K 28672 x 8192: 2 rows 33.1 ->
// 31.4 us against gemv_kernel, but 3 and 4 rows 37.5 and 43.2 us against
// 29.8 and 30.6 us on the matrix cores (the dot2 work grows with the rows).
constexpr int kStreamMaxBatch = 2;

template <class F>
__host__ __device__ __forceinline__ size_t stream_stage_bytes(int batch, int nu) {
  const size_t b = (size_t)batch * F::kWords * staged_stride<F>(nu) * 16 +
                   (size_t)batch * nu * F::kSums * 4;
  return (b + 15) & ~(size_t)15;
}

template <class F, int B, int DR>
__global__ void __launch_bounds__(kStreamThreads)
gemv_stream_kernel(const uint8_t *__restrict__ W, int64_t row_bytes, int nu,
                   const float *__restrict__ x, int64_t ldx, float *__restrict__ y, int64_t ldy,
                   int64_t N) {
  constexpr int T = F::kWords;
  constexpr int NI = kStreamLoads;
  static_assert((DR - 1) * NI <= 63, "load counter range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  u32x4 *xs = reinterpret_cast<u32x4 *>(smem);  // slot (b*T + t)*NS + u
  const int NS = staged_stride<F>(nu);
  float *sums = reinterpret_cast<float *>(smem + (size_t)B * T * NS * 16);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  uint8_t *const ring = smem + stream_stage_bytes<F>(B, nu) + (size_t)wave * DR * kStreamSlot;
  const int64_t nwaves = (int64_t)gridDim.x * kStreamWaves;
  // Row bookkeeping in 32 bits (N <= 2^31, so every row index and count
  // below stays under 2^32): wave-uniform, so it runs on the scalar unit
  // (64-bit signed compares have no scalar form and took vector
  // instructions in the chunk loop).
  const uint32_t nw32 = (uint32_t)nwaves, n32 = (uint32_t)N;
  const uint32_t wave_id = blockIdx.x * (uint32_t)kStreamWaves + (uint32_t)wave;
  const uint32_t n_rows = wave_id < n32 ? (n32 - wave_id + nw32 - 1) / nw32 : 0u;
  // Chunks per row: Q4_K 1 or 2, kept a run-time value, so that the chunk
  // loop below stays a loop (the compiler keeps it within 128 VGPRs); the
  // Q4_0 pair form takes one chunk per row (with a second one it spilled).
  constexpr bool kOneChunk = std::is_same<F, FmtQ4_0x2>::value;
  static_assert(B <= kStreamMaxBatch, "activation rows");
  const int cpr = kOneChunk ? 1 : (nu + kWave - 1) / kWave;
  auto chunk_units = [&](int c) {  // units in chunk c of a row: cpr - 1 full chunks, a last one
    return nu - c * kWave < kWave ? nu - c * kWave : kWave;
  };

  // Request item `issued` (chunk ic of row irow) into ring slot `slot`.
  uint32_t irow = wave_id, issued = 0;
  int ic = 0;
  auto issue = [&](int slot) {
    const bool live = issued < n_rows * (uint32_t)cpr;
    const uint32_t r = irow < n32 ? irow : n32 - 1;
    const rsrc_t rs = make_rsrc(W + (int64_t)r * row_bytes + (int64_t)ic * kStreamChunk,
                                live ? (uint32_t)(chunk_units(ic) * kStreamUnitBytes) : 0u);
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ring + slot * kStreamSlot + k * (kWave * 16), 16,
                                               k * (kWave * 16) + lane * 16, 0, 0,
                                               2 /* non-temporal */);
    }
    ++issued;
    if (++ic == cpr) {
      ic = 0;
      irow += nw32;
    }
  };
  // Stage the activation words and the per-(b, u) sums of gemv_kernel; at
  // batch 1 each lane then copies those of its first unit into registers.
  // The barriers wait for LDS operations only, not for chunk requests.
  // Two orders (shuffled A/B on MI355X, cold HBM):
  // - Q4_K, and Q4_0 pairs at batch 2: each thread loads its (at most two)
  //   words before the first chunks are requested, since loads return in
  //   order and words loaded behind the chunks would wait for them. The
  //   thread holding the first word of a group of kSumWords words adds the
  //   group's sums from its neighbours' partial sums (lanes hold a group's
  //   words in order, and the additions follow word_sums' order), so one
  //   barrier covers words and sums. Q4_K 28672 x 8192: 25.85 -> 25.5 us
  //   at batch 1, 32.0 -> 31.2 us at batch 2; Q4_0 12288 x 4096 batch 2:
  //   10.1 -> 9.65 us.
  // - Q4_0 pairs at batch 1: chunks first, then gemv_kernel's staging and a
  //   second pass for the sums. The first order measured 0.3-0.5 us slower
  //   there (8.0 -> 8.3 us at 11008 and 12288 x 4096).
  constexpr bool kWordsFirst = !kOneChunk || B == 2;
  static_assert(kStreamMaxBatch * kStreamMaxUPL * kWave * T <= 2 * kStreamThreads,
                "two staged words per thread cover every streamed input");
  if (kWordsFirst) {
    const int xtotal = B * nu * T;  // at most 2 * kStreamThreads (see the assertion above)
    XWord xw[2];
    int xdst[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + k * kStreamThreads;
      const int ic = i < xtotal ? i : xtotal - 1;
      const int t = ic % T, r = ic / T;
      const int b = r % B, u = r / B;
      xw[k] = load_xword<F>(x, ldx, b, u, t);
      xdst[k] = i < xtotal ? (b * T + t) * NS + u : -1;
    }
#pragma unroll
    for (int k = 0; k < DR; ++k) issue(k);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 wd = pack_xword(xw[k]);
      if (xdst[k] >= 0) xs[xdst[k]] = wd;
      const half2_t ha = as_half2(wd.x), hb = as_half2(wd.y), hc = as_half2(wd.z),
                    hd = as_half2(wd.w);
      const float plo = ((float)ha.x + (float)ha.y) + ((float)hc.x + (float)hc.y);
      const float phi = ((float)hb.x + (float)hb.y) + ((float)hd.x + (float)hd.y);
      float slo = 0.0f, shi = 0.0f;
#pragma unroll
      for (int j = 0; j < F::kSumWords; ++j) {
        slo += __shfl(plo, lane + j < kWave ? lane + j : lane);
        shi += __shfl(phi, lane + j < kWave ? lane + j : lane);
      }
      const int i = tid + k * kStreamThreads;
      const int t = i % T, r = i / T;
      if (i < xtotal && t % F::kSumWords == 0)
        F::stage_sums(sums, (r % B) * nu + r / B, t / F::kSumWords, slo, shi);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
#pragma unroll
    for (int k = 0; k < DR; ++k) issue(k);
    stage_words<F, kStreamThreads, 1>(xs, B, nu, x, ldx,
                                      [&](int b, int u, int t) { return (b * T + t) * NS + u; });
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int i = tid; i < B * nu; i += kStreamThreads) {
      const int u = i % nu, b = i / nu;
#pragma unroll
      for (int g = 0; g < T / F::kSumWords; ++g) {
        float slo = 0.0f, shi = 0.0f;
#pragma unroll
        for (int t = g * F::kSumWords; t < (g + 1) * F::kSumWords; ++t)
          word_sums(xs[(b * T + t) * NS + u], slo, shi);
        F::stage_sums(sums, i, g, slo, shi);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // At batch 1, registers hold the first chunk's activations; those of a
  // second chunk, and all of them at larger batches, stay in LDS (there are
  // no registers left for them).
  u32x4 xr[B == 1 ? T : 1];
  float sr[2];
  if (B == 1) {
    const int u = lane < nu ? lane : nu - 1;
#pragma unroll
    for (int t = 0; t < T; ++t) xr[t] = xs[t * NS + u];
    sr[0] = sums[2 * u];
    sr[1] = sums[2 * u + 1];
  }

  // Lane's unit of the chunk in `slot` (clamped into the chunk).
  auto read_unit = [&](int slot, int nuc, typename F::Raw &r) {
    r = F::read_stream_unit(reinterpret_cast<const u32x4 *>(ring + slot * kStreamSlot),
                            lane < nuc ? lane : nuc - 1);
  };

  const UnpackMasks kmask;
  int slot = 0;
  uint32_t crow = wave_id;
  for (uint32_t rr = 0; rr < n_rows; ++rr) {
    float acc[1][B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[0][b] = 0.0f;
#pragma nounroll
    for (int c = 0; c < cpr; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      // this chunk has landed (the next DR - 1 may still be in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DR - 1) * NI) : "memory");
      typename F::Raw rw[1];
      read_unit(slot, chunk_units(c), rw[0]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(slot);
      slot = slot + 1 == DR ? 0 : slot + 1;
      const int nuc = chunk_units(c);
      const bool valid = lane < nuc;
      const int u = c * kWave + (valid ? lane : 0);
      if (B == 1 && c == 0)
        F::template compute_with<B, 1>(
            rw, [&](int, int t) { return xr[B == 1 ? t : 0]; }, [&](int, int h) { return sr[h]; },
            u, valid, kmask, acc);
      else
        F::template compute_with<B, 1>(
            rw, [&](int b, int t) { return xs[(b * T + t) * NS + u]; },
            [&](int b, int h) { return sums[2 * (b * nu + u) + h]; }, u, valid, kmask, acc);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = group_sum(acc[0][b], kWave);
      if (lane == kWave - 1) y[b * ldy + (int64_t)crow] = v;
    }
    crow += nw32;
  }
  // no buffer-to-LDS load may be left in flight when the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class F, int B, int DR>
hipError_t launch_stream(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                         hipStream_t stream) {
  auto kern = gemv_stream_kernel<F, B, DR>;
  const hipError_t e = ensure_max_lds<gemv_stream_kernel<F, B, DR>>(kMaxLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kStreamThreads), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.nu, x, pl.ldx, y, pl.ldy, pl.N);
  return hipGetLastError();
}

template <class F>
hipError_t launch_stream_b(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                           hipStream_t s) {
  if (pl.batch == 1) return launch_stream<F, 1, kStreamDepth>(pl, W, x, y, s);
  if (pl.batch == 2) return launch_stream<F, 2, kStreamDepth>(pl, W, x, y, s);
  return hipErrorInvalidValue;
}

template <class F, int B, int R, int U, bool FULL>
hipError_t launch_valu(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                       hipStream_t stream) {
  auto kern = gemv_kernel<F, B, R, U, FULL>;
  const hipError_t e = ensure_max_lds<gemv_kernel<F, B, R, U, FULL>>(kMaxGemvLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.unit0, pl.nu, x, pl.ldx, y, pl.ldy, pl.N, pl.lpr_log2,
                     pl.accumulate);
  return hipGetLastError();
}

template <class C, int U, int KS, int D>
hipError_t launch_coal(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                       hipStream_t stream) {
  auto kern = gemv_coal_kernel<C, U, KS, D>;
  const hipError_t e = ensure_max_lds<gemv_coal_kernel<C, U, KS, D>>(kMaxLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.unit0, pl.nu, x, pl.ldx, y, pl.ldy, pl.N, pl.batch,
                     pl.accumulate);
  return hipGetLastError();
}

// Coalesced-kernel instances: U in {1, 2}, KS in {1, 2, 4, 8}, depth 2, 3, 4
// or 6 chunks in flight per wave.
template <class C, int U, int D>
hipError_t launch_coal_ks(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                          hipStream_t s) {
  switch (pl.ksplit) {
    case 1: return launch_coal<C, U, 1, D>(pl, W, x, y, s);
    case 2: return launch_coal<C, U, 2, D>(pl, W, x, y, s);
    case 4: return launch_coal<C, U, 4, D>(pl, W, x, y, s);
    default: return launch_coal<C, U, 8, D>(pl, W, x, y, s);
  }
}
template <class C, int U>
hipError_t launch_coal_d(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                         hipStream_t s) {
  switch (pl.depth) {
    case 2: return launch_coal_ks<C, U, 2>(pl, W, x, y, s);
    case 3: return launch_coal_ks<C, U, 3>(pl, W, x, y, s);
    case 4: return launch_coal_ks<C, U, 4>(pl, W, x, y, s);
    default: return launch_coal_ks<C, U, 6>(pl, W, x, y, s);
  }
}
template <class C>
hipError_t launch_coal_fmt(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                           hipStream_t s) {
  if (pl.units_per_lane == 2) return launch_coal_d<C, 2>(pl, W, x, y, s);
  return launch_coal_d<C, 1>(pl, W, x, y, s);
}

// Activations-in-registers instances: CPS in {1, 2, 3, 4} super-chunks per
// k-slice, KS in {1, 2, 4, 8}, a ring of kCoalrRing chunks per wave.
template <class C, int CPS, int KS>
hipError_t launch_coalr(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                        hipStream_t stream) {
  auto kern = gemv_coalr_kernel<C, CPS, KS, kCoalrRing>;
  const hipError_t e = ensure_max_lds<gemv_coalr_kernel<C, CPS, KS, kCoalrRing>>(kMaxLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.unit0, pl.nu, x, pl.ldx, y, pl.ldy, pl.N, pl.batch,
                     pl.accumulate);
  return hipGetLastError();
}
template <class C, int CPS>
hipError_t launch_coalr_ks(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                           hipStream_t s) {
  switch (pl.ksplit) {
    case 1: return launch_coalr<C, CPS, 1>(pl, W, x, y, s);
    case 2: return launch_coalr<C, CPS, 2>(pl, W, x, y, s);
    case 4: return launch_coalr<C, CPS, 4>(pl, W, x, y, s);
    default: return launch_coalr<C, CPS, 8>(pl, W, x, y, s);
  }
}
template <class C>
hipError_t launch_coalr_fmt(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                            hipStream_t s) {
  switch (pl.cps) {
    case 1: return launch_coalr_ks<C, 1>(pl, W, x, y, s);
    case 2: return launch_coalr_ks<C, 2>(pl, W, x, y, s);
    case 3: return launch_coalr_ks<C, 3>(pl, W, x, y, s);
    default: return launch_coalr_ks<C, 4>(pl, W, x, y, s);
  }
}

template <class F, int R, int U, int KS, int NW>
hipError_t launch_mfma(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                       hipStream_t stream) {
  auto kern = gemv_mfma_kernel<F, R, U, KS, NW>;
  const hipError_t e = ensure_max_lds<gemv_mfma_kernel<F, R, U, KS, NW>>(kMaxGemvLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(NW * kWave), pl.lds_bytes, stream, W,
                     pl.row_bytes, pl.unit0, pl.nu, x, pl.ldx, y, pl.ldy, pl.N, pl.batch,
                     pl.accumulate);
  return hipGetLastError();
}

// (rows per lane, units per lane per chunk) shapes that are instantiated.
template <class F, int B, bool FULL>
hipError_t launch_ru(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                     hipStream_t s) {
  const int r = pl.rows_per_lane, u = pl.units_per_lane;
  if (r == 1 && u == 4) return launch_valu<F, B, 1, 4, FULL>(pl, W, x, y, s);
  if (r == 1) return launch_valu<F, B, 1, 2, FULL>(pl, W, x, y, s);
  if (r == 2 && u == 1) return launch_valu<F, B, 2, 1, FULL>(pl, W, x, y, s);
  return launch_valu<F, B, 2, 2, FULL>(pl, W, x, y, s);
}

// Matrix-core launches (Q4_0 and Q4_K).
template <class F>
hipError_t launch_fmt_mfma(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                           hipStream_t s) {
  const int u = pl.units_per_lane;
  if (pl.lds_stage) {
    if (pl.xregs) {
      if (pl.cps < 1 || pl.cps > 4) return hipErrorInvalidValue;
      if (std::is_same<F, FmtQ4_K>::value) return launch_coalr_fmt<CoalQ4_K>(pl, W, x, y, s);
      return launch_coalr_fmt<CoalQ4_0>(pl, W, x, y, s);
    }
    if (std::is_same<F, FmtQ4_K>::value) return launch_coal_fmt<CoalQ4_K>(pl, W, x, y, s);
    return launch_coal_fmt<CoalQ4_0>(pl, W, x, y, s);
  }
  if (pl.waves == 16) {
    switch (pl.ksplit) {
      case 4: return u == 4 ? launch_mfma<F, 1, 4, 4, 16>(pl, W, x, y, s)
                            : launch_mfma<F, 1, 2, 4, 16>(pl, W, x, y, s);
      case 8: return u == 4 ? launch_mfma<F, 1, 4, 8, 16>(pl, W, x, y, s)
                            : launch_mfma<F, 1, 2, 8, 16>(pl, W, x, y, s);
      default: return u == 4 ? launch_mfma<F, 1, 4, 16, 16>(pl, W, x, y, s)
                             : launch_mfma<F, 1, 2, 16, 16>(pl, W, x, y, s);
    }
  }
  switch (pl.ksplit) {
    case 1: return u == 4 ? launch_mfma<F, 1, 4, 1, 8>(pl, W, x, y, s)
                          : launch_mfma<F, 1, 2, 1, 8>(pl, W, x, y, s);
    case 2: return u == 4 ? launch_mfma<F, 1, 4, 2, 8>(pl, W, x, y, s)
                          : launch_mfma<F, 1, 2, 2, 8>(pl, W, x, y, s);
    case 4: return u == 4 ? launch_mfma<F, 1, 4, 4, 8>(pl, W, x, y, s)
                          : launch_mfma<F, 1, 2, 4, 8>(pl, W, x, y, s);
    default: return u == 4 ? launch_mfma<F, 1, 4, 8, 8>(pl, W, x, y, s)
                           : launch_mfma<F, 1, 2, 8, 8>(pl, W, x, y, s);
  }
}

template <class F>
hipError_t launch_fmt(const GemvPlan &pl, const uint8_t *W, const float *x, float *y,
                      hipStream_t s) {
  if constexpr (std::is_same<F, FmtQ4_0x2>::value) {  // VALU mode only
    if (pl.mfma || pl.lds_stage) return hipErrorInvalidValue;
  } else {
    if (pl.mfma) return launch_fmt_mfma<F>(pl, W, x, y, s);
  }
  if constexpr (std::is_same<F, FmtQ4_K>::value || std::is_same<F, FmtQ4_0x2>::value) {
    if (pl.stream) {
      // the whole row in one launch, at most kStreamMaxUPL chunks
      const int upl = (pl.nu + kWave - 1) / kWave;
      if (pl.unit0 != 0 || pl.accumulate || upl > kStreamMaxUPL) return hipErrorInvalidValue;
      return launch_stream_b<F>(pl, W, x, y, s);
    }
  }
  const bool full = pl.lpr_log2 == 6;
  if (pl.batch == 1)
    return full ? launch_ru<F, 1, true>(pl, W, x, y, s) : launch_ru<F, 1, false>(pl, W, x, y, s);
  return full ? launch_ru<F, 2, true>(pl, W, x, y, s) : launch_ru<F, 2, false>(pl, W, x, y, s);
}

}  // namespace

template <class F>
size_t staged_bytes(bool mfma, int batch, int nu) {
  if (mfma) return (size_t)F::kWords * staged_stride<F>(nu * batch) * 16;
  return (size_t)batch * F::kWords * staged_stride<F>(nu) * 16 + (size_t)batch * nu * F::kSums * 4;
}

size_t gemv_lds_bytes(GemvFormat f, bool mfma, int batch, int nu) {
  switch (f) {
    case GemvFormat::Q4_0: return staged_bytes<FmtQ4_0>(mfma, batch, nu);
    case GemvFormat::Q4_0x2: return staged_bytes<FmtQ4_0x2>(mfma, batch, nu);
    default: return staged_bytes<FmtQ4_K>(mfma, batch, nu);
  }
}

size_t gemv_mfma_reduce_bytes(int waves) { return (size_t)waves * kWave * 16; }

bool gemv_coalr_fits(GemvFormat f, int cps, int batch) {
  const int T = f == GemvFormat::Q4_K ? FmtQ4_K::kWords : FmtQ4_0::kWords;
  const int scu = f == GemvFormat::Q4_K ? CoalQ4_K::kUnitsPerSC : CoalQ4_0::kUnitsPerSC;
  const int ts = f == GemvFormat::Q4_K ? staged_stride<FmtQ4_K>(cps * scu * batch)
                                       : staged_stride<FmtQ4_0>(cps * scu * batch);
  return (size_t)T * ts * 16 <= (size_t)kCoalrRing * 3 * kWave * 16;
}

size_t gemv_coalr_lds_bytes() {
  return (size_t)kWavesPerWg * kCoalrRing * 3 * kWave * 16 + (size_t)2 * kWavesPerWg * kWave * 16;
}

size_t gemv_stream_lds_bytes(GemvFormat f, int batch, int nu) {
  const size_t stage = f == GemvFormat::Q4_K ? stream_stage_bytes<FmtQ4_K>(batch, nu)
                                             : stream_stage_bytes<FmtQ4_0x2>(batch, nu);
  return stage + (size_t)kStreamWaves * kStreamDepth * kStreamSlot;
}

int gemv_stream_max_batch() { return kStreamMaxBatch; }

int gemv_stream_max_units(GemvFormat f) {
  return (f == GemvFormat::Q4_K ? kStreamMaxUPL : 1) * kWave;
}

int gemv_stream_waves() { return kStreamWaves; }

size_t gemv_coal_stage_bytes(int u) {
  return (size_t)kWavesPerWg * ((16 * 9 * u + 63) / 64) * kWave * 16;
}

int gemv_unit_weights(GemvFormat f) {
  switch (f) {
    case GemvFormat::Q4_0: return FmtQ4_0::kUnitWeights;
    case GemvFormat::Q4_0x2: return FmtQ4_0x2::kUnitWeights;
    case GemvFormat::Q4_K: return FmtQ4_K::kUnitWeights;
    case GemvFormat::Q8_0: return 32;   // FmtQ8_0: one block
    case GemvFormat::Q6_K: return 128;  // FmtQ6_K: half a super-block
    case GemvFormat::Q2_K: return 128;  // FmtQ2_K: half a super-block
    case GemvFormat::I4G32: return 32;  // FmtI4G32: one group
    case GemvFormat::Q1_0: return 32;   // FmtQ1_0: one block
  }
  return 32;
}

int gemv_threads() { return kGemvThreads; }

hipError_t gemv_launch(GemvFormat f, const GemvPlan &pl, const uint8_t *W, const float *x,
                       float *y, hipStream_t stream) {
  if (f == GemvFormat::Q4_0) return launch_fmt<FmtQ4_0>(pl, W, x, y, stream);
  if (f == GemvFormat::Q4_0x2) return launch_fmt<FmtQ4_0x2>(pl, W, x, y, stream);
  return launch_fmt<FmtQ4_K>(pl, W, x, y, stream);
}

}  // namespace lqmm

// Q8_0 x fp16 GEMM for prefill: Y[m][n] = sum_k X[m][k] * W[n][k], fp32
// accumulation, fp16 output, on the gfx950 fp16 matrix cores.
//
// This is the matmul case of "Resumo Tecnico: Llamas na Web", section
// "Design de Shader Consciente de Quantizacao": quantized blocks are loaded
// into shared memory (the CU's LDS), dequantized and reused by every row of
// the M tile.
//
// * One workgroup of NWAVES waves (8; 7 as a tuning override) per
//   128 x (32 * NWAVES) output tile; wave w owns columns 32w .. 32w+31
//   of the tile and all 128 rows, as 4 tiles of v_mfma_f32_32x32x16_f16 (two
//   waves per SIMD, so one wave's vector-ALU dequantization overlaps the
//   other's matrix-core work).
// * (K % 64 == 0; otherwise the LDS-tile kernel of gemm_lds.hip runs.) K advances 64 (two Q8_0 blocks) per step. The X tile (128
//   rows x 64 fp16) goes through a ring of NS LDS stages, written by
//   buffer-to-LDS loads issued NS - 1 steps ahead and shared by the
//   workgroup. Each wave brings the raw Q8_0 bytes of its own 32 weight rows
//   into its own LDS records with buffer-to-LDS loads two steps ahead (three
//   record buffers): raw bytes cost about half the LDS write bandwidth of
//   dequantized fp16, and LDS writes run at about half the rate of LDS reads
//   on this GPU.
// * Each wave dequantizes its own columns once per step, from its records
//   straight into MFMA B operands (so each weight is dequantized once per
//   workgroup and reused by all 128 rows): q ^ 0x80 placed in the mantissa
//   of 1024.0 with v_perm_b32 is exactly 1152 + q; a packed subtract gives q
//   and a packed multiply gives fp16(d*q), one rounding.
// * K order inside a step: MFMA slice s (16 k) takes, in lane half h, the
//   codes 8s .. 8s+7 of block h. A operands (X) are read in the same order;
//   the X tile is stored with 16-byte chunks permuted per row pair so that
//   those reads are free of LDS bank conflicts.
#include <stdlib.h>

#include "lqmm_device.hpp"
#include "lqmm_internal.hpp"

namespace lqmm {
namespace {

constexpr int BM = 128, BK = 64;
constexpr int NS = 4;                        // LDS stages of the X tile
constexpr int kXStageBytes = BM * BK * 2;    // 16 KB
constexpr int kXInstr = kXStageBytes / 1024;  // buffer-to-LDS loads per stage (1 KB each)
// Raw W: each wave owns 32 rows of the tile. A step is 68 bytes of a row,
// fetched as five 16-byte pieces at byte 0, 16, 32, 36 and 52 (pieces 2
// and 3 overlap, so nothing past the row's step is read and block 1's codes
// are exactly pieces 3 and 4): piece p of the wave's
// 160 goes to byte 16 p of the step's record buffer, i.e. an 80-byte record
// per row. Buffer-to-LDS load i writes 64 consecutive pieces, so a record
// buffer spans kWLoads KB (the last load's spare lanes write its padding).
constexpr int kWRows = 32;                   // weight rows per wave
constexpr int kWRec = 80;                    // LDS bytes per row record
constexpr int kWPieces = 5;
constexpr int kWLoads = (kWRows * kWPieces + 63) / 64;  // 16-byte loads per lane per step
constexpr int kWBufs = 3;                              // record buffers per wave
constexpr int kWBufBytes = kWLoads * 1024;
constexpr int kWWaveBytes = kWBufs * kWBufBytes;

template <int NWAVES>
struct Tile {
  static constexpr int BN = kWRows * NWAVES;
  static constexpr int kThreads = 64 * NWAVES;
  // X loads per wave per step: wave w issues loads w, w + NWAVES, ... of the
  // stage's kXInstr, so the first kXInstr % NWAVES waves issue one more.
  static constexpr int kXMax = (kXInstr + NWAVES - 1) / NWAVES;
  static constexpr int kLdsBytes = NS * kXStageBytes + NWAVES * kWWaveBytes;
  static_assert(NS == 4 && 2 * kXMax + kWLoads <= 63, "pipeline depths and vmcnt range");
};

// Slot of 16-byte chunk c (0..7) of X tile row r: chunks permuted per row
// pair, so that the 16 rows one ds_read_b128 phase touches hit 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int xslot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Wait until at most N of this wave's vector-memory loads are outstanding
// and all its LDS operations are done, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// fp16 weights d*q of 4 int8 codes (one dword) as two fp16 pairs.
__device__ __forceinline__ void dequant_word(uint32_t w, half2_t d2, uint32_t &lo, uint32_t &hi) {
  const half2_t bias = {(half_t)1152.0f, (half_t)1152.0f};
  const uint32_t u = w ^ 0x80808080u;
  half2_t l = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  half2_t h = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
  lo = as_u32((l - bias) * d2);
  hi = as_u32((h - bias) * d2);
}

template <int NWAVES>
__global__ void __launch_bounds__(64 * NWAVES)
gemm_q8_0_kernel(const uint8_t *__restrict__ W, const uint16_t *__restrict__ X,
                 uint16_t *__restrict__ Y, int64_t M, int64_t N, int64_t K, int tiles_n) {
  using TT = Tile<NWAVES>;
  constexpr int BN = TT::BN;
  constexpr int kXMax = TT::kXMax;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
  // L2. Renumber so that consecutive logical tiles (the M tiles that share
  // one weight N tile) run on the same XCD and share its L2. (32-bit scalar
  // arithmetic: the host keeps the tile count below 2^31, and the buffer
  // resources built from these values must stay in scalar registers.)
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int ntiles = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if (ntiles % 8 == 0) tile = (tile % 8) * (ntiles / 8) + tile / 8;
  tile = __builtin_amdgcn_readfirstlane(tile);
  const int64_t m0 = (int64_t)(tile % tiles_m) * BM, n0 = (int64_t)(tile / tiles_m) * BN;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const uint32_t Ku = (uint32_t)K;
  const uint32_t row_bytes = Ku / 32 * 34;
  const int nk = (int)(K / BK);  // K % 64 == 0 here

  // Buffer resources over the tile's rows, ending at the last row of each
  // tensor: rows past M or N read zeros (their results are never stored).
  const int64_t xrows = M - m0 < BM ? M - m0 : BM;
  const int64_t wrows = N - n0 < BN ? N - n0 : BN;
  const rsrc_t xr = make_rsrc(X + m0 * K, (uint32_t)(xrows * K * 2));
  const rsrc_t wr = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)(wrows * row_bytes));

  // Per-lane source offsets within the tile (VGPRs); the step's offset goes
  // in the scalar offset. Every byte a step reads lies inside its own row
  // (K % 64 == 0), and rows past M or N start past the end of the resource.
  // X: buffer-to-LDS load j = wave + i * NWAVES (j < kXInstr) fills 64
  // consecutive 16-byte slots of the stage; lane L fills slot L.
  const int nx = (kXInstr - wave + NWAVES - 1) / NWAVES;  // this wave's X loads per step
  uint32_t xoff[kXMax];
#pragma unroll
  for (int i = 0; i < kXMax; ++i) {
    const int j = wave + i * NWAVES;
    const int slot = (j < kXInstr ? j : 0) * 64 + lane;
    const int r = slot >> 3, c = xslot(r, slot & 7);  // slot & 7 holds chunk c of row r
    xoff[i] = (uint32_t)r * Ku * 2 + 16 * c;
  }
  // W: piece p = 64 i + lane of this wave's kWRows * 5 pieces (lanes past the
  // last piece repeat it): row p / 5, piece p % 5, kept at byte 16 p of the
  // wave's record area (80 bytes a row).
  uint32_t woff[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    int p = 64 * i + lane;
    p = p < kWRows * kWPieces ? p : kWRows * kWPieces - 1;
    const int rr = p / kWPieces, k = p % kWPieces;
    woff[i] = (uint32_t)(wave * kWRows + rr) * row_bytes + (k < 3 ? 16 * k : k == 3 ? 36 : 52);
  }
  uint8_t *const wl = smem + NS * kXStageBytes + wave * kWWaveBytes;  // this wave's W records

  // This wave's X loads of step kt (the test is wave-uniform, and absent
  // when every wave issues kXMax).
  auto issue_x = [&](int kt) {
    const int ks = kt < nk ? kt : nk - 1;  // past the end: reload the last step, never read
    uint8_t *st = smem + (kt % NS) * kXStageBytes;
#pragma unroll
    for (int i = 0; i < kXMax; ++i)
      if (kXInstr % NWAVES == 0 || i < nx)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, st + (wave + i * NWAVES) * 1024, 16,
                                                 (int)xoff[i], ks * (BK * 2), 0, 0);
  };
  // This wave's W pieces of step kt into record buffer kt % kWBufs.
  auto issue_w = [&](int kt) {
    const int ks = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, wl + (kt % kWBufs) * kWBufBytes + i * 1024, 16,
                                               (int)woff[i], ks * 68, 0, 0);
  };
  // B operands of one step from this wave's W records: this lane's column
  // (row l % 32 of the wave) and block h; slice s uses codes 8s .. 8s+7.
  // Record pieces: 0 = step bytes 0..15, 1 = 16..31, 2 = 32..47, 3 = 36..51,
  // 4 = 52..67. The lane reads three whole pieces with 16-byte LDS reads
  // (the 80-byte record stride keeps eight consecutive lanes on distinct
  // banks; 4-byte reads at that stride conflicted about 4-way): block 0
  // takes pieces 0, 1, 2 (d in the low half of dword 0, codes from byte 2),
  // block 1 takes pieces 3, 4, 2 (codes from byte 0, d in the high half of
  // the third piece's first dword), so code dword j is alignbyte(D[j + 1],
  // D[j], 2 - 2h) in both halves.
  auto dequant_step = [&](int buf, half8_t (&b)[4]) {
    const uint8_t *rec = wl + buf * kWBufBytes + l32 * kWRec;
    const u32x4 r0 = *reinterpret_cast<const u32x4 *>(rec + 48 * h);
    const u32x4 r1 = *reinterpret_cast<const u32x4 *>(rec + 16 + 48 * h);
    const u32x4 r2 = *reinterpret_cast<const u32x4 *>(rec + 32);
    const uint32_t q[9] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w, r2.x};
    const uint32_t dword = h ? r2.x : r0.x;
    const half_t dh = __builtin_bit_cast(half_t, (uint16_t)__builtin_amdgcn_ubfe(dword, 16 * h, 16));
    const half2_t d2 = {dh, dh};
    const uint32_t shift = 2 - 2 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w0 = __builtin_amdgcn_alignbyte(q[2 * s + 1], q[2 * s], shift);
      const uint32_t w1 = __builtin_amdgcn_alignbyte(q[2 * s + 2], q[2 * s + 1], shift);
      uint32_t p0, p1, p2, p3;
      dequant_word(w0, d2, p0, p1);
      dequant_word(w1, d2, p2, p3);
      b[s] = __builtin_bit_cast(half8_t, u32x4{p0, p1, p2, p3});
    }
  };

  // Each wave owns a 128 x 32 block of the tile as 4 tiles of
  // v_mfma_f32_32x32x16_f16: lane l supplies row (or column) l % 32 and the
  // 8 k values 8 * (l / 32) .. +7 of each operand. Two waves share each
  // SIMD, so one wave's dequantization overlaps the other's MFMAs.
  float16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // Pipeline (all loads are buffer-to-LDS). Iteration kt issues W of step
  // kt + 2, then X of step kt + 3 (NS - 1 ahead; shared by the workgroup,
  // one barrier per step). W records are wave-private: only this wave reads
  // them, so they need no barrier, and the record buffer refilled in step
  // kt was last read (into registers) in step kt - 1. Loads complete in issue
  // order; when step kt starts, the loads issued after its W are X of step
  // kt + 1 and W and X of step kt + 1's iteration, and X of step kt was
  // issued before its W. The prologue issues in the same order.
  issue_x(0);
  issue_w(0);
  issue_x(1);
  issue_w(1);
  issue_x(2);
  for (int kt = 0; kt < nk; ++kt) {
    if (kXInstr % NWAVES == 0 || nx == kXMax)
      wait_and_barrier<2 * kXMax + kWLoads>();
    else
      wait_and_barrier<2 * (kXMax - 1) + kWLoads>();
    issue_w(kt + 2);
    issue_x(kt + NS - 1);
    __builtin_amdgcn_sched_barrier(0);
    half8_t b[4];
    dequant_step(kt % kWBufs, b);
    const uint8_t *st = smem + (kt % NS) * kXStageBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * i + l32;
        a[i] = *reinterpret_cast<const half8_t *>(st + row * 128 + 16 * xslot(row, 4 * h + s));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[s], acc[i], 0, 0, 0);
    }
  }
  // Drain the loads issued past the end before the workgroup exits.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // D layout of v_mfma_f32_32x32x16_f16: lane l holds column l % 32 and rows
  // 8 * (v / 4) + 4 * (l / 32) + v % 4 for v = 0..15.
  const int64_t col = n0 + wave * 32 + l32;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < M && col < N)
        Y[row * N + col] = __builtin_bit_cast(uint16_t, (half_t)acc[i][v]);
    }
}


template <int NWAVES>
hipError_t launch_fast(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
  using TT = Tile<NWAVES>;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + TT::BN - 1) / TT::BN;
  const int64_t tiles = tiles_m * tiles_n;
  // Load offsets (and the out-of-range marker 2^31) must fit in 31 bits.
  if (tiles > 0x7fffffff || (int64_t)BM * K * 2 >= ((int64_t)1 << 31) ||
      (int64_t)TT::BN * (K / 32 * 34) >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  const hipError_t e = ensure_max_lds<gemm_q8_0_kernel<NWAVES>>(TT::kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_q8_0_kernel<NWAVES>, dim3((unsigned)tiles), dim3(TT::kThreads),
                     TT::kLdsBytes, stream, W, X, Y, M, N, K, (int)tiles_n);
  return hipGetLastError();
}

// Tuning override for sweeps: LQMM_TUNE_GEMM_WAVES = 7 or 8.
int env_waves_override() {
  const char *s = getenv("LQMM_TUNE_GEMM_WAVES");
  return s && *s ? atoi(s) : -1;
}

}  // namespace

hipError_t gemm_q8_0_launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M,
                            int64_t N, int64_t K, int num_cus, hipStream_t stream) {
  (void)num_cus;
  // K % 64 == 32: rows are not whole dwords per 64-k step; the kernel that
  // dequantizes each step's blocks into fp16 LDS tiles (gemm_lds.hip) takes
  // exact-size block loads and a ragged last step.
  if (K % 64 != 0) return gemm_lds_launch(GemmFormat::Q8_0, W, X, Y, M, N, K, stream);
  // Eight waves (128 x 256 tiles). Seven (128 x 224) fill more CUs at some
  // shapes (512 x 14336: 256 tiles instead of 224), but a seven-wave tile
  // takes as long as an eight-wave one (three of its SIMDs still run two
  // waves) and measured slower there; it stays available as a tuning
  // override (LQMM_TUNE_GEMM_WAVES = 7).
  const bool seven = env_waves_override() == 7;
  return seven ? launch_fast<7>(W, X, Y, M, N, K, stream) : launch_fast<8>(W, X, Y, M, N, K, stream);
}

}  // namespace lqmm

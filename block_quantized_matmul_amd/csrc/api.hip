// C entry points of liblqmm: argument validation, launch planning, dispatch.
// Every check runs on the host before the first HIP call; the only HIP calls
// are the per-device property query (cached) and the kernel launches.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdlib.h>
#include <string.h>

#include "lqmm.h"
#include "lqmm_internal.hpp"

namespace {

// Split-K workspace of the allocation-free GEMV entry point: a static
// device array, one copy per GPU, zero-initialized when the code object is
// loaded and kept until the process ends. In host code `scratch` is only a
// stand-in symbol; its device address on each GPU comes from
// hipGetSymbolAddress (below) and only that address is ever passed on.
constexpr size_t kScratchBytes = LQMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceInfo {
  std::once_flag once;
  bool ok = false;
  int num_cus = 0;
  void *scratch_ptr = nullptr;  // this device's copy of `scratch`
};
DeviceInfo g_dev[lqmm::kMaxDevices];

// Current device, checked to be gfx950; CU count and the device address of
// the static scratch array cached per device (set up once, with the device
// current).
lqmm_status current_device(int *num_cus, void **scratch_ptr = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= lqmm::kMaxDevices) return LQMM_ERR_DEVICE;
  DeviceInfo &di = g_dev[dev];
  std::call_once(di.once, [&]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
    di.scratch_ptr = p;
    di.num_cus = prop.multiProcessorCount;
    di.ok = di.num_cus > 0;
  });
  if (!di.ok) return LQMM_ERR_DEVICE;
  *num_cus = di.num_cus;
  if (scratch_ptr) *scratch_ptr = di.scratch_ptr;
  return LQMM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool dim_ok(int64_t v) { return v > 0 && v <= LQMM_MAX_DIM; }

// Optional tuning override (benchmark sweeps only): integer env var or -1.
int env_int(const char *name) {
  const char *s = getenv(name);
  if (!s || !*s) return -1;
  return atoi(s);
}

// ---- small problems -----------------------------------------------------------
// The latency-bound kernel takes problems of at most this many 64-weight
// units (4096 x 4096 Q4_0: 262,144 units, 9.4 MB) at up to four activation
// rows: there the whole matrix is a few memory round trips' worth of data.
constexpr int64_t kSmallMaxUnits = 262144;
// Activation rows it takes by default; up to kSmallMaxBatch when forced
// (LQMM_TUNE_GEMV_SMALL=1). Measured at 4096 x 4096 Q4_0: batch 1 5.75 ->
// 5.54 us against the kernels below, batch 4 6.7 -> 10.3 us (the dot2 work
// grows with the rows; the matrix cores take it from three rows up).
constexpr int kSmallBatch = 2;
constexpr int kSmallMaxBatch = 4;
constexpr size_t kWsAlign = 256;

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Plan the small-problem kernel for one pass of B <= 4 activation rows.
// Slices: the fewest (a power of two) that let one wave cover a row slice
// (at most 64 lanes x U units); LQMM_TUNE_GEMV_SPLITK forces more. Waves per
// workgroup: the most (4, 2, 1) that still give every CU a workgroup.
// Returns false when the problem is not small (or the override disables the
// kernel); the workspace the plan needs is *ws_need (0 for one slice).
// Formats that run on the small-problem kernel only (at any size).
bool small_only(lqmm::GemvFormat f) {
  using lqmm::GemvFormat;
  return f == GemvFormat::Q8_0 || f == GemvFormat::Q6_K || f == GemvFormat::Q2_K ||
         f == GemvFormat::I4G32 || f == GemvFormat::Q1_0;
}

// Bytes per row of N x K weights in format f.
int64_t gemv_row_bytes(lqmm::GemvFormat f, int64_t K) {
  using lqmm::GemvFormat;
  switch (f) {
    case GemvFormat::Q4_0:
    case GemvFormat::Q4_0x2: return K / 32 * 18;
    case GemvFormat::Q4_K: return K / 256 * 144;
    case GemvFormat::Q8_0: return K / 32 * 34;
    case GemvFormat::Q6_K: return K / 256 * 210;
    case GemvFormat::Q2_K: return K / 256 * 84;
    case GemvFormat::I4G32: return K / 2;
    case GemvFormat::Q1_0: return K / 32 * 6;
  }
  return 0;
}

bool plan_small(lqmm::GemvFormat fmt, int64_t N, int64_t K, int B, int num_cus,
                lqmm::SmallGemvPlan *pl, size_t *ws_need) {
  using lqmm::GemvFormat;
  const int env_small = env_int("LQMM_TUNE_GEMV_SMALL");
  const int env_splitk = env_int("LQMM_TUNE_GEMV_SPLITK");
  const int env_u = env_int("LQMM_TUNE_GEMV_SMALL_U");
  const int env_nw = env_int("LQMM_TUNE_GEMV_SMALL_WAVES");
  const bool only = small_only(fmt);
  if (!only && (env_small == 0 || B > (env_small == 1 ? kSmallMaxBatch : kSmallBatch)))
    return false;
  if (B < 1 || B > kSmallMaxBatch) return false;
  const GemvFormat f = fmt == GemvFormat::Q4_0 && K % 64 == 0 ? GemvFormat::Q4_0x2 : fmt;
  const int uw = lqmm::gemv_unit_weights(f);
  const int64_t nu64 = K / uw;
  if (!only && env_small != 1 && N * (K / 64) > kSmallMaxUnits) return false;
  if (nu64 > (1 << 24)) return false;
  const int nu = (int)nu64;
  // slices start on super-blocks: Q4_K (4 units each), Q6_K and Q2_K (2)
  const int step = f == GemvFormat::Q4_K ? 4 : (f == GemvFormat::Q6_K || f == GemvFormat::Q2_K) ? 2 : 1;
  // Units per lane: one; for the formats that run here at any size, two when
  // that saves a split-K pass over a large matrix (4 * num_cus rows or more).
  int U = env_u == 2 ? 2 : 1;
  if (env_u != 1 && env_u != 2 && only && nu > 64 && nu <= 128 && N >= 4 * (int64_t)num_cus) U = 2;
  auto slice_units = [&](int S) {
    int n = (nu + S - 1) / S;
    return (n + step - 1) / step * step;
  };
  int S = 1;
  while (slice_units(S) > 64 * U) S *= 2;
  if (env_splitk > S) S = env_splitk;
  int nus = slice_units(S);
  S = (nu + nus - 1) / nus;  // slices actually covered
  int lpr_log2 = 0;
  while ((1 << lpr_log2) * U < nus) ++lpr_log2;
  const int rows_per_wave = 64 >> lpr_log2;
  const size_t lds = lqmm::gemv_small_lds_bytes(f, B, nus);
  if (lds > lqmm::gemv_small_max_lds()) return false;
  auto blocks = [&](int nw) { return (N + (int64_t)rows_per_wave * nw - 1) / ((int64_t)rows_per_wave * nw); };
  // The widest workgroups that still leave a quarter of the CUs one: each
  // workgroup stages its x slice once, so wider ones move less from L2, and
  // these problems are bound by latency, not by the CUs' load bandwidth.
  // Measured at batch 1: 4096 x 4096 with 4096 one-wave workgroups 7.6 us,
  // 2048 two-wave 6.1, 1024 four-wave 5.5, 512 eight-wave 5.35, 256
  // sixteen-wave 5.15; 1024 x 1024 with 256 one-wave workgroups 3.9-4.2 us,
  // 64 four-wave 3.66, 32 eight-wave 3.75. 8 and 16 waves for one unit per
  // lane at one or two rows.
  const bool wide = B <= 2;
  int nw = 1;
  for (int c : {16, 8, 4, 2}) {
    if ((c <= 4 || wide) && blocks(c) * S * 4 >= num_cus) {
      nw = c;
      break;
    }
  }
  if (env_nw == 1 || env_nw == 2 || env_nw == 4 || (wide && (env_nw == 8 || env_nw == 16)))
    nw = env_nw;
  const int64_t rb = blocks(nw);
  if (rb * S > 0x7fffffff) return false;
  pl->f = f;
  pl->batch = B;
  pl->units_per_lane = U;
  pl->lpr_log2 = lpr_log2;
  pl->slices = S;
  pl->nu = nu;
  pl->nus = nus;
  pl->waves = nw;
  pl->row_blocks = (int)rb;
  pl->grid = (int)(rb * S);
  pl->lds_bytes = lds;
  pl->row_bytes = gemv_row_bytes(f, K);
  pl->N = N;
  // counters (one int per row block), then S * B * N partial sums
  *ws_need = S == 1 ? 0 : align_up((size_t)rb * 4) + (size_t)S * B * (size_t)N * 4;
  return true;
}

// static_ws: ws is the device's static scratch (allocation-free entry
// point): a split-K plan that needs more than it holds is refused, and the
// plan's counters are zeroed by a kernel before each split-K launch.
lqmm_status gemv_common(lqmm::GemvFormat fmt, const void *W, const float *x, float *y,
                        int64_t N, int64_t K, int64_t batch, void *ws, size_t ws_bytes,
                        hipStream_t stream, bool static_ws = false) {
  using lqmm::GemvFormat;
  const int blk = fmt == GemvFormat::Q4_0 ? 32 : 256;
  const int blk_bytes = fmt == GemvFormat::Q4_0 ? 18 : 144;
  if (!W || !x || !y) return LQMM_ERR_NULL;
  if (!dim_ok(N) || !dim_ok(K) || !dim_ok(batch) || K % blk != 0) return LQMM_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(x) || !aligned16(y)) return LQMM_ERR_ALIGN;
  if (ws && !aligned16(ws)) return LQMM_ERR_ALIGN;

  int num_cus = 0;
  void *scratch_ptr = nullptr;
  lqmm_status st = current_device(&num_cus, &scratch_ptr);
  if (st != LQMM_OK) return st;
  if (static_ws) {
    ws = scratch_ptr;
    ws_bytes = kScratchBytes;
  }

  // Small problems (all rows in passes of at most four): the latency-bound
  // kernel, when its split-K workspace (if it needs one) is there.
  if (batch <= kSmallMaxBatch) {  // (plan_small applies the default limit)
    lqmm::SmallGemvPlan sp;
    size_t need = 0;
    if (plan_small(fmt, N, K, (int)batch, num_cus, &sp, &need)) {
      if (need > 0 && (!ws || ws_bytes < need)) {
        if (static_ws || env_int("LQMM_TUNE_GEMV_SPLITK") > 1) return LQMM_ERR_WORKSPACE;
      } else {
        sp.ldx = K;
        sp.ldy = N;
        int *cnt = need ? static_cast<int *>(ws) : nullptr;
        float *part = need ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                       align_up((size_t)sp.row_blocks * 4))
                           : nullptr;
        if (need && static_ws) {
          hipError_t e = lqmm::gemv_small_clear_counters(cnt, sp.row_blocks, stream);
          if (e != hipSuccess) return LQMM_ERR_LAUNCH;
        }
        hipError_t e = lqmm::gemv_small_launch(sp, static_cast<const uint8_t *>(W), x, y, part,
                                               cnt, stream);
        return e == hipSuccess ? LQMM_OK : LQMM_ERR_LAUNCH;
      }
    }
  }

  const int64_t units_total = K / lqmm::gemv_unit_weights(fmt);
  const int64_t row_bytes = K / blk * blk_bytes;
  const int threads = lqmm::gemv_threads();
  const int waves_per_wg = threads / 64;
  const int env_r = env_int("LQMM_TUNE_GEMV_R");
  const int env_u = env_int("LQMM_TUNE_GEMV_U");
  const int env_grid = env_int("LQMM_TUNE_GEMV_GRID");
  const int env_mfma = env_int("LQMM_TUNE_GEMV_MFMA");
  const int env_wgcu = env_int("LQMM_TUNE_GEMV_WG_PER_CU");
  const int env_ks = env_int("LQMM_TUNE_GEMV_KS");
  const int env_waves = env_int("LQMM_TUNE_GEMV_WAVES");
  const int env_ldsk = env_int("LQMM_TUNE_GEMV_LDSK");
  const int env_depth = env_int("LQMM_TUNE_GEMV_DEPTH");
  const int env_pair = env_int("LQMM_TUNE_GEMV_Q4_0_PAIR");
  const int env_xregs = env_int("LQMM_TUNE_GEMV_XREGS");
  const int env_stream = env_int("LQMM_TUNE_GEMV_STREAM");
  const int env_stream_batch = env_int("LQMM_TUNE_GEMV_STREAM_BATCH");
  const int env_whole = env_int("LQMM_TUNE_GEMV_WHOLE");
  const int64_t tiles = (N + 15) / 16;  // 16-row tiles of the matrix-core kernels

  // K-slices per tile of the coalesced kernel (one workgroup per CU): the
  // number that gives each wave the fewest units, counting the last, partly
  // filled pass of workgroups over the CUs as a whole one; ties go to more
  // slices. With the activations in registers (xr), at most four
  // super-chunks per slice. Then the tuning override; every slice must hold
  // a whole chunk of uu super-chunks (uu drops to 1 for rows shorter than a
  // chunk).
  auto coal_slices = [&](int64_t nu, int &uu, bool xr, int sc_units) -> int {
    int ks = 1;
    int64_t best = -1;
    for (int k = 8; k >= 1; k /= 2) {
      if (xr && (nu / sc_units + k - 1) / k > 4) continue;
      const int64_t wgs = (tiles * k + 7) / 8;
      const int64_t grid_k = wgs < (int64_t)num_cus ? wgs : (int64_t)num_cus;
      const int64_t upc = (int64_t)sc_units * uu;  // units per chunk
      const int64_t slice = ((nu + k - 1) / k + upc - 1) / upc * upc;
      const int64_t cost = (wgs + grid_k - 1) / grid_k * slice;
      if (best < 0 || cost < best) {
        best = cost;
        ks = k;
      }
    }
    if (env_ks >= 1 && env_ks <= 8 && (env_ks & (env_ks - 1)) == 0) ks = env_ks;
    while (ks > 1 && (nu / ks) < sc_units * uu) ks /= 2;
    if (nu < sc_units * uu) uu = 1;
    while (xr && (nu / sc_units + ks - 1) / ks > 4 && ks < 8) ks *= 2;
    return ks;
  };

  for (int64_t b0 = 0; b0 < batch; ) {
    const int64_t left = batch - b0;
    // Matrix cores from three activation rows up: their cost per weight does
    // not grow with the batch, the dot2 path's does.
    bool mfma = left >= 3;
    if (env_mfma == 0 || env_mfma == 1) mfma = env_mfma == 1;
    // VALU-mode Q4_0 takes two blocks per unit when K % 64 == 0: 36-byte,
    // 4-byte-aligned loads instead of an 18-byte block per lane. Measured:
    // faster when there are more rows than one workgroup per CU covers (a
    // wave per two rows), slower with only one workgroup per CU.
    const int64_t rows_one_wg_per_cu = (int64_t)num_cus * waves_per_wg * 2;
    auto pair_for = [&](bool valu) {
      if (env_pair == 0 || env_pair == 1)
        return fmt == GemvFormat::Q4_0 && valu && K % 64 == 0 && env_pair == 1;
      return fmt == GemvFormat::Q4_0 && valu && K % 64 == 0 && N > rows_one_wg_per_cu;
    };
    // The kernel that streams rows through LDS (one workgroup per CU, whole
    // K in one launch) takes rows of at most 8192 weights (Q4_K) or 4096
    // (Q4_0, two blocks per unit) at up to two activation rows (the second
    // row reads its activations from LDS), when every wave gets at least two
    // weight rows. Measured on Q4_K at batch 1: 4% faster at 28672 x 8192
    // and 8% at 14336 x 4096, even at 8192 x 8192 (two rows per wave), 4%
    // slower at 4096 x 4096 (one); at batch 2 4-5% faster (Q4_K 28672 x
    // 8192, Q4_0 12288 x 4096). Overrides: LQMM_TUNE_GEMV_STREAM 0 off, 1 on
    // whatever N is; LQMM_TUNE_GEMV_STREAM_BATCH 1 or 2.
    const int64_t stream_waves_total = (int64_t)num_cus * lqmm::gemv_stream_waves();
    const GemvFormat fs = pair_for(true) ? GemvFormat::Q4_0x2 : fmt;
    int stream_batch = lqmm::gemv_stream_max_batch();
    if (env_stream_batch >= 1 && env_stream_batch <= lqmm::gemv_stream_max_batch())
      stream_batch = env_stream_batch;
    const int64_t units_s = K / lqmm::gemv_unit_weights(fs);
    const bool streamed =
        (fs == GemvFormat::Q4_K || fs == GemvFormat::Q4_0x2) && env_stream != 0 && env_mfma != 1 &&
        left <= stream_batch && units_s <= lqmm::gemv_stream_max_units(fs) &&
        (env_stream == 1 || N >= 2 * stream_waves_total) &&
        lqmm::gemv_stream_lds_bytes(fs, (int)left, (int)units_s) <= (size_t)lqmm::kMaxLds;
    if (streamed) mfma = false;
    const int bmax = mfma ? 16 : streamed ? stream_batch : 2;
    const int B = (int)(left < bmax ? left : bmax);
    // Matrix-core kernel that requests each workgroup's whole weight share at
    // once, when it fits (rows of at most 16 super-chunks, at most three
    // tiles per CU, all of x in one batch of loads). By default only at one
    // tile per CU. Measured against the coalesced kernel (cold, same
    // process): Q4_0 4096 x 4096 batch 4 6.50 -> 5.92 us with it;
    // 11008 and 12288 x 4096 batch 4 (three tiles per CU) 11.1 and 11.5 us
    // against 10.4 and 10.7 us, slower. LQMM_TUNE_GEMV_WHOLE: 0 off, 1 on
    // wherever it fits.
    const bool whole_default = tiles <= (int64_t)num_cus;
    if (mfma && env_whole != 0 && (env_whole == 1 || whole_default) &&
        (fmt == GemvFormat::Q4_0 || fmt == GemvFormat::Q4_K) &&
        K % 256 == 0 && 16 * row_bytes < ((int64_t)1 << 31)) {
      const int64_t nsc = K / 256;
      const int ks = 8;
      const int cps = (int)((nsc + ks - 1) / ks);
      const int64_t nu = K / lqmm::gemv_unit_weights(fmt);
      const int64_t grid = tiles < num_cus ? tiles : num_cus;
      const int64_t maxt = (tiles + grid - 1) / grid;
      if (cps <= 2 && maxt <= 3 && (int64_t)B * nu * (fmt == GemvFormat::Q4_K ? 8 : 4) <=
                                       lqmm::gemv_whole_max_words() &&
          lqmm::gemv_whole_lds_bytes(fmt, cps, (int)maxt, (int)nu, B) <= (size_t)lqmm::kMaxLds) {
        lqmm::GemvPlan pw{};
        pw.mfma = 1;
        pw.batch = B;
        pw.ksplit = ks;
        pw.cps = cps;
        pw.depth = (int)maxt;
        pw.grid = (int)grid;
        pw.row_bytes = row_bytes;
        pw.ldx = K;
        pw.ldy = N;
        pw.N = N;
        hipError_t e = lqmm::gemv_whole_launch(fmt, pw, static_cast<const uint8_t *>(W),
                                               x + b0 * K, y + b0 * N, stream);
        if (e != hipSuccess) return LQMM_ERR_LAUNCH;
        b0 += B;
        continue;
      }
    }
    const GemvFormat f = streamed ? fs : pair_for(!mfma) ? GemvFormat::Q4_0x2 : fmt;
    const int uw = lqmm::gemv_unit_weights(f);
    const int64_t units = K / uw;
    // MFMA mode uses the coalesced kernel (loads staged through LDS, 8
    // waves) when rows are whole 256-weight super-chunks of 144 bytes and a
    // 16-row tile spans less than 2 GiB (32-bit load offsets); otherwise, or
    // when disabled for tuning, the MFMA-layout kernel.
    const int sc_units = fmt == GemvFormat::Q4_K ? 4 : 8;  // units per super-chunk
    const bool lds_stage = mfma && env_ldsk != 0 && units_total % sc_units == 0 &&
                           16 * row_bytes < ((int64_t)1 << 31);
    // Its variant with the activations in registers takes the whole K in one
    // launch when k-slices of at most four super-chunks cover a row (up to 32
    // super-chunks, with eight slices) and a slice's activations fit in one
    // wave's chunk ring for staging. Measured: faster when every wave
    // computes at least 12 chunks (Q4_K 28672 x 8192 at 8 rows: 28), slower
    // below about 6 (its per-wave staging comes before the first chunk
    // request).
    bool xregs = lds_stage && env_xregs != 0 && units_total / sc_units <= 32;
    if (xregs) {
      int uu1 = 1;
      const int ks = coal_slices(units, uu1, true, sc_units);
      const int64_t cps = (units / sc_units + ks - 1) / ks;
      xregs = lqmm::gemv_coalr_fits(fmt, (int)cps, B);
      const int64_t wgs = (tiles * ks + 7) / 8;
      const int64_t grid = wgs < (int64_t)num_cus ? wgs : (int64_t)num_cus;
      const int64_t tiles_per_wave = (tiles + grid * (8 / ks) - 1) / (grid * (8 / ks));
      if (env_xregs != 1) xregs = xregs && tiles_per_wave * cps >= 12;
    }
    // Other MFMA launches: 16-wave workgroups when the staged activations
    // leave room for only one workgroup per CU, so that more loads are in
    // flight.
    int waves = 8;
    if (mfma && !lds_stage) {
      const int64_t per_unit = (int64_t)lqmm::gemv_lds_bytes(fmt, true, B, 1);
      if (per_unit * units_total > 80 * 1024) waves = 16;
      if (env_waves == 8 || env_waves == 16) waves = env_waves;
    }
    // One super-chunk per row per chunk, two for large N at up to six
    // activation rows (long K-slices; the staged activations leave room).
    const int lds_u = xregs ? 1
                      : lds_stage ? ((env_u == 1 || env_u == 2)
                                       ? env_u
                                       : (B <= 6 && N > 6 * 16 * (int64_t)num_cus ? 2 : 1))
                                : 0;
    // LDS beyond the staged activations: the coalesced kernel's per-wave
    // weight staging areas (its k-split reduction reuses them), or the other
    // MFMA kernel's reduction buffer.
    const int64_t red_bytes =
        !mfma ? 0
              : lds_stage ? (int64_t)lqmm::gemv_coal_stage_bytes(lds_u)
                          : (int64_t)lqmm::gemv_mfma_reduce_bytes(waves);
    const int64_t lds_cap = lds_stage ? lqmm::kMaxLds : lqmm::kMaxGemvLds;
    // per-unit cost taken over many units, where the row padding is negligible
    int64_t max_units = units;
    if (!xregs && !streamed) {
      max_units = (lds_cap - red_bytes) * 4096 / (int64_t)lqmm::gemv_lds_bytes(f, mfma, B, 4096);
      // K-split launches start on whole Q4_K super-blocks, and on whole
      // super-chunks for the coalesced kernel.
      const int64_t ustep = lds_stage ? sc_units : fmt == GemvFormat::Q4_K ? 4 : 1;
      max_units -= max_units % ustep;
      // the staged rows are padded: step back until they fit
      while (max_units > ustep &&
             (int64_t)lqmm::gemv_lds_bytes(f, mfma, B, (int)max_units) + red_bytes > lds_cap)
        max_units -= ustep;
      if (max_units < ustep) return LQMM_ERR_SHAPE;
    }
    for (int64_t u0 = 0; u0 < units; u0 += max_units) {
      const int64_t nu64 = units - u0 < max_units ? units - u0 : max_units;
      const int nu = (int)nu64;
      lqmm::GemvPlan pl;
      pl.mfma = mfma;
      pl.batch = B;
      int lpr_log2 = 0;
      while ((1 << lpr_log2) < nu && lpr_log2 < 6) ++lpr_log2;
      pl.lpr_log2 = lpr_log2;
      pl.lds_bytes = xregs    ? lqmm::gemv_coalr_lds_bytes()
                     : streamed ? lqmm::gemv_stream_lds_bytes(f, B, nu)
                              : lqmm::gemv_lds_bytes(f, mfma, B, nu) + red_bytes;
      int64_t wg_per_cu = (int64_t)(160 * 1024) / (int64_t)(pl.lds_bytes ? pl.lds_bytes : 1);
      // The coalesced kernel runs one workgroup per CU: each workgroup stages
      // all of x, so more workgroups mostly add staging traffic.
      const int64_t wg_cap = env_wgcu > 0 ? env_wgcu : (lds_stage || streamed ? 1 : 2);
      if (wg_per_cu > wg_cap) wg_per_cu = wg_cap;
      if (wg_per_cu < 1) wg_per_cu = 1;
      int64_t wg_needed;
      if (mfma) {
        // R = 1 tile of 16 rows per team; KS waves share a tile along K so
        // that small N still gives every CU several waves.
        int uu = lds_stage ? lds_u : 2, ks = waves == 16 ? 4 : 1;
        const int ksmax = waves == 16 ? 16 : 8;
        if (lds_stage) {
          ks = coal_slices(nu, uu, xregs, sc_units);
        } else {
          while (ks < ksmax && tiles * ks < (int64_t)num_cus * 8 && nu >= 2 * ks * 4 * uu) ks *= 2;
          if (env_u == 2 || env_u == 4) uu = env_u;
          if (env_ks >= (waves == 16 ? 4 : 1) && env_ks <= ksmax && (env_ks & (env_ks - 1)) == 0)
            ks = env_ks;
        }
        pl.rows_per_lane = 1;
        pl.units_per_lane = uu;
        pl.ksplit = ks;
        pl.waves = waves;
        pl.lds_stage = lds_stage;
        pl.xregs = xregs;
        pl.cps = xregs ? (nu / sc_units + ks - 1) / ks : 0;
        pl.stream = 0;
        pl.depth = (env_depth == 2 || env_depth == 3 || env_depth == 4 || env_depth == 6) ? env_depth : 2;
        const int teams = waves / ks;
        wg_needed = (tiles + teams - 1) / teams;
      } else {
        const int slots = 64 >> lpr_log2;
        // Rows per lane R and units per lane per chunk U.
        int r = 2, uu = 1;
        if (env_r == 1 || env_r == 2) r = env_r;
        if (env_u == 1 || env_u == 2 || env_u == 4) uu = env_u;
        if (r == 1 && uu == 1) uu = 2;
        if (r == 2 && uu == 4) uu = 2;
        pl.rows_per_lane = r;
        pl.units_per_lane = uu;
        pl.ksplit = 1;
        pl.waves = waves_per_wg;
        pl.lds_stage = 0;
        pl.xregs = 0;
        pl.cps = 0;
        pl.depth = 2;
        pl.stream = streamed;
        // the streamed kernel: one row per wave at a time
        const int64_t groups = streamed ? N : (N + (int64_t)slots * r - 1) / ((int64_t)slots * r);
        const int wpw = streamed ? lqmm::gemv_stream_waves() : waves_per_wg;
        wg_needed = (groups + wpw - 1) / wpw;
      }
      pl.nu = nu;
      pl.unit0 = u0;
      pl.row_bytes = row_bytes;
      pl.ldx = K;
      pl.ldy = N;
      pl.N = N;
      // Persistent grid: at most wg_per_cu workgroups per CU, no more than
      // there is work for.
      int64_t grid = wg_needed < num_cus * wg_per_cu ? wg_needed : num_cus * wg_per_cu;
      if (env_grid > 0) grid = env_grid;
      pl.grid = (int)grid;
      pl.accumulate = u0 > 0;
      const uint8_t *Wb = static_cast<const uint8_t *>(W);
      hipError_t e = lqmm::gemv_launch(f, pl, Wb, x + b0 * K + u0 * uw, y + b0 * N, stream);
      if (e != hipSuccess) return LQMM_ERR_LAUNCH;
    }
    b0 += B;
  }
  return LQMM_OK;
}

// GEMV over the formats that run on the small-problem kernel only: passes of
// up to four activation rows; split-K plans (rows longer than one wave's
// slice) need the workspace.
lqmm_status gemv_more(lqmm::GemvFormat f, int blk, const void *W, const float *aux_a,
                      const float *aux_b, const float *x, float *y, int64_t N, int64_t K,
                      int64_t batch, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!W || !x || !y) return LQMM_ERR_NULL;
  if (f == lqmm::GemvFormat::I4G32 && (!aux_a || !aux_b)) return LQMM_ERR_NULL;
  if (!dim_ok(N) || !dim_ok(K) || !dim_ok(batch) || K % blk != 0) return LQMM_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(x) || !aligned16(y)) return LQMM_ERR_ALIGN;
  if (aux_a && (!aligned16(aux_a) || !aligned16(aux_b))) return LQMM_ERR_ALIGN;
  if (ws && !aligned16(ws)) return LQMM_ERR_ALIGN;
  int num_cus = 0;
  lqmm_status st = current_device(&num_cus);
  if (st != LQMM_OK) return st;
  for (int64_t b0 = 0; b0 < batch; b0 += kSmallMaxBatch) {
    const int B = (int)(batch - b0 < kSmallMaxBatch ? batch - b0 : kSmallMaxBatch);
    lqmm::SmallGemvPlan sp;
    size_t need = 0;
    if (!plan_small(f, N, K, B, num_cus, &sp, &need)) return LQMM_ERR_SHAPE;
    if (need > 0 && (!ws || ws_bytes < need)) return LQMM_ERR_WORKSPACE;
    sp.ldx = K;
    sp.ldy = N;
    sp.aux_a = aux_a;
    sp.aux_b = aux_b;
    sp.aux_groups = K / 32;
    int *cnt = need ? static_cast<int *>(ws) : nullptr;
    float *part = need ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                   align_up((size_t)sp.row_blocks * 4))
                       : nullptr;
    hipError_t e = lqmm::gemv_small_launch(sp, static_cast<const uint8_t *>(W), x + b0 * K,
                                           y + b0 * N, part, cnt, stream);
    if (e != hipSuccess) return LQMM_ERR_LAUNCH;
  }
  return LQMM_OK;
}

}  // namespace

extern "C" {

lqmm_status lqmm_sgemm(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
                       void *stream) {
  if (!A || !B || !C) return LQMM_ERR_NULL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return LQMM_ERR_SHAPE;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return LQMM_ERR_ALIGN;
  int num_cus = 0;
  lqmm_status st = current_device(&num_cus);
  if (st != LQMM_OK) return st;
  hipError_t e = lqmm::sgemm_launch(A, B, C, M, N, K, num_cus, (hipStream_t)stream);
  return e == hipSuccess ? LQMM_OK : LQMM_ERR_LAUNCH;
}

lqmm_status lqmm_gemv_q4_0(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_common(lqmm::GemvFormat::Q4_0, W, x, y, N, K, batch, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

lqmm_status lqmm_gemv_q4_0_noalloc(const void *W, const float *x, float *y, int64_t N,
                                   int64_t K, int64_t batch, void *stream) {
  return gemv_common(lqmm::GemvFormat::Q4_0, W, x, y, N, K, batch, nullptr, 0,
                     (hipStream_t)stream, true);
}

lqmm_status lqmm_gemv_q4_k(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_common(lqmm::GemvFormat::Q4_K, W, x, y, N, K, batch, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

lqmm_status lqmm_gemv_q8_0(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_more(lqmm::GemvFormat::Q8_0, 32, W, nullptr, nullptr, x, y, N, K, batch, workspace,
                   workspace_bytes, (hipStream_t)stream);
}

lqmm_status lqmm_gemv_q6_k(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_more(lqmm::GemvFormat::Q6_K, 256, W, nullptr, nullptr, x, y, N, K, batch, workspace,
                   workspace_bytes, (hipStream_t)stream);
}

lqmm_status lqmm_gemv_q2_k(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_more(lqmm::GemvFormat::Q2_K, 256, W, nullptr, nullptr, x, y, N, K, batch, workspace,
                   workspace_bytes, (hipStream_t)stream);
}

lqmm_status lqmm_gemv_q1_0(const void *W, const float *x, float *y, int64_t N, int64_t K,
                           int64_t batch, void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_more(lqmm::GemvFormat::Q1_0, 32, W, nullptr, nullptr, x, y, N, K, batch, workspace,
                   workspace_bytes, (hipStream_t)stream);
}

lqmm_status lqmm_gemv_i4g32(const uint32_t *Wq, const float *scales, const float *zeros,
                            const float *x, float *y, int64_t N, int64_t K, int64_t batch,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return gemv_more(lqmm::GemvFormat::I4G32, 32, Wq, scales, zeros, x, y, N, K, batch, workspace,
                   workspace_bytes, (hipStream_t)stream);
}

lqmm_status lqmm_gemm_q8_0_f16(const void *W, const uint16_t *X, uint16_t *Y, int64_t M,
                               int64_t N, int64_t K, void *stream) {
  if (!W || !X || !Y) return LQMM_ERR_NULL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || K % 32 != 0) return LQMM_ERR_SHAPE;
  if (K >= LQMM_GEMM_MAX_K) return LQMM_ERR_SHAPE;  // 31-bit load offsets within a tile
  if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return LQMM_ERR_ALIGN;
  int num_cus = 0;
  lqmm_status st = current_device(&num_cus);
  if (st != LQMM_OK) return st;
  hipError_t e = lqmm::gemm_q8_0_launch(static_cast<const uint8_t *>(W), X, Y, M, N, K, num_cus,
                                        (hipStream_t)stream);
  return e == hipSuccess ? LQMM_OK : LQMM_ERR_LAUNCH;
}

static lqmm_status gemm_lds_common(lqmm::GemmFormat f, int blk, const void *W, const uint16_t *X,
                                   uint16_t *Y, int64_t M, int64_t N, int64_t K, void *stream) {
  if (!W || !X || !Y) return LQMM_ERR_NULL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || K % blk != 0) return LQMM_ERR_SHAPE;
  if (K >= LQMM_GEMM_MAX_K) return LQMM_ERR_SHAPE;  // 31-bit load offsets within a tile
  if (!aligned16(W) || !aligned16(X) || !aligned16(Y)) return LQMM_ERR_ALIGN;
  int num_cus = 0;
  lqmm_status st = current_device(&num_cus);
  if (st != LQMM_OK) return st;
  hipError_t e = lqmm::gemm_lds_launch(f, static_cast<const uint8_t *>(W), X, Y, M, N, K,
                                       (hipStream_t)stream);
  return e == hipSuccess ? LQMM_OK : LQMM_ERR_LAUNCH;
}

lqmm_status lqmm_gemm_q4_0_f16(const void *W, const uint16_t *X, uint16_t *Y, int64_t M,
                               int64_t N, int64_t K, void *stream) {
  return gemm_lds_common(lqmm::GemmFormat::Q4_0, 32, W, X, Y, M, N, K, stream);
}

lqmm_status lqmm_gemm_q4_k_f16(const void *W, const uint16_t *X, uint16_t *Y, int64_t M,
                               int64_t N, int64_t K, void *stream) {
  return gemm_lds_common(lqmm::GemmFormat::Q4_K, 256, W, X, Y, M, N, K, stream);
}

size_t lqmm_gemv_workspace_bytes(int64_t N, int64_t K, int64_t batch) {
  // The largest need of any GEMV format's call of these sizes (passes of at
  // most four activation rows), for the most row blocks any device's plan
  // can have.
  if (!dim_ok(N) || !dim_ok(K) || !dim_ok(batch)) return 0;
  using lqmm::GemvFormat;
  size_t best = 0;
  for (GemvFormat f : {GemvFormat::Q4_0, GemvFormat::Q4_K, GemvFormat::Q8_0, GemvFormat::Q6_K,
                       GemvFormat::Q2_K, GemvFormat::I4G32, GemvFormat::Q1_0}) {
    const int blk = (f == GemvFormat::Q4_K || f == GemvFormat::Q6_K || f == GemvFormat::Q2_K) ? 256 : 32;
    if (K % blk != 0) continue;
    const int64_t B = small_only(f) && batch > kSmallMaxBatch ? kSmallMaxBatch : batch;
    if (B > kSmallMaxBatch) continue;
    lqmm::SmallGemvPlan sp;
    size_t need = 0;
    if (plan_small(f, N, K, (int)B, 1 << 30, &sp, &need) && need > best) best = need;
  }
  return best;
}

const char *lqmm_status_string(int s) {
  switch (s) {
    case LQMM_OK: return "LQMM_OK";
    case LQMM_ERR_NULL: return "LQMM_ERR_NULL: a required pointer is NULL";
    case LQMM_ERR_SHAPE: return "LQMM_ERR_SHAPE: a size is out of range or not a block multiple";
    case LQMM_ERR_ALIGN: return "LQMM_ERR_ALIGN: a pointer is not 16-byte aligned";
    case LQMM_ERR_WORKSPACE: return "LQMM_ERR_WORKSPACE: the call needs a larger workspace";
    case LQMM_ERR_DEVICE: return "LQMM_ERR_DEVICE: no usable gfx950 device";
    case LQMM_ERR_LAUNCH: return "LQMM_ERR_LAUNCH: kernel launch failed";
  }
  return "LQMM: unknown status";
}

int lqmm_version(void) { return 100; }

}  // extern "C"

// Host-side interface between the C entry points (api.hip) and the kernel
// translation units. Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace lqmm {

// Devices the per-device state below covers (device ids 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;

// Raise kernel KERN's dynamic-LDS limit to `bytes`, once per device and
// kernel instance, thread-safe (std::call_once per device); later calls
// return the first call's result. KERN is a template argument so that every
// kernel instance has its own flags.
template <auto KERN>
hipError_t ensure_max_lds(int bytes) {
  struct PerDevice {
    std::once_flag once;
    hipError_t err = hipSuccess;
  };
  static PerDevice state[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return hipErrorInvalidDevice;
  PerDevice &d = state[dev];
  std::call_once(d.once, [&]() {
    d.err = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return d.err;
}

// ---- GEMV -------------------------------------------------------------------
// Q4_0x2: Q4_0 weights taken two blocks (64 weights, 36 bytes) per unit, used
// by the VALU-mode kernel when K % 64 == 0.
// Q8_0, Q6_K, Q2_K, I4G32 (the int4 group-32 layout) and Q1_0 (1-bit codes)
// run on the small-problem kernel only.
enum class GemvFormat { Q4_0, Q4_K, Q4_0x2, Q8_0, Q6_K, Q2_K, I4G32, Q1_0 };

// Largest dynamic LDS one GEMV launch may use (staged activations + sums).
constexpr int kMaxGemvLds = 144 * 1024;

struct GemvPlan {
  int mfma;           // 1: matrix-core mode (batch up to 16), 0: VALU dot2 mode (batch 1 or 2)
  int batch;          // activation rows in this launch
  int rows_per_lane;  // 1, 2 or 4
  int units_per_lane; // units each lane loads per chunk: VALU (R, U) in {(1,2),(1,4),(2,1),(2,2)}
  int ksplit;         // MFMA mode: waves sharing one tile along K (1..8; 4..16 with 16 waves)
  int waves;          // MFMA mode: waves per workgroup (8 or 16)
  int lds_stage;      // MFMA mode: coalesced loads staged through LDS (8 waves; units_per_lane = U
                      // super-chunks of 256 weights per row per chunk)
  int depth;          // lds_stage: chunks in flight per wave (2, 3, 4 or 6)
  int xregs;          // lds_stage: activations in registers (whole K in one launch, U = 1)
  int cps;            // xregs: super-chunks per k-slice (1..4)
  int stream;         // VALU mode, Q4_K or Q4_0x2: the kernel that streams rows through LDS
                      // (batch 1 or 2, whole K in one launch)
  int lpr_log2;       // log2(lanes sharing one weight row)
  int nu;             // units (of gemv_unit_weights weights) per row in this launch
  int64_t unit0;      // first unit of each row covered by this launch
  int64_t row_bytes;  // bytes per weight row
  int64_t ldx, ldy;   // row strides of x and y, in elements
  int64_t N;          // weight rows
  int grid;           // workgroups
  size_t lds_bytes;   // dynamic LDS
  int accumulate;     // 1: y += result
};

size_t gemv_lds_bytes(GemvFormat f, bool mfma, int batch, int nu);
size_t gemv_mfma_reduce_bytes(int waves);  // extra LDS of an MFMA-mode launch
size_t gemv_coal_stage_bytes(int u);        // per-workgroup staging of the coalesced MFMA kernel
size_t gemv_coalr_lds_bytes();              // LDS of the coalesced kernel with activations in registers
size_t gemv_stream_lds_bytes(GemvFormat f, int batch, int nu);  // LDS of the streamed kernel
int gemv_stream_max_batch();                      // the most activation rows it takes
int gemv_stream_waves();                          // its waves per workgroup
int gemv_stream_max_units(GemvFormat f);          // the longest row it takes, in 64-weight units
// whether a k-slice of cps super-chunks of `batch` activation rows can be
// staged in one wave's chunk ring (the activations-in-registers kernel)
bool gemv_coalr_fits(GemvFormat f, int cps, int batch);
constexpr int kMaxLds = 160 * 1024;         // LDS per workgroup on gfx950
int gemv_unit_weights(GemvFormat f);
int gemv_threads();
hipError_t gemv_launch(GemvFormat f, const GemvPlan &plan, const uint8_t *W, const float *x,
                       float *y, hipStream_t stream);

// Matrix-core kernel that requests each workgroup's whole weight share at
// once (gemv_whole.hip): Q4_0 or Q4_K rows of whole 256-weight super-chunks,
// `ksplit` waves per 16-row tile (cps super-chunks each, ksplit * cps
// covering the row), one tile per workgroup at a time and `depth` tiles per
// workgroup (1..3), all of x staged (at most gemv_whole_max_words() words).
// Uses plan fields batch, row_bytes, ldx, ldy, N, grid, ksplit, cps, depth.
size_t gemv_whole_lds_bytes(GemvFormat f, int cps, int maxt, int nu, int nb);
int gemv_whole_max_words();
int gemv_whole_waves();
hipError_t gemv_whole_launch(GemvFormat f, const GemvPlan &plan, const uint8_t *W, const float *x,
                             float *y, hipStream_t stream);

// Latency-bound kernel for small problems (gemv_small.hip): one workgroup of
// `waves` waves per (row block, K slice); each lane takes units_per_lane
// units of its row's slice; slices > 1 splits K across workgroups (partial
// sums in a workspace, fixed-order reduction by the last arrival).
struct SmallGemvPlan {
  GemvFormat f;       // Q4_0, Q4_0x2 or Q4_K
  int batch;          // activation rows (1..4)
  int units_per_lane; // 1 or 2
  int lpr_log2;       // log2(lanes per row)
  int slices;         // K slices (workgroups per row block)
  int nu;             // units per row
  int nus;            // units per slice
  int waves;          // waves per workgroup: 1, 2 or 4
  int grid;           // workgroups = row blocks * slices
  int row_blocks;
  size_t lds_bytes;
  int64_t row_bytes, ldx, ldy, N;
  // per-group arrays of formats that keep them apart (I4G32: scales, zeros)
  const float *aux_a = nullptr, *aux_b = nullptr;
  int64_t aux_groups = 0;  // groups per row
};
size_t gemv_small_lds_bytes(GemvFormat f, int batch, int nus);
// the further formats' instances (gemv_small_more.hip)
size_t gemv_small_lds_bytes_more(GemvFormat f, int batch, int nus);
hipError_t gemv_small_launch_more(const SmallGemvPlan &plan, const uint8_t *W, const float *x,
                                  float *y, float *partials, int *counters, hipStream_t stream);
size_t gemv_small_max_lds();  // the most dynamic LDS a small-kernel plan may use
hipError_t gemv_small_launch(const SmallGemvPlan &plan, const uint8_t *W, const float *x, float *y,
                             float *partials, int *counters, hipStream_t stream);
// Zero the first n arrival counters of a workspace (a kernel launch).
hipError_t gemv_small_clear_counters(int *counters, int n, hipStream_t stream);

// ---- Q8_0 x fp16 GEMM ---------------------------------------------------------
hipError_t gemm_q8_0_launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M,
                            int64_t N, int64_t K, int num_cus, hipStream_t stream);

// ---- quantized x fp16 GEMM with dequantized fp16 weight tiles in LDS ----------
enum class GemmFormat { Q8_0, Q4_0, Q4_K };
hipError_t gemm_lds_launch(GemmFormat f, const uint8_t *W, const uint16_t *X, uint16_t *Y,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

// ---- fp32 GEMM ----------------------------------------------------------------
hipError_t sgemm_launch(const float *A, const float *B, float *C, int64_t M, int64_t N,
                        int64_t K, int num_cus, hipStream_t stream);

}  // namespace lqmm

// Host-side interface between the C entry points (api.hip) and the kernel
// translation units. Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lqmm {

// ---- GEMV -------------------------------------------------------------------
// Q4_0x2: Q4_0 weights taken two blocks (64 weights, 36 bytes) per unit, used
// by the VALU-mode kernel when K % 64 == 0.
enum class GemvFormat { Q4_0, Q4_K, Q4_0x2 };

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

// ---- Q8_0 x fp16 GEMM ---------------------------------------------------------
hipError_t gemm_q8_0_launch(const uint8_t *W, const uint16_t *X, uint16_t *Y, int64_t M,
                            int64_t N, int64_t K, int num_cus, hipStream_t stream);

// ---- fp32 GEMM ----------------------------------------------------------------
hipError_t sgemm_launch(const float *A, const float *B, float *C, int64_t M, int64_t N,
                        int64_t K, int num_cus, hipStream_t stream);

}  // namespace lqmm

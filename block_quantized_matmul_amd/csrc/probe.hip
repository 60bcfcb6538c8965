// Streaming-read probes: the HBM read rate plain kernels reach on this GPU,
// reported by the benchmark as context for the GEMV kernels' rates (which are
// stated against the 8 TB/s datasheet peak). Every 16-byte word of the buffer
// is read once, with non-temporal loads, in one of two orders:
// * grid stride: thread i reads words i, i + G, i + 2G, ... (G = all
//   threads), eight in flight per thread;
// * wave blocks: each wave reads whole 4 KB blocks (four 1 KB loads of 64
//   consecutive 16-byte words), the blocks strided over all waves.
// Also two empty marker kernels that bracket the benchmark's timed region in
// kernel traces. Built as its own library (liblqmm_probe.so); not part of the
// lqmm interface.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kDepth = 8;

__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const u32x4 *__restrict__ p, int64_t n16, uint32_t *out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kDepth - 1) * stride < n16; i += kDepth * stride) {
    u32x4 v[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kDepth; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // The loads must not be optimized away; this store almost never happens.
  if (acc == 0x9E3779B9u) out[0] = acc;
}

constexpr int kBlockLoads = 4;  // 1 KB loads per wave block

__global__ void __launch_bounds__(kThreads)
block_read_kernel(const u32x4 *__restrict__ p, int64_t n16, uint32_t *out) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int64_t nblk = n16 / (kBlockLoads * 64);
  uint32_t acc = 0;
  for (int64_t b = wave; b < nblk; b += nw) {
    const u32x4 *q = p + b * (kBlockLoads * 64) + lane;
    u32x4 v[kBlockLoads];
#pragma unroll
    for (int k = 0; k < kBlockLoads; ++k) v[k] = __builtin_nontemporal_load(q + k * 64);
#pragma unroll
    for (int k = 0; k < kBlockLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // the words after the last whole block
  for (int64_t i = nblk * (kBlockLoads * 64) + (int64_t)blockIdx.x * kThreads + threadIdx.x;
       i < n16; i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// Empty kernels whose names mark the start and the end of the benchmark's
// timed region in a kernel trace.
__global__ void timed_region_begin_marker() {}
__global__ void timed_region_end_marker() {}

}  // namespace

// Launch the begin (which == 0) or end (which != 0) marker kernel on
// `stream`. Returns 0, or the HIP error code of the launch.
extern "C" int lqmm_probe_marker(int which, void *stream) {
  if (which == 0)
    hipLaunchKernelGGL(timed_region_begin_marker, dim3(1), dim3(64), 0, (hipStream_t)stream);
  else
    hipLaunchKernelGGL(timed_region_end_marker, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

// Read `bytes` (a multiple of 16) from the 16-byte aligned device buffer p on
// `stream` with `grid` workgroups of 256 threads, in grid-stride order
// (blocks == 0) or in wave blocks (blocks != 0); `out` is a device word the
// kernel may write. Returns 0, or the HIP error code of the launch.
extern "C" int lqmm_probe_stream_read(const void *p, int64_t bytes, void *out, int grid,
                                      int blocks, void *stream) {
  if (!p || !out || bytes < 16 || bytes % 16 != 0 || grid < 1) return (int)hipErrorInvalidValue;
  if (blocks)
    hipLaunchKernelGGL(block_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(p), bytes / 16, static_cast<uint32_t *>(out));
  else
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(p), bytes / 16, static_cast<uint32_t *>(out));
  return (int)hipGetLastError();
}

// Measurement aid of gemmf32: the FP32 matrix-core ceiling of the device at the clock it
// actually runs at, so that a GEMM's throughput can be set against a measured limit as
// well as against the 157.3 TFLOP/s specification (which assumes the 2.4 GHz peak clock).
//
// Every wave issues nothing but v_mfma_f32_32x32x2_f32 (4096 FLOP each) on register
// operands, four independent accumulators deep, and records how many shader-clock cycles
// (s_memtime) and how many 100 MHz wall-clock ticks (s_memrealtime) its loop took.  The
// ratio of the two is the shader clock during the loop; the cycles per instruction show
// the matrix pipe's issue rate.  The kernel reads no memory and writes one float per lane
// (to keep the arithmetic live) and one record per wave.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_common.h"

namespace gemmf32 {

constexpr int kPeakThreads = 256;          // 4 waves per workgroup
constexpr int kPeakWaves = kPeakThreads / 64;
constexpr int kPeakMfmaPerIter = 16;       // 4 accumulators x 4 instructions
constexpr int kPeakMaxBlocks = 65536;
constexpr int kPeakMaxIters = 1 << 20;

__global__ void __launch_bounds__(kPeakThreads)
gemm_f32_peak_kernel(int iters, float* __restrict__ out, uint64_t* __restrict__ rec) {
  const float a = 1.0f / (float)(1 + (threadIdx.x & 7));
  const float b = 1.0f / (float)(2 + (threadIdx.x & 3));
  floatx16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kPeakMfmaPerIter; ++u)
      acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[u & 3], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  // The store depends on every accumulator, so the clocks below are read after the last
  // matrix instruction has finished.
  const int64_t gid = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  out[gid] = s;
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  if ((threadIdx.x & 63) == 0) {
    const int64_t w = (int64_t)blockIdx.x * kPeakWaves + threadIdx.x / 64;
    rec[2 * w] = c1 - c0;
    rec[2 * w + 1] = w1 - w0;
  }
}

}  // namespace gemmf32

// Shader clock under matrix-core load.  The published bf16 peak assumes the
// chip's top clock; under a sustained MFMA stream it runs lower, and the
// measured clock gives the peak a pure MFMA stream can approach (kernels that
// also spend time on vector and memory work draw less power and may hold a
// higher clock).  Every SIMD runs two waves of independent 32x32x16 bf16
// MFMAs (the occupancy of the forward and dQ passes) for about 8 ms, long
// enough to pass a short boost at the start; lane 0 of each wave reads the
// shader-clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) around its stream, and the ratio of the sums is the clock.

#include <vector>

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kClkThreads = 256;                 // four waves: one per SIMD
constexpr int kClkMaxGroups = 1024;              // two per CU, up to 512 CUs
constexpr int kClkIters = 32768;                 // x 8 MFMAs per wave (about 8 ms)
constexpr double kRealtimeGHz = 0.1;             // s_memrealtime rate

// [group][wave][shader ticks, realtime ticks]; module memory, no allocation
__device__ unsigned long long g_clk[kClkMaxGroups * (kClkThreads / 64) * 2];

__global__ __launch_bounds__(kClkThreads, 2) void sclk_kernel(int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)((threadIdx.x + i) & 15));
    b[i] = (__bf16)(1e-3f * (float)i);
  }
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const int w = threadIdx.x >> 6;
  unsigned long long* rec = g_clk + ((int64_t)blockIdx.x * (kClkThreads / 64) + w) * 2;
  if ((threadIdx.x & 63) == 0) {
    rec[0] = t1 - t0;
    rec[1] = r1 - r0;
  }
  if (s < 0.0f) rec[0] = 0;   // never taken (the products are non-negative); keeps them live
}

}  // namespace
}  // namespace prism

using namespace prism;

extern "C" int prism_sclk_probe(double* ghz, prism_stream stream) {
  if (ghz == nullptr) return PRISM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)sclk_kernel, kClkThreads, 0) != hipSuccess)
    return PRISM_EHIP;
  int groups = (cus > 0 ? cus : 1) * (per_cu < 2 ? (per_cu > 0 ? per_cu : 1) : 2);
  if (groups > kClkMaxGroups) groups = kClkMaxGroups;
  hipLaunchKernelGGL(sclk_kernel, dim3(groups), dim3(kClkThreads), 0, s, kClkIters);
  if (hipGetLastError() != hipSuccess) return PRISM_EHIP;
  std::vector<unsigned long long> host((size_t)groups * (kClkThreads / 64) * 2);
  const size_t bytes = host.size() * sizeof(unsigned long long);
  if (hipMemcpyFromSymbolAsync(host.data(), HIP_SYMBOL(g_clk), bytes, 0, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return PRISM_EHIP;
  double shader = 0.0, real = 0.0;
  for (int i = 0; i < groups * (kClkThreads / 64); ++i) {
    shader += (double)host[2 * i];
    real += (double)host[2 * i + 1];
  }
  if (real <= 0.0) return PRISM_EHIP;
  *ghz = shader / real * kRealtimeGHz;
  return PRISM_OK;
}

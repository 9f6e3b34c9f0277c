// Audio-to-video norm producer: a_n = |h-hat_n|_2 for every video token, the
// guidance map that the next layer's zone statistics read (Prism guide (pt),
// Método 1, second paragraph: the norms of the audio-to-video cross-attention
// output, cached from the previous layer).
//
// A streaming row reduction, bound by HBM reads of h-hat (2 bytes per value).
// A row of C bf16 values is C/8 16-byte chunks; a group of G lanes (G a power
// of two, at most 64, at most C/8) reads one row with 16-byte loads, so a
// wave covers 64/G rows per load instruction and every load instruction
// reads whole contiguous runs.  Each wave keeps U such row groups in flight.
// Squares of bf16 values are exact in float64 and their float64 sum is within
// one rounding of the exact sum, so the float32 result is the correctly
// rounded norm except within a hair of a rounding midpoint.

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kWaves = 4;   // waves per workgroup
constexpr int kSteps = 4;   // row groups in flight per wave

__device__ __forceinline__ double sq8(uint4 x, double acc) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = (double)__uint_as_float(w[i] << 16);
    const double hi = (double)__uint_as_float(w[i] & 0xffff0000u);
    acc = __builtin_fma(lo, lo, acc);
    acc = __builtin_fma(hi, hi, acc);
  }
  return acc;
}

template <int LG>
__global__ __launch_bounds__(kWaves * 64) void a2v_norm_kernel(const uint16_t* __restrict__ h, int64_t n,
                                                                int chunks, int64_t stride,
                                                                float* __restrict__ a) {
  constexpr int G = 1 << LG;
  constexpr int RPW = 64 / G;  // rows per wave per step
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (G - 1);
  const int64_t base = ((int64_t)blockIdx.x * kWaves + wave) * (RPW * kSteps) + (lane >> LG);

  double acc[kSteps];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) acc[u] = 0.0;

  for (int c = sub; c < chunks; c += G) {
    uint4 x[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t row = base + (int64_t)u * RPW;
      x[u] = row < n ? *reinterpret_cast<const uint4*>(h + row * stride + (int64_t)c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) acc[u] = sq8(x[u], acc[u]);
  }

#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) acc[u] += __shfl_xor(acc[u], o, 64);
  }
  if (sub == 0) {
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t row = base + (int64_t)u * RPW;
      if (row < n) a[row] = (float)__builtin_sqrt(acc[u]);
    }
  }
}

template <int LG>
hipError_t launch_lg(const uint16_t* h, int64_t n, int chunks, int64_t stride, float* a, hipStream_t s) {
  constexpr int rows_per_block = kWaves * (64 >> LG) * kSteps;
  const int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(a2v_norm_kernel<LG>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, s, h, n, chunks, stride, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_a2v_norms(const uint16_t* h_hat, int64_t n, int channels, int64_t stride, float* a,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int chunks = channels / 8;
  int lg = 0;
  while (lg < 6 && (2 << lg) <= chunks) ++lg;
  switch (lg) {
    case 0: return launch_lg<0>(h_hat, n, chunks, stride, a, s);
    case 1: return launch_lg<1>(h_hat, n, chunks, stride, a, s);
    case 2: return launch_lg<2>(h_hat, n, chunks, stride, a, s);
    case 3: return launch_lg<3>(h_hat, n, chunks, stride, a, s);
    case 4: return launch_lg<4>(h_hat, n, chunks, stride, a, s);
    case 5: return launch_lg<5>(h_hat, n, chunks, stride, a, s);
    default: return launch_lg<6>(h_hat, n, chunks, stride, a, s);
  }
}

}  // namespace prism

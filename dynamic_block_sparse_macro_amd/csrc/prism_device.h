// Device-side helpers shared by the Prism HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int kZone = 8;          // macro-zone edge
constexpr int kZoneTokens = 512;  // tokens per macro-zone
constexpr int kTile = 64;         // token sub-tile of the attention kernels
constexpr int kNumShapes = 16;

// Candidate block shapes: edges in {2,4,8}, volume in {64,128,256}, ordered by
// volume then (b_T, b_H, b_W).  Enumerated, not tabulated by hand.
struct ShapeTable {
  uint8_t e[kNumShapes][3];
  uint16_t vol[kNumShapes];
};

__host__ __device__ constexpr ShapeTable make_shape_table() {
  ShapeTable t{};
  int n = 0;
  const int vols[3] = {64, 128, 256};
  const int edges[3] = {2, 4, 8};
  for (int vi = 0; vi < 3; ++vi)
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b)
        for (int c = 0; c < 3; ++c)
          if (edges[a] * edges[b] * edges[c] == vols[vi]) {
            t.e[n][0] = (uint8_t)edges[a];
            t.e[n][1] = (uint8_t)edges[b];
            t.e[n][2] = (uint8_t)edges[c];
            t.vol[n] = (uint16_t)vols[vi];
            ++n;
          }
  return t;
}

// Operand tiles of the attention kernels are 64 rows x D bf16, row-major, with
// the 16-byte chunk c of row r stored at chunk position swz_chunk<D>(r, c) =
// c ^ f(r).  For D = 128 (16 chunks = all 64 banks per row) f permutes the bits
// of r mod 16 so that (a) 16 consecutive rows get 16 different f (16-byte row
// reads of 16 lanes hit distinct banks) and (b) the four rows read together by
// a transposing 8-byte read differ in bits 2-3 of f (the 4 x 4 chunks two
// 16-lane groups touch land on 16 distinct positions).  For D = 64 (a row is
// half the banks) f has the same two properties per bank half.  The tile can
// be copied to LDS verbatim.
template <int D>
__host__ __device__ __forceinline__ constexpr int swz_chunk(int r, int c) {
  return D == 128 ? (c ^ (((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)))
                  : (c ^ ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Workgroup-wide reductions (blockDim.x a multiple of 64, <= 1024).
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_max(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T y = __shfl_xor(x, o, 64);
    x = y > x ? y : x;
  }
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_min(T x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T y = __shfl_xor(x, o, 64);
    x = y < x ? y : x;
  }
  return x;
}

// red must hold blockDim.x / 64 elements; all threads get the result.
template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T x, T* red, Op op) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if (lane == 0) red[wid] = x;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < nw; ++i) r = op(r, red[i]);
  return r;
}

struct OpAdd {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
  template <typename T>
  __device__ T operator()(T a, T b) const { return b > a ? b : a; }
};
struct OpMin {
  template <typename T>
  __device__ T operator()(T a, T b) const { return b < a ? b : a; }
};

// Block containing 64-token sub-tile `tile` of one head: largest b with
// blk_start[b] <= tile, searched over the head's n_b blocks.
__device__ __forceinline__ int block_of_tile(const int32_t* __restrict__ bs, int nb, int tile) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (bs[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace prism

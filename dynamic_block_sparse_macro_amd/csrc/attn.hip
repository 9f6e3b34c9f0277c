// Variable-block-size block-sparse flash attention, forward and backward.
//
// Prism (pt reading guide), Método 3: an online-softmax kernel runs attention
// only over the attended set S_i of each query block.  Prism (zh reading guide),
// 常见问题: gradients flow only through the sparse attention on the selected
// blocks.  Prism (sd114.wiki post), 工作原理 step 4: results are restored to the
// original T x H x W layout.
//
// CDNA4 design:
//  * every block is 1, 2 or 4 sub-tiles of 64 tokens, so one code path serves
//    64/128/256-token blocks; a workgroup owns one 64-token tile (query tile in
//    the forward and dQ passes, key tile in the dK/dV pass), two waves of 32
//    rows each;
//  * v_mfma_f32_32x32x16_bf16 for every product, computed transposed
//    (S^T = K Q^T, O^T = V^T P^T, ...) so that the accumulator of one product
//    is, register for register, the B operand of the next: no shuffles between
//    the two GEMMs;
//  * operands come from the two-part layout written by the permutation
//    (row tiles and 64-token column tiles), so LDS staging is a plain copy;
//  * float32 online softmax in the log2 domain, float32 accumulation;
//  * the backward runs a query-major pass (dQ) and a key-major pass over the
//    transposed block index (dK, dV), so no float atomics are needed and the
//    result is bitwise reproducible.

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles.  Row tiles are [64][D] with an 8-element pad, column tiles
// [D][64] with a 4-element pad, which keeps the 16-byte and 8-byte operand
// reads of a wave free of bank conflicts.
template <int D>
struct RowTile {
  static constexpr int LD = D + 8;
  uint16_t x[kTile * LD];
  __device__ uint16_t* row(int r) { return x + r * LD; }
};
template <int D>
struct ColTile {
  static constexpr int LD = kTile + 4;
  uint16_t x[D * LD];
  __device__ uint16_t* row(int c) { return x + c * LD; }
};

// copy a contiguous 64 x D row tile into LDS
template <int D, int NT>
__device__ __forceinline__ void stage_rows(RowTile<D>& t, const uint16_t* __restrict__ src) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int c = threadIdx.x; c < kTile * CH; c += NT) {
    const int r = c / CH, k = c % CH;
    *(uint4*)(t.row(r) + k * 8) = *(const uint4*)(src + c * 8);
  }
}
// copy a contiguous D x 64 column tile into LDS
template <int D, int NT>
__device__ __forceinline__ void stage_cols(ColTile<D>& t, const uint16_t* __restrict__ src) {
#pragma unroll
  for (int c = threadIdx.x; c < D * 8; c += NT) {
    const int d = c >> 3, k = c & 7;
    *(uint4*)(t.row(d) + k * 8) = *(const uint4*)(src + c * 8);
  }
}

// 16-byte A-operand read from a row tile: row r, columns 16 s + 8 g .. + 7
template <int D>
__device__ __forceinline__ bf16x8 rd_row(RowTile<D>& t, int r, int s, int g) {
  return *(const bf16x8*)(t.row(r) + 16 * s + 8 * g);
}
// A-operand read from a column tile for k-step (kk, hh): keys
// 32 kk + 16 hh + 4 g + {0..3} and the same + 8, matching the register order
// of a 32x32 accumulator used as the B operand.
template <int D>
__device__ __forceinline__ bf16x8 rd_col(ColTile<D>& t, int c, int kk, int hh, int g) {
  const uint16_t* p = t.row(c) + 32 * kk + 16 * hh + 4 * g;
  return cat4(*(const bf16x4*)p, *(const bf16x4*)(p + 8));
}

// write a [64][D] bf16 tile held in LDS to THW rows through perm
template <int D, int NT>
__device__ __forceinline__ void store_rows_thw(RowTile<D>& t, uint16_t* __restrict__ out, const Geometry& g, int h,
                                               int64_t tile, const int32_t* __restrict__ perm) {
  constexpr int CH = D / 8;
  const int64_t p0 = (int64_t)h * g.N + tile * kTile;
#pragma unroll
  for (int c = threadIdx.x; c < kTile * CH; c += NT) {
    const int r = c / CH, k = c % CH;
    const int64_t n = perm ? (int64_t)perm[p0 + r] : tile * kTile + r;
    *(uint4*)(out + (int64_t)h * g.hstride + n * g.tstride + k * 8) = *(const uint4*)(t.row(r) + k * 8);
  }
}

// accumulator (rows = D dims in tiles of 32, column = lane's row of the tile)
// -> bf16 into an LDS row tile at row `r`
template <int D>
__device__ __forceinline__ void acc_to_rowtile(RowTile<D>& t, const floatx16* acc, int r, int g, float mul) {
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * u + 8 * j + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(acc[u][4 * j] * mul, acc[u][4 * j + 1] * mul);
      v.y = pack_bf16x2(acc[u][4 * j + 2] * mul, acc[u][4 * j + 3] * mul);
      *(uint2*)(t.row(r) + d0) = v;
    }
}

struct KeyRange {
  int e0, e1;
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D>
struct FwdSmem {
  RowTile<D> k;
  ColTile<D> vt;
};

template <int D, bool DENSE>
__global__ __launch_bounds__(128) void attn_fwd_kernel(Geometry g, float sl2, const uint16_t* __restrict__ qp,
                                                       const uint16_t* __restrict__ kp,
                                                       const uint16_t* __restrict__ vp,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ blk_start,
                                                       const int32_t* __restrict__ n_blocks,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx, uint16_t* __restrict__ o,
                                                       float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;
  const int h = blockIdx.y;
  const int64_t qt = xcd_remap(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g32 = lane >> 5, l32 = lane & 31;
  const int64_t hN = (int64_t)h * g.N;
  const uint16_t* Qr = qp + hN * D;
  const uint16_t* Kr = kp + hN * D;
  const uint16_t* Vc = vp + ((int64_t)g.heads * g.N + hN) * D;

  const int64_t qrow = qt * kTile + 32 * w + l32;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qreg[s] = *(const bf16x8*)(Qr + qrow * D + 16 * s + 8 * g32);

  floatx16 oacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[u][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  auto tile_step = [&](int64_t kt) {
    __syncthreads();
    stage_rows<D, 128>(sm.k, Kr + kt * kTile * D);
    stage_cols<D, 128>(sm.vt, Vc + kt * kTile * D);
    __syncthreads();
    floatx16 sacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kk][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) sacc[kk] = mfma32(rd_row(sm.k, 32 * kk + l32, s, g32), qreg[s], sacc[kk]);
    }
    float mloc = sacc[0][0];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[kk][i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc * sl2);
    const float alpha = fast_exp2(m_run - m_new);
    bf16x8 pb[4];
    float lsum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // the normaliser sums the same bf16-rounded weights the PV product uses
        const __bf16 pr = (__bf16)fast_exp2(__builtin_fmaf(sacc[kk][i], sl2, -m_new));
        lsum += (float)pr;
        pb[kk * 2 + (i >> 3)][i & 7] = pr;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[u][i] *= alpha;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          oacc[u] = mfma32(rd_col(sm.vt, 32 * u + l32, kk, hh, g32), pb[kk * 2 + hh], oacc[u]);
  };

  if (DENSE) {
    for (int64_t kt = 0; kt < g.tiles; ++kt) tile_step(kt);
  } else {
    const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
    const int nb = n_blocks[h];
    const int i = block_of_tile(bs, nb, (int)qt);
    const int32_t* rp = row_ptr + (int64_t)h * (g.tiles + 1);
    const int e0 = rp[i], e1 = rp[i + 1];
    for (int e = e0; e < e1; ++e) {
      const int j = col_idx[e];
      const int t1 = bs[j + 1];
      for (int kt = bs[j]; kt < t1; ++kt) tile_step(kt);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (g32 == 0) lse[hN + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  __syncthreads();
  acc_to_rowtile(sm.k, oacc, 32 * w + l32, g32, inv);
  __syncthreads();
  store_rows_thw<D, 128>(sm.k, o, g, h, qt, perm);
}

// ---------------------------------------------------------------------------
// backward pre-pass: dO into the operand layout, delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(Geometry g, const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dout,
                                                      const int32_t* __restrict__ perm, uint16_t* __restrict__ dop,
                                                      float* __restrict__ delta) {
  constexpr int CH = D / 8;
  __shared__ __attribute__((aligned(16))) RowTile<D> tb;
  const int64_t tile = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t p0 = (int64_t)h * g.N + tile * kTile;
  uint16_t* rows = dop + p0 * D;
  uint16_t* cols = dop + (int64_t)g.heads * g.N * D + p0 * D;
  for (int c = tid; c < kTile * CH; c += 256) {
    const int r = c / CH, k = c % CH;
    const int64_t n = perm ? (int64_t)perm[p0 + r] : tile * kTile + r;
    const int64_t off = (int64_t)h * g.hstride + n * g.tstride + k * 8;
    const uint4 dv = *(const uint4*)(dout + off);
    const uint4 ov = *(const uint4*)(o + off);
    *(uint4*)(tb.row(r) + k * 8) = dv;
    *(uint4*)(rows + (int64_t)r * D + k * 8) = dv;
    const uint32_t a4[4] = {dv.x, dv.y, dv.z, dv.w}, b4[4] = {ov.x, ov.y, ov.z, ov.w};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += bf16_to_f32((uint16_t)(a4[e] & 0xFFFF)) * bf16_to_f32((uint16_t)(b4[e] & 0xFFFF));
      acc += bf16_to_f32((uint16_t)(a4[e] >> 16)) * bf16_to_f32((uint16_t)(b4[e] >> 16));
    }
#pragma unroll
    for (int off2 = CH / 2; off2 > 0; off2 >>= 1) acc += __shfl_xor(acc, off2, CH);
    if (k == 0) delta[p0 + r] = acc;
  }
  __syncthreads();
  for (int q = tid; q < D * 8; q += 256) {
    const int c = q >> 3, r0 = (q & 7) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = (uint32_t)tb.row(r0 + 2 * e)[c] | ((uint32_t)tb.row(r0 + 2 * e + 1)[c] << 16);
    *(uint4*)(cols + c * kTile + r0) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// ---------------------------------------------------------------------------
// backward, query-major pass: dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqSmem {
  RowTile<D> k, v;
  ColTile<D> kt;
};

template <int D, bool DENSE>
__global__ __launch_bounds__(128) void attn_bwd_dq_kernel(Geometry g, float scale, float sl2,
                                                          const uint16_t* __restrict__ qp,
                                                          const uint16_t* __restrict__ kp,
                                                          const uint16_t* __restrict__ vp,
                                                          const uint16_t* __restrict__ dop,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ delta,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ blk_start,
                                                          const int32_t* __restrict__ n_blocks,
                                                          const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx,
                                                          uint16_t* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) DqSmem<D> sm;
  const int h = blockIdx.y;
  const int64_t qt = xcd_remap(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g32 = lane >> 5, l32 = lane & 31;
  const int64_t hN = (int64_t)h * g.N;
  const int64_t part1 = (int64_t)g.heads * g.N * D;
  const uint16_t* Kr = kp + hN * D;
  const uint16_t* Kc = kp + part1 + hN * D;
  const uint16_t* Vr = vp + hN * D;

  const int64_t qrow = qt * kTile + 32 * w + l32;
  bf16x8 qreg[D / 16], dreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qreg[s] = *(const bf16x8*)(qp + (hN + qrow) * D + 16 * s + 8 * g32);
    dreg[s] = *(const bf16x8*)(dop + (hN + qrow) * D + 16 * s + 8 * g32);
  }
  const float lse2 = lse[hN + qrow] * kLog2e;
  const float dlt = delta[hN + qrow];
  floatx16 dqacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[u][i] = 0.0f;

  auto tile_step = [&](int64_t kt) {
    __syncthreads();
    stage_rows<D, 128>(sm.k, Kr + kt * kTile * D);
    stage_rows<D, 128>(sm.v, Vr + kt * kTile * D);
    stage_cols<D, 128>(sm.kt, Kc + kt * kTile * D);
    __syncthreads();
    floatx16 sacc[2], pacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kk][i] = pacc[kk][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc[kk] = mfma32(rd_row(sm.k, 32 * kk + l32, s, g32), qreg[s], sacc[kk]);
        pacc[kk] = mfma32(rd_row(sm.v, 32 * kk + l32, s, g32), dreg[s], pacc[kk]);
      }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(__builtin_fmaf(sacc[kk][i], sl2, -lse2));
        dsb[kk * 2 + (i >> 3)][i & 7] = (__bf16)(pv * (pacc[kk][i] - dlt));
      }
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          dqacc[u] = mfma32(rd_col(sm.kt, 32 * u + l32, kk, hh, g32), dsb[kk * 2 + hh], dqacc[u]);
  };

  if (DENSE) {
    for (int64_t kt = 0; kt < g.tiles; ++kt) tile_step(kt);
  } else {
    const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
    const int i = block_of_tile(bs, n_blocks[h], (int)qt);
    const int32_t* rp = row_ptr + (int64_t)h * (g.tiles + 1);
    const int e0 = rp[i], e1 = rp[i + 1];
    for (int e = e0; e < e1; ++e) {
      const int j = col_idx[e];
      const int t1 = bs[j + 1];
      for (int kt = bs[j]; kt < t1; ++kt) tile_step(kt);
    }
  }
  __syncthreads();
  acc_to_rowtile(sm.k, dqacc, 32 * w + l32, g32, scale);
  __syncthreads();
  store_rows_thw<D, 128>(sm.k, dq, g, h, qt, perm);
}

// ---------------------------------------------------------------------------
// backward, key-major pass: dK and dV
// ---------------------------------------------------------------------------
template <int D>
struct DkvSmem {
  RowTile<D> q, d;
  ColTile<D> qt, dt;
  float lse2[kTile], dlt[kTile];
};

template <int D, bool DENSE>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_kernel(Geometry g, float scale, float sl2,
                                                            const uint16_t* __restrict__ qp,
                                                            const uint16_t* __restrict__ kp,
                                                            const uint16_t* __restrict__ vp,
                                                            const uint16_t* __restrict__ dop,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ delta,
                                                            const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ blk_start,
                                                            const int32_t* __restrict__ n_blocks,
                                                            const int32_t* __restrict__ t_row_ptr,
                                                            const int32_t* __restrict__ t_col_idx,
                                                            uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  __shared__ __attribute__((aligned(16))) DkvSmem<D> sm;
  const int h = blockIdx.y;
  const int64_t kt = xcd_remap(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g32 = lane >> 5, l32 = lane & 31;
  const int64_t hN = (int64_t)h * g.N;
  const int64_t part1 = (int64_t)g.heads * g.N * D;
  const uint16_t* Qr = qp + hN * D;
  const uint16_t* Qc = qp + part1 + hN * D;
  const uint16_t* Dr = dop + hN * D;
  const uint16_t* Dc = dop + part1 + hN * D;

  const int64_t krow = kt * kTile + 32 * w + l32;
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kreg[s] = *(const bf16x8*)(kp + (hN + krow) * D + 16 * s + 8 * g32);
    vreg[s] = *(const bf16x8*)(vp + (hN + krow) * D + 16 * s + 8 * g32);
  }
  floatx16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[u][i] = dvacc[u][i] = 0.0f;

  auto tile_step = [&](int64_t qt) {
    __syncthreads();
    stage_rows<D, 128>(sm.q, Qr + qt * kTile * D);
    stage_rows<D, 128>(sm.d, Dr + qt * kTile * D);
    stage_cols<D, 128>(sm.qt, Qc + qt * kTile * D);
    stage_cols<D, 128>(sm.dt, Dc + qt * kTile * D);
    if (threadIdx.x < kTile) {
      sm.lse2[threadIdx.x] = lse[hN + qt * kTile + threadIdx.x] * kLog2e;
    } else {
      sm.dlt[threadIdx.x - kTile] = delta[hN + qt * kTile + threadIdx.x - kTile];
    }
    __syncthreads();
    floatx16 sacc[2], pacc[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[qq][i] = pacc[qq][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc[qq] = mfma32(rd_row(sm.q, 32 * qq + l32, s, g32), kreg[s], sacc[qq]);
        pacc[qq] = mfma32(rd_row(sm.d, 32 * qq + l32, s, g32), vreg[s], pacc[qq]);
      }
    }
    bf16x8 pb[4], dsb[4];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q0 = 32 * qq + 8 * j + 4 * g32;
        const float4 l4 = *(const float4*)(sm.lse2 + q0);
        const float4 d4 = *(const float4*)(sm.dlt + q0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          const float pv = fast_exp2(__builtin_fmaf(sacc[qq][i], sl2, -lv[e]));
          pb[qq * 2 + (i >> 3)][i & 7] = (__bf16)pv;
          dsb[qq * 2 + (i >> 3)][i & 7] = (__bf16)(pv * (pacc[qq][i] - dvv[e]));
        }
      }
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          dvacc[u] = mfma32(rd_col(sm.dt, 32 * u + l32, qq, hh, g32), pb[qq * 2 + hh], dvacc[u]);
          dkacc[u] = mfma32(rd_col(sm.qt, 32 * u + l32, qq, hh, g32), dsb[qq * 2 + hh], dkacc[u]);
        }
  };

  if (DENSE) {
    for (int64_t qt = 0; qt < g.tiles; ++qt) tile_step(qt);
  } else {
    const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
    const int j = block_of_tile(bs, n_blocks[h], (int)kt);
    const int32_t* tp = t_row_ptr + (int64_t)h * (g.tiles + 1);
    const int e0 = tp[j], e1 = tp[j + 1];
    for (int e = e0; e < e1; ++e) {
      const int i = t_col_idx[e];
      const int t1 = bs[i + 1];
      for (int qt = bs[i]; qt < t1; ++qt) tile_step(qt);
    }
  }
  __syncthreads();
  acc_to_rowtile(sm.q, dkacc, 32 * w + l32, g32, scale);
  acc_to_rowtile(sm.d, dvacc, 32 * w + l32, g32, 1.0f);
  __syncthreads();
  store_rows_thw<D, 128>(sm.q, dk, g, h, kt, perm);
  store_rows_thw<D, 128>(sm.d, dv, g, h, kt, perm);
}

template <int D, bool DENSE>
hipError_t fwd_impl(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp, const uint16_t* vp,
                    const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks, const int32_t* row_ptr,
                    const int32_t* col_idx, uint16_t* o, float* lse, hipStream_t s) {
  dim3 grid((unsigned)g.tiles, (unsigned)g.heads);
  hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE>), grid, dim3(128), 0, s, g, scale * kLog2e, qp, kp, vp, perm,
                     blk_start, n_blocks, row_ptr, col_idx, o, lse);
  return hipGetLastError();
}

template <int D, bool DENSE>
hipError_t bwd_impl(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp, const uint16_t* vp,
                    const uint16_t* dop, const float* lse, const float* delta, const int32_t* perm,
                    const int32_t* blk_start, const int32_t* n_blocks, const int32_t* row_ptr,
                    const int32_t* col_idx, const int32_t* t_row_ptr, const int32_t* t_col_idx, uint16_t* dq,
                    uint16_t* dk, uint16_t* dv, hipStream_t s) {
  dim3 grid((unsigned)g.tiles, (unsigned)g.heads);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, DENSE>), grid, dim3(128), 0, s, g, scale, scale * kLog2e, qp, kp, vp,
                     dop, lse, delta, perm, blk_start, n_blocks, row_ptr, col_idx, dq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, DENSE>), grid, dim3(128), 0, s, g, scale, scale * kLog2e, qp, kp, vp,
                     dop, lse, delta, perm, blk_start, n_blocks, t_row_ptr, t_col_idx, dk, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const int32_t* perm, const int32_t* blk_start,
                           const int32_t* n_blocks, const int32_t* row_ptr, const int32_t* col_idx, uint16_t* o,
                           float* lse, hipStream_t s) {
  const bool dense = row_ptr == nullptr;
  if (g.D == 128)
    return dense ? fwd_impl<128, true>(g, scale, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, lse, s)
                 : fwd_impl<128, false>(g, scale, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, lse, s);
  return dense ? fwd_impl<64, true>(g, scale, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, lse, s)
               : fwd_impl<64, false>(g, scale, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, lse, s);
}

hipError_t launch_bwd_pre(const Geometry& g, const uint16_t* o, const uint16_t* dout, const int32_t* perm,
                          uint16_t* dop, float* delta, hipStream_t s) {
  dim3 grid((unsigned)g.tiles, (unsigned)g.heads);
  if (g.D == 128) hipLaunchKernelGGL(bwd_pre_kernel<128>, grid, dim3(256), 0, s, g, o, dout, perm, dop, delta);
  else hipLaunchKernelGGL(bwd_pre_kernel<64>, grid, dim3(256), 0, s, g, o, dout, perm, dop, delta);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const uint16_t* dop, const float* lse, const float* delta,
                           const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks,
                           const int32_t* row_ptr, const int32_t* col_idx, const int32_t* t_row_ptr,
                           const int32_t* t_col_idx, uint16_t* dq, uint16_t* dk, uint16_t* dv, hipStream_t s) {
  const bool dense = row_ptr == nullptr;
#define PRISM_BWD(DD, DN)                                                                                         \
  bwd_impl<DD, DN>(g, scale, qp, kp, vp, dop, lse, delta, perm, blk_start, n_blocks, row_ptr, col_idx, t_row_ptr, \
                   t_col_idx, dq, dk, dv, s)
  if (g.D == 128) return dense ? PRISM_BWD(128, true) : PRISM_BWD(128, false);
  return dense ? PRISM_BWD(64, true) : PRISM_BWD(64, false);
#undef PRISM_BWD
}

}  // namespace prism

// Zone statistics and shape planning for Prism dynamic sparse attention.
//
// Prism (pt reading guide), Método 1: per 8x8x8 macro-zone, the variance of the
// mean-pooled value slices along T, H and W (sigma^2_v,d), its normalised ratio
// r_v,d, the audio coupling a-bar and directional audio variance v-hat_a,d
// from the cached A2V norms, and g_d = r_v,d + a-bar * v-hat_a,d + eps.
// Método 2: density rho against tau_128 / tau_256 gives the volume B(m);
// l*_d = -1/2 log2 g_d + 1/3 (log2 B + 1/2 sum_d' log2 g_d'); the block
// shape is the candidate of that volume nearest to l* in log2 distance.
//
// All statistics and decisions in float64.  A zone's sums of bfloat16 values
// (512 terms within 36 binades of each other) and of float32 values (within 20
// binades) are exact in float64, so per-zone statistics do not depend on
// summation order for such inputs; this file is built without floating-point
// contraction so that the decision arithmetic is the plain sequence of IEEE
// operations.

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {

namespace {

constexpr ShapeTable kShapes = make_shape_table();
__constant__ ShapeTable c_shapes = kShapes;

// ---------------------------------------------------------------------------
// zone statistics: one workgroup of 256 threads per (zone, head)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void zone_stats_kernel(Geometry g, const uint16_t* __restrict__ v,
                                                         const float* __restrict__ a, double* __restrict__ zstats) {
  constexpr int LPT = D / 2;     // threads per token row, two channels each
  constexpr int G = 256 / LPT;   // token groups
  constexpr int TPG = 8 / G;     // T-planes per group
  __shared__ double shT[8][D], shH[8][D], shW[8][D];
  __shared__ double acube[512];
  __shared__ double red[4];
  __shared__ double aslice[3][8];

  const int m = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int znh = g.H / kZone, znw = g.W / kZone;
  const int zt = m / (znh * znw), zh = (m / znw) % znh, zw = m % znw;
  const int cp = tid % LPT, grp = tid / LPT;
  const uint16_t* vb = v + (int64_t)h * g.hstride + 2 * cp;

  // the zone's audio norms (64 threads x 8 values) are loaded first, so their
  // latency overlaps that of the value loads
  float apre[8];
  if (tid < 64) {
    const int eta = tid >> 3, om = tid & 7;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
      apre[tau] = a ? a[((int64_t)(zt * kZone + tau) * g.H + zh * kZone + eta) * g.W + zw * kZone + om] : 0.0f;
  }

  double sT[TPG][2], sH[8][2], sW[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) sH[i][0] = sH[i][1] = sW[i][0] = sW[i][1] = 0.0;
#pragma unroll
  for (int i = 0; i < TPG; ++i) sT[i][0] = sT[i][1] = 0.0;

#pragma unroll
  for (int tl = 0; tl < TPG; ++tl) {
    const int t = zt * kZone + grp * TPG + tl;
    // the plane's 64 loads are issued before its sums: more bytes in flight
    // per wave (the kernel is bound by HBM latency x parallelism)
    uint32_t pl[8][8];
#pragma unroll
    for (int eta = 0; eta < 8; ++eta) {
      const int64_t row = ((int64_t)t * g.H + zh * kZone + eta) * g.W + zw * kZone;
#pragma unroll
      for (int om = 0; om < 8; ++om) pl[eta][om] = *(const uint32_t*)(vb + (row + om) * g.tstride);
    }
#pragma unroll
    for (int eta = 0; eta < 8; ++eta) {
      const uint32_t* pr = pl[eta];
#pragma unroll
      for (int om = 0; om < 8; ++om) {
        const double x0 = (double)bf16_to_f32((uint16_t)(pr[om] & 0xFFFFu));
        const double x1 = (double)bf16_to_f32((uint16_t)(pr[om] >> 16));
        sT[tl][0] += x0; sT[tl][1] += x1;
        sH[eta][0] += x0; sH[eta][1] += x1;
        sW[om][0] += x0; sW[om][1] += x1;
      }
    }
  }
  // T slices are owned by one group each; H and W slices are summed over the
  // groups in a fixed order.
#pragma unroll
  for (int tl = 0; tl < TPG; ++tl) {
    shT[grp * TPG + tl][2 * cp] = sT[tl][0];
    shT[grp * TPG + tl][2 * cp + 1] = sT[tl][1];
  }
  for (int gi = 0; gi < G; ++gi) {
    if (grp == gi) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (gi == 0) {
          shH[i][2 * cp] = sH[i][0]; shH[i][2 * cp + 1] = sH[i][1];
          shW[i][2 * cp] = sW[i][0]; shW[i][2 * cp + 1] = sW[i][1];
        } else {
          shH[i][2 * cp] += sH[i][0]; shH[i][2 * cp + 1] += sH[i][1];
          shW[i][2 * cp] += sW[i][0]; shW[i][2 * cp + 1] += sW[i][1];
        }
      }
    }
    __syncthreads();
  }

  // audio cube (a shared by all heads)
  if (tid < 64) {
    const int eta = tid >> 3, om = tid & 7;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) acube[(tau * 8 + eta) * 8 + om] = (double)apre[tau];
  }

  // per-channel variance of the slice means, per axis
  double vT = 0.0, vH = 0.0, vW = 0.0;
  if (tid < D) {
    const int c = tid;
    double mT[8], mH[8], mW[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mT[i] = shT[i][c] / 64.0;
      mH[i] = shH[i][c] / 64.0;
      mW[i] = shW[i][c] / 64.0;
    }
    double muT = 0.0, muH = 0.0, muW = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) { muT += mT[i]; muH += mH[i]; muW += mW[i]; }
    muT /= 8.0; muH /= 8.0; muW /= 8.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double dT = mT[i] - muT, dH = mH[i] - muH, dW = mW[i] - muW;
      vT += dT * dT; vH += dH * dH; vW += dW * dW;
    }
    vT /= 8.0; vH /= 8.0; vW /= 8.0;
  }
  const double sumT = block_reduce(vT, red, OpAdd());
  const double sumH = block_reduce(vH, red, OpAdd());
  const double sumW = block_reduce(vW, red, OpAdd());

  if (tid < 24) {
    const int d = tid >> 3, i = tid & 7;
    double s = 0.0;
    for (int j = 0; j < 8; ++j)
      for (int k = 0; k < 8; ++k) {
        const int tau = d == 0 ? i : j, eta = d == 1 ? i : (d == 0 ? j : k), om = d == 2 ? i : k;
        s += acube[(tau * 8 + eta) * 8 + om];
      }
    aslice[d][i] = s / 64.0;
  }
  __syncthreads();
  if (tid == 0) {
    // zone total from the eight T-slice sums (exact, like the slice sums, for
    // norms within 20 binades of each other, so the grouping does not matter)
    double tot = 0.0;
    for (int i = 0; i < 8; ++i) tot += aslice[0][i] * 64.0;
    double sa[3];
    for (int d = 0; d < 3; ++d) {
      double mu = 0.0;
      for (int i = 0; i < 8; ++i) mu += aslice[d][i];
      mu /= 8.0;
      double s = 0.0;
      for (int i = 0; i < 8; ++i) {
        const double dd = aslice[d][i] - mu;
        s += dd * dd;
      }
      sa[d] = s / 8.0;
    }
    double* z = zstats + ((int64_t)h * g.Z + m) * 8;
    z[0] = sumT / (double)D;
    z[1] = sumH / (double)D;
    z[2] = sumW / (double)D;
    z[3] = sa[0];
    z[4] = sa[1];
    z[5] = sa[2];
    z[6] = tot / 512.0;
    z[7] = 0.0;
  }
}

// One workgroup per head: density normalisation, audio coupling and g_d.
__global__ __launch_bounds__(1024) void zone_finalize_kernel(Geometry g, prism_params p, double* __restrict__ zstats,
                                                             double* __restrict__ gout, double* __restrict__ rho) {
  __shared__ double red[16];
  const int h = blockIdx.x;
  double* zs = zstats + (int64_t)h * g.Z * 8;
  double emax = 0.0, amin = INFINITY, amax = -INFINITY;
  for (int64_t m = threadIdx.x; m < g.Z; m += blockDim.x) {
    const double* z = zs + m * 8;
    const double E = (z[0] + z[1]) + z[2];
    emax = E > emax ? E : emax;
    amin = z[6] < amin ? z[6] : amin;
    amax = z[6] > amax ? z[6] : amax;
  }
  emax = block_reduce(emax, red, OpMax());
  amin = block_reduce(amin, red, OpMin());
  amax = block_reduce(amax, red, OpMax());
  for (int64_t m = threadIdx.x; m < g.Z; m += blockDim.x) {
    double* z = zs + m * 8;
    const double E = (z[0] + z[1]) + z[2];
    const double Sa = (z[3] + z[4]) + z[5];
    const double abar = amax > amin ? (z[6] - amin) / (amax - amin) : 0.0;
    double r[3], vh[3];
    for (int d = 0; d < 3; ++d) {
      r[d] = E > 0.0 ? z[d] / E : 1.0 / 3.0;
      vh[d] = Sa > 0.0 ? z[3 + d] / Sa : 1.0 / 3.0;
    }
    double* go = gout + ((int64_t)h * g.Z + m) * 3;
    for (int d = 0; d < 3; ++d) {
      double x;
      if (p.variant & PRISM_VARIANT_VISUAL_ONLY) x = r[d];
      else if (p.variant & PRISM_VARIANT_AUDIO_ONLY) x = abar * vh[d];
      else x = r[d] + abar * vh[d];
      go[d] = x + p.eps;
    }
    double rh = emax > 0.0 ? E / emax : 0.0;
    if ((p.variant & PRISM_VARIANT_RHO_MAX_AUDIO) && abar > rh) rh = abar;
    rho[(int64_t)h * g.Z + m] = rh;
    z[7] = abar;
  }
}

// ---------------------------------------------------------------------------
// shape planning
// ---------------------------------------------------------------------------
__device__ int choose_shape(const double* gm, double rho, const prism_params& p) {
  if (p.variant & PRISM_VARIANT_FIXED_SHAPE) return p.fixed_shape;
  const int vol = rho < p.tau256 ? 256 : (rho < p.tau128 ? 128 : 64);
  double lg[3];
  for (int d = 0; d < 3; ++d) lg[d] = log2(gm[d]);
  const double S = log2((double)vol);
  const double c = (S + 0.5 * ((lg[0] + lg[1]) + lg[2])) / 3.0;
  double ell[3];
  for (int d = 0; d < 3; ++d) ell[d] = -0.5 * lg[d] + c;
  int best = -1;
  double bestd = 0.0;
  for (int s = 0; s < kNumShapes; ++s) {
    if (c_shapes.vol[s] != vol) continue;
    double dd[3];
    for (int d = 0; d < 3; ++d) {
      const int e = c_shapes.e[s][d];
      const double le = e == 2 ? 1.0 : (e == 4 ? 2.0 : 3.0);
      dd[d] = le - ell[d];
    }
    const double dist = (dd[0] * dd[0] + dd[1] * dd[1]) + dd[2] * dd[2];
    if (best < 0 || dist < bestd) { best = s; bestd = dist; }
  }
  return best;
}

// One workgroup per head: shapes, block starts (a scan of blocks per zone) and
// the block count.
__global__ __launch_bounds__(1024) void plan_kernel(Geometry g, prism_params p, const double* __restrict__ gin,
                                                    const double* __restrict__ rho, uint8_t* __restrict__ shape_id,
                                                    int32_t* __restrict__ blk_start, int32_t* __restrict__ n_blocks) {
  __shared__ int scan[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
  int carry = 0;
  for (int64_t m0 = 0; m0 < g.Z; m0 += blockDim.x) {
    const int64_t m = m0 + tid;
    int sid = 0, nbz = 0;
    if (m < g.Z) {
      sid = choose_shape(gin + ((int64_t)h * g.Z + m) * 3, rho[(int64_t)h * g.Z + m], p);
      nbz = kZoneTokens / c_shapes.vol[sid];
      shape_id[(int64_t)h * g.Z + m] = (uint8_t)sid;
    }
    scan[tid] = nbz;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int x = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int base = carry + scan[tid] - nbz;
    if (m < g.Z) {
      const int step = c_shapes.vol[sid] / kTile;
      for (int b = 0; b < nbz; ++b) bs[base + b] = (int32_t)(m * (kZoneTokens / kTile) + b * step);
    }
    carry += scan[blockDim.x - 1];
    __syncthreads();
  }
  for (int64_t b = carry + tid; b <= g.tiles; b += blockDim.x) bs[b] = (int32_t)g.tiles;
  if (tid == 0) n_blocks[h] = carry;
}

// perm[p] for every block-order position p.
__global__ __launch_bounds__(256) void perm_kernel(Geometry g, const uint8_t* __restrict__ shape_id,
                                                   int32_t* __restrict__ perm) {
  const int h = blockIdx.y;
  const int64_t pidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (pidx >= g.N) return;
  const int64_t m = pidx / kZoneTokens;
  const int q = (int)(pidx % kZoneTokens);
  const int sid = shape_id[(int64_t)h * g.Z + m];
  const int bT = c_shapes.e[sid][0], bH = c_shapes.e[sid][1], bW = c_shapes.e[sid][2];
  const int vol = c_shapes.vol[sid];
  const int lb = q / vol, e = q % vol;
  const int nH = kZone / bH, nW = kZone / bW;
  const int it = lb / (nH * nW), ih = (lb / nW) % nH, iw = lb % nW;
  const int tau = e / (bH * bW), eta = (e / bW) % bH, om = e % bW;
  const int znh = g.H / kZone, znw = g.W / kZone;
  const int64_t zt = m / (znh * znw), zh = (m / znw) % znh, zw = m % znw;
  const int64_t t = zt * kZone + it * bT + tau, hh = zh * kZone + ih * bH + eta, w = zw * kZone + iw * bW + om;
  perm[(int64_t)h * g.N + pidx] = (int32_t)((t * g.H + hh) * g.W + w);
}

}  // namespace

hipError_t launch_zone_stats(const Geometry& g, const prism_params& p, const uint16_t* v, const float* a,
                             double* zstats, double* gout, double* rho, hipStream_t s) {
  dim3 grid((unsigned)g.Z, (unsigned)g.heads);
  if (g.D == 128) hipLaunchKernelGGL(zone_stats_kernel<128>, grid, dim3(256), 0, s, g, v, a, zstats);
  else hipLaunchKernelGGL(zone_stats_kernel<64>, grid, dim3(256), 0, s, g, v, a, zstats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zone_finalize_kernel, dim3(g.heads), dim3(1024), 0, s, g, p, zstats, gout, rho);
  return hipGetLastError();
}

hipError_t launch_plan_shapes(const Geometry& g, const prism_params& p, const double* gin, const double* rho,
                              uint8_t* shape_id, int32_t* perm, int32_t* blk_start, int32_t* n_blocks,
                              hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(g.heads), dim3(1024), 0, s, g, p, gin, rho, shape_id, blk_start, n_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((g.N + 255) / 256), (unsigned)g.heads);
  hipLaunchKernelGGL(perm_kernel, grid, dim3(256), 0, s, g, shape_id, perm);
  return hipGetLastError();
}

}  // namespace prism

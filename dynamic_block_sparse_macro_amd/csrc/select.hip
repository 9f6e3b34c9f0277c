// Token permutation, block pooling and hybrid Top-k / Top-p block selection.
//
// Prism (sd114.wiki post), 工作原理 step 4: tokens are regrouped so that every
// block is contiguous, and results are restored to the T x H x W layout later.
// Prism (pt reading guide), Método 3: key blocks are mean-pooled into
// representatives Kbar_j and scored against the (mean-pooled) query blocks; the
// block probabilities P_i give S_i = Top-k(P_i, k) U Top-p(P_i, p).
//
// Block means and scores are float64 (the sums of bfloat16 inputs are exact);
// every row is sorted in LDS (bitonic) by (score descending, index ascending);
// Top-k and Top-p are two prefixes of that order, so S_i is the longer one,
// optionally trimmed to a key-token budget that never goes below Top-k.

#include <vector>

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {

namespace {

constexpr int kPanelRows = 2048;   // score rows held in the workspace at once
// threads per selection row: 512 keep four rows' workgroups on a CU (1,024 kept
// two) and took the selection stage from 1.77 to 1.62 ms at 2K
constexpr int kSelectThreads = 512;

// ---------------------------------------------------------------------------
// permutation into the operand layout (+ float64 tile sums)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void permute_kernel(Geometry g, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ perm, uint16_t* __restrict__ xp,
                                                      double* __restrict__ tile_sums) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int LD = D + 8;          // padded LDS row
  __shared__ __attribute__((aligned(16))) uint16_t tb[kTile * LD];
  const int64_t tile = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t p0 = (int64_t)h * g.N + tile * kTile;
  uint16_t* rows = xp + p0 * D;
  for (int c = tid; c < kTile * CH; c += 256) {
    const int r = c / CH, k = c % CH;
    const int64_t n = perm ? (int64_t)perm[p0 + r] : tile * kTile + r;
    const uint4 val = *(const uint4*)(x + (int64_t)h * g.hstride + n * g.tstride + k * 8);
    *(uint4*)(rows + (int64_t)r * D + swz_chunk<D>(r, k) * 8) = val;
    if (tile_sums) *(uint4*)(tb + r * LD + k * 8) = val;
  }
  if (!tile_sums) return;
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    for (int r = 0; r < kTile; ++r) s += (double)bf16_to_f32(tb[r * LD + tid]);
    tile_sums[((int64_t)h * g.tiles + tile) * D + tid] = s;
  }
}

// ---------------------------------------------------------------------------
// Block means from tile sums: Kbar_b = sum over the block's tiles / size.
__global__ void pool_finalize_kernel(Geometry g, const double* __restrict__ tile_sums,
                                     const int32_t* __restrict__ blk_start, const int32_t* __restrict__ n_blocks,
                                     double* __restrict__ pooled) {
  const int h = blockIdx.y;
  const int64_t b = blockIdx.x;
  if (b >= n_blocks[h]) return;
  const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
  const int t0 = bs[b], t1 = bs[b + 1];
  for (int c = threadIdx.x; c < g.D; c += blockDim.x) {
    double s = 0.0;
    for (int t = t0; t < t1; ++t) s += tile_sums[((int64_t)h * g.tiles + t) * g.D + c];
    pooled[((int64_t)h * g.tiles + b) * g.D + c] = s / (double)((t1 - t0) * kTile);
  }
}

// ---------------------------------------------------------------------------
// float64 block scores of one row panel: S[r][j] = scale * qbar[row0+r] . kbar[j]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar,
                                                    int D, int nb, int row0, int rows, double scale,
                                                    double* __restrict__ S, int64_t ldS) {
  __shared__ double As[16][65], Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int r0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  if (r0 >= rows || j0 >= nb) return;
  double acc[4][4] = {};
  // this thread's four elements of each 64 x 16 chunk; the next chunk's are
  // loaded while the current one is multiplied
  double pa[4], pb[4];
  auto load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = threadIdx.x + u * 256, rr = e >> 4, kk = e & 15;
      pa[u] = (r0 + rr < rows) ? qbar[(int64_t)(row0 + r0 + rr) * D + c0 + kk] : 0.0;
      pb[u] = (j0 + rr < nb) ? kbar[(int64_t)(j0 + rr) * D + c0 + kk] : 0.0;
    }
  };
  load(0);
  for (int c0 = 0; c0 < D; c0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = threadIdx.x + u * 256, rr = e >> 4, kk = e & 15;
      As[kk][rr] = pa[u];
      Bs[kk][rr] = pb[u];
    }
    __syncthreads();
    if (c0 + 16 < D) load(c0 + 16);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[kk][ty * 4 + i]; bv[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + ty * 4 + i, c = j0 + tx * 4 + j;
      if (r < rows && c < nb) S[(int64_t)r * ldS + c] = scale * acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// per-row selection
// ---------------------------------------------------------------------------
// Sort key: the score's order-preserving bits, complemented for descending
// order, cut to 48 bits, then the 16-bit block index (ascending on ties).
__device__ __forceinline__ uint64_t desc_key(double s, int j) {
  uint64_t u = (uint64_t)__double_as_longlong(s);
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return ((~u) & 0xFFFFFFFFFFFF0000ull) | (uint64_t)j;
}

template <typename T>
__device__ T block_exclusive_scan(T x, T* wtot, T* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  T inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) wtot[wid] = inc;
  __syncthreads();
  T off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wid) off += wtot[w];
    tot += wtot[w];
  }
  *total = tot;
  return off + inc - x;
}

// The rank-th smallest (1-based) of the distinct keys keys[0, nb): eight
// passes over 8-bit digits, most significant first, each counting the keys
// that still match the digits fixed so far in an LDS histogram.
__device__ uint64_t radix_select(const uint64_t* keys, int nb, int rank, int* hist, int* sel) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += nt) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < nb; j += nt) {
      const uint64_t k = keys[j];
      if ((k & pmask) == prefix) atomicAdd(&hist[(int)((k >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid < 64) {   // one wave: the digit whose bucket holds the rank-th key
      int c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[4 * tid + i];
        sum += c[i];
      }
      int inc = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (tid >= o) inc += y;
      }
      const int exc = inc - sum;
      if (rank > exc && rank <= inc) {
        int r = rank - exc, b = 4 * tid + 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (r <= c[i]) {
            b = 4 * tid + i;
            break;
          }
          r -= c[i];
        }
        sel[0] = b;
        sel[1] = r;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sel[0] << shift;
    pmask |= 255ull << shift;
    rank = sel[1];
    __syncthreads();   // sel and hist are rewritten by the next pass
  }
  return prefix;
}

constexpr int kSelectMaxKeysPerThread = 16384 / kSelectThreads;   // the largest row, in LDS

__global__ __launch_bounds__(kSelectThreads) void select_kernel(const double* __restrict__ S, int64_t ldS, int nb, int npow2,
                                                      int row0, const int32_t* __restrict__ bs, int top_k,
                                                      double top_p, double cap, int64_t N, int variant,
                                                      uint32_t* __restrict__ bitmap, int nbw,
                                                      int32_t* __restrict__ row_len) {
  extern __shared__ __attribute__((aligned(16))) uint64_t keys[];
  uint32_t* bits = (uint32_t*)(keys + npow2);
  __shared__ double redd[16];
  __shared__ int64_t redl[16];
  __shared__ int redi[16];
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const double* srow = S + (int64_t)r * ldS;

  double mx = -INFINITY;
  for (int j = tid; j < nb; j += nt) mx = fmax(mx, srow[j]);
  mx = block_reduce(mx, redd, OpMax());
  double z = 0.0;
  for (int j = tid; j < npow2; j += nt) {
    if (j < nb) {
      const double s = srow[j];
      z += exp(s - mx);
      keys[j] = desc_key(s, j);
    } else {
      keys[j] = ~0ull;
    }
  }
  for (int w = tid; w < nbw; w += nt) bits[w] = 0u;
  const double Z = block_reduce(z, redd, OpAdd());

  // Under a density cap only the first U / 64 positions of the sorted order
  // can be selected (every block holds at least one 64-token tile), besides
  // the top k: the M smallest keys are found by a radix select, moved to the
  // front and sorted; the rest is never read.  The sorted prefix is the same
  // as that of a sort of the whole row.
  int nsort = npow2, nvalid = nb;
  if (cap < 1.0) {
    const int64_t U = (int64_t)floor(cap * (double)N);
    const int mcap = (int)(U / kTile < (int64_t)nb ? U / kTile : (int64_t)nb);
    const int M = max(min(top_k, nb), mcap);
    int m2 = 1;
    while (m2 < M) m2 <<= 1;
    if (m2 < npow2 && M > 0 && nb <= kSelectMaxKeysPerThread * nt) {   // (every row fits: N <= 2^20)
      __shared__ int s_hist[256], s_sel[2], s_cnt;
      const uint64_t T = radix_select(keys, nb, M, s_hist, s_sel);
      uint64_t kv[kSelectMaxKeysPerThread];
#pragma unroll
      for (int i = 0; i < kSelectMaxKeysPerThread; ++i) {
        const int j = tid + i * nt;
        kv[i] = j < nb ? keys[j] : ~0ull;
      }
      if (tid == 0) s_cnt = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSelectMaxKeysPerThread; ++i)
        if (tid + i * nt < nb && kv[i] <= T) keys[atomicAdd(&s_cnt, 1)] = kv[i];
      for (int q = M + tid; q < m2; q += nt) keys[q] = ~0ull;
      nsort = m2;
      nvalid = M;
    }
  }

  // bitonic sort, ascending
  for (int k = 2; k <= nsort; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      __syncthreads();
      for (int t = tid; t < (nsort >> 1); t += nt) {
        const int i = 2 * t - (t & (jj - 1));
        const int ixj = i + jj;
        const uint64_t a = keys[i], b = keys[ixj];
        const bool up = (i & k) == 0;
        if ((a > b) == up) { keys[i] = b; keys[ixj] = a; }
      }
    }
  }
  __syncthreads();

  // prefix mass C(n) and prefix key tokens T(n) in sorted order
  // (chunks over the whole row, so that the sums over the first positions are
  // grouped as in a full sort)
  const int chunk = (nb + nt - 1) / nt;
  const int r0 = tid * chunk, r1 = min(nvalid, r0 + chunk);
  double pl = 0.0;
  int64_t tl = 0;
  for (int q = r0; q < r1; ++q) {
    const int j = (int)(keys[q] & 0xFFFFu);
    pl += exp(srow[j] - mx) / Z;
    tl += (int64_t)(bs[j + 1] - bs[j]) * kTile;
  }
  double ptot;
  int64_t ttot;
  double poff = block_exclusive_scan(pl, redd, &ptot);
  int64_t toff = block_exclusive_scan(tl, redl, &ttot);
  const int64_t U = (int64_t)floor(cap * (double)N);
  int np_c = nb, ncap_c = 0;
  for (int q = r0; q < r1; ++q) {
    const int j = (int)(keys[q] & 0xFFFFu);
    poff += exp(srow[j] - mx) / Z;
    toff += (int64_t)(bs[j + 1] - bs[j]) * kTile;
    if (poff >= top_p && np_c == nb) np_c = q + 1;
    if (toff <= U) ++ncap_c;
  }
  int n_p = block_reduce(np_c, redi, OpMin());
  int n_cap = block_reduce(ncap_c, redi, OpAdd());
  if (top_p >= 1.0) n_p = nb;
  if (cap >= 1.0) n_cap = nb;
  const int n_k = top_k < nb ? top_k : nb;
  int L;
  if (variant & PRISM_VARIANT_TOPK_ONLY) L = n_k;
  else if (variant & PRISM_VARIANT_TOPP_ONLY) L = max(1, min(n_p, n_cap));
  else L = max(n_k, min(n_p, n_cap));

  __syncthreads();
  for (int q = tid; q < L; q += nt) {
    const int j = (int)(keys[q] & 0xFFFFu);
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t* brow = bitmap + (int64_t)(row0 + r) * nbw;
  for (int w = tid; w < nbw; w += nt) brow[w] = bits[w];
  if (tid == 0) row_len[row0 + r] = L;
}

// Exclusive scan of per-head lengths into local pointers; tail entries repeat
// the total.  One workgroup per head.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ len, int64_t len_stride,
                                                    const int32_t* __restrict__ n_blocks, int64_t tiles,
                                                    int32_t* __restrict__ ptr, int32_t* __restrict__ total) {
  __shared__ int wt[16];
  const int h = blockIdx.x, nb = n_blocks[h];
  const int32_t* l = len + (int64_t)h * len_stride;
  int32_t* p = ptr + (int64_t)h * (tiles + 1);
  int carry = 0;
  for (int i0 = 0; i0 < nb; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    const int x = i < nb ? l[i] : 0;
    int tot;
    const int ex = block_exclusive_scan(x, wt, &tot);
    if (i < nb) p[i] = carry + ex;
    carry += tot;
  }
  for (int64_t i = nb + threadIdx.x; i <= tiles; i += blockDim.x) p[i] = carry;
  if (threadIdx.x == 0) total[h] = carry;
}

__device__ __forceinline__ int64_t head_base(const int32_t* total, int h) {
  int64_t b = 0;
  for (int i = 0; i < h; ++i) b += total[i];
  return b;
}

// Query-major column lists, ascending, from the bitmap rows.
__global__ __launch_bounds__(64) void emit_rows_kernel(const uint32_t* __restrict__ bitmap, int64_t head_bitmap,
                                                       int nbw, const int32_t* __restrict__ n_blocks,
                                                       const int32_t* __restrict__ ptr, int64_t tiles,
                                                       const int32_t* __restrict__ total, int32_t* __restrict__ col) {
  const int h = blockIdx.y, i = blockIdx.x, lane = threadIdx.x;
  if (i >= n_blocks[h]) return;
  const uint32_t* brow = bitmap + h * head_bitmap + (int64_t)i * nbw;
  int64_t out = head_base(total, h) + ptr[(int64_t)h * (tiles + 1) + i];
  for (int w0 = 0; w0 < nbw; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = w < nbw ? brow[w] : 0u;
    const int c = __popc(word);
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    int64_t pos = out + inc - c;
    while (word) {
      const int b = __ffs(word) - 1;
      word &= word - 1;
      col[pos++] = w * 32 + b;
    }
    out += __shfl(inc, 63, 64);
  }
}

constexpr int kTRows = 256;   // rows of the selection bitmap per transpose chunk

// Key-major index from the selection bitmap, in chunks of kTRows query-block
// rows: one wave per (32-column word, row chunk, head).  Count pass (fill =
// false): t_cnt[h][c][j] = entries of column j in chunk c.  Fill pass: the
// rows of column j in chunk c go, ascending, to t_col from
// t_ptr[h][j] + t_cnt[h][c][j] on (t_cnt then holds offsets within the
// column, see chunk_scan_kernel).
__global__ __launch_bounds__(64) void transpose_kernel(const uint32_t* __restrict__ bitmap, int64_t head_bitmap,
                                                       int nbw, const int32_t* __restrict__ n_blocks, bool fill,
                                                       int32_t* __restrict__ t_cnt, const int32_t* __restrict__ t_ptr,
                                                       int64_t tiles, const int32_t* __restrict__ total,
                                                       int32_t* __restrict__ t_col) {
  const int h = blockIdx.z, w = blockIdx.x, c = blockIdx.y, lane = threadIdx.x;
  const int nb = n_blocks[h];
  const int i_lo = c * kTRows, i_hi = min(nb, i_lo + kTRows);
  if (w * 32 >= nb || i_lo >= nb) return;
  const uint32_t* bm = bitmap + h * head_bitmap;
  const int nchunk = (int)((tiles + kTRows - 1) / kTRows);
  int32_t* cnt_row = t_cnt + ((int64_t)h * nchunk + c) * tiles;
  const int j = w * 32 + lane;
  int64_t off = 0;
  if (fill && lane < 32 && j < nb) off = head_base(total, h) + t_ptr[(int64_t)h * (tiles + 1) + j] + cnt_row[j];
  int cnt = 0;
  for (int i0 = i_lo; i0 < i_hi; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t word = i < i_hi ? bm[(int64_t)i * nbw + w] : 0u;
    for (int b = 0; b < 32; ++b) {
      const uint64_t m = __ballot((word >> b) & 1u);
      if (fill) {
        const int64_t before = __shfl(off, b, 64);
        if ((word >> b) & 1u) t_col[before + __popcll(m & ((1ull << lane) - 1ull))] = i;
        if (lane == b) off += __popcll(m);
      } else if (lane == b) {
        cnt += __popcll(m);
      }
    }
  }
  if (!fill && lane < 32 && j < nb) cnt_row[j] = cnt;
}

// Per column j: t_cnt[h][c][j] -> exclusive sum over chunks c' < c, and the
// column's length into t_len[h][j].
__global__ __launch_bounds__(256) void chunk_scan_kernel(int32_t* __restrict__ t_cnt,
                                                         const int32_t* __restrict__ n_blocks, int64_t tiles,
                                                         int32_t* __restrict__ t_len) {
  const int h = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int nb = n_blocks[h];
  if (j >= nb) return;
  const int nchunk = (int)((tiles + kTRows - 1) / kTRows);
  const int used = (nb + kTRows - 1) / kTRows;
  int32_t* col = t_cnt + (int64_t)h * nchunk * tiles + j;
  int run = 0;
  for (int c = 0; c < used; ++c) {
    const int x = col[(int64_t)c * tiles];
    col[(int64_t)c * tiles] = run;
    run += x;
  }
  t_len[(int64_t)h * tiles + j] = run;
}

// Final pointers: local offsets plus the head's base in the shared index array.
__global__ void add_base_kernel(const int32_t* __restrict__ local, int32_t* __restrict__ ptr, int64_t tiles,
                                const int32_t* __restrict__ total) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > tiles) return;
  ptr[(int64_t)h * (tiles + 1) + i] = local[(int64_t)h * (tiles + 1) + i] + (int32_t)head_base(total, h);
}

template <typename T>
T* carve(char*& p, size_t count) {
  T* out = (T*)p;
  p += (count * sizeof(T) + 255) & ~(size_t)255;
  return out;
}

}  // namespace

struct SelectWs {
  double* panel;
  uint32_t* bitmap;
  int32_t* row_len;
  int32_t* t_len;
  int32_t* t_cnt;   // [heads][row chunk][column] counts, then offsets within the column
  int32_t* row_local;
  int32_t* t_local;
  int32_t* nnz;
  int32_t* t_nnz;
};

static SelectWs carve_select(const Geometry& g, char* base, size_t* bytes) {
  const int64_t nbmax = g.tiles;
  const int64_t nbw = (nbmax + 31) / 32;
  const int64_t rows = nbmax < kPanelRows ? nbmax : kPanelRows;
  char* p = base;
  SelectWs w;
  w.panel = carve<double>(p, rows * nbmax);
  w.bitmap = carve<uint32_t>(p, g.heads * nbmax * nbw);
  w.row_len = carve<int32_t>(p, g.heads * nbmax);
  w.t_len = carve<int32_t>(p, g.heads * nbmax);
  w.t_cnt = carve<int32_t>(p, g.heads * ((nbmax + kTRows - 1) / kTRows) * nbmax);
  w.row_local = carve<int32_t>(p, g.heads * (nbmax + 1));
  w.t_local = carve<int32_t>(p, g.heads * (nbmax + 1));
  w.nnz = carve<int32_t>(p, g.heads);
  w.t_nnz = carve<int32_t>(p, g.heads);
  *bytes = (size_t)(p - base);
  return w;
}

size_t select_workspace_bytes(const Geometry& g) {
  size_t b = 0;
  carve_select(g, nullptr, &b);
  return b;
}

hipError_t launch_permute(const Geometry& g, const uint16_t* x, const int32_t* perm, uint16_t* xp,
                          double* tile_sums, hipStream_t s) {
  dim3 grid((unsigned)g.tiles, (unsigned)g.heads);
  if (g.D == 128) hipLaunchKernelGGL(permute_kernel<128>, grid, dim3(256), 0, s, g, x, perm, xp, tile_sums);
  else hipLaunchKernelGGL(permute_kernel<64>, grid, dim3(256), 0, s, g, x, perm, xp, tile_sums);
  return hipGetLastError();
}

hipError_t launch_pool_finalize(const Geometry& g, const double* tile_sums, const int32_t* blk_start,
                                const int32_t* n_blocks, double* pooled, hipStream_t s) {
  hipLaunchKernelGGL(pool_finalize_kernel, dim3((unsigned)g.tiles, (unsigned)g.heads), dim3(128), 0, s, g, tile_sums,
                     blk_start, n_blocks, pooled);
  return hipGetLastError();
}

#define PRISM_TRY(x)                 \
  do {                               \
    hipError_t e_ = (x);             \
    if (e_ != hipSuccess) return e_; \
  } while (0)

hipError_t run_selection(const Geometry& g, const prism_params& p, const int32_t* blk_start,
                         const int32_t* n_blocks, const double* qbar, const double* kbar, int32_t* row_ptr,
                         int32_t* col_idx, int64_t col_cap, int32_t* t_row_ptr, int32_t* t_col_idx,
                         int64_t* nnz_host, char* ws, int* status, hipStream_t s) {
  size_t bytes = 0;
  SelectWs w = carve_select(g, ws, &bytes);
  const int64_t nbmax = g.tiles, nbw = (nbmax + 31) / 32;
  *status = PRISM_OK;

  std::vector<int32_t> nbh(g.heads), nz(g.heads);
  PRISM_TRY(hipMemcpyAsync(nbh.data(), n_blocks, sizeof(int32_t) * g.heads, hipMemcpyDeviceToHost, s));
  PRISM_TRY(hipStreamSynchronize(s));
  const double scale = p.scale > 0 ? p.scale : 1.0 / sqrt((double)g.D);

  for (int h = 0; h < g.heads; ++h) {
    const int nb = nbh[h];
    int npow2 = 1;
    while (npow2 < nb) npow2 <<= 1;
    const size_t lds = (size_t)npow2 * 8 + (size_t)nbw * 4;
    const double* qh = qbar + (int64_t)h * g.tiles * g.D;
    const double* kh = kbar + (int64_t)h * g.tiles * g.D;
    const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
    for (int r0 = 0; r0 < nb; r0 += kPanelRows) {
      const int rows = nb - r0 < kPanelRows ? nb - r0 : kPanelRows;
      dim3 grid((unsigned)((nb + 63) / 64), (unsigned)((rows + 63) / 64));
      hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, s, qh, kh, g.D, nb, r0, rows, scale, w.panel,
                         (int64_t)nb);
      PRISM_TRY(hipGetLastError());
      PRISM_TRY(hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(select_kernel, dim3(rows), dim3(kSelectThreads), lds, s, w.panel, (int64_t)nb, nb, npow2, r0, bs,
                         p.top_k, p.top_p, p.density_cap, g.N, p.variant,
                         w.bitmap + (int64_t)h * nbmax * nbw, (int)nbw, w.row_len + (int64_t)h * nbmax);
      PRISM_TRY(hipGetLastError());
    }
  }
  hipLaunchKernelGGL(scan_kernel, dim3(g.heads), dim3(1024), 0, s, w.row_len, nbmax, n_blocks, g.tiles, w.row_local,
                     w.nnz);
  PRISM_TRY(hipGetLastError());
  PRISM_TRY(hipMemcpyAsync(nz.data(), w.nnz, sizeof(int32_t) * g.heads, hipMemcpyDeviceToHost, s));
  PRISM_TRY(hipStreamSynchronize(s));
  int64_t total = 0;
  for (int h = 0; h < g.heads; ++h) {
    nnz_host[h] = nz[h];
    total += nz[h];
  }
  if (total > col_cap || total > (int64_t)INT32_MAX) {
    *status = PRISM_ECAPACITY;
    return hipSuccess;
  }
  hipLaunchKernelGGL(emit_rows_kernel, dim3((unsigned)nbmax, (unsigned)g.heads), dim3(64), 0, s, w.bitmap,
                     nbmax * nbw, (int)nbw, n_blocks, w.row_local, g.tiles, w.nnz, col_idx);
  PRISM_TRY(hipGetLastError());
  dim3 gb((unsigned)((g.tiles + 1 + 255) / 256), (unsigned)g.heads);
  if (t_row_ptr == nullptr) {  // forward-only caller: no key-major index
    hipLaunchKernelGGL(add_base_kernel, gb, dim3(256), 0, s, w.row_local, row_ptr, g.tiles, w.nnz);
    return hipGetLastError();
  }
  const unsigned nchunk = (unsigned)((nbmax + kTRows - 1) / kTRows);
  const dim3 gt((unsigned)nbw, nchunk, (unsigned)g.heads);
  hipLaunchKernelGGL(transpose_kernel, gt, dim3(64), 0, s, w.bitmap, nbmax * nbw, (int)nbw, n_blocks, false, w.t_cnt,
                     w.t_local, g.tiles, w.nnz, t_col_idx);
  PRISM_TRY(hipGetLastError());
  hipLaunchKernelGGL(chunk_scan_kernel, dim3((unsigned)((nbmax + 255) / 256), (unsigned)g.heads), dim3(256), 0, s,
                     w.t_cnt, n_blocks, g.tiles, w.t_len);
  PRISM_TRY(hipGetLastError());
  hipLaunchKernelGGL(scan_kernel, dim3(g.heads), dim3(1024), 0, s, w.t_len, nbmax, n_blocks, g.tiles, w.t_local,
                     w.t_nnz);
  PRISM_TRY(hipGetLastError());
  hipLaunchKernelGGL(transpose_kernel, gt, dim3(64), 0, s, w.bitmap, nbmax * nbw, (int)nbw, n_blocks, true, w.t_cnt,
                     w.t_local, g.tiles, w.t_nnz, t_col_idx);
  PRISM_TRY(hipGetLastError());
  hipLaunchKernelGGL(add_base_kernel, gb, dim3(256), 0, s, w.row_local, row_ptr, g.tiles, w.nnz);
  PRISM_TRY(hipGetLastError());
  hipLaunchKernelGGL(add_base_kernel, gb, dim3(256), 0, s, w.t_local, t_row_ptr, g.tiles, w.t_nnz);
  return hipGetLastError();
}

}  // namespace prism

// Variable-block-size block-sparse flash attention, forward and backward.
//
// Prism (pt reading guide), Método 3: an online-softmax kernel runs attention
// only over the attended set S_i of each query block.  Prism (zh reading guide),
// 常见问题: gradients flow only through the sparse attention on the selected
// blocks.  Prism (sd114.wiki post), 工作原理 step 4: results are restored to the
// original T x H x W layout.
//
// CDNA4 design:
//  * every block is 1, 2 or 4 tiles of 64 tokens, so one code path serves
//    64/128/256-token blocks.  A workgroup (4 waves) owns a pair of 64-token
//    tiles of one zone (query tiles 2p, 2p + 1 in the forward and dQ passes;
//    key tiles in the dK/dV pass, paired by list overlap in key_pairs_kernel);
//    each wave owns 32 rows.  The two tiles of a pair lie in one block or in
//    two 64-token blocks of the same zone; the workgroup walks the union of
//    their block lists and each wave pair computes only the tiles its own list
//    holds;
//  * v_mfma_f32_32x32x16_bf16 for every product, computed transposed
//    (S^T = K Q^T, O^T = V^T P^T, ...) so that the accumulator of one product
//    is, register for register, the B operand of the next;
//  * operand tiles live in HBM exactly as they sit in LDS (row-major, XOR
//    swizzled 16-byte chunks), so staging is an asynchronous copy into LDS
//    (buffer_load_dwordx4 ... lds, addressed from scalar registers),
//    double-buffered behind the MFMA work; the forward's walk is software
//    pipelined inside each wave (S of one tile and PV of the tile two back
//    interleaved with the softmax of the tile between);
//  * operands that need a tile's columns (V^T, K^T, Q^T, dO^T) are read from
//    the same row tiles with the transposing LDS read ds_read_b64_tr_b16;
//  * float32 online softmax in the log2 domain with lazy rescaling (the
//    running maximum moves only when a score exceeds it by 2^8);
//  * the backward runs a query-major pass (dQ) and a key-major pass over the
//    transposed block index (dK, dV): no float atomics, bitwise reproducible;
//  * persistent workgroups: the grid holds as many workgroups as the chip
//    keeps resident, and each takes tile pairs from a work queue, first the
//    queue of its own XCD (one contiguous eighth of every head's pairs, so
//    neighbouring query blocks, which share most key blocks, meet in one L2),
//    then the others.  Rows differ widely in length, so this balances the
//    XCDs and leaves no slot waiting on the dispatcher.  Each queue runs
//    longest work first; when all heads' K/V (or Q/dO) exceed the last-level
//    cache it runs head by head, so that the chip works on one head's
//    operands at a time.

#include <limits.h>

#include <type_traits>

#include "prism_device.h"
#include "prism_internal.h"

namespace prism {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;   // log2 headroom before the running max moves
constexpr int kThreads = 256;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4v;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's global->LDS copies have landed
}

template <int D>
struct TileGeo {
  static constexpr int ROWB = D * 2;            // bytes per row
  static constexpr int BYTES = kTile * ROWB;    // bytes per tile
  static constexpr int CHUNKS = BYTES / 16;     // 16-byte chunks per tile
  // one pipeline stage: two operand tiles, sized to also hold the 128-row
  // output staging area (128 x (D + 8) bf16) of the epilogue
  static constexpr int STAGE = 2 * BYTES + 2048;
};

// The two pipeline stages are separate LDS objects (stage0, stage1) so
// that the compiler can tell the prefetch into one stage from the reads of
// the other; with a single array it makes every read of the current stage
// wait for the prefetch as well, which exposes the full memory latency.
#define PRISM_STAGE(B, s0, s1) ((B) ? (s1) : (s0))

// Copies into LDS go through buffer loads: the copy's base address sits in
// a scalar buffer descriptor (record count = the copy's size), the per-lane
// offset is a loop-invariant vector register and the wave's part of the
// offset a scalar, and M0 (the LDS address) is scalar too, so a copy costs
// no vector ALU work.
constexpr int kRsrcFlags = 0x00020000;   // descriptor word 3: 32-bit data format

// buffer resource covering one contiguous operand tile
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* src) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, TileGeo<D>::BYTES, kRsrcFlags);
}
// copy instructions per wave of one tile copy
template <int D>
constexpr int kCopyOpsOf = TileGeo<D>::CHUNKS / kThreads;
// instruction `op` of this wave's share of an asynchronous tile copy into LDS
template <int D>
__device__ __forceinline__ void dma_tile_op(__amdgpu_buffer_rsrc_t r, char* lds, int op) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int chunk0 = op * kThreads + w * 64;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + chunk0 * 16), 16, lane * 16, chunk0 * 16, 0, 0);
}
// asynchronous copy of one contiguous operand tile into LDS (all 256 threads)
template <int D>
__device__ __forceinline__ void dma_tile(char* lds, const uint16_t* __restrict__ src) {
  const __amdgpu_buffer_rsrc_t r = tile_rsrc<D>(src);
#pragma unroll
  for (int op = 0; op < kCopyOpsOf<D>; ++op) dma_tile_op<D>(r, lds, op);
}
// asynchronous copy of 64 floats (one per tile row) into LDS
// (called by one whole wave; lane l copies float l)
__device__ __forceinline__ void dma_vec64(char* lds, const float* __restrict__ src) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, 64 * 4, kRsrcFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, lane * 4, 0, 0, 0);
}

// Per-lane LDS byte offsets inside an operand tile.  With the XOR swizzle of
// swz_chunk the chunk a lane touches depends only on its row modulo 16, so one
// set of offsets serves every 32-row block of a tile (added as immediates).
//  row[s]    16-byte row read: row l32, columns 16 s + 8 g .. + 7 (A or B
//            operand whose lanes index tile rows)
//  tr[h][u]  8-byte transposing read of rows 8 h + 4 g + {0..3} (plus the
//            32-row / 16-row block base), columns 32 u + 16 (l/16 & 1) + 4 (l%16 & 3)
//            .. + 3: in each 16-lane group lane i then holds column
//            32 u + 16 (l/16 & 1) + i of those four rows.
template <int D>
struct LaneOff {
  static constexpr int ROWB = D * 2;
  int row[D / 16];
  int tr[2][D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, l32 = lane & 31, gg = lane >> 4, a = lane & 15;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) row[s] = l32 * ROWB + swz_chunk<D>(l32, 2 * s + g) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
        const int r = 8 * h + 4 * g + (a >> 2);
        const int col = 32 * u + 16 * (gg & 1) + 4 * (a & 3);
        tr[h][u] = r * ROWB + swz_chunk<D>(r, col >> 3) * 16 + (col & 7) * 2;
      }
  }
};

// operand whose lanes index tile rows 32 kk + l32 (k-step s over columns)
template <int D>
__device__ __forceinline__ bf16x8 lds_row(const char* tile, const LaneOff<D>& o, int kk, int s) {
  return *(const bf16x8*)(tile + kk * 32 * LaneOff<D>::ROWB + o.row[s]);
}

// Column operand of a 32x32x16 MFMA from a row tile: lane l takes column
// 32 u + l % 32 and, for k-step (kk, hh), rows 32 kk + 16 hh + 4 g + {0..3}
// and the same + 8 (g = l / 32): the register order of a 32x32 accumulator
// used as the B operand of the next product.
template <int D>
__device__ __forceinline__ bf16x8 lds_col(const char* tile, const LaneOff<D>& o, int u, int kk, int hh) {
  const char* p = tile + (32 * kk + 16 * hh) * LaneOff<D>::ROWB;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + o.tr[0][u]));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + o.tr[1][u]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// register operand from an operand tile in HBM (row r, swizzled layout)
template <int D>
__device__ __forceinline__ bf16x8 ld_row(const uint16_t* __restrict__ tile, int r, int s, int g) {
  return *(const bf16x8*)(tile + r * D + swz_chunk<D>(r, 2 * s + g) * 8);
}

// accumulator (rows = D dims in tiles of 32, column = the lane's row) -> bf16
// into a padded LDS staging area at row r
template <int D>
__device__ __forceinline__ void acc_to_stage(uint16_t* st, const floatx16* acc, int r, int g, float mul) {
  constexpr int LD = D + 8;
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * u + 8 * j + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(acc[u][4 * j] * mul, acc[u][4 * j + 1] * mul);
      v.y = pack_bf16x2(acc[u][4 * j + 2] * mul, acc[u][4 * j + 3] * mul);
      *(uint2*)(st + r * LD + d0) = v;
    }
}

// the same rows' low parts: bf16(x - hi) with hi = bf16(x), x = acc * mul,
// so that hi + lo carries O to about 16 significant bits
template <int D>
__device__ __forceinline__ void acc_to_stage_lo(uint16_t* st, const floatx16* acc, int r, int g, float mul) {
  constexpr int LD = D + 8;
  auto lo = [](float x) { return x - bf16_to_f32(f32_to_bf16(x)); };
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * u + 8 * j + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(lo(acc[u][4 * j] * mul), lo(acc[u][4 * j + 1] * mul));
      v.y = pack_bf16x2(lo(acc[u][4 * j + 2] * mul), lo(acc[u][4 * j + 3] * mul));
      *(uint2*)(st + r * LD + d0) = v;
    }
}

// write 128 staged rows to 128 contiguous rows of D (block order)
template <int D>
__device__ __forceinline__ void store_pair_rows(const uint16_t* st, uint16_t* __restrict__ out) {
  constexpr int CH = D / 8, LD = D + 8;
  for (int c = threadIdx.x; c < 2 * kTile * CH; c += kThreads) {
    const int r = c / CH, k = c % CH;
    *(uint4*)(out + (int64_t)r * D + k * 8) = *(const uint4*)(st + r * LD + k * 8);
  }
}

// write 128 staged rows (two tiles) to THW rows through perm
template <int D>
__device__ __forceinline__ void store_pair_thw(const uint16_t* st, uint16_t* __restrict__ out, const Geometry& g,
                                               int h, int64_t tile0, const int32_t* __restrict__ perm) {
  constexpr int CH = D / 8, LD = D + 8;
  const int64_t p0 = (int64_t)h * g.N + tile0 * kTile;
  for (int c = threadIdx.x; c < 2 * kTile * CH; c += kThreads) {
    const int r = c / CH, k = c % CH;
    const int64_t n = perm ? (int64_t)perm[p0 + r] : tile0 * kTile + r;
    *(uint4*)(out + (int64_t)h * g.hstride + n * g.tstride + k * 8) = *(const uint4*)(st + r * LD + k * 8);
  }
}

// the same for two tiles anywhere in the head: staged rows 0..63 are tile
// ta, rows 64..127 tile tb
template <int D>
__device__ __forceinline__ void store_tiles_thw(const uint16_t* st, uint16_t* __restrict__ out, const Geometry& g,
                                                int h, int64_t ta, int64_t tb, const int32_t* __restrict__ perm) {
  constexpr int CH = D / 8, LD = D + 8;
  for (int c = threadIdx.x; c < 2 * kTile * CH; c += kThreads) {
    const int r = c / CH, k = c % CH;
    const int64_t p = (r < kTile ? ta : tb) * kTile + (r & (kTile - 1));
    const int64_t n = perm ? (int64_t)perm[(int64_t)h * g.N + p] : p;
    *(uint4*)(out + (int64_t)h * g.hstride + n * g.tstride + k * 8) = *(const uint4*)(st + r * LD + k * 8);
  }
}

// A window on an ascending block list: lane i holds entry base + i (block
// index and its tile range, loaded together), so the iterator reads the next
// block with a lane read instead of two dependent memory round trips, and
// refills once per 64 blocks.
struct ListWin {
  const int32_t* idx;
  int n, base, pos;
  int vj, vs, ve;   // per lane: block index, first tile, end tile of entry base + lane

  __device__ __forceinline__ void refill(const int32_t* __restrict__ bs) {
    base = pos;
    const int e = base + (int)(threadIdx.x & 63);
    vj = INT_MAX;
    vs = ve = 0;
    if (e < n) {
      vj = idx[e];
      vs = bs[vj];
      ve = bs[vj + 1];
    }
  }
  // block index at the current position (INT_MAX past the end)
  __device__ __forceinline__ int peek(const int32_t* __restrict__ bs) {
    if (pos >= n) return INT_MAX;
    if (pos - base >= 64) refill(bs);
    return __builtin_amdgcn_readlane(vj, pos - base);
  }
  __device__ __forceinline__ int start() const { return __builtin_amdgcn_readlane(vs, pos - base); }
  __device__ __forceinline__ int end() const { return __builtin_amdgcn_readlane(ve, pos - base); }
};

// Walks the tiles of the union of two ascending block lists (one per tile of
// the pair), in ascending block order, with a flag per list.  Uniform across
// the workgroup.
struct PairIter {
  ListWin a, b;
  const int32_t* bs;
  bool same, dense;
  int kt, kt_end;
  bool ua, ub;

  __device__ bool next(int& tile, bool& use_a, bool& use_b) {
    if (kt >= kt_end) {
      if (dense) return false;
      const int ja = a.peek(bs);
      const int jb = same ? ja : b.peek(bs);
      const int j = ja < jb ? ja : jb;
      if (j == INT_MAX) return false;
      ua = ja == j;
      ub = jb == j;
      if (ua) {
        kt = a.start();
        kt_end = a.end();
        ++a.pos;
      } else {
        kt = b.start();
        kt_end = b.end();
      }
      if (!same && ub) ++b.pos;
    }
    tile = kt++;
    use_a = ua;
    use_b = ub;
    return true;
  }
};

// the key (or query) lists of tiles ta and tb (a work item's two tiles) of head h
__device__ __forceinline__ PairIter make_iter(const Geometry& g, int h, int ta, int tb, const int32_t* __restrict__ blk_start,
                                              const int32_t* __restrict__ n_blocks,
                                              const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx) {
  PairIter it;
  it.kt = 0;
  it.kt_end = 0;
  it.ua = it.ub = true;
  if (ptr == nullptr) {          // dense: every tile, both lists
    it.dense = true;
    it.same = true;
    it.kt_end = (int)g.tiles;
    it.bs = nullptr;
    it.a.n = it.b.n = 0;
    return it;
  }
  it.dense = false;
  const int32_t* bs = blk_start + (int64_t)h * (g.tiles + 1);
  const int nbk = n_blocks[h];
  const int ba = block_of_tile(bs, nbk, ta);
  const int bb = block_of_tile(bs, nbk, tb);
  const int32_t* rp = ptr + (int64_t)h * (g.tiles + 1);
  it.bs = bs;
  it.same = ba == bb;
  it.a.idx = idx + rp[ba];
  it.a.n = rp[ba + 1] - rp[ba];
  it.a.pos = 0;
  it.a.refill(bs);
  it.b.idx = idx + rp[bb];
  it.b.n = rp[bb + 1] - rp[bb];
  it.b.pos = 0;
  if (!it.same) it.b.refill(bs);
  return it;
}

template <int B>
using Parity = std::integral_constant<int, B>;

// Work queues of a persistent launch: queue positions 0..total-1 split into
// 8 contiguous ranges, one per XCD, each with a counter in cnt[0..7] (zero at
// launch); order[pos] (NULL = identity) is the work item at a position.  A
// workgroup drains the queue of the XCD it runs on, then the others in turn;
// every call on an exhausted queue moves on, so each workgroup makes at most
// total + 8 attempts and always ends.
struct WorkQueue {
  int* cnt;
  const int32_t* order;
  int total, per, xq, qi;

  __device__ __forceinline__ void init(int* c, const int32_t* ord, int n) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    cnt = c;
    order = ord;
    total = n;
    per = (n + 7) / 8;
    xq = (int)(x & 7);
    qi = 0;
  }
  // next work item or -1 (called by one thread)
  __device__ __forceinline__ int next() {
    while (qi < 8) {
      const int q = (xq + qi) & 7;
      const int lo = q * per;
      const int hi = lo + per < total ? lo + per : total;
      if (lo < hi) {
        const int i = atomicAdd(&cnt[q], 1);
        if (lo + i < hi) return order ? order[lo + i] : lo + i;
      }
      ++qi;
    }
    return -1;
  }
};

// ---- queue order: head by head, longest work first, inside each XCD's range ----
// Cost of a work item (a pair of 64-token tiles): the key (or query) tiles
// its lists walk, estimated as the longer of the two lists in tiles.

// tiles[h][b]: sum of the sizes (in tiles) of the blocks in list b of head h
__global__ __launch_bounds__(256) void list_tiles_kernel(const int32_t* __restrict__ blk_start,
                                                          const int32_t* __restrict__ n_blocks,
                                                          const int32_t* __restrict__ ptr,
                                                          const int32_t* __restrict__ idx, int64_t tiles,
                                                          int32_t* __restrict__ out) {
  const int h = blockIdx.y;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= n_blocks[h]) return;
  const int32_t* bs = blk_start + (int64_t)h * (tiles + 1);
  const int32_t* rp = ptr + (int64_t)h * (tiles + 1);
  int sum = 0;
  for (int e = rp[b] + lane; e < rp[b + 1]; e += 64) {
    const int j = idx[e];
    sum += bs[j + 1] - bs[j];
  }
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) out[(int64_t)h * tiles + b] = sum;
}

// Tile-weighted size of the intersection of the lists of blocks ba and bb
// (ascending block indices): one wave, every lane gets the sum.
__device__ __forceinline__ int list_overlap(const int32_t* __restrict__ bs, const int32_t* __restrict__ rp,
                                            const int32_t* __restrict__ idx, int ba, int bb) {
  const int lane = threadIdx.x & 63;
  const int32_t* B = idx + rp[bb];
  const int nB = rp[bb + 1] - rp[bb];
  int sum = 0;
  for (int e = rp[ba] + lane; e < rp[ba + 1]; e += 64) {
    const int j = idx[e];
    int lo = 0, hi = nB;   // first position with B[pos] >= j
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (B[mid] < j) lo = mid + 1; else hi = mid;
    }
    if (lo < nB && B[lo] == j) sum += bs[j + 1] - bs[j];
  }
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  return sum;
}

// Key-tile pairs of the key-major pass, one workgroup per 8-tile zone, one
// wave per candidate pair.  A zone of eight one-tile blocks (volume 64)
// pairs its tiles either as (2i, 2i + 1) or as (i, i + 4), whichever walks
// fewer union steps: the two tiles of a pair share a work item, so the query
// tiles in one list but not the other leave half of the workgroup idle.
// Other zones keep (2i, 2i + 1), which lie in one block and share its list.
// pairs[h][p] = (ta, tb); cost[h][p] = the union's length in tiles.
__global__ __launch_bounds__(512) void key_pairs_kernel(const int32_t* __restrict__ blk_start,
                                                        const int32_t* __restrict__ n_blocks,
                                                        const int32_t* __restrict__ ptr,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ list_tiles, int64_t tiles,
                                                        int32_t* __restrict__ pairs, int32_t* __restrict__ cost) {
  __shared__ int s_u[8];   // union lengths: pairs (2i, 2i + 1), then (i, i + 4)
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 8;
  const int wv = threadIdx.x >> 6;   // one wave per candidate pair
  const int32_t* bs = blk_start + (int64_t)h * (tiles + 1);
  const int32_t* rp = ptr + (int64_t)h * (tiles + 1);
  const int32_t* lt = list_tiles + (int64_t)h * tiles;
  const int nb = n_blocks[h];
  const int b0 = block_of_tile(bs, nb, t0);
  const bool single = block_of_tile(bs, nb, t0 + 7) - b0 == 7;
  auto uni = [&](int ta, int tb) {
    const int ba = single ? b0 + ta : block_of_tile(bs, nb, t0 + ta);
    const int bb = single ? b0 + tb : block_of_tile(bs, nb, t0 + tb);
    return ba == bb ? lt[ba] : lt[ba] + lt[bb] - list_overlap(bs, rp, idx, ba, bb);
  };
  if (wv < 4 || single) {
    const int u = wv < 4 ? uni(2 * wv, 2 * wv + 1) : uni(wv - 4, wv);
    if ((threadIdx.x & 63) == 0) s_u[wv] = u;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const int i = threadIdx.x;
    const bool by4 = single && s_u[4] + s_u[5] + s_u[6] + s_u[7] < s_u[0] + s_u[1] + s_u[2] + s_u[3];
    const int64_t p = (int64_t)h * (tiles / 2) + t0 / 2 + i;
    const int ta = by4 ? i : 2 * i;
    pairs[2 * p] = t0 + ta;
    pairs[2 * p + 1] = t0 + ta + (by4 ? 4 : 1);
    cost[p] = by4 ? s_u[4 + i] : s_u[i];
  }
}

constexpr int kSortMax = 4096;   // largest XCD range sorted in LDS
constexpr int64_t kLastLevelCache = 256LL << 20;   // MI355X's memory-side cache, bytes

// Work item at position s of the head-interleaved sequence: the pairs are cut
// into eighths, and each eighth lists every head's pairs of that eighth, head
// by head.  XCD range x then holds eighth x of every head.
__device__ __forceinline__ int seq_item(int s, int npair, int heads) {
  auto a = [&](int e) { return (e * npair + 7) / 8; };
  int e = 0;
  while (e < 7 && s >= heads * a(e + 1)) ++e;
  const int c = a(e + 1) - a(e);
  const int r = s - heads * a(e);
  return (r / c) * npair + a(e) + r % c;
}

// order[pos] for the XCD range of this workgroup: head by head (by_head) or
// all heads together, by cost descending inside, ties by position (a bitonic
// sort of 64-bit keys in LDS).  The cost of an item is pair_cost[item] when given, else the longer
// list of its tiles (2 pair, 2 pair + 1).
__global__ __launch_bounds__(1024) void queue_order_kernel(const int32_t* __restrict__ blk_start,
                                                            const int32_t* __restrict__ n_blocks,
                                                            const int32_t* __restrict__ list_tiles,
                                                            const int32_t* __restrict__ pair_cost, int64_t tiles,
                                                            int npair, int total, bool by_head,
                                                            int32_t* __restrict__ order) {
  __shared__ uint64_t key[kSortMax];
  const int heads = total / npair;
  const int per = (total + 7) / 8;
  const int lo = blockIdx.x * per;
  const int hi = lo + per < total ? lo + per : total;
  const int n = hi > lo ? hi - lo : 0;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += blockDim.x) {
    uint64_t k = ~0ull;   // padding sorts last
    if (i < n) {
      const int w = seq_item(lo + i, npair, heads);
      const int h = w / npair, pair = w % npair;
      uint32_t cost;
      if (pair_cost != nullptr) {
        cost = (uint32_t)pair_cost[w];
      } else {
        const int32_t* bs = blk_start + (int64_t)h * (tiles + 1);
        const int nb = n_blocks[h];
        const int ba = block_of_tile(bs, nb, 2 * pair);
        const int bb = block_of_tile(bs, nb, 2 * pair + 1);
        const int32_t* lt = list_tiles + (int64_t)h * tiles;
        const int ca = lt[ba], cb = lt[bb];
        cost = (uint32_t)(ca > cb ? ca : cb);
      }
      k = ((uint64_t)(by_head ? h : 0) << 56) | ((uint64_t)(0xffffffu - (cost < 0xffffffu ? cost : 0xffffffu)) << 32) |
          (uint32_t)i;
    }
    key[i] = k;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n2; i += blockDim.x) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint64_t a = key[i], b = key[j];
          if ((a > b) == up) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < n; i += blockDim.x) order[lo + i] = seq_item(lo + (int)(uint32_t)key[i], npair, heads);
}

// the workgroup's next work item (uniform), -1 when all queues are empty
__device__ __forceinline__ int fetch_work(WorkQueue& wq, int* slot) {
  if (threadIdx.x == 0) *slot = wq.next();
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);   // uniform: scalar registers from here on
}

__global__ void zero_kernel(int* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// Workgroup barrier without a memory fence: __syncthreads() would also wait
// for every copy in flight (its release covers LDS written by the copies).
// The loop's LDS reads are all consumed before the barrier and the explicit
// wait before it orders the copies; the empty asm statements keep the
// compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Forward: each wave's walk over the key tiles is software pipelined three
// deep.  Iteration j computes S(j) = K(j) Q^T and the PV product of tile
// j - 2 as one-MFMA chunks (S and PV alternating), and between them the
// softmax of tile j - 1, so the wave's own vector work runs while its matrix
// products execute; the other workgroup on the CU fills the rest.  Stage
// j & 1 holds K(j) and V(j - 2); after the barrier of iteration j the copy of
// K(j + 1) and V(j - 1) goes into the other stage.  Per tile the running
// output takes the same operations in the same order as a walk without the
// pipeline: PV(t - 1) is added, then the rescale decided by the softmax of
// t, then PV(t).
constexpr int kReadAhead = 2;   // forward: chunks between an operand's LDS read and its MFMA
constexpr int kCopyStride = 4;   // forward: chunks between two copy instructions

template <int D, bool DENSE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    Geometry g, float sl2, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_start,
    const int32_t* __restrict__ n_blocks, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    uint16_t* __restrict__ o, uint16_t* __restrict__ o_lo, float* __restrict__ lse, int* __restrict__ cnt,
    const int32_t* __restrict__ order) {
  constexpr int TB = TileGeo<D>::BYTES;
  __shared__ __attribute__((aligned(16))) char stage0[TileGeo<D>::STAGE];   // K(j), V(j - 2) of even j
  __shared__ __attribute__((aligned(16))) char stage1[TileGeo<D>::STAGE];   // K(j), V(j - 2) of odd j
  __shared__ int s_work;
  const int npair = (int)(g.tiles / 2);
  WorkQueue wq;
  wq.init(cnt, order, npair * g.heads);
  for (;;) {
  const int wk = fetch_work(wq, &s_work);
  if (wk < 0) break;
  const int h = wk / npair;
  const int pair = wk % npair;
  const int lane = threadIdx.x & 63, g32 = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const bool second = w >= 2;
  const int64_t hN = (int64_t)h * g.N;
  const int64_t qt = 2 * pair + (second ? 1 : 0);
  const int rloc = 32 * (w & 1) + l32;          // row within the query tile
  const uint16_t* Kb = kp + hN * D;
  const uint16_t* Vb = vp + hN * D;
  LaneOff<D> off;
  off.init(lane);

  bf16x8 qreg[D / 16];
  {
    const uint16_t* Qt = qp + (hN + qt * kTile) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = ld_row<D>(Qt, rloc, s, g32);
  }
  floatx16 oacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[u][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f, r_run = 0.0f;

  PairIter it = make_iter(g, h, 2 * pair, 2 * pair + 1, blk_start, n_blocks, DENSE ? nullptr : row_ptr, col_idx);
  // next tile of the walk: e = it exists, m = this wave's query tile attends
  // to it; past the end t = 0 (tile 0 of the head: the source of copies made
  // only so that every slot a masked product reads holds finite values)
  auto fetch = [&](int& t, bool& e, bool& m) {
    bool ua, ub;
    e = it.next(t, ua, ub);
    m = e && (second ? ub : ua);
    if (!e) t = 0;
  };
  // pipeline state: tiles j (S), j - 1 (softmax, and its V copy), j - 2
  // (PV); the look-ahead tile j + 1, whose K is copied during iteration j
  int tS, t1, tX = 0;
  bool eS, mS, e1, m1, eX = false, mX = false, eP = false;
  fetch(tS, eS, mS);
  fetch(t1, e1, m1);
  dma_tile<D>(stage0, Kb + (int64_t)tS * kTile * D);
  dma_tile<D>(stage0 + TB, Vb);
  floatx16 sc[2][2];   // S^T of the tiles of even / odd index (two 32-key halves)
  bf16x8 pw[2][4];     // their bf16 weights, the B operands of PV
  // the first two iterations run the softmax and PV of tiles -1, -2 masked
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[b2][kk][i] = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[b2][v][i] = (__bf16)0.0f;
  }

  auto step = [&](auto par) {
    constexpr int B = decltype(par)::value, X = B ^ 1;   // parities of j and j - 1
    int t2;
    bool e2, m2;
    fetch(t2, e2, m2);                         // tile j + 2
    wait_dma();                                // this wave's copies of K(j), V(j - 2) have landed
    barrier_nofence();                         // ... and every wave's; stage B ^ 1 is free
    // copies of K(j + 1) and V(j - 1) into the other stage: one copy
    // instruction every kCopyStride chunks of the loop below, so that the
    // first products of the iteration are not queued behind them
    char* const nx = PRISM_STAGE(B ^ 1, stage0, stage1);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc<D>(Kb + (int64_t)t1 * kTile * D);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc<D>(Vb + (int64_t)tX * kTile * D);
    constexpr int kCopyOps = kCopyOpsOf<D>;
    const char* Kt = PRISM_STAGE(B, stage0, stage1);
    const char* Vt = Kt + TB;
    // a wave whose query tile does not attend to a tile still runs its
    // products, masked through the data: that tile's softmax takes the
    // maximum +inf, so its weights are 0 and PV adds exact zeros (the output
    // accumulators never hold -0); the running maximum and sums stay as they are
    const bool doX = eX && mX;
    float alpha = 1.0f, lsum = 0.0f, rsum = 0.0f;
    bool resc = false;
    {
      constexpr int NS = D / 8;   // S products (two 32-key halves x D/16 k-steps)
      constexpr int NC = 2 * NS;  // chunks: S and PV products alternating
      bf16x8 kop[NS], vop[NS];
      auto read = [&](int c) {
        const int i = c >> 1;
        if ((c & 1) == 0) kop[i] = lds_row<D>(Kt, off, i & 1, i >> 1);
        else vop[i] = lds_col<D>(Vt, off, i % (D / 32), i / (2 * (D / 32)), (i / (D / 32)) & 1);
      };
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[B][kk][i] = 0.0f;
#pragma unroll
      for (int c = 0; c < kReadAhead; ++c) read(c);
      float mloc = 0.0f, m_use = 0.0f;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c % kCopyStride == 0 && c / kCopyStride < 2 * kCopyOps) {
          const int ci = c / kCopyStride, tile = ci / kCopyOps;   // tile 0: K(j + 1), 1: V(j - 1)
          dma_tile_op<D>(tile ? rv : rk, nx + tile * TB, ci % kCopyOps);
        }
        if (c + kReadAhead < NC) read(c + kReadAhead);
        const int i = c >> 1;
        if ((c & 1) == 0) sc[B][i & 1] = mfma32(kop[i], qreg[i >> 1], sc[B][i & 1]);
        else {
          const int kk = i / (2 * (D / 32)), hh = (i / (D / 32)) & 1, u = i % (D / 32);
          oacc[u] = mfma32(vop[i], pw[B][kk * 2 + hh], oacc[u]);
        }
        if (c == 0) {
          mloc = sc[X][0][0];
#pragma unroll
          for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sc[X][0][e]);
        } else if (c == 1) {
#pragma unroll
          for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sc[X][1][e]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
          mloc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
          resc = __any(mloc > m_run + kRescale) & doX;
          const float m_new = resc ? fmaxf(m_run, mloc) : m_run;
          alpha = fast_exp2(m_run - m_new);   // used only when resc
          m_run = m_new;
          m_use = doX ? m_run : INFINITY;
        } else {
#pragma unroll
          for (int e = ((c - 2) * 32) / (NC - 2); e < ((c - 1) * 32) / (NC - 2); ++e) {
            const int kk = e >> 4, ii = e & 15;
            const float pv = fast_exp2(__builtin_fmaf(sc[X][kk][ii], sl2, -m_use));
            lsum += pv;
            pw[X][kk * 2 + (ii >> 3)][ii & 7] = (__bf16)pv;
            asm volatile("" : "+v"(lsum));
            if ((e & 7) == 7) {
              const int v = e >> 3;
              rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw[X][v], pw[X][v], 0, 1), ones, rsum, false);
              rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw[X][v], pw[X][v], 2, 3), ones, rsum, false);
              rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw[X][v], pw[X][v], 4, 5), ones, rsum, false);
              rsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw[X][v], pw[X][v], 6, 7), ones, rsum, false);
              asm volatile("" : "+v"(rsum), "+v"(pw[X][v]));
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (resc) {   // rare: the running sums and output move to the new maximum
      l_run *= alpha;
      r_run *= alpha;
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[u][i] *= alpha;
    }
    {
#pragma clang fp contract(off)
      l_run += lsum;
      r_run += rsum;
    }
    eP = eX;
    eX = eS;
    mX = mS;
    tX = tS;
    eS = e1;
    mS = m1;
    tS = t1;
    t1 = t2;
    e1 = e2;
    m1 = m2;
  };
  while (eS || eX || eP) {
    step(Parity<0>{});
    if (!(eS || eX || eP)) break;
    step(Parity<1>{});
  }
  wait_dma();   // the last copies have landed before stage0 becomes the staging area
  __syncthreads();

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / (r_run + __shfl_xor(r_run, 32, 64));
  if (lse != nullptr && g32 == 0) lse[hN + qt * kTile + rloc] = (m_run + __log2f(l_tot)) * kLn2;
  uint16_t* st = (uint16_t*)stage0;       // 128 x (D + 8) staging rows
  acc_to_stage<D>(st, oacc, 32 * w + l32, g32, inv);
  __syncthreads();
  store_pair_thw<D>(st, o, g, h, 2 * (int64_t)pair, perm);
  if (o_lo != nullptr) {   // the low parts, block order (for the backward's Delta)
    __syncthreads();
    acc_to_stage_lo<D>(st, oacc, 32 * w + l32, g32, inv);
    __syncthreads();
    store_pair_rows<D>(st, o_lo + (hN + 2 * (int64_t)pair * kTile) * D);
  }
  __syncthreads();   // staging area and s_work are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// backward pre-pass: dO into the operand layout, -delta = -rowsum(dO * O),
// lse2 = lse * log2(e).  O is the bf16 output plus, when the forward kept
// them (o_lo != NULL, block order), its low parts: Delta from the bf16 O
// alone carries its rounding (up to 2^-8 relative) into every dS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(Geometry g, const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ o_lo,
                                                      const uint16_t* __restrict__ dout,
                                                      const int32_t* __restrict__ perm,
                                                      const float* __restrict__ lse, uint16_t* __restrict__ dop,
                                                      float* __restrict__ delta, float* __restrict__ lse2) {
  constexpr int CH = D / 8;
  const int64_t tile = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t p0 = (int64_t)h * g.N + tile * kTile;
  uint16_t* rows = dop + p0 * D;
  for (int c = tid; c < kTile * CH; c += 256) {
    const int r = c / CH, k = c % CH;
    const int64_t n = perm ? (int64_t)perm[p0 + r] : tile * kTile + r;
    const int64_t off = (int64_t)h * g.hstride + n * g.tstride + k * 8;
    const uint4 dv = *(const uint4*)(dout + off);
    const uint4 ov = *(const uint4*)(o + off);
    const uint4 lv = o_lo != nullptr ? *(const uint4*)(o_lo + (p0 + r) * D + k * 8) : make_uint4(0, 0, 0, 0);
    *(uint4*)(rows + (int64_t)r * D + swz_chunk<D>(r, k) * 8) = dv;
    const uint32_t a4[4] = {dv.x, dv.y, dv.z, dv.w}, b4[4] = {ov.x, ov.y, ov.z, ov.w}, c4[4] = {lv.x, lv.y, lv.z, lv.w};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += bf16_to_f32((uint16_t)(a4[e] & 0xFFFF)) *
             (bf16_to_f32((uint16_t)(b4[e] & 0xFFFF)) + bf16_to_f32((uint16_t)(c4[e] & 0xFFFF)));
      acc += bf16_to_f32((uint16_t)(a4[e] >> 16)) *
             (bf16_to_f32((uint16_t)(b4[e] >> 16)) + bf16_to_f32((uint16_t)(c4[e] >> 16)));
    }
#pragma unroll
    for (int off2 = CH / 2; off2 > 0; off2 >>= 1) acc += __shfl_xor(acc, off2, CH);
    if (k == 0) {
      delta[p0 + r] = -acc;   // stored negated: it seeds the dP accumulators
      lse2[p0 + r] = lse[p0 + r] * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// backward, query-major pass: dQ (in 32-key halves of each key tile)
// ---------------------------------------------------------------------------
constexpr int kReadAheadQ = 2;   // dQ pass: chunks between an operand's LDS read and its MFMA

template <int D, bool DENSE>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_kernel(
    Geometry g, float scale, float sl2, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const uint16_t* __restrict__ dop, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_start,
    const int32_t* __restrict__ n_blocks, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    uint16_t* __restrict__ dq, int* __restrict__ cnt, const int32_t* __restrict__ order) {
  constexpr int TB = TileGeo<D>::BYTES;
  __shared__ __attribute__((aligned(16))) char stage0[TileGeo<D>::STAGE];   // K, V of even steps
  __shared__ __attribute__((aligned(16))) char stage1[TileGeo<D>::STAGE];   // K, V of odd steps
  __shared__ int s_work;
  const int npair = (int)(g.tiles / 2);
  WorkQueue wq;
  wq.init(cnt, order, npair * g.heads);
  for (;;) {
  const int wk = fetch_work(wq, &s_work);
  if (wk < 0) break;
  const int h = wk / npair;
  const int pair = wk % npair;
  const int lane = threadIdx.x & 63, g32 = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const bool second = w >= 2;
  const int64_t hN = (int64_t)h * g.N;
  const int64_t qt = 2 * pair + (second ? 1 : 0);
  const int rloc = 32 * (w & 1) + l32;
  const uint16_t* Kb = kp + hN * D;
  const uint16_t* Vb = vp + hN * D;
  LaneOff<D> off;
  off.init(lane);

  bf16x8 qreg[D / 16], dreg[D / 16];
  {
    const uint16_t* Qt = qp + (hN + qt * kTile) * D;
    const uint16_t* Dt = dop + (hN + qt * kTile) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qreg[s] = ld_row<D>(Qt, rloc, s, g32);
      dreg[s] = ld_row<D>(Dt, rloc, s, g32);
    }
  }
  const float l2 = lse2[hN + qt * kTile + rloc];
  const float nd = delta[hN + qt * kTile + rloc];   // -delta of this lane's query row: dP starts here
  floatx16 dqacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[u][i] = 0.0f;

  PairIter it = make_iter(g, h, 2 * pair, 2 * pair + 1, blk_start, n_blocks, DENSE ? nullptr : row_ptr, col_idx);
  int kt, kt_next = 0;
  bool ua, ub, ua_n = false, ub_n = false;
  bool have = it.next(kt, ua, ub);
  if (have) {
    dma_tile<D>(stage0, Kb + (int64_t)kt * kTile * D);
    dma_tile<D>(stage0 + TB, Vb + (int64_t)kt * kTile * D);
  }
  auto step = [&](auto par) {
    constexpr int B = decltype(par)::value;
    const bool have_next = it.next(kt_next, ua_n, ub_n);
    wait_dma();
    __syncthreads();
    if (have_next) {
      char* nx = PRISM_STAGE(B ^ 1, stage0, stage1);
      dma_tile<D>(nx, Kb + (int64_t)kt_next * kTile * D);
      dma_tile<D>(nx + TB, Vb + (int64_t)kt_next * kTile * D);
    }
    if (second ? ub : ua) {
      const char* Kt = PRISM_STAGE(B, stage0, stage1);
      const char* Vt = Kt + TB;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        floatx16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[i] = 0.0f;
          pacc[i] = nd;
        }
        {
          // one-MFMA chunks, K and V row operands read kReadAheadQ chunks
          // ahead (left to itself the compiler reads each operand into the
          // same registers right before its product and waits for it)
          constexpr int NC = D / 8;   // S and dP products alternating
          bf16x8 op[NC];
          auto read = [&](int c) { op[c] = lds_row<D>((c & 1) ? Vt : Kt, off, kk, c >> 1); };
#pragma unroll
          for (int c = 0; c < kReadAheadQ; ++c) read(c);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if (c + kReadAheadQ < NC) read(c + kReadAheadQ);
            if ((c & 1) == 0) sacc = mfma32(op[c], qreg[c >> 1], sacc);
            else pacc = mfma32(op[c], dreg[c >> 1], pacc);   // dP - delta
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        bf16x8 ka[2][D / 32];   // K^T operands, read before the dS arithmetic
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int u = 0; u < D / 32; ++u) ka[hh][u] = lds_col<D>(Kt, off, u, kk, hh);
        bf16x8 dsb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = fast_exp2(__builtin_fmaf(sacc[i], sl2, -l2));
          dsb[i >> 3][i & 7] = (__bf16)(pv * pacc[i]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int u = 0; u < D / 32; ++u) dqacc[u] = mfma32(ka[hh][u], dsb[hh], dqacc[u]);
      }
    }
    kt = kt_next;
    ua = ua_n;
    ub = ub_n;
    have = have_next;
  };
  while (have) {
    step(Parity<0>{});
    if (!have) break;
    step(Parity<1>{});
  }
  __syncthreads();
  uint16_t* st = (uint16_t*)stage0;
  acc_to_stage<D>(st, dqacc, 32 * w + l32, g32, scale);
  __syncthreads();
  store_pair_thw<D>(st, dq, g, h, 2 * (int64_t)pair, perm);
  __syncthreads();   // staging area and s_work are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// backward, key-major pass: dK and dV (in 32-query halves of each query tile)
// ---------------------------------------------------------------------------
template <int D, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dkdv_kernel(
    Geometry g, float scale, float sl2, const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const uint16_t* __restrict__ dop, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ perm, const int32_t* __restrict__ blk_start,
    const int32_t* __restrict__ n_blocks, const int32_t* __restrict__ t_row_ptr,
    const int32_t* __restrict__ t_col_idx, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int* __restrict__ cnt, const int32_t* __restrict__ order, const int32_t* __restrict__ pairs) {
  constexpr int TB = TileGeo<D>::BYTES;
  // Q, dO, then lse2 and delta (64 floats each) of even / odd steps
  __shared__ __attribute__((aligned(16))) char stage0[TileGeo<D>::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[TileGeo<D>::STAGE];
  __shared__ int s_work;
  const int npair = (int)(g.tiles / 2);
  WorkQueue wq;
  wq.init(cnt, order, npair * g.heads);
  for (;;) {
  const int wk = fetch_work(wq, &s_work);
  if (wk < 0) break;
  const int h = wk / npair;
  const int pair = wk % npair;
  const int lane = threadIdx.x & 63, g32 = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const bool second = w >= 2;
  const int64_t hN = (int64_t)h * g.N;
  // the work item's key tiles: (2 pair, 2 pair + 1) or the pair table's
  int ta = 2 * pair, tb = 2 * pair + 1;
  if (!DENSE && pairs != nullptr) {
    ta = pairs[2 * ((int64_t)h * npair + pair)];
    tb = pairs[2 * ((int64_t)h * npair + pair) + 1];
  }
  const int64_t kt = second ? tb : ta;
  const int rloc = 32 * (w & 1) + l32;
  const uint16_t* Qb = qp + hN * D;
  const uint16_t* Db = dop + hN * D;
  LaneOff<D> off;
  off.init(lane);

  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const uint16_t* Kt = kp + (hN + kt * kTile) * D;
    const uint16_t* Vt = vp + (hN + kt * kTile) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kreg[s] = ld_row<D>(Kt, rloc, s, g32);
      vreg[s] = ld_row<D>(Vt, rloc, s, g32);
    }
  }
  floatx16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[u][i] = dvacc[u][i] = 0.0f;

  PairIter it = make_iter(g, h, ta, tb, blk_start, n_blocks, DENSE ? nullptr : t_row_ptr, t_col_idx);
  int qt, qt_next = 0;
  bool ua, ub, ua_n = false, ub_n = false;
  bool have = it.next(qt, ua, ub);
  auto issue = [&](auto par, int tq) {
    constexpr int B = decltype(par)::value;
    char* st = PRISM_STAGE(B, stage0, stage1);
    dma_tile<D>(st, Qb + (int64_t)tq * kTile * D);
    dma_tile<D>(st + TB, Db + (int64_t)tq * kTile * D);
    // even waves copy lse2, odd waves delta (each copy is made twice, with
    // equal values; no branch around the copy)
    dma_vec64(st + 2 * TB + (w & 1) * 4 * kTile, ((w & 1) ? delta : lse2) + hN + (int64_t)tq * kTile);
  };
  if (have) issue(Parity<0>{}, qt);
  auto step = [&](auto par) {
    constexpr int B = decltype(par)::value;
    const bool have_next = it.next(qt_next, ua_n, ub_n);
    wait_dma();
    __syncthreads();
    if (have_next) issue(Parity<B ^ 1>{}, qt_next);
    if (second ? ub : ua) {
      const char* Qt = PRISM_STAGE(B, stage0, stage1);
      const char* Dt = Qt + TB;
      const float* sl = (const float*)(Qt + 2 * TB);     // lse2
      const float* sd = sl + kTile;                         // delta
      // Software pipeline over the two 32-query halves h0, h1 of the tile:
      //   A: S, dP of h0 while the row operands of h1 load;
      //   B: S, dP of h1 while the column operands of h0 load and h0's
      //      softmax (P, dS) runs;
      //   C: dV, dK of h0 while the column operands of h1 load and h1's
      //      softmax runs;
      //   D: dV, dK of h1 (still in flight when the next step starts).
      // Each phase is written as chunks of one matrix product plus its share
      // of loads and vector work, fenced by scheduling barriers, so that the
      // products issue evenly between the other instructions (one wave per
      // SIMD here: nothing else hides a gap in the matrix pipe).
      floatx16 sacc[2], pacc[2];
      bf16x8 qa[2][D / 16], da[2][D / 16];
      bf16x8 dta[2][2][D / 32], qta[2][2][D / 32];
      bf16x8 pb[2][2], dsb[2][2];
      auto rows = [&](int qq) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          qa[qq][s] = lds_row<D>(Qt, off, qq, s);
          da[qq][s] = lds_row<D>(Dt, off, qq, s);
        }
      };
      auto seed = [&](int qq) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // dP starts at -delta of each query row (rows 32 qq + 8 j + 4 g + e)
          const float4 d4 = *(const float4*)(&sd[32 * qq + 8 * j + 4 * g32]);
          pacc[qq][4 * j] = d4.x;
          pacc[qq][4 * j + 1] = d4.y;
          pacc[qq][4 * j + 2] = d4.z;
          pacc[qq][4 * j + 3] = d4.w;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qq][i] = 0.0f;
      };
      constexpr int NM = D / 8;   // products per phase (one per chunk)
      // one matrix product of a phase: S (even m) or dP (odd m) of half qq
      auto sdp1 = [&](int qq, int m) {
        const int s = m >> 1;
        if (m & 1) pacc[qq] = mfma32(da[qq][s], vreg[s], pacc[qq]);   // dP - delta
        else sacc[qq] = mfma32(qa[qq][s], kreg[s], sacc[qq]);
      };
      auto row1 = [&](int qq, int m) {
        const int s = m >> 1;
        if (m & 1) da[qq][s] = lds_row<D>(Dt, off, qq, s);
        else qa[qq][s] = lds_row<D>(Qt, off, qq, s);
      };
      // product m of dV (even) / dK (odd) for half qq, and the column load it needs
      auto dvdk1 = [&](int qq, int m) {
        const int hh = (m >> 1) / (D / 32), u = (m >> 1) % (D / 32);
        if (m & 1) dkacc[u] = mfma32(qta[qq][hh][u], dsb[qq][hh], dkacc[u]);
        else dvacc[u] = mfma32(dta[qq][hh][u], pb[qq][hh], dvacc[u]);
      };
      auto col1 = [&](int qq, int m) {
        const int hh = (m >> 1) / (D / 32), u = (m >> 1) % (D / 32);
        if (m & 1) qta[qq][hh][u] = lds_col<D>(Qt, off, u, qq, hh);
        else dta[qq][hh][u] = lds_col<D>(Dt, off, u, qq, hh);
      };
      float lv[16];
      auto lse_load = [&](int qq) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 l4 = *(const float4*)(&sl[32 * qq + 8 * j + 4 * g32]);
          lv[4 * j] = l4.x;
          lv[4 * j + 1] = l4.y;
          lv[4 * j + 2] = l4.z;
          lv[4 * j + 3] = l4.w;
        }
      };
      // P and dS of elements i, i + 1 of half qq
      auto soft2 = [&](int qq, int i) {
#pragma unroll
        for (int e = i; e < i + 2; ++e) {
          const float pv = fast_exp2(__builtin_fmaf(sacc[qq][e], sl2, -lv[e]));
          pb[qq][e >> 3][e & 7] = (__bf16)pv;
          dsb[qq][e >> 3][e & 7] = (__bf16)(pv * pacc[qq][e]);
        }
      };
      // softmax pairs of chunk m: 8 pairs over NM chunks
      auto soft_chunk = [&](int qq, int m) {
        if constexpr (NM >= 8) {
          if ((m % (NM / 8)) == NM / 8 - 1) soft2(qq, 2 * (m / (NM / 8)));
        } else {
#pragma unroll
          for (int p = 0; p < 8 / NM; ++p) soft2(qq, 2 * (m * (8 / NM) + p));
        }
      };
      // A: S, dP of h0; row loads of h1
      rows(0);
      seed(0);
      seed(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        sdp1(0, m);
        row1(1, m);
        __builtin_amdgcn_sched_barrier(0);
      }
      // B: S, dP of h1; column loads and softmax of h0
      lse_load(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        sdp1(1, m);
        col1(0, m);
        soft_chunk(0, m);
        __builtin_amdgcn_sched_barrier(0);
      }
      // C: dV, dK of h0; column loads and softmax of h1
      lse_load(1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        dvdk1(0, m);
        col1(1, m);
        soft_chunk(1, m);
        __builtin_amdgcn_sched_barrier(0);
      }
      // D: dV, dK of h1
#pragma unroll
      for (int m = 0; m < NM; ++m) dvdk1(1, m);
    }
    qt = qt_next;
    ua = ua_n;
    ub = ub_n;
    have = have_next;
  };
  while (have) {
    step(Parity<0>{});
    if (!have) break;
    step(Parity<1>{});
  }
  uint16_t* st = (uint16_t*)stage0;
  __syncthreads();
  acc_to_stage<D>(st, dkacc, 32 * w + l32, g32, scale);
  __syncthreads();
  store_tiles_thw<D>(st, dk, g, h, ta, tb, perm);
  __syncthreads();
  acc_to_stage<D>(st, dvacc, 32 * w + l32, g32, 1.0f);
  __syncthreads();
  store_tiles_thw<D>(st, dv, g, h, ta, tb, perm);
  __syncthreads();   // staging area and s_work are reused by the next item
  }
}

// workgroups of `kernel` the chip keeps resident at once (the persistent grid)
hipError_t resident_grid(const void* kernel, unsigned* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0);
  if (e != hipSuccess) return e;
  *grid = (unsigned)((cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1));
  return hipSuccess;
}

// Queue order of a sparse launch over the lists (ptr, idx): longest work
// first inside each XCD's range (head by head for large launches).  Returns NULL (identity order) for a dense
// launch or when a range is too long to sort in LDS.
// With `pairs` (scratch of 3 heads * tiles / 2 ints) the key tiles are also
// paired by key_pairs_kernel (*pairs_out = the table, cost = union length).
hipError_t queue_order(const Geometry& g, const int32_t* blk_start, const int32_t* n_blocks, const int32_t* ptr,
                       const int32_t* idx, int32_t* list_tiles, int32_t* order, const int32_t** out,
                       int32_t* pairs, const int32_t** pairs_out, hipStream_t s) {
  *out = nullptr;
  if (pairs_out) *pairs_out = nullptr;
  const int npair = (int)(g.tiles / 2);
  const int total = npair * g.heads;
  if (ptr == nullptr || order == nullptr) return hipSuccess;
  hipLaunchKernelGGL(list_tiles_kernel, dim3((unsigned)((g.tiles + 3) / 4), (unsigned)g.heads), dim3(256), 0, s,
                     blk_start, n_blocks, ptr, idx, g.tiles, list_tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int32_t* cost = nullptr;
  if (pairs != nullptr) {
    cost = pairs + 2 * (int64_t)total;
    hipLaunchKernelGGL(key_pairs_kernel, dim3((unsigned)(g.tiles / 8), (unsigned)g.heads), dim3(512), 0, s, blk_start,
                       n_blocks, ptr, idx, list_tiles, g.tiles, pairs, cost);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    *pairs_out = pairs;
  }
  if ((total + 7) / 8 > kSortMax) return hipSuccess;
  // head by head only when the operands the passes re-read (K and V, or Q
  // and dO) of all heads exceed the 256 MB last-level cache: otherwise the
  // order only lengthens the tail
  const bool by_head = (int64_t)g.heads * 2 * g.N * g.D * 2 > kLastLevelCache;
  hipLaunchKernelGGL(queue_order_kernel, dim3(8), dim3(1024), 0, s, blk_start, n_blocks, list_tiles, cost, g.tiles,
                     npair, total, by_head, order);
  e = hipGetLastError();
  if (e == hipSuccess) *out = order;
  return e;
}

template <int D, bool DENSE>
hipError_t fwd_impl(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp, const uint16_t* vp,
                    const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks, const int32_t* row_ptr,
                    const int32_t* col_idx, uint16_t* o, uint16_t* o_lo, float* lse, int* queues, int32_t* sched,
                    hipStream_t s) {
  const void* k = (const void*)attn_fwd_kernel<D, DENSE>;
  unsigned grid = 0;
  hipError_t e = resident_grid(k, &grid);
  if (e != hipSuccess) return e;
  const int32_t* order = nullptr;
  if (sched != nullptr) {
    e = queue_order(g, blk_start, n_blocks, row_ptr, col_idx, sched, sched + g.heads * g.tiles, &order, nullptr,
                    nullptr, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, queues, 8);
  hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE>), dim3(grid), dim3(kThreads), 0, s, g, scale * kLog2e, qp, kp, vp,
                     perm, blk_start, n_blocks, row_ptr, col_idx, o, o_lo, lse, queues, order);
  return hipGetLastError();
}

template <int D, bool DENSE>
hipError_t bwd_impl(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp, const uint16_t* vp,
                    const uint16_t* dop, const float* lse2, const float* delta, const int32_t* perm,
                    const int32_t* blk_start, const int32_t* n_blocks, const int32_t* row_ptr,
                    const int32_t* col_idx, const int32_t* t_row_ptr, const int32_t* t_col_idx, uint16_t* dq,
                    uint16_t* dk, uint16_t* dv, int* queues, int32_t* sched, hipStream_t s) {
  unsigned grid_q = 0, grid_k = 0;
  hipError_t e = resident_grid((const void*)attn_bwd_dq_kernel<D, DENSE>, &grid_q);
  if (e == hipSuccess) e = resident_grid((const void*)attn_bwd_dkdv_kernel<D, DENSE>, &grid_k);
  if (e != hipSuccess) return e;
  const int32_t *order_q = nullptr, *order_k = nullptr, *pairs_k = nullptr;
  if (sched != nullptr) {
    const int64_t lt = (int64_t)g.heads * g.tiles, npairs = (int64_t)g.heads * (g.tiles / 2);
    e = queue_order(g, blk_start, n_blocks, row_ptr, col_idx, sched, sched + lt, &order_q, nullptr, nullptr, s);
    if (e == hipSuccess)
      e = queue_order(g, blk_start, n_blocks, t_row_ptr, t_col_idx, sched, sched + lt + npairs, &order_k,
                      sched + lt + 2 * npairs, &pairs_k, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, queues, 16);
  // the key-major pass first: 0.8% faster at 2K than the other order (same box)
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, DENSE>), dim3(grid_k), dim3(kThreads), 0, s, g, scale, scale * kLog2e,
                     qp, kp, vp, dop, lse2, delta, perm, blk_start, n_blocks, t_row_ptr, t_col_idx, dk, dv,
                     queues + 8, order_k, pairs_k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, DENSE>), dim3(grid_q), dim3(kThreads), 0, s, g, scale, scale * kLog2e, qp,
                     kp, vp, dop, lse2, delta, perm, blk_start, n_blocks, row_ptr, col_idx, dq, queues, order_q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const int32_t* perm, const int32_t* blk_start,
                           const int32_t* n_blocks, const int32_t* row_ptr, const int32_t* col_idx, uint16_t* o,
                           uint16_t* o_lo, float* lse, int* queues, int32_t* sched, hipStream_t s) {
  const bool dense = row_ptr == nullptr;
#define PRISM_FWD(DD, DN) \
  fwd_impl<DD, DN>(g, scale, qp, kp, vp, perm, blk_start, n_blocks, row_ptr, col_idx, o, o_lo, lse, queues, sched, s)
  if (g.D == 128) return dense ? PRISM_FWD(128, true) : PRISM_FWD(128, false);
  return dense ? PRISM_FWD(64, true) : PRISM_FWD(64, false);
#undef PRISM_FWD
}

hipError_t launch_bwd_pre(const Geometry& g, const uint16_t* o, const uint16_t* o_lo, const uint16_t* dout,
                          const int32_t* perm, const float* lse, uint16_t* dop, float* delta, float* lse2,
                          hipStream_t s) {
  dim3 grid((unsigned)g.tiles, (unsigned)g.heads);
  if (g.D == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, grid, dim3(256), 0, s, g, o, o_lo, dout, perm, lse, dop, delta, lse2);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, grid, dim3(256), 0, s, g, o, o_lo, dout, perm, lse, dop, delta, lse2);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const uint16_t* dop, const float* lse2, const float* delta,
                           const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks,
                           const int32_t* row_ptr, const int32_t* col_idx, const int32_t* t_row_ptr,
                           const int32_t* t_col_idx, uint16_t* dq, uint16_t* dk, uint16_t* dv, int* queues,
                           int32_t* sched, hipStream_t s) {
  const bool dense = row_ptr == nullptr;
#define PRISM_BWD(DD, DN)                                                                                          \
  bwd_impl<DD, DN>(g, scale, qp, kp, vp, dop, lse2, delta, perm, blk_start, n_blocks, row_ptr, col_idx, t_row_ptr, \
                   t_col_idx, dq, dk, dv, queues, sched, s)
  if (g.D == 128) return dense ? PRISM_BWD(128, true) : PRISM_BWD(128, false);
  return dense ? PRISM_BWD(64, true) : PRISM_BWD(64, false);
#undef PRISM_BWD
}

}  // namespace prism

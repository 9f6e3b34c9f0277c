// Host-side launchers of the Prism kernels (one translation unit per stage).
// Arguments have been validated by the C-ABI layer; every launcher returns the
// hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prism.h"

namespace prism {

struct Geometry {
  int T, H, W, heads, D;
  int64_t N;          // tokens per head
  int64_t Z;          // zones per head
  int64_t tiles;      // N / 64
  int64_t hstride, tstride;
};

// ---- zone statistics and plan (zone_plan.hip) ----
hipError_t launch_zone_stats(const Geometry& g, const prism_params& p, const uint16_t* v, const float* a,
                             double* zstats, double* gout, double* rho, hipStream_t s);
hipError_t launch_plan_shapes(const Geometry& g, const prism_params& p, const double* gin, const double* rho,
                              uint8_t* shape_id, int32_t* perm, int32_t* blk_start, int32_t* n_blocks,
                              hipStream_t s);

// ---- permutation, pooling and block selection (select.hip) ----
// Gathers THW rows of x through perm (NULL = identity) into the operand
// layout (swizzled 64-row tiles); when pool_sums != NULL also writes per-tile
// float64 channel sums [heads][tiles][D].
hipError_t launch_permute(const Geometry& g, const uint16_t* x, const int32_t* perm, uint16_t* xp,
                          double* pool_sums, hipStream_t s);
hipError_t launch_pool_finalize(const Geometry& g, const double* tile_sums, const int32_t* blk_start,
                                const int32_t* n_blocks, double* pooled, hipStream_t s);
size_t select_workspace_bytes(const Geometry& g);
// Scores, selects and writes the query-major index (and, when t_row_ptr is
// not NULL, the key-major one).  Sets *status to PRISM_ECAPACITY, writing no
// index, when the pairs exceed col_cap.  Synchronises the stream.
hipError_t run_selection(const Geometry& g, const prism_params& p, const int32_t* blk_start,
                         const int32_t* n_blocks, const double* qbar, const double* kbar, int32_t* row_ptr,
                         int32_t* col_idx, int64_t col_cap, int32_t* t_row_ptr, int32_t* t_col_idx,
                         int64_t* nnz_host, char* ws, int* status, hipStream_t s);

// ---- attention (attn.hip) ----
// Sparse when row_ptr != NULL, dense over all tiles (64-token blocks, identity
// perm) otherwise.  lse and o_lo may be NULL (not stored).  `queues` is device scratch
// of kQueueInts ints for the persistent work queues (cleared here, on s);
// `sched` (NULL: work in index order) is scratch of sched_ints(g, backward)
// ints for the longest-first queue order (and, backward, the key-tile pairs).
constexpr int kQueueInts = 64;
inline int64_t sched_ints(const Geometry& g, bool backward) {
  return (int64_t)g.heads * g.tiles + (backward ? 5 : 1) * (int64_t)g.heads * (g.tiles / 2);
}
hipError_t launch_attn_fwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const int32_t* perm, const int32_t* blk_start,
                           const int32_t* n_blocks, const int32_t* row_ptr, const int32_t* col_idx, uint16_t* o,
                           uint16_t* o_lo, float* lse, int* queues, int32_t* sched, hipStream_t s);
// o_lo (NULL: not used): the low bf16 parts of O, [heads][N][D] in block order
hipError_t launch_bwd_pre(const Geometry& g, const uint16_t* o, const uint16_t* o_lo, const uint16_t* dout,
                          const int32_t* perm, const float* lse, uint16_t* dop, float* delta, float* lse2,
                          hipStream_t s);
hipError_t launch_attn_bwd(const Geometry& g, float scale, const uint16_t* qp, const uint16_t* kp,
                           const uint16_t* vp, const uint16_t* dop, const float* lse2, const float* delta,
                           const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks,
                           const int32_t* row_ptr, const int32_t* col_idx, const int32_t* t_row_ptr,
                           const int32_t* t_col_idx, uint16_t* dq, uint16_t* dk, uint16_t* dv, int* queues,
                           int32_t* sched, hipStream_t s);

// ---- audio-to-video norm producer (a2v.hip) ----
hipError_t launch_a2v_norms(const uint16_t* h_hat, int64_t n, int channels, int64_t stride, float* a,
                            hipStream_t s);

}  // namespace prism

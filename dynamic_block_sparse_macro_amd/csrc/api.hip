// C ABI of the Prism library: argument validation, workspace sizing and
// stream-ordered orchestration of the kernels.  Every argument is checked
// before the first HIP call, so a rejected call launches and writes nothing.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "prism_internal.h"

using prism::Geometry;

namespace {

// The selection sorts one row of block scores (up to N / 64 of them, 8-byte
// keys) in LDS: 16,384 keys fill 128 KB of the 160 KB.  This also keeps block
// indices within the 16 bits of the sort key.
constexpr int64_t kMaxTokens = 16384LL * 64;

int check_problem(const prism_problem* pr, Geometry* g) {
  if (!pr) return PRISM_EINVAL;
  if (pr->T <= 0 || pr->H <= 0 || pr->W <= 0 || pr->T % 8 || pr->H % 8 || pr->W % 8) return PRISM_EGRID;
  if (pr->heads < 1) return PRISM_EINVAL;
  if (pr->head_dim != 64 && pr->head_dim != 128) return PRISM_EDIM;
  if (pr->token_stride < pr->head_dim || pr->token_stride % 8 || pr->head_stride < 0 || pr->head_stride % 8)
    return PRISM_EINVAL;
  const int64_t N = (int64_t)pr->T * pr->H * pr->W;
  if (N > kMaxTokens) return PRISM_EINVAL;
  if ((int64_t)pr->heads * N > (int64_t)INT32_MAX / 2) return PRISM_EINVAL;
  g->T = pr->T;
  g->H = pr->H;
  g->W = pr->W;
  g->heads = pr->heads;
  g->D = pr->head_dim;
  g->N = N;
  g->Z = N / 512;
  g->tiles = N / 64;
  g->hstride = pr->head_stride;
  g->tstride = pr->token_stride;
  return PRISM_OK;
}

int check_params(const prism_params* p) {
  if (!p) return PRISM_EINVAL;
  if (!(p->eps > 0.0) || !isfinite(p->eps)) return PRISM_EPARAM;
  if (!isfinite(p->tau128) || !isfinite(p->tau256) || !(p->tau256 <= p->tau128)) return PRISM_EPARAM;
  if (p->top_k < 1) return PRISM_EPARAM;
  if (!(p->top_p > 0.0 && p->top_p <= 1.0)) return PRISM_EPARAM;
  if (!(p->density_cap > 0.0 && p->density_cap <= 1.0)) return PRISM_EPARAM;
  if (!(p->scale >= 0.0) || !isfinite(p->scale)) return PRISM_EPARAM;
  const int known = PRISM_VARIANT_FIXED_SHAPE | PRISM_VARIANT_TOPK_ONLY | PRISM_VARIANT_TOPP_ONLY |
                    PRISM_VARIANT_VISUAL_ONLY | PRISM_VARIANT_AUDIO_ONLY | PRISM_VARIANT_RHO_MAX_AUDIO;
  if (p->variant & ~known) return PRISM_EPARAM;
  if ((p->variant & PRISM_VARIANT_TOPK_ONLY) && (p->variant & PRISM_VARIANT_TOPP_ONLY)) return PRISM_EPARAM;
  if ((p->variant & PRISM_VARIANT_VISUAL_ONLY) && (p->variant & PRISM_VARIANT_AUDIO_ONLY)) return PRISM_EPARAM;
  if ((p->variant & PRISM_VARIANT_FIXED_SHAPE) && (p->fixed_shape < 0 || p->fixed_shape > 15)) return PRISM_EPARAM;
  if (p->pass_heads < 0) return PRISM_EPARAM;
  return PRISM_OK;
}

#define CHECK(x)                  \
  do {                            \
    const int st_ = (x);          \
    if (st_ != PRISM_OK) return st_; \
  } while (0)

#define HIPCALL(x)                              \
  do {                                          \
    if ((x) != hipSuccess) return PRISM_EHIP;   \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

float attn_scale(const prism_params& p, int D) { return p.scale > 0 ? (float)p.scale : 1.0f / sqrtf((float)D); }

// workspace of prism_select_blocks: tile sums (q, k), pooled means (q, k),
// then the selection scratch
size_t select_ws(const Geometry& g) {
  const size_t pooled = align256(sizeof(double) * g.heads * g.tiles * g.D);
  return 4 * pooled + prism::select_workspace_bytes(g);
}

size_t operand_bytes(const Geometry& g) { return align256(sizeof(uint16_t) * g.heads * g.N * g.D); }

size_t bwd_ws(const Geometry& g) { return operand_bytes(g) + 2 * align256(sizeof(float) * g.heads * g.N); }

// work-queue counters of the persistent attention kernels, and the scratch
// of their longest-first queue order
constexpr size_t kQueueBytes = sizeof(int) * prism::kQueueInts;
size_t sched_bytes(const Geometry& g, bool backward) {
  return align256(sizeof(int32_t) * (size_t)prism::sched_ints(g, backward));
}

// ---- forward-only inference path ----
// Heads run in passes of `group` heads, enough for the attention grid to
// fill the chip (about 2048 workgroups of two 64-token tiles); the workspace
// holds one pass and is reused by the next.  Inside a pass the float64 tile
// sums, pooled means and selection scratch are dead once the index is built,
// so the permuted V rows are written over them.
struct InferLayout {
  int group;
  int64_t lmax;  // largest possible selected blocks per query block
  size_t zst, gv, rho, shape, perm, bs, nb, qp, kp, region, rp, col, queues, sched, total;
};

int64_t max_row_blocks(const Geometry& g, const prism_params& p) {
  const int64_t tiles = g.tiles;
  if (p.variant & PRISM_VARIANT_TOPK_ONLY) return p.top_k < tiles ? p.top_k : tiles;
  if (p.density_cap >= 1.0 || p.top_p >= 1.0) return tiles;
  // the cap admits at most floor(cap N) key tokens beyond Top-k, and every
  // block holds at least 64 tokens
  const int64_t cap_blocks = (int64_t)floor(p.density_cap * (double)g.N) / 64;
  int64_t l = cap_blocks > p.top_k ? cap_blocks : p.top_k;
  if (l < 1) l = 1;
  return l < tiles ? l : tiles;
}

InferLayout infer_layout(const Geometry& geo, const prism_params& p) {
  InferLayout L;
  const int64_t want = p.pass_heads > 0 ? p.pass_heads : (4096 + geo.tiles - 1) / geo.tiles;
  L.group = (int)(want < geo.heads ? want : geo.heads);
  Geometry g = geo;
  g.heads = L.group;
  const int64_t G = L.group;
  L.lmax = max_row_blocks(geo, p);
  L.zst = align256(sizeof(double) * G * g.Z * 8);
  L.gv = align256(sizeof(double) * G * g.Z * 3);
  L.rho = align256(sizeof(double) * G * g.Z);
  L.shape = align256(G * g.Z);
  L.perm = align256(sizeof(int32_t) * G * g.N);
  L.bs = align256(sizeof(int32_t) * G * (g.tiles + 1));
  L.nb = align256(sizeof(int32_t) * G);
  L.qp = operand_bytes(g);
  L.kp = operand_bytes(g);
  const size_t sel = select_ws(g);
  L.region = sel > operand_bytes(g) ? sel : operand_bytes(g);
  L.rp = align256(sizeof(int32_t) * G * (g.tiles + 1));
  L.col = align256(sizeof(int32_t) * G * g.tiles * L.lmax);
  L.queues = align256(kQueueBytes);
  L.sched = sched_bytes(g, false);
  L.total = L.zst + L.gv + L.rho + L.shape + L.perm + L.bs + L.nb + L.qp + L.kp + L.region + L.rp + L.col + L.queues +
            L.sched;
  return L;
}

// ---- allocation-free forward (prism_attn_fwd_noalloc) ----
// Its scratch is this array: one copy per GPU, held until the process ends.
// Host code must not take the array's name as a device address; the address
// comes from hipGetSymbolAddress, once per device.
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (NULL: not looked up yet)

// `scratch`'s address on the current device
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* prism_strerror(int status) {
  switch (status) {
    case PRISM_OK: return "success";
    case PRISM_EINVAL: return "invalid argument (NULL pointer, size or stride)";
    case PRISM_EGRID: return "T, H and W must be positive multiples of 8";
    case PRISM_EDIM: return "head_dim must be 64 or 128";
    case PRISM_EPARAM: return "invalid hyper-parameter";
    case PRISM_ECAPACITY: return "col_cap is smaller than the number of selected block pairs";
    case PRISM_EWORKSPACE: return "workspace missing or too small";
    case PRISM_EHIP: return "HIP runtime error";
    case PRISM_EINDEX: return "the block index breaks an invariant (prism_check_index)";
    default: return "unknown status";
  }
}

int prism_a2v_norms(const prism_bf16* h_hat, int64_t n_tokens, int32_t channels, int64_t token_stride, float* a,
                    prism_stream stream) {
  if (!h_hat || !a || ((uintptr_t)h_hat & 15)) return PRISM_EINVAL;
  if (n_tokens < 0 || n_tokens > INT32_MAX || channels <= 0 || channels % 8) return PRISM_EINVAL;
  if (token_stride < channels || token_stride % 8) return PRISM_EINVAL;
  HIPCALL(prism::launch_a2v_norms(h_hat, n_tokens, channels, token_stride, a, (hipStream_t)stream));
  return PRISM_OK;
}

int prism_zone_stats(const prism_problem* prob, const prism_params* par, const prism_bf16* v, const float* a,
                     double* zstats, double* g, double* rho, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!v || !zstats || !g || !rho) return PRISM_EINVAL;
  HIPCALL(prism::launch_zone_stats(geo, *par, v, a, zstats, g, rho, (hipStream_t)stream));
  return PRISM_OK;
}

int prism_plan_shapes(const prism_problem* prob, const prism_params* par, const double* g, const double* rho,
                      uint8_t* shape_id, int32_t* perm, int32_t* blk_start, int32_t* n_blocks, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!g || !rho || !shape_id || !perm || !blk_start || !n_blocks) return PRISM_EINVAL;
  HIPCALL(prism::launch_plan_shapes(geo, *par, g, rho, shape_id, perm, blk_start, n_blocks, (hipStream_t)stream));
  return PRISM_OK;
}

int prism_select_blocks(const prism_problem* prob, const prism_params* par, const prism_bf16* q,
                        const prism_bf16* k, const prism_bf16* v, const int32_t* perm, const int32_t* blk_start,
                        const int32_t* n_blocks, prism_bf16* qp, prism_bf16* kp, prism_bf16* vp, int32_t* row_ptr,
                        int32_t* col_idx, int64_t col_cap, int32_t* t_row_ptr, int32_t* t_col_idx,
                        int64_t* nnz_host, void* ws, size_t* ws_bytes, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const size_t need = select_ws(geo);
  if (!ws) {
    *ws_bytes = need;
    return PRISM_OK;
  }
  if (*ws_bytes < need) return PRISM_EWORKSPACE;
  if (!q || !k || !v || !perm || !blk_start || !n_blocks || !qp || !kp || !vp || !row_ptr || !col_idx ||
      !t_row_ptr || !t_col_idx || !nnz_host || col_cap < 0)
    return PRISM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const size_t pooled = align256(sizeof(double) * geo.heads * geo.tiles * geo.D);
  char* w = (char*)ws;
  double* qsum = (double*)w;
  double* ksum = (double*)(w + pooled);
  double* qbar = (double*)(w + 2 * pooled);
  double* kbar = (double*)(w + 3 * pooled);
  char* sel = w + 4 * pooled;
  HIPCALL(prism::launch_permute(geo, q, perm, qp, qsum, s));
  HIPCALL(prism::launch_permute(geo, k, perm, kp, ksum, s));
  HIPCALL(prism::launch_permute(geo, v, perm, vp, nullptr, s));
  HIPCALL(prism::launch_pool_finalize(geo, qsum, blk_start, n_blocks, qbar, s));
  HIPCALL(prism::launch_pool_finalize(geo, ksum, blk_start, n_blocks, kbar, s));
  int status = PRISM_OK;
  HIPCALL(prism::run_selection(geo, *par, blk_start, n_blocks, qbar, kbar, row_ptr, col_idx, col_cap, t_row_ptr,
                               t_col_idx, nnz_host, sel, &status, s));
  return status;
}

int prism_attn_fwd(const prism_problem* prob, const prism_params* par, const prism_bf16* qp, const prism_bf16* kp,
                   const prism_bf16* vp, const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks,
                   const int32_t* row_ptr, const int32_t* col_idx, prism_bf16* o, prism_bf16* o_lo, float* lse,
                   void* ws, size_t* ws_bytes, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const size_t need = align256(kQueueBytes) + sched_bytes(geo, false);
  if (!ws) {
    *ws_bytes = need;
    return PRISM_OK;
  }
  if (*ws_bytes < need) return PRISM_EWORKSPACE;
  if (!qp || !kp || !vp || !perm || !blk_start || !n_blocks || !row_ptr || !col_idx || !o || !lse)
    return PRISM_EINVAL;
  HIPCALL(prism::launch_attn_fwd(geo, attn_scale(*par, geo.D), qp, kp, vp, perm, blk_start, n_blocks, row_ptr,
                                 col_idx, o, o_lo, lse, (int*)ws, (int32_t*)((char*)ws + align256(kQueueBytes)),
                                 (hipStream_t)stream));
  return PRISM_OK;
}

int prism_attn_fwd_noalloc(const prism_problem* prob, const prism_params* par, const prism_bf16* qp,
                           const prism_bf16* kp, const prism_bf16* vp, const int32_t* perm, const int32_t* blk_start,
                           const int32_t* n_blocks, const int32_t* row_ptr, const int32_t* col_idx, prism_bf16* o,
                           prism_bf16* o_lo, float* lse, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!qp || !kp || !vp || !perm || !blk_start || !n_blocks || !row_ptr || !col_idx || !o || !lse)
    return PRISM_EINVAL;
  if (align256(kQueueBytes) + sched_bytes(geo, false) > kStaticScratchBytes) return PRISM_EWORKSPACE;
  void* ws = nullptr;
  HIPCALL(static_scratch(&ws));
  // the queue counters are cleared by a kernel inside launch_attn_fwd; the
  // queue order is written before it is read
  HIPCALL(prism::launch_attn_fwd(geo, attn_scale(*par, geo.D), qp, kp, vp, perm, blk_start, n_blocks, row_ptr,
                                 col_idx, o, o_lo, lse, (int*)ws, (int32_t*)((char*)ws + align256(kQueueBytes)),
                                 (hipStream_t)stream));
  return PRISM_OK;
}

int prism_attn_bwd(const prism_problem* prob, const prism_params* par, const prism_bf16* qp, const prism_bf16* kp,
                   const prism_bf16* vp, const prism_bf16* o, const prism_bf16* o_lo, const prism_bf16* dout,
                   const float* lse, const int32_t* perm, const int32_t* blk_start, const int32_t* n_blocks,
                   const int32_t* row_ptr,
                   const int32_t* col_idx, const int32_t* t_row_ptr, const int32_t* t_col_idx, prism_bf16* dq,
                   prism_bf16* dk, prism_bf16* dv, void* ws, size_t* ws_bytes, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const size_t need = bwd_ws(geo) + align256(kQueueBytes) + sched_bytes(geo, true);
  if (!ws) {
    *ws_bytes = need;
    return PRISM_OK;
  }
  if (*ws_bytes < need) return PRISM_EWORKSPACE;
  if (!qp || !kp || !vp || !o || !dout || !lse || !perm || !blk_start || !n_blocks || !row_ptr || !col_idx ||
      !t_row_ptr || !t_col_idx || !dq || !dk || !dv)
    return PRISM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* dop = (uint16_t*)ws;
  float* delta = (float*)((char*)ws + operand_bytes(geo));
  float* lse2 = (float*)((char*)delta + align256(sizeof(float) * geo.heads * geo.N));
  int* queues = (int*)((char*)ws + bwd_ws(geo));
  int32_t* sched = (int32_t*)((char*)queues + align256(kQueueBytes));
  HIPCALL(prism::launch_bwd_pre(geo, o, o_lo, dout, perm, lse, dop, delta, lse2, s));
  HIPCALL(prism::launch_attn_bwd(geo, attn_scale(*par, geo.D), qp, kp, vp, dop, lse2, delta, perm, blk_start,
                                 n_blocks, row_ptr, col_idx, t_row_ptr, t_col_idx, dq, dk, dv, queues, sched, s));
  return PRISM_OK;
}

int prism_infer_fwd(const prism_problem* prob, const prism_params* par, const prism_bf16* q, const prism_bf16* k,
                    const prism_bf16* v, const float* a, prism_bf16* o, void* ws, size_t* ws_bytes,
                    prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const InferLayout L = infer_layout(geo, *par);
  if ((int64_t)L.group * geo.tiles * L.lmax > (int64_t)INT32_MAX) return PRISM_EINVAL;
  if (!ws) {
    *ws_bytes = L.total;
    return PRISM_OK;
  }
  if (*ws_bytes < L.total) return PRISM_EWORKSPACE;
  if (!q || !k || !v || !o) return PRISM_EINVAL;
  // o may be q, k or v itself: a pass consumes its heads' inputs (zone
  // statistics, permutation) before its attention writes their outputs

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  auto take = [&w](size_t b) {
    char* r = w;
    w += b;
    return r;
  };
  double* zst = (double*)take(L.zst);
  double* gv = (double*)take(L.gv);
  double* rho = (double*)take(L.rho);
  uint8_t* shape = (uint8_t*)take(L.shape);
  int32_t* perm = (int32_t*)take(L.perm);
  int32_t* bs = (int32_t*)take(L.bs);
  int32_t* nb = (int32_t*)take(L.nb);
  uint16_t* qp = (uint16_t*)take(L.qp);
  uint16_t* kp = (uint16_t*)take(L.kp);
  char* region = take(L.region);
  int32_t* rp = (int32_t*)take(L.rp);
  int32_t* col = (int32_t*)take(L.col);
  int* queues = (int*)take(L.queues);
  int32_t* sched = (int32_t*)take(L.sched);
  uint16_t* vp = (uint16_t*)region;

  const float scale = attn_scale(*par, geo.D);
  std::vector<int64_t> nnz(L.group);
  for (int h0 = 0; h0 < geo.heads; h0 += L.group) {
    Geometry g = geo;
    g.heads = geo.heads - h0 < L.group ? geo.heads - h0 : L.group;
    const int64_t off = (int64_t)h0 * geo.hstride;
    const size_t pooled = align256(sizeof(double) * g.heads * g.tiles * g.D);
    double* qsum = (double*)region;
    double* ksum = (double*)(region + pooled);
    double* qbar = (double*)(region + 2 * pooled);
    double* kbar = (double*)(region + 3 * pooled);
    char* sel = region + 4 * pooled;
    HIPCALL(prism::launch_zone_stats(g, *par, v + off, a, zst, gv, rho, s));
    HIPCALL(prism::launch_plan_shapes(g, *par, gv, rho, shape, perm, bs, nb, s));
    HIPCALL(prism::launch_permute(g, q + off, perm, qp, qsum, s));
    HIPCALL(prism::launch_permute(g, k + off, perm, kp, ksum, s));
    HIPCALL(prism::launch_pool_finalize(g, qsum, bs, nb, qbar, s));
    HIPCALL(prism::launch_pool_finalize(g, ksum, bs, nb, kbar, s));
    int status = PRISM_OK;
    HIPCALL(prism::run_selection(g, *par, bs, nb, qbar, kbar, rp, col, (int64_t)g.heads * g.tiles * L.lmax, nullptr,
                                 nullptr, nnz.data(), sel, &status, s));
    if (status != PRISM_OK) return status;
    HIPCALL(prism::launch_permute(g, v + off, perm, vp, nullptr, s));
    HIPCALL(prism::launch_attn_fwd(g, scale, qp, kp, vp, perm, bs, nb, rp, col, o + off, nullptr, nullptr, queues,
                                   sched, s));
  }
  return PRISM_OK;
}

int prism_dense_attn_fwd(const prism_problem* prob, const prism_params* par, const prism_bf16* q,
                         const prism_bf16* k, const prism_bf16* v, prism_bf16* o, float* lse, void* ws,
                         size_t* ws_bytes, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const size_t need = 3 * operand_bytes(geo) + align256(kQueueBytes);
  if (!ws) {
    *ws_bytes = need;
    return PRISM_OK;
  }
  if (*ws_bytes < need) return PRISM_EWORKSPACE;
  if (!q || !k || !v || !o || !lse) return PRISM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* qp = (uint16_t*)ws;
  uint16_t* kp = (uint16_t*)((char*)ws + operand_bytes(geo));
  uint16_t* vp = (uint16_t*)((char*)ws + 2 * operand_bytes(geo));
  HIPCALL(prism::launch_permute(geo, q, nullptr, qp, nullptr, s));
  HIPCALL(prism::launch_permute(geo, k, nullptr, kp, nullptr, s));
  HIPCALL(prism::launch_permute(geo, v, nullptr, vp, nullptr, s));
  int* queues = (int*)((char*)ws + 3 * operand_bytes(geo));
  HIPCALL(prism::launch_attn_fwd(geo, attn_scale(*par, geo.D), qp, kp, vp, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, o, nullptr, lse, queues, nullptr, s));
  return PRISM_OK;
}

int prism_dense_attn_bwd(const prism_problem* prob, const prism_params* par, const prism_bf16* q,
                         const prism_bf16* k, const prism_bf16* v, const prism_bf16* o, const prism_bf16* dout,
                         const float* lse, prism_bf16* dq, prism_bf16* dk, prism_bf16* dv, void* ws,
                         size_t* ws_bytes, prism_stream stream) {
  Geometry geo;
  CHECK(check_problem(prob, &geo));
  CHECK(check_params(par));
  if (!ws_bytes) return PRISM_EINVAL;
  const size_t need = 3 * operand_bytes(geo) + bwd_ws(geo) + align256(kQueueBytes);
  if (!ws) {
    *ws_bytes = need;
    return PRISM_OK;
  }
  if (*ws_bytes < need) return PRISM_EWORKSPACE;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return PRISM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const size_t ob = operand_bytes(geo);
  uint16_t* qp = (uint16_t*)ws;
  uint16_t* kp = (uint16_t*)((char*)ws + ob);
  uint16_t* vp = (uint16_t*)((char*)ws + 2 * ob);
  uint16_t* dop = (uint16_t*)((char*)ws + 3 * ob);
  float* delta = (float*)((char*)ws + 4 * ob);
  float* lse2 = (float*)((char*)delta + align256(sizeof(float) * geo.heads * geo.N));
  HIPCALL(prism::launch_permute(geo, q, nullptr, qp, nullptr, s));
  HIPCALL(prism::launch_permute(geo, k, nullptr, kp, nullptr, s));
  HIPCALL(prism::launch_permute(geo, v, nullptr, vp, nullptr, s));
  int* queues = (int*)((char*)ws + 3 * ob + bwd_ws(geo));
  HIPCALL(prism::launch_bwd_pre(geo, o, nullptr, dout, nullptr, lse, dop, delta, lse2, s));
  HIPCALL(prism::launch_attn_bwd(geo, attn_scale(*par, geo.D), qp, kp, vp, dop, lse2, delta, nullptr, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, queues, nullptr, s));
  return PRISM_OK;
}

}  // extern "C"

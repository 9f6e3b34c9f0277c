"""Plain CPU oracle of Prism's dynamic sparse video self-attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Written from the Prism pages ("Prism: Dynamic Sparse Attention for Native 2K
Joint Video-Audio Generation Model Training"); citations name the page and the
section on it:
  [pt/M1] Portuguese reading guide (xyznot.com/pt), "Método", part 1
          (variation indicator: sigma^2_v,d, r_v,d, a_t,h,w, a-bar, v-hat, g_d)
  [pt/M2] same page, "Método", part 2 (block volume and shape quantisation:
          rho, tau_128, tau_256, the information-loss model, l*_d, s*)
  [pt/M3] same page, "Método", part 3 (hybrid Top-k / Top-p attention, S_i)
  [pt/IC] same page, "Ideias centrais" (8x8x8 macro-zones, 16 candidate shapes,
          volumes {64, 128, 256})
  [zh/FAQ] Chinese reading guide (xyznot.com/zh), "常见问题" (block sizes stay
          multiples of 64 tokens; statistics and P_i are detached constants,
          gradients flow only through sparse attention on the selected blocks)
  [blog/4] sd114.wiki post, "工作原理", step 4 (attention runs on the selected
          blocks only and the result is restored to the original layout)

Precision: every statistic and every discrete decision in float64; attention
in float64.  Inputs are the bfloat16-rounded values the GPU receives, upcast
exactly.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  R1  a is a per-token float32 norm map supplied by the caller; absent = 0.
  R2  v-hat_a,d: variance of the slice means of a along d, normalised to sum
      to 1 over d (1/3 each when all three are 0).  Pinned by closed forms
      (a map varying along one axis; a flat map).
  R3  a-bar(m): min-max normalisation of the zone mean of a over all zones
      (0 everywhere when max == min).  Pinned by zones of known means.
  R4  epsilon = 1e-6.
  R5  rho(m) = E(m) / max_m' E(m'), E = sum_d sigma^2_v,d, per head (0 when
      max E == 0).  Pinned by closed-form variances and constant zones.
  R6  rho < tau_256 -> 256; else rho < tau_128 -> 128; else 64.
  R7  candidate shapes: edges in {2, 4, 8}, volume in {64, 128, 256}
      (exactly 16 of them), canonical order by volume, then (b_T, b_H, b_W).
  R8  distance in log2 space; exact ties go to the lowest canonical index.
  R9  permuted order: zones ascending, blocks in raster order (T outermost)
      inside a zone, tokens in raster order inside a block.
  R10 query blocks are mean-pooled like key blocks.
  R11 block score s_ij = scale * Qbar_i . Kbar_j, scale = 1/sqrt(D) by default.
  R12 block order: score descending, then block index ascending.
  R13 Top-p: the shortest prefix whose cumulative probability reaches p,
      crossing block included; all blocks if it never does; p >= 1 selects
      all blocks.
  R14 density cap (optional): at most floor(cap * N) key tokens per query
      block; it trims only the Top-p extension, never below Top-k.  Pinned by
      brute force over every prefix of small rows.
  R15 statistics, shapes and the block index are per head; a is shared.
  R16 no causal mask; the log-sum-exp uses the natural log.
  R17 no block is forced into S_i.
  R21 ablation variants (sd114.wiki post, "测试结果" items 2-3, which compare
      fixed block shapes, video-only and audio-only guidance, and Top-k-only
      or adaptive-threshold-only selection): a fixed shape replaces the plan
      in every zone; Top-k alone keeps min(k, n_b) blocks; Top-p alone keeps
      the (capped) nucleus, at least one block; video-only guidance drops the
      a-bar v-hat term, audio-only guidance drops r; max(rho, a-bar) is an
      alternative density.  Each is pinned: the k best scores, the brute-force
      nucleus, the union identity, the silent-audio identity, and a
      three-zone map whose rho and a-bar are known exactly.
  R22 the A2V norm a_n = |h-hat_n|_2 is taken over the bf16 values of h-hat
      in float64 (squares exact) and rounded once to float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "ZONE", "TOL_SCORE", "TOL_MASS", "TOL_DIST", "TOL_RHO",
    "candidate_shapes", "CANDIDATES", "CANDIDATE_VOLUMES",
    "zone_grid", "to_zones", "video_variation", "audio_terms", "a2v_norms",
    "composite_indicator", "information_density", "zone_statistics",
    "block_volume", "ell_star", "quantise_shape", "plan_shapes", "shape_tie_set",
    "partition", "permute_tokens", "unpermute_tokens",
    "pool_blocks", "block_scores", "block_probabilities", "select_row", "select_blocks",
    "csr_from_rows", "csr_transpose",
    "sparse_attention_fwd", "sparse_attention_bwd", "sparse_attention_key_block_grad",
    "dense_attention", "dense_attention_bwd",
    "masked_attention_thw", "token_block_map",
    "Params", "run_pipeline", "row_tie_affected", "row_is_valid_alternative",
    "attention_flops", "selected_pairs",
    "VARIANT_FIXED_SHAPE", "VARIANT_TOPK_ONLY", "VARIANT_TOPP_ONLY", "VARIANT_VISUAL_ONLY", "VARIANT_AUDIO_ONLY",
    "VARIANT_RHO_MAX_AUDIO",
]

ZONE = 8                      # Z_T = Z_H = Z_W = 8 [pt/IC]
TOL_SCORE = 1e-6              # block-score ties (absolute)
TOL_MASS = 1e-9               # cumulative-probability ties at the Top-p cut
TOL_DIST = 1e-6               # shape-distance ties
TOL_RHO = 1e-6                # density ties at tau_128 / tau_256


# Variant switches (bit flags; 0 = the method as the pages describe it).  The
# pages' ablations compare against fixed block shapes, Top-k-only and
# Top-p-only selection, and guidance from the video or the audio signal alone
# (sd114.wiki post, 测试结果 items 2-3); RHO_MAX_AUDIO lets the audio coupling
# raise the density (an alternative reading of "information density").
VARIANT_FIXED_SHAPE = 1
VARIANT_TOPK_ONLY = 2
VARIANT_TOPP_ONLY = 4
VARIANT_VISUAL_ONLY = 8
VARIANT_AUDIO_ONLY = 16
VARIANT_RHO_MAX_AUDIO = 32


@dataclass(frozen=True)
class Params:
    """Hyper-parameters of one Prism layer ([pt/M1], [pt/M2], [pt/M3])."""
    eps: float = 1e-6
    tau128: float = 0.5
    tau256: float = 0.25
    top_k: int = 16
    top_p: float = 0.9
    density_cap: float = 1.0
    scale: float = 0.0            # 0 -> 1 / sqrt(head_dim)
    variant: int = 0              # VARIANT_* bits
    fixed_shape: int = 0          # candidate index used with VARIANT_FIXED_SHAPE

    def score_scale(self, head_dim: int) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(head_dim)


# ----------------------------------------------------------------------------
# candidate block shapes [pt/IC], R7
# ----------------------------------------------------------------------------

def candidate_shapes() -> np.ndarray:
    """All (b_T, b_H, b_W) with edges in {2, 4, 8} and volume in {64, 128, 256},
    ordered by volume, then lexicographically."""
    out = []
    for vol in (64, 128, 256):
        for bt in (2, 4, 8):
            for bh in (2, 4, 8):
                for bw in (2, 4, 8):
                    if bt * bh * bw == vol:
                        out.append((bt, bh, bw))
    return np.array(out, dtype=np.int64)


CANDIDATES = candidate_shapes()
CANDIDATE_VOLUMES = CANDIDATES.prod(axis=1)


# ----------------------------------------------------------------------------
# macro-zones [pt/IC]
# ----------------------------------------------------------------------------

def zone_grid(T: int, H: int, W: int) -> tuple[int, int, int]:
    if T % ZONE or H % ZONE or W % ZONE:
        raise ValueError("T, H and W must be multiples of the 8-token macro-zone edge")
    return T // ZONE, H // ZONE, W // ZONE


def to_zones(x: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """[..., N, C] in THW order -> [..., Z, 8(tau), 8(eta), 8(omega), C].

    Zone m = (z_t * H/8 + z_h) * W/8 + z_w; (tau, eta, omega) are the local
    coordinates inside it."""
    zt, zh, zw = zone_grid(T, H, W)
    lead = x.shape[:-2]
    C = x.shape[-1]
    y = x.reshape(*lead, zt, ZONE, zh, ZONE, zw, ZONE, C)
    n = len(lead)
    y = y.transpose(*range(n), n, n + 2, n + 4, n + 1, n + 3, n + 5, n + 6)
    return y.reshape(*lead, zt * zh * zw, ZONE, ZONE, ZONE, C)


def _slice_means(xz: np.ndarray) -> list[np.ndarray]:
    """Mean-pooled slices along T, H and W: [..., Z, 8, 8, 8, C] -> 3 x [..., Z, 8, C]."""
    return [xz.mean(axis=(-3, -2)), xz.mean(axis=(-4, -2)), xz.mean(axis=(-4, -3))]


def video_variation(v: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """sigma^2_v,d(m) for d = T, H, W ([pt/M1], first equation).

    For each axis: the slice means of V along that axis (each slice is the
    mean over the other two axes), their per-channel population variance over
    the Z_d = 8 slices around their mean mu^(d), averaged over the D channels.
    v: [heads][N][D]; returns [heads][Z][3]."""
    vz = to_zones(np.asarray(v, dtype=np.float64), T, H, W)
    out = []
    for vbar in _slice_means(vz):                 # [heads][Z][8][D]
        mu = vbar.mean(axis=-2, keepdims=True)    # mu^(d)_{m,c}
        out.append(((vbar - mu) ** 2).mean(axis=-2).mean(axis=-1))
    return np.stack(out, axis=-1)


def _normalise_over_axes(x: np.ndarray) -> np.ndarray:
    s = x.sum(axis=-1, keepdims=True)
    safe = np.where(s > 0, s, 1.0)
    return np.where(s > 0, x / safe, 1.0 / 3.0)


def a2v_norms(h_hat: np.ndarray) -> np.ndarray:
    """a_{t,h,w} = || h-hat_{t,h,w} ||_2 of the audio-to-video cross-attention
    output ([pt/M1], second paragraph).  h_hat: [N][C] -> [N]."""
    h = np.asarray(h_hat, dtype=np.float64)
    return np.sqrt((h * h).sum(axis=-1))


def audio_terms(a: np.ndarray | None, T: int, H: int, W: int):
    """Audio coupling strength a-bar(m) in [0, 1] and normalised directional
    variance v-hat_a,d(m) from the cached A2V norm map ([pt/M1]; readings R2, R3).

    Returns (abar [Z], vhat [Z][3], mu_a [Z], sigma^2_a [Z][3])."""
    zt, zh, zw = zone_grid(T, H, W)
    Z = zt * zh * zw
    if a is None:
        a = np.zeros(T * H * W)
    az = to_zones(np.asarray(a, dtype=np.float64).reshape(-1, 1), T, H, W)[..., 0]   # [Z][8][8][8]
    means = [az.mean(axis=(-2, -1)), az.mean(axis=(-3, -1)), az.mean(axis=(-3, -2))]
    mu_a = az.mean(axis=(-3, -2, -1))
    sa2 = np.stack([((m - m.mean(axis=-1, keepdims=True)) ** 2).mean(axis=-1) for m in means], axis=-1)
    vhat = _normalise_over_axes(sa2)
    lo, hi = mu_a.min(), mu_a.max()
    abar = (mu_a - lo) / (hi - lo) if hi > lo else np.zeros(Z)
    return abar, vhat, mu_a, sa2


def composite_indicator(r: np.ndarray, abar: np.ndarray, vhat: np.ndarray, eps: float) -> np.ndarray:
    """g_d(m) = r_v,d(m) + a-bar(m) * v-hat_a,d(m) + eps ([pt/M1], last equation)."""
    return r + abar[..., :, None] * vhat + eps


def information_density(sv2: np.ndarray) -> np.ndarray:
    """rho(m): E(m) = sum_d sigma^2_v,d(m) divided by its maximum over the
    head's zones (reading R5).  sv2: [heads][Z][3] -> [heads][Z]."""
    E = sv2.sum(axis=-1)
    mx = E.max(axis=-1, keepdims=True)
    return np.where(mx > 0, E / np.where(mx > 0, mx, 1.0), 0.0)


def zone_statistics(v: np.ndarray, a: np.ndarray | None, T: int, H: int, W: int, eps: float = 1e-6,
                    variant: int = 0) -> dict:
    """Everything the zone-statistics step produces, per head.  With
    VARIANT_VISUAL_ONLY the audio term is dropped (g = r + eps), with
    VARIANT_AUDIO_ONLY the video ratio (g = a-bar v-hat + eps); with
    VARIANT_RHO_MAX_AUDIO the density is max(rho, a-bar)."""
    sv2 = video_variation(v, T, H, W)
    r = _normalise_over_axes(sv2)                # r_v,d(m) [pt/M1]
    abar, vhat, mu_a, sa2 = audio_terms(a, T, H, W)
    if variant & VARIANT_VISUAL_ONLY:
        g = r + eps
    elif variant & VARIANT_AUDIO_ONLY:
        g = np.broadcast_to(abar[:, None] * vhat, r.shape) + eps
    else:
        g = composite_indicator(r, abar, vhat, eps)
    rho = information_density(sv2)
    if variant & VARIANT_RHO_MAX_AUDIO:
        rho = np.maximum(rho, abar[None, :])
    return dict(sv2=sv2, r=r, E=sv2.sum(-1), abar=abar, vhat=vhat, mu_a=mu_a, sa2=sa2, g=g, rho=rho)


# ----------------------------------------------------------------------------
# block volume and shape [pt/M2]
# ----------------------------------------------------------------------------

def block_volume(rho: np.ndarray, tau128: float = 0.5, tau256: float = 0.25) -> np.ndarray:
    """B(m) in {64, 128, 256} from rho against tau_128 and tau_256 (R6)."""
    rho = np.asarray(rho)
    return np.where(rho < tau256, 256, np.where(rho < tau128, 128, 64)).astype(np.int64)


def ell_star(g: np.ndarray, vol) -> np.ndarray:
    """l*_d = -1/2 log2 g_d + 1/3 (S + 1/2 (log2 g_T + log2 g_H + log2 g_W)),
    S = log2 B(m) ([pt/M2]).  g: [..., 3]; vol broadcast over [...]."""
    lg = np.log2(np.asarray(g, dtype=np.float64))
    S = np.log2(np.asarray(vol, dtype=np.float64))
    c = (S + 0.5 * ((lg[..., 0] + lg[..., 1]) + lg[..., 2])) / 3.0
    return -0.5 * lg + c[..., None]


def _shape_distances(ell: np.ndarray, vol: int) -> tuple[np.ndarray, np.ndarray]:
    idx = np.nonzero(CANDIDATE_VOLUMES == vol)[0]
    e = np.log2(CANDIDATES[idx].astype(np.float64))
    d = e - ell[None, :]
    dist = (d[:, 0] ** 2 + d[:, 1] ** 2) + d[:, 2] ** 2
    return idx, dist


def quantise_shape(ell: np.ndarray, vol: int) -> tuple[int, float, np.ndarray, np.ndarray]:
    """s* = the candidate of volume B nearest to l* in Euclidean (log2) distance;
    exact ties go to the lowest canonical index (R8).
    Returns (shape index, margin to the runner-up, candidate indices, distances)."""
    idx, dist = _shape_distances(ell, vol)
    best = int(np.argmin(dist))
    srt = np.sort(dist)
    margin = float(srt[1] - srt[0]) if len(srt) > 1 else math.inf
    return int(idx[best]), margin, idx, dist


def plan_shapes(g: np.ndarray, rho: np.ndarray, tau128: float = 0.5, tau256: float = 0.25,
                forced_shape: np.ndarray | None = None) -> dict:
    """Per head and zone: volume, continuous optimum, chosen shape and margins.

    g: [heads][Z][3], rho: [heads][Z].  forced_shape (same shape as rho, -1 =
    free) overrides a decision, which the tests use only for zones whose
    decision is a tie within tolerance."""
    heads, Z = rho.shape
    vol = block_volume(rho, tau128, tau256)
    shape_id = np.zeros((heads, Z), np.int64)
    dmargin = np.zeros((heads, Z))
    vmargin = np.minimum(np.abs(rho - tau128), np.abs(rho - tau256))
    ell = np.zeros((heads, Z, 3))
    for h in range(heads):
        for m in range(Z):
            if forced_shape is not None and forced_shape[h, m] >= 0:
                sid = int(forced_shape[h, m])
                vol[h, m] = CANDIDATE_VOLUMES[sid]
                ell[h, m] = ell_star(g[h, m], vol[h, m])
                shape_id[h, m] = sid
                dmargin[h, m] = math.inf
                continue
            ell[h, m] = ell_star(g[h, m], vol[h, m])
            sid, mg, _, _ = quantise_shape(ell[h, m], int(vol[h, m]))
            shape_id[h, m] = sid
            dmargin[h, m] = mg
    return dict(vol=vol, ell=ell, shape_id=shape_id, dist_margin=dmargin, vol_margin=vmargin)


def shape_tie_set(g_m: np.ndarray, rho_m: float, tau128: float = 0.5, tau256: float = 0.25,
                  tol_rho: float = TOL_RHO, tol_dist: float = TOL_DIST) -> set[int]:
    """Every shape index an implementation may choose for one zone when its
    volume or shape decision is within tolerance of a tie."""
    vols = {int(block_volume(rho_m, tau128, tau256))}
    for t, lo_vol, hi_vol in ((tau256, 256, 128), (tau128, 128, 64)):
        if abs(rho_m - t) <= tol_rho:
            vols |= {lo_vol, hi_vol}
    out = set()
    for vol in vols:
        idx, dist = _shape_distances(ell_star(g_m, vol), vol)
        out |= {int(i) for i, d in zip(idx, dist) if d <= dist.min() + tol_dist}
    return out


# ----------------------------------------------------------------------------
# partition and permutation [blog/4], R9
# ----------------------------------------------------------------------------

def partition(shape_id: np.ndarray, T: int, H: int, W: int) -> tuple[np.ndarray, np.ndarray]:
    """Tile each macro-zone with its block shape and list the tokens in
    permuted (block-contiguous) order.

    shape_id: [Z].  Returns perm [N] (permuted position -> THW token index)
    and blk_start [n_b + 1] (block starts in units of 64 tokens)."""
    zt, zh, zw = zone_grid(T, H, W)
    N = T * H * W
    perm = np.empty(N, np.int64)
    starts = []
    p = 0
    for m in range(zt * zh * zw):
        mt, rem = divmod(m, zh * zw)
        mh, mw = divmod(rem, zw)
        bt, bh, bw = CANDIDATES[int(shape_id[m])]
        for it in range(ZONE // bt):
            for ih in range(ZONE // bh):
                for iw in range(ZONE // bw):
                    t = mt * ZONE + it * bt + np.arange(bt)
                    h = mh * ZONE + ih * bh + np.arange(bh)
                    w = mw * ZONE + iw * bw + np.arange(bw)
                    idx = ((t[:, None, None] * H + h[None, :, None]) * W + w[None, None, :]).reshape(-1)
                    starts.append(p // 64)
                    perm[p:p + idx.size] = idx
                    p += idx.size
    starts.append(N // 64)
    return perm, np.array(starts, np.int64)


def permute_tokens(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x_p[p] = x[perm[p]] along the token axis (-2)."""
    return np.take(x, perm, axis=-2)


def unpermute_tokens(xp: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Scatter back to THW order: x[perm[p]] = x_p[p] [blog/4]."""
    out = np.empty_like(xp)
    out[..., perm, :] = xp
    return out


def token_block_map(perm: np.ndarray, blk_start: np.ndarray) -> np.ndarray:
    """THW token index -> block index."""
    N = perm.size
    sizes = np.diff(blk_start) * 64
    blk_of_pos = np.repeat(np.arange(sizes.size), sizes)
    out = np.empty(N, np.int64)
    out[perm] = blk_of_pos
    return out


# ----------------------------------------------------------------------------
# pooled block scores and hybrid Top-k / Top-p selection [pt/M3]
# ----------------------------------------------------------------------------

def pool_blocks(xp: np.ndarray, blk_start: np.ndarray) -> np.ndarray:
    """Mean of each block's token vectors (K-bar_j; Q-bar_i likewise, R10).
    xp: [N][D] in permuted order -> [n_b][D] float64."""
    x = np.asarray(xp, dtype=np.float64)
    st = blk_start[:-1] * 64
    sizes = np.diff(blk_start) * 64
    return np.add.reduceat(x, st, axis=0) / sizes[:, None]


def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = scale * Q-bar_i . K-bar_j (R11)."""
    return scale * (qbar @ kbar.T)


def block_probabilities(s: np.ndarray) -> np.ndarray:
    """P_i = softmax over all key blocks j of s_ij ([pt/M3])."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _sorted_order(s_row: np.ndarray) -> np.ndarray:
    """Key blocks by score descending, then index ascending (R12)."""
    return np.lexsort((np.arange(s_row.size), -s_row))


def select_row(s_row: np.ndarray, P_row: np.ndarray, sizes: np.ndarray, top_k: int, top_p: float,
               density_cap: float, N: int, variant: int = 0) -> dict:
    """S_i = Top-k(P_i, k) U Top-p(P_i, p) ([pt/M3]; R12-R14).

    Both parts are prefixes of the same descending order, so the union is
    the longer prefix; the optional density cap limits the Top-p extension.
    VARIANT_TOPK_ONLY keeps Top-k alone; VARIANT_TOPP_ONLY keeps the (capped)
    Top-p prefix alone, at least one block."""
    nb = s_row.size
    order = _sorted_order(s_row)
    C = np.cumsum(P_row[order])
    if top_p >= 1.0:
        n_p = nb
    else:
        hit = np.nonzero(C >= top_p)[0]
        n_p = int(hit[0]) + 1 if hit.size else nb
    n_k = min(int(top_k), nb)
    if density_cap >= 1.0:
        n_cap = nb
    else:
        U = math.floor(density_cap * N)
        tok = np.cumsum(sizes[order])
        n_cap = int(np.searchsorted(tok, U, side="right"))
    if variant & VARIANT_TOPK_ONLY:
        L = n_k
    elif variant & VARIANT_TOPP_ONLY:
        L = max(1, min(n_p, n_cap))
    else:
        L = max(n_k, min(n_p, n_cap))
    return dict(order=order, C=C, n_p=n_p, n_k=n_k, n_cap=n_cap, L=L, cols=np.sort(order[:L]), variant=variant)


def row_tie_affected(s_row: np.ndarray, sel: dict, top_p: float, capped: bool,
                     tol_s: float = TOL_SCORE, tol_m: float = TOL_MASS) -> bool:
    """True when a rounding-level change of a score or a cumulative mass could
    change this row's selected set."""
    order, L, nb = sel["order"], sel["L"], s_row.size
    ss = s_row[order]

    def gap(r):  # gap between sorted positions r and r + 1 (1-based r)
        return ss[r - 1] - ss[r] if 1 <= r < nb else math.inf

    if gap(L) <= tol_s:
        return True
    uses_p = not (sel.get("variant", 0) & VARIANT_TOPK_ONLY)
    if uses_p and top_p < 1.0 and L == sel["n_p"]:
        C = sel["C"]
        n_p = sel["n_p"]
        if abs(C[n_p - 1] - top_p) <= tol_m or (n_p >= 2 and abs(C[n_p - 2] - top_p) <= tol_m):
            return True
    if uses_p and capped and L == sel["n_cap"]:
        if gap(sel["n_cap"] + 1) <= tol_s or gap(sel["n_cap"]) <= tol_s:
            return True
    return False


def row_is_valid_alternative(s_row: np.ndarray, cols: np.ndarray, sel: dict, tol_s: float = TOL_SCORE) -> bool:
    """For a tie-affected row: is `cols` a selection some rounding of the scores
    could produce?  It must keep the Top-k floor (one block for Top-p
    alone), be a prefix of the score
    order up to the tie tolerance, and have a length within two of the
    oracle's."""
    cols = np.asarray(cols)
    floor = 1 if sel.get("variant", 0) & VARIANT_TOPP_ONLY else sel["n_k"]
    if cols.size < floor or abs(cols.size - sel["L"]) > 2:
        return False
    if np.unique(cols).size != cols.size or (np.diff(cols) <= 0).any():
        return False
    inside = np.zeros(s_row.size, bool)
    inside[cols] = True
    if inside.all():
        return True
    return s_row[~inside].max() <= s_row[inside].min() + tol_s


def select_blocks(qp: np.ndarray, kp: np.ndarray, blk_start: np.ndarray, params: Params, N: int,
                  rows: np.ndarray | None = None) -> dict:
    """Pool, score and select for one head.  qp, kp: [N][D] permuted order.
    rows: optional subset of query blocks (default all)."""
    D = qp.shape[-1]
    qbar = pool_blocks(qp, blk_start)
    kbar = pool_blocks(kp, blk_start)
    sizes = np.diff(blk_start) * 64
    nb = sizes.size
    rows = np.arange(nb) if rows is None else np.asarray(rows)
    scale = params.score_scale(D)
    out_rows, ties = {}, []
    capped = params.density_cap < 1.0
    for i in rows:
        s_row = block_scores(qbar[i:i + 1], kbar, scale)[0]
        P_row = block_probabilities(s_row)
        sel = select_row(s_row, P_row, sizes, params.top_k, params.top_p, params.density_cap, N, params.variant)
        sel["s"] = s_row
        sel["tie"] = row_tie_affected(s_row, sel, params.top_p, capped)
        out_rows[int(i)] = sel
        if sel["tie"]:
            ties.append(int(i))
    return dict(qbar=qbar, kbar=kbar, sizes=sizes, rows=out_rows, ties=ties)


def csr_from_rows(cols_per_row: list[np.ndarray]) -> tuple[np.ndarray, np.ndarray]:
    row_ptr = np.zeros(len(cols_per_row) + 1, np.int64)
    row_ptr[1:] = np.cumsum([c.size for c in cols_per_row])
    col = np.concatenate(cols_per_row) if cols_per_row else np.zeros(0, np.int64)
    return row_ptr, col.astype(np.int64)


def csr_transpose(row_ptr: np.ndarray, col_idx: np.ndarray, n_cols: int) -> tuple[np.ndarray, np.ndarray]:
    """Key-major copy of the block index: for each key block, the query blocks
    that selected it, ascending."""
    rows = np.repeat(np.arange(row_ptr.size - 1), np.diff(row_ptr))
    order = np.lexsort((rows, col_idx))
    t_ptr = np.zeros(n_cols + 1, np.int64)
    t_ptr[1:] = np.cumsum(np.bincount(col_idx, minlength=n_cols))
    return t_ptr, rows[order]


# ----------------------------------------------------------------------------
# sparse attention on the selected blocks [pt/M3], [zh/FAQ], R16
# ----------------------------------------------------------------------------

def _key_tokens(cols: np.ndarray, blk_start: np.ndarray) -> np.ndarray:
    return np.concatenate([np.arange(blk_start[j] * 64, blk_start[j + 1] * 64) for j in cols])


def sparse_attention_fwd(qp, kp, vp, blk_start, row_ptr, col_idx, scale, rows=None):
    """o_p = softmax_t(scale q_p . k_t) v_t over the tokens t of the key blocks
    in S_i, for every token p of query block i; lse_p = ln sum_t exp(...).
    All arrays in permuted order, float64.  Returns (o_p [N][D], lse [N]);
    with `rows`, only those query blocks are computed (the rest stay 0)."""
    qp = np.asarray(qp, np.float64)
    kp = np.asarray(kp, np.float64)
    vp = np.asarray(vp, np.float64)
    o = np.zeros_like(qp)
    lse = np.zeros(qp.shape[0])
    for i in (range(blk_start.size - 1) if rows is None else rows):
        qs = slice(blk_start[i] * 64, blk_start[i + 1] * 64)
        kt = _key_tokens(col_idx[row_ptr[i]:row_ptr[i + 1]], blk_start)
        s = scale * (qp[qs] @ kp[kt].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[qs] = (e / z) @ vp[kt]
        lse[qs] = (m + np.log(z))[:, 0]
    return o, lse


def sparse_attention_bwd(qp, kp, vp, op, dop, lse, blk_start, row_ptr, col_idx, scale, rows=None):
    """Gradients of sum(O * dO) with the selection held fixed ([zh/FAQ]: the
    statistics, shapes and P_i are constants).  Returns (dq_p, dk_p, dv_p);
    with `rows`, only the contributions of those query blocks."""
    qp, kp, vp, op, dop = (np.asarray(x, np.float64) for x in (qp, kp, vp, op, dop))
    dq = np.zeros_like(qp)
    dk = np.zeros_like(kp)
    dv = np.zeros_like(vp)
    for i in (range(blk_start.size - 1) if rows is None else rows):
        qs = slice(blk_start[i] * 64, blk_start[i + 1] * 64)
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        kt = _key_tokens(cols, blk_start)
        P = np.exp(scale * (qp[qs] @ kp[kt].T) - lse[qs][:, None])
        dP = dop[qs] @ vp[kt].T
        delta = (dop[qs] * op[qs]).sum(axis=1, keepdims=True)
        dS = P * (dP - delta)
        dq[qs] = scale * (dS @ kp[kt])
        dk_part = scale * (dS.T @ qp[qs])
        dv_part = P.T @ dop[qs]
        off = 0
        for j in cols:
            n = (blk_start[j + 1] - blk_start[j]) * 64
            ks = slice(blk_start[j] * 64, blk_start[j + 1] * 64)
            dk[ks] += dk_part[off:off + n]
            dv[ks] += dv_part[off:off + n]
            off += n
    return dq, dk, dv


def sparse_attention_key_block_grad(qp, kp, vp, op, dop, lse, blk_start, qrows, j, scale):
    """dK and dV of the tokens of key block j alone ([zh/FAQ]: with S fixed,
    gradients reach a key token only from the query blocks whose S_i holds
    its block).  qrows: those query blocks (the column of j in the key-major
    index).  op and lse need only be valid on the tokens of qrows.  Per query
    token p and key token t of j:
        P_pt = exp(scale q_p . k_t - lse_p),  dS_pt = P_pt (dO_p . v_t - dO_p . o_p),
        dV_t = sum_p P_pt dO_p,  dK_t = scale sum_p dS_pt q_p.
    Returns (dk_j, dv_j), each [|B_j|][D], float64."""
    ks = slice(blk_start[j] * 64, blk_start[j + 1] * 64)
    k = np.asarray(kp[ks], np.float64)
    v = np.asarray(vp[ks], np.float64)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in qrows:
        qs = slice(blk_start[i] * 64, blk_start[i + 1] * 64)
        q = np.asarray(qp[qs], np.float64)
        o = np.asarray(op[qs], np.float64)
        do = np.asarray(dop[qs], np.float64)
        P = np.exp(scale * (q @ k.T) - np.asarray(lse[qs], np.float64)[:, None])
        dS = P * (do @ v.T - (do * o).sum(axis=1, keepdims=True))
        dv += P.T @ do
        dk += scale * (dS.T @ q)
    return dk, dv


def dense_attention(q, k, v, scale):
    """Full softmax attention (the quadratic baseline the method replaces)."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[:, 0]


def dense_attention_bwd(q, k, v, o, do, lse, scale):
    q, k, v, o, do = (np.asarray(x, np.float64) for x in (q, k, v, o, do))
    P = np.exp(scale * (q @ k.T) - lse[:, None])
    dS = P * (do @ v.T - (do * o).sum(axis=1, keepdims=True))
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ do


def masked_attention_thw(q, k, v, blk_of_token, row_ptr, col_idx, scale):
    """Independent route to the sparse forward: dense attention in THW order
    with an additive -inf mask built from the token -> block map, no permuted
    tensors.  Returns (o [N][D], lse [N])."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    nb = row_ptr.size - 1
    allowed = np.zeros((nb, nb), bool)
    for i in range(nb):
        allowed[i, col_idx[row_ptr[i]:row_ptr[i + 1]]] = True
    mask = allowed[blk_of_token[:, None], blk_of_token[None, :]]
    s = np.where(mask, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[:, 0]


def selected_pairs(blk_start: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray) -> int:
    """Number of (query token, key token) pairs attended."""
    sizes = np.diff(blk_start) * 64
    rows = np.repeat(np.arange(sizes.size), np.diff(row_ptr))
    return int((sizes[rows] * sizes[col_idx]).sum())


def attention_flops(pairs: int, head_dim: int) -> tuple[int, int]:
    """Algorithmic FLOPs: forward 2 GEMMs (4 D per pair), backward 5 GEMMs
    (10 D per pair: the recomputed scores, dP, dV, dQ, dK)."""
    return 4 * head_dim * pairs, 10 * head_dim * pairs


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def run_pipeline(q, k, v, a, T, H, W, params: Params, do=None, attention: bool = True,
                 forced_shape: np.ndarray | None = None) -> dict:
    """Run every step for all heads.  q, k, v, do: [heads][N][D] (bf16 values
    as float32/float64), a: [N] or None.  Returns per-step results."""
    heads, N, D = q.shape
    zs = zone_statistics(v, a, T, H, W, params.eps, params.variant)
    if params.variant & VARIANT_FIXED_SHAPE:
        forced_shape = np.full(zs["rho"].shape, params.fixed_shape, np.int64)
    plan = plan_shapes(zs["g"], zs["rho"], params.tau128, params.tau256, forced_shape)
    scale = params.score_scale(D)
    res = dict(zone=zs, plan=plan, heads=[])
    for h in range(heads):
        perm, blk_start = partition(plan["shape_id"][h], T, H, W)
        qp, kp = permute_tokens(q[h], perm), permute_tokens(k[h], perm)
        sel = select_blocks(qp, kp, blk_start, params, N)
        nb = blk_start.size - 1
        row_ptr, col_idx = csr_from_rows([sel["rows"][i]["cols"] for i in range(nb)])
        t_ptr, t_col = csr_transpose(row_ptr, col_idx, nb)
        hr = dict(perm=perm, blk_start=blk_start, n_blocks=nb, sel=sel, row_ptr=row_ptr, col_idx=col_idx,
                  t_row_ptr=t_ptr, t_col_idx=t_col, pairs=selected_pairs(blk_start, row_ptr, col_idx))
        if attention:
            vp = permute_tokens(v[h], perm)
            op, lse = sparse_attention_fwd(qp, kp, vp, blk_start, row_ptr, col_idx, scale)
            hr.update(o=unpermute_tokens(op, perm), lse_p=lse, o_p=op)
            if do is not None:
                dop = permute_tokens(do[h], perm)
                dq, dk, dv = sparse_attention_bwd(qp, kp, vp, op, dop, lse, blk_start, row_ptr, col_idx, scale)
                hr.update(dq=unpermute_tokens(dq, perm), dk=unpermute_tokens(dk, perm),
                          dv=unpermute_tokens(dv, perm))
        res["heads"].append(hr)
    return res

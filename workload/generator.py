"""Seeded synthetic video-latent workloads for Prism sparse video self-attention.

The Prism pages evaluate on real 2K clips (their 2K-Bench), which are not
available; these generators stand in for them with the structure the pages
describe: hundreds of thousands of video tokens on a T x H x W latent grid,
large repetitive static background, content that varies along one direction
inside a local region, and compact sounding regions that carry the
audio-to-video coupling.  Nothing here computes any step of the method; both
the CPU oracle and the GPU path receive the same bfloat16-rounded arrays.

Recipe (one numpy PCG64 stream per workload, fixed draw order):
  1. zone attributes: static-zone subset (exactly round(f*Z) zones), a field
     axis per zone (uniform over T/H/W; static zones use H or W only, so they
     are near-constant along T), and an amplitude A_m ~ U[0, 2];
  2. noise q, k, v ~ N(0, 1), float32, per head in THW token order;
  3. per-(head, zone) direction vectors u (shared by q and k, so that pooled
     block scores show locality) and w (for v), N(0, I_D);
  4. sound-blob centres, uniform over the grid;
  5. the dispersed-query subset (exactly round(f*Z) zones), whose q is replaced
     by 0.02 * its noise and gets no field, so its block scores are nearly
     uniform;
  6. dO ~ N(0, 1) for workloads with a backward pass;
  7. for the tiny workload, random directions z_n ~ N(0, I_64) that give the
     audio-to-video output vectors h_n = a_n * z_n / |z_n|.
The smooth field added to q and k is A_m * phi(i) * u_m and to v
A_m * phi(i) * w_m, phi(i) = cos(pi (i + 1/2) / 8), i the zone-local
coordinate along the zone's axis.  The audio norm map is
a = base + sum_b exp(-|x - c_b|^2 / (2 sigma^2)), x = (t, h, w) in token units.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

ZONE = 8  # macro-zone edge (tokens) along T, H and W


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    seed: int
    static_frac: float
    n_blobs: int
    blob_sigma: float
    a_base: float
    top_k: int
    top_p: float
    density_cap: float = 1.0          # 1.0 means no cap
    backward: bool = True
    dispersed_frac: float = 0.0
    h_hat_dim: int = 0                # > 0: also draw the A2V output vectors
    note: str = ""

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def Z(self) -> int:
        return (self.T // ZONE) * (self.H // ZONE) * (self.W // ZONE)

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS: dict[str, WorkloadConfig] = {
    # the small case the oracle runs in well under a second
    "tiny": WorkloadConfig("tiny", 8, 16, 16, 1, 64, 1, 0.0, 1, 3.0, 0.1, 2, 0.9,
                           h_hat_dim=64, note="tiny oracle case, 2,048 tokens"),
    "720p": WorkloadConfig("720p", 16, 48, 80, 4, 128, 720, 0.2, 2, 6.0, 0.05, 8, 0.9,
                           backward=False, note="720p-shaped forward, 61,440 tokens"),
    "1080p": WorkloadConfig("1080p", 16, 72, 120, 2, 128, 1080, 0.4, 2, 6.0, 0.05, 8, 0.9,
                            note="1080p-shaped training step, 138,240 tokens"),
    "2k": WorkloadConfig("2k", 32, 88, 160, 2, 128, 2048, 0.6, 3, 8.0, 0.05, 16, 0.9,
                         density_cap=0.10, note="2K headline, 450,560 tokens"),
    "long": WorkloadConfig("long", 64, 88, 160, 1, 128, 4096, 0.6, 3, 8.0, 0.05, 16, 0.95,
                           density_cap=0.15, dispersed_frac=0.5,
                           note="2K long-clip stress, 901,120 tokens"),
    # parity cases: several tiles, mixed block sizes, ragged row lengths
    "par_small": WorkloadConfig("par_small", 16, 24, 32, 2, 128, 11, 0.4, 2, 4.0, 0.05, 4, 0.9,
                                note="12,288 tokens, 24 zones"),
    "par_cap": WorkloadConfig("par_cap", 8, 32, 40, 2, 128, 12, 0.3, 2, 4.0, 0.05, 4, 0.95,
                              density_cap=0.2, dispersed_frac=0.5,
                              note="10,240 tokens, cap-bound dispersed rows"),
    "par_d64": WorkloadConfig("par_d64", 16, 16, 24, 1, 64, 13, 0.3, 1, 3.0, 0.1, 3, 0.8,
                              note="6,144 tokens, head_dim 64"),
    "one_zone": WorkloadConfig("one_zone", 8, 8, 8, 1, 128, 14, 0.0, 1, 2.0, 0.1, 1, 0.5,
                               note="a single macro-zone"),
    "par_heads": WorkloadConfig("par_heads", 8, 24, 40, 5, 128, 15, 0.3, 2, 4.0, 0.05, 4, 0.9,
                                density_cap=0.3, dispersed_frac=0.3,
                                note="7,680 tokens, five heads (60 tile pairs each: uneven queue eighths)"),
    # many heads of a small grid: all heads' K and V (277 MB) exceed the 256 MB
    # last-level cache, so the attention work queues run head by head, at a
    # size the oracle checks in full
    "many_heads": WorkloadConfig("many_heads", 8, 32, 48, 44, 128, 16, 0.3, 2, 4.0, 0.05, 4, 0.9,
                                 density_cap=0.1, dispersed_frac=0.25,
                                 note="12,288 tokens, 44 heads (head-by-head queue order)"),
    # the largest grid the library accepts (1,048,576 tokens); with every zone
    # cut into 64-token blocks it has the most blocks a selection row can hold
    "max_grid": WorkloadConfig("max_grid", 16, 128, 512, 1, 128, 4097, 0.6, 3, 8.0, 0.05, 16, 0.9,
                               density_cap=0.02, note="largest accepted grid, 1,048,576 tokens"),
}


# ----------------------------------------------------------------------------
# bfloat16 helpers (storage format of the GPU inputs; round to nearest even)
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    cfg: WorkloadConfig
    q_bits: np.ndarray            # [heads][N][D] uint16 (bf16), THW token order
    k_bits: np.ndarray
    v_bits: np.ndarray
    a: np.ndarray                 # [N] float32 audio-to-video norm map
    do_bits: np.ndarray | None    # [heads][N][D] uint16 or None
    h_hat: np.ndarray | None      # [N][h_hat_dim] float32 or None
    zone_axis: np.ndarray         # [Z] int (0 = T, 1 = H, 2 = W)
    zone_amp: np.ndarray          # [Z] float
    static_mask: np.ndarray       # [Z] bool
    dispersed_mask: np.ndarray    # [Z] bool
    extras: dict = field(default_factory=dict)

    def f32(self, name: str) -> np.ndarray:
        """The exact float32 values of a bf16 tensor ("q", "k", "v", "do")."""
        return bf16_bits_to_f32(getattr(self, name + "_bits"))


def _phi(i: np.ndarray) -> np.ndarray:
    return np.cos(np.pi * (i + 0.5) / ZONE)


def _token_zone_and_local(T: int, H: int, W: int):
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    zone = ((t // ZONE) * (H // ZONE) + h // ZONE) * (W // ZONE) + w // ZONE
    return zone.reshape(-1), np.stack([t % ZONE, h % ZONE, w % ZONE]).reshape(3, -1), (t, h, w)


def generate(cfg: WorkloadConfig | str, *, keep_fp32: bool = False) -> Workload:
    """Draw one workload.  All tensors are returned in THW token order."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    T, H, W, D, heads = cfg.T, cfg.H, cfg.W, cfg.head_dim, cfg.heads
    if T % ZONE or H % ZONE or W % ZONE:
        raise ValueError("grid must be a multiple of 8 along T, H and W")
    N, Z = cfg.N, cfg.Z
    rng = np.random.Generator(np.random.PCG64(cfg.seed))

    # 1. zone attributes
    n_static = int(round(cfg.static_frac * Z))
    static_mask = np.zeros(Z, bool)
    if n_static:
        static_mask[rng.choice(Z, n_static, replace=False)] = True
    axis_any = rng.integers(0, 3, Z)
    axis_static = rng.integers(1, 3, Z)
    zone_axis = np.where(static_mask, axis_static, axis_any)
    zone_amp = rng.uniform(0.0, 2.0, Z)

    # 2. noise
    q = rng.standard_normal((heads, N, D), dtype=np.float32)
    k = rng.standard_normal((heads, N, D), dtype=np.float32)
    v = rng.standard_normal((heads, N, D), dtype=np.float32)

    # 3. per-(head, zone) directions
    u = rng.standard_normal((heads, Z, D)).astype(np.float32)
    w_dir = rng.standard_normal((heads, Z, D)).astype(np.float32)

    # 4. sound-blob centres
    centres = rng.uniform(0.0, 1.0, (cfg.n_blobs, 3)) * np.array([T, H, W], np.float64)

    # 5. dispersed-query zones
    dispersed_mask = np.zeros(Z, bool)
    n_disp = int(round(cfg.dispersed_frac * Z))
    if n_disp:
        dispersed_mask[rng.choice(Z, n_disp, replace=False)] = True

    # 6. upstream gradient
    do = rng.standard_normal((heads, N, D), dtype=np.float32) if cfg.backward else None

    # 7. A2V output directions (tiny workload only)
    z_dirs = rng.standard_normal((N, cfg.h_hat_dim)) if cfg.h_hat_dim else None

    # smooth zone fields
    tok_zone, local, (tt, hh, ww) = _token_zone_and_local(T, H, W)
    coef = (zone_amp[tok_zone] * _phi(local[zone_axis[tok_zone], np.arange(N)])).astype(np.float32)
    tok_disp = dispersed_mask[tok_zone]
    for hd in range(heads):
        uf = u[hd][tok_zone]
        uf *= coef[:, None]
        q[hd] += uf
        k[hd] += uf
        if n_disp:
            q[hd][tok_disp] = 0.02 * (q[hd][tok_disp] - uf[tok_disp])
        del uf
        wf = w_dir[hd][tok_zone]
        wf *= coef[:, None]
        v[hd] += wf
        del wf

    # audio-to-video norm map
    x = np.stack([tt.reshape(-1), hh.reshape(-1), ww.reshape(-1)], axis=1).astype(np.float64)
    a64 = np.full(N, cfg.a_base, np.float64)
    for c in centres:
        a64 += np.exp(-np.sum((x - c) ** 2, axis=1) / (2.0 * cfg.blob_sigma ** 2))
    a = a64.astype(np.float32)
    h_hat = None
    if z_dirs is not None:
        h_hat = (a64[:, None] * z_dirs / np.linalg.norm(z_dirs, axis=1, keepdims=True)).astype(np.float32)

    wl = Workload(cfg=cfg, q_bits=bf16_round(q), k_bits=bf16_round(k), v_bits=bf16_round(v), a=a,
                  do_bits=bf16_round(do) if do is not None else None, h_hat=h_hat,
                  zone_axis=zone_axis, zone_amp=zone_amp, static_mask=static_mask,
                  dispersed_mask=dispersed_mask)
    if keep_fp32:
        wl.extras.update(q32=q, k32=k, v32=v, do32=do)
    return wl


def a2v_output(wl: Workload, channels: int, token_stride: int | None = None) -> np.ndarray:
    """Synthetic audio-to-video cross-attention output h-hat [N][channels]
    (bf16 bit patterns, rows padded to token_stride values) for a workload
    of any size: h_n = a_n * z_n / sqrt(channels) with z_n ~ N(0, I) from a
    stream of its own (seed + 7919 * channels), so the workload's other draws
    do not change and |h_n| is close to a_n.  The padding holds bf16 NaN,
    which no reader may touch."""
    N = wl.cfg.N
    stride = channels if token_stride is None else token_stride
    rng = np.random.Generator(np.random.PCG64(wl.cfg.seed + 7919 * channels))
    out = np.full((N, stride), 0x7FC0, np.uint16)
    step = 1 << 16
    for s0 in range(0, N, step):
        z = rng.standard_normal((min(step, N - s0), channels), dtype=np.float32)
        z *= (wl.a[s0:s0 + z.shape[0]] / np.float32(np.sqrt(channels)))[:, None]
        out[s0:s0 + z.shape[0], :channels] = bf16_round(z)
    return out

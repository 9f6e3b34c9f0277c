"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare every step with the CPU oracle.

Discrete decisions (volumes, shapes, selected blocks) must match bit for bit,
except where the oracle records a tie within tolerance (a density within
1e-6 of a threshold, a shape distance margin within 1e-6, block scores within
1e-6 at a cut, cumulative mass within 1e-9 of p): there the GPU's choice must
be one of the tied options and the oracle adopts it for the later steps.
"""

from __future__ import annotations

import math
import time

import numpy as np

import oracle as O
from workload import Workload

FWD_MAX_ABS = 2e-2      # bf16 GPU output vs float64 oracle
FWD_MEAN_ABS = 2e-3
GRAD_REL_L2 = 1e-2
LSE_MAX_ABS = 2e-3


def log(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)


def oracle_params(cfg, **over) -> O.Params:
    d = dict(top_k=cfg.top_k, top_p=cfg.top_p, density_cap=cfg.density_cap)
    d.update(over)
    return O.Params(**d)


def binding_params(cfg, **over):
    from dynamic_block_sparse_macro_amd import binding as B
    d = dict(top_k=cfg.top_k, top_p=cfg.top_p, density_cap=cfg.density_cap)
    d.update(over)
    return B.make_params(**d)


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_dev_to_f32(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)


class LayerOnGpu:
    """One pass of the whole layer on the GPU, with host copies of every output."""

    def __init__(self, wl: Workload, params=None, backward: bool | None = None, layer_kw=None):
        import torch
        from dynamic_block_sparse_macro_amd.pipeline import LayerShape, PrismLayer
        c = wl.cfg
        self.cfg = c
        self.params = params if params is not None else binding_params(c)
        self.shape = LayerShape(c.T, c.H, c.W, c.heads, c.head_dim)
        self.layer = PrismLayer(self.shape, self.params, **(layer_kw or {}))
        self.q, self.k, self.v = (to_dev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
        self.a = torch.from_numpy(wl.a).cuda()
        self.o = torch.empty_like(self.q)
        self.nnz = self.layer.forward(self.q, self.k, self.v, self.a, self.o)
        backward = c.backward if backward is None else backward
        self.backward = backward and wl.do_bits is not None
        if self.backward:
            self.do = to_dev(wl.do_bits)
            self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
            self.layer.attn_bwd(self.o, self.do, self.dq, self.dk, self.dv)
        torch.cuda.synchronize()

    def host(self):
        L = self.layer
        out = dict(zstats=L.zstats.cpu().numpy(), g=L.g.cpu().numpy(), rho=L.rho.cpu().numpy(),
                   shape_id=L.shape_id.cpu().numpy().astype(np.int64), index=L.index_host(),
                   o=bf16_dev_to_f32(self.o), lse=L.lse.cpu().numpy())
        if self.backward:
            out.update(dq=bf16_dev_to_f32(self.dq), dk=bf16_dev_to_f32(self.dk), dv=bf16_dev_to_f32(self.dv))
        return out


# ----------------------------------------------------------------------------
# step checks
# ----------------------------------------------------------------------------

def check_zone_stats(gpu: dict, zs: dict, rtol=1e-12):
    z = gpu["zstats"]
    np.testing.assert_allclose(z[..., 0:3], zs["sv2"], rtol=rtol, atol=1e-300)
    np.testing.assert_allclose(z[0, :, 3:6], zs["sa2"], rtol=rtol, atol=1e-300)
    np.testing.assert_allclose(z[0, :, 6], zs["mu_a"], rtol=rtol, atol=1e-300)
    np.testing.assert_allclose(z[0, :, 7], zs["abar"], rtol=rtol, atol=1e-15)
    np.testing.assert_allclose(gpu["g"], zs["g"], rtol=rtol, atol=0)
    np.testing.assert_allclose(gpu["rho"], zs["rho"], rtol=rtol, atol=1e-300)


def reconcile_shapes(gpu_shape: np.ndarray, zs: dict, plan: dict, op: O.Params):
    """Exact match outside ties; for tied zones the GPU's choice must be in
    the tie set.  Returns (forced-shape array, number of tied zones)."""
    heads, Z = gpu_shape.shape
    forced = np.full((heads, Z), -1, np.int64)
    ties = 0
    for h in range(heads):
        for m in range(Z):
            tied = plan["dist_margin"][h, m] <= O.TOL_DIST or plan["vol_margin"][h, m] <= O.TOL_RHO
            if gpu_shape[h, m] == plan["shape_id"][h, m]:
                continue
            assert tied, f"head {h} zone {m}: GPU shape {gpu_shape[h, m]} vs oracle {plan['shape_id'][h, m]}"
            allowed = O.shape_tie_set(zs["g"][h, m], zs["rho"][h, m], op.tau128, op.tau256)
            assert int(gpu_shape[h, m]) in allowed, (h, m, allowed)
            forced[h, m] = gpu_shape[h, m]
            ties += 1
    return forced, ties


def check_partition(gidx: dict, perm: np.ndarray, blk_start: np.ndarray):
    assert gidx["n_blocks"] == blk_start.size - 1
    np.testing.assert_array_equal(gidx["blk_start"], blk_start)
    np.testing.assert_array_equal(gidx["perm"], perm)


def unswizzle_tiles(stored: np.ndarray, D: int) -> np.ndarray:
    """Operand layout -> plain rows.  Each 64-row tile is row-major with the
    16-byte chunk c of row r stored at chunk position c ^ f(r), with
    f(r) = ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1) for D = 128
    and f(r) = (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)
    for D = 64."""
    n = stored.shape[0]
    ch = D // 8
    t = stored.reshape(n // 64, 64, ch, 8)
    r = np.arange(64)
    if D == 128:
        f = ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)
    else:
        f = (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1)
    pos = np.arange(ch)[None, :] ^ f[:, None]            # [64][ch]: stored position of logical chunk c
    return t[:, r[:, None], pos, :].reshape(n, D)


def check_operands(layer, h: int, wl: Workload, perm: np.ndarray):
    """The operand buffers hold the permuted rows, bitwise, in the swizzled
    64-row tile layout."""
    import torch
    D = wl.cfg.head_dim
    for name, buf in (("q", layer.qp), ("k", layer.kp), ("v", layer.vp)):
        bits = getattr(wl, name + "_bits")[h]
        host = buf.view(torch.int16).cpu().numpy().view(np.uint16)[h]
        np.testing.assert_array_equal(unswizzle_tiles(host, D), bits[perm])


def compare_rows(gidx: dict, osel: dict, rows) -> dict:
    """Selected key blocks of each query-block row: bit-exact outside ties."""
    rp, col = gidx["row_ptr"], gidx["col_idx"]
    ties, alt = 0, 0
    for i in rows:
        g_cols = col[rp[i]:rp[i + 1]]
        r = osel["rows"][int(i)]
        if np.array_equal(g_cols, r["cols"]):
            ties += int(r["tie"])
            continue
        assert r["tie"], f"row {i}: GPU selected {g_cols.size} blocks, oracle {r['cols'].size}, not a tie"
        assert O.row_is_valid_alternative(r["s"], g_cols, r), f"row {i}: not a valid tie alternative"
        ties += 1
        alt += 1
    return dict(tie_rows=ties, alternative_rows=alt)


def check_transpose(gidx: dict):
    tp, tc = O.csr_transpose(gidx["row_ptr"], gidx["col_idx"], gidx["n_blocks"])
    np.testing.assert_array_equal(gidx["t_row_ptr"], tp)
    np.testing.assert_array_equal(gidx["t_col_idx"], tc)


def check_f32_rounding(gpu: np.ndarray, ref: np.ndarray, rel_tie: float = 1e-12) -> int:
    """gpu (float32) must be ref (float64) rounded to nearest; where ref lies
    within rel_tie of the midpoint between two float32 values either
    neighbour is accepted.  Returns the number of such ties taken the other
    way."""
    gpu = np.asarray(gpu, np.float32)
    near = ref.astype(np.float32)
    bad = gpu != near
    if not bad.any():
        return 0
    g, r, n = gpu[bad], ref[bad], near[bad]
    up, down = np.nextafter(n, np.float32(np.inf)), np.nextafter(n, np.float32(-np.inf))
    assert ((g == up) | (g == down)).all(), "GPU value more than one float32 step from the reference"
    mid = (g.astype(np.float64) + n.astype(np.float64)) / 2
    assert (np.abs(r - mid) <= rel_tie * np.abs(r)).all(), "GPU value is not a correct rounding"
    return int(bad.sum())


def fwd_errors(o_gpu: np.ndarray, o_ref: np.ndarray) -> tuple[float, float]:
    d = np.abs(o_gpu.astype(np.float64) - o_ref)
    return float(d.max()), float(d.mean())


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(x.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def oracle_index_to_device(layer, idx_per_head: list[dict]):
    """Upload an oracle block index into the layer's index buffers (global
    offsets across heads, tail entries repeated), so that the GPU attention
    runs on exactly the oracle's selection."""
    import torch
    tiles = layer.shape.tiles
    heads = layer.shape.heads
    rp = np.zeros((heads, tiles + 1), np.int32)
    trp = np.zeros((heads, tiles + 1), np.int32)
    cols, tcols = [], []
    base = 0
    for h, ix in enumerate(idx_per_head):
        nb = ix["blk_start"].size - 1
        rp[h, :nb + 1] = ix["row_ptr"] + base
        rp[h, nb + 1:] = ix["row_ptr"][-1] + base
        trp[h, :nb + 1] = ix["t_row_ptr"] + base
        trp[h, nb + 1:] = ix["t_row_ptr"][-1] + base
        cols.append(ix["col_idx"])
        tcols.append(ix["t_col_idx"])
        base += int(ix["row_ptr"][-1])
    col = np.concatenate(cols).astype(np.int32)
    tcol = np.concatenate(tcols).astype(np.int32)
    layer.row_ptr.copy_(torch.from_numpy(rp))
    layer.t_row_ptr.copy_(torch.from_numpy(trp))
    if col.size > layer.col_cap:
        layer.col_cap = col.size
        layer.col_idx = torch.empty(col.size, dtype=torch.int32, device=layer.device)
        layer.t_col_idx = torch.empty_like(layer.col_idx)
    layer.col_idx[:col.size].copy_(torch.from_numpy(col))
    layer.t_col_idx[:tcol.size].copy_(torch.from_numpy(tcol))

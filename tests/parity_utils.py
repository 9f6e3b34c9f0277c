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
import os
import time
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import get_context, shared_memory

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

    def __init__(self, wl: Workload, params=None, backward: bool | None = None, layer_kw=None,
                 fill_nan: bool = False):
        """fill_nan: every output buffer (O, its low parts, LSE, dQ, dK, dV)
        starts as NaN, so an element no work item wrote stays NaN."""
        import torch
        from dynamic_block_sparse_macro_amd.pipeline import LayerShape, PrismLayer
        c = wl.cfg
        self.cfg = c
        self.params = params if params is not None else binding_params(c)
        self.shape = LayerShape(c.T, c.H, c.W, c.heads, c.head_dim)
        self.layer = PrismLayer(self.shape, self.params, **(layer_kw or {}))
        self.q, self.k, self.v = (to_dev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits))
        self.a = torch.from_numpy(wl.a).cuda()

        def out_like(t):
            return torch.full_like(t, float("nan")) if fill_nan else torch.empty_like(t)

        self.o = out_like(self.q)
        if fill_nan:
            self.layer.lse.fill_(float("nan"))
            self.layer.o_lo.fill_(float("nan"))
        self.nnz = self.layer.forward(self.q, self.k, self.v, self.a, self.o)
        backward = c.backward if backward is None else backward
        self.backward = backward and wl.do_bits is not None
        if self.backward:
            self.do = to_dev(wl.do_bits)
            self.dq, self.dk, self.dv = (out_like(self.q) for _ in range(3))
            self.layer.attn_bwd(self.o, self.do, self.dq, self.dk, self.dv)
        torch.cuda.synchronize()

    def check_index(self):
        """prism_check_index on a host copy of the index the layer holds."""
        check_device_index(self.layer)

    def host(self):
        L = self.layer
        self.check_index()
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


def fwd_row_bound(vp: np.ndarray, blk_start: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray) -> np.ndarray:
    """Per-token forward error bound (block order) from bf16 rounding alone:
    the weights are rounded to bf16 before the PV product and in their sum
    (bf16 keeps 8 significant bits: up to 2^-8 relative each, so at most
    2^-7 of the largest |v| among the row's selected keys), and O is rounded
    to bf16 on output (up to 2^-8 of |O|, itself at most that |v|); plus 1e-3
    for float32 accumulation: 3 * 2^-8 * max over the row's keys of |v| +
    1e-3.  It exceeds the fixed 2e-2 bar only where outputs approach the
    largest values (for |O| >= 8 half a bf16 step, 2^-5, is already above
    2e-2)."""
    bound = np.zeros(vp.shape[0])
    vmax = np.abs(vp).max(axis=1)
    for i in range(blk_start.size - 1):
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        m = max(float(vmax[blk_start[j] * 64:blk_start[j + 1] * 64].max()) for j in cols)
        bound[blk_start[i] * 64:blk_start[i + 1] * 64] = 3 * 2.0 ** -8 * m + 1e-3
    return bound


def check_fwd_elements(o_gpu: np.ndarray, o_ref: np.ndarray, bound_thw: np.ndarray) -> tuple[int, float]:
    """Every element within max(2e-2, its row's bf16 rounding bound); returns
    the number of elements beyond 2e-2 and the largest error / bound."""
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    allowed = np.maximum(FWD_MAX_ABS, bound_thw)[:, None]
    assert (err <= allowed).all(), f"forward error {err.max():.3e} beyond its row bound"
    return int((err > FWD_MAX_ABS).sum()), float((err / allowed).max())


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
    check_device_index(layer)


def check_device_index(layer):
    """The index a layer's attention calls will read (perm, block starts,
    both block lists, as held on the device) passes prism_check_index."""
    from dynamic_block_sparse_macro_amd import binding as B
    host = lambda t: np.ascontiguousarray(t.cpu().numpy().astype(np.int32))
    B.prism_check_index(layer.prob, host(layer.perm), host(layer.blk_start), host(layer.n_blocks),
                        host(layer.row_ptr), host(layer.col_idx), host(layer.t_row_ptr), host(layer.t_col_idx),
                        layer.col_idx.numel())


# ----------------------------------------------------------------------------
# oracle work spread over worker processes (full-size checks)
# ----------------------------------------------------------------------------
# Workers are spawned (fresh interpreters that never touch the GPU); the large
# arrays reach them through shared memory, and each works on a chunk of
# query-block rows with the oracle's own functions.

def oracle_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(12, n - 2))


class SharedArrays:
    """numpy arrays copied into shared memory, attachable by name."""

    def __init__(self, **arrays):
        self.shm, self.spec = [], {}
        for name, a in arrays.items():
            a = np.ascontiguousarray(a)
            m = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, a.dtype, buffer=m.buf)[...] = a
            self.shm.append(m)
            self.spec[name] = (m.name, a.shape, a.dtype.str)

    def close(self):
        for m in self.shm:
            m.close()
            m.unlink()
        self.shm = []


_W: dict = {}


def _attach(spec: dict, extra: dict, threads: int = 1):
    from threadpoolctl import threadpool_limits
    _W.clear()
    _W["_limits"] = threadpool_limits(threads)   # BLAS threads of this worker
    _W["_shm"] = []
    for name, (sname, shape, dt) in spec.items():
        m = shared_memory.SharedMemory(name=sname)
        _W["_shm"].append(m)
        _W[name] = np.ndarray(shape, np.dtype(dt), buffer=m.buf)
    _W.update(extra)


def _select_chunk(rows):
    """Oracle selection of some query-block rows: (cols, tie, full row when tied)."""
    sel = O.select_blocks(_W["qp"], _W["kp"], _W["bs"], _W["params"], _W["N"], rows=rows)
    out = {}
    for i, r in sel["rows"].items():
        out[i] = (r["cols"], bool(r["tie"]), r if r["tie"] else None)
    return out


def _fwd_chunk(rows):
    """Oracle forward of some query blocks over their whole rows: o and lse of their tokens."""
    bs = _W["bs"]
    o, lse = O.sparse_attention_fwd(_W["qp"], _W["kp"], _W["vp"], bs, _W["rp"], _W["ci"], _W["scale"], rows=rows)
    tok = np.concatenate([np.arange(bs[i] * 64, bs[i + 1] * 64) for i in rows])
    return tok, o[tok], lse[tok]


def _pool(arrays: SharedArrays, extra: dict, workers: int):
    """A spawned process pool; each worker runs its share of the host's cores
    as BLAS threads."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return ProcessPoolExecutor(workers, mp_context=get_context("spawn"), initializer=_attach,
                               initargs=(arrays.spec, extra, max(1, cores // workers)))


def _progress(results, what: str, total: int):
    """Yield from results, logging every few finished chunks (long oracle
    runs keep printing)."""
    t0 = time.perf_counter()
    for n, r in enumerate(results, 1):
        if n == total or n % max(1, total // 6) == 0:
            log(f"  oracle {what}: {n} of {total} chunks ({time.perf_counter() - t0:.1f} s)")
        yield r


def _chunks(rows, n):
    rows = np.asarray(rows)
    return [c for c in np.array_split(rows, max(1, min(len(rows), n))) if c.size]


def oracle_select_all(qp, kp, blk_start, params: O.Params, N: int, workers: int | None = None) -> dict:
    """Oracle selection of every query-block row of one head, in parallel.
    Returns {row: (cols, tie, row dict when tied)}."""
    workers = workers or oracle_workers()
    nb = blk_start.size - 1
    sh = SharedArrays(qp=qp, kp=kp, bs=blk_start)
    try:
        with _pool(sh, dict(params=params, N=N), workers) as ex:
            out = {}
            chunks = _chunks(np.arange(nb), 6 * workers)
            for r in _progress(ex.map(_select_chunk, chunks), "selection", len(chunks)):
                out.update(r)
    finally:
        sh.close()
    return out


def oracle_fwd_rows(qp, kp, vp, blk_start, row_ptr, col_idx, scale, rows, workers: int | None = None):
    """Oracle forward of the query blocks `rows` (whole rows), in parallel.
    Returns (o, lse) over all tokens, valid on the tokens of `rows`."""
    workers = workers or oracle_workers()
    sh = SharedArrays(qp=qp, kp=kp, vp=vp, bs=blk_start, rp=row_ptr, ci=col_idx)
    o = np.zeros((qp.shape[0], qp.shape[1]))
    lse = np.zeros(qp.shape[0])
    try:
        with _pool(sh, dict(scale=scale), workers) as ex:
            chunks = _chunks(sorted(int(i) for i in rows), 3 * workers)
            for tok, ot, lt in _progress(ex.map(_fwd_chunk, chunks), "forward rows", len(chunks)):
                o[tok] = ot
                lse[tok] = lt
    finally:
        sh.close()
    return o, lse


def compare_all_rows(gidx: dict, osel: dict) -> dict:
    """Every query-block row of the GPU index against the oracle's selection:
    bit-exact outside ties, a valid tied alternative inside."""
    rp, col = gidx["row_ptr"], gidx["col_idx"]
    ties, alt = 0, 0
    for i in range(rp.size - 1):
        g_cols = col[rp[i]:rp[i + 1]]
        cols, tie, r = osel[i]
        if np.array_equal(g_cols, cols):
            ties += int(tie)
            continue
        assert tie, f"row {i}: GPU selected {g_cols.size} blocks, oracle {cols.size}, not a tie"
        assert O.row_is_valid_alternative(r["s"], g_cols, r), f"row {i}: not a valid tie alternative"
        ties += 1
        alt += 1
    return dict(tie_rows=ties, alternative_rows=alt)


def _pipeline_head(h):
    """The oracle's whole pipeline for head h alone, with that head's shapes
    given (from the all-head plan): per-head results as in run_pipeline."""
    W = _W
    res = O.run_pipeline(W["q"][h:h + 1], W["k"][h:h + 1], W["v"][h:h + 1], W["a"], W["T"], W["H"], W["W"],
                         W["params"], do=W["do"][h:h + 1], forced_shape=W["shape"][h:h + 1])
    hr = res["heads"][0]
    for nm in ("o", "dq", "dk", "dv", "o_p"):
        hr[nm] = hr[nm].astype(np.float32)
    return hr


def oracle_pipeline_heads(wl: Workload, params: O.Params, workers: int | None = None) -> dict:
    """O.run_pipeline for every head of a workload, heads spread over worker
    processes: zone statistics and the plan of all heads here (a and a-bar
    are shared by the heads), then each head's partition, selection, forward
    and backward in a worker with its planned shapes."""
    c = wl.cfg
    zs = O.zone_statistics(wl.f32("v"), wl.a, c.T, c.H, c.W, params.eps, params.variant)
    forced = None
    if params.variant & O.VARIANT_FIXED_SHAPE:
        forced = np.full(zs["rho"].shape, params.fixed_shape, np.int64)
    plan = O.plan_shapes(zs["g"], zs["rho"], params.tau128, params.tau256, forced)
    workers = workers or oracle_workers()
    sh = SharedArrays(q=wl.f32("q"), k=wl.f32("k"), v=wl.f32("v"), do=wl.f32("do"),
                      a=wl.a if wl.a is not None else np.zeros(c.N, np.float32), shape=plan["shape_id"])
    try:
        with _pool(sh, dict(params=params, T=c.T, H=c.H, W=c.W), workers) as ex:
            heads = list(_progress(ex.map(_pipeline_head, range(c.heads)), "heads", c.heads))
    finally:
        sh.close()
    return dict(zone=zs, plan=plan, heads=heads)

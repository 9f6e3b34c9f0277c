"""GPU parity: every step of the HIP path (through the C ABI) against the CPU
oracle on seeded workloads small enough for the oracle to run in full."""

import math

import numpy as np
import pytest

import oracle as O
from workload import generate

from parity_utils import (FWD_MAX_ABS, FWD_MEAN_ABS, GRAD_REL_L2, LSE_MAX_ABS, LayerOnGpu, check_operands,
                          check_partition, check_transpose, check_zone_stats, compare_rows, fwd_errors, fwd_row_bound,
                          log,
                          oracle_index_to_device, oracle_params, reconcile_shapes, rel_l2)

pytestmark = pytest.mark.gpu

CASES = ["tiny", "one_zone", "par_d64", "par_small", "par_cap", "par_heads"]


def _oracle_head(wl, plan, h, op):
    c = wl.cfg
    perm, bs = O.partition(plan["shape_id"][h], c.T, c.H, c.W)
    qp = O.permute_tokens(wl.f32("q")[h], perm)
    kp = O.permute_tokens(wl.f32("k")[h], perm)
    sel = O.select_blocks(qp, kp, bs, op, c.N)
    nb = bs.size - 1
    rp, col = O.csr_from_rows([sel["rows"][i]["cols"] for i in range(nb)])
    trp, tcol = O.csr_transpose(rp, col, nb)
    return dict(perm=perm, blk_start=bs, sel=sel, row_ptr=rp, col_idx=col, t_row_ptr=trp, t_col_idx=tcol)


@pytest.mark.parametrize("name", CASES)
def test_pipeline_parity(name):
    _pipeline_parity(generate(name), {})


# (workload, variant switches, fixed shape index): the ablation baselines
VARIANTS = [
    ("par_small", O.VARIANT_FIXED_SHAPE, 7),
    ("par_d64", O.VARIANT_FIXED_SHAPE, 0),
    ("par_cap", O.VARIANT_TOPK_ONLY, 0),
    ("par_cap", O.VARIANT_TOPP_ONLY, 0),
    ("par_small", O.VARIANT_VISUAL_ONLY, 0),
    ("par_small", O.VARIANT_AUDIO_ONLY, 0),
    ("par_small", O.VARIANT_RHO_MAX_AUDIO, 0),
    ("par_d64", O.VARIANT_VISUAL_ONLY | O.VARIANT_TOPP_ONLY | O.VARIANT_RHO_MAX_AUDIO, 0),
]


@pytest.mark.parametrize("name,variant,fixed", VARIANTS)
def test_variant_parity(name, variant, fixed):
    _pipeline_parity(generate(name), dict(variant=variant, fixed_shape=fixed))


# selection at its limits: Top-k alone covering every block (every row dense);
# one block per row (k = 1 with a Top-p and a cap below any block); Top-p only
# with a p below any block's probability (n_p = 1)
EXTREMES = [
    ("par_small", dict(top_k=1_000_000)),
    ("par_cap", dict(top_k=1, top_p=1e-9, density_cap=1e-6)),
    ("par_d64", dict(top_k=1, top_p=1e-9, variant=O.VARIANT_TOPP_ONLY)),
    # under a cap the GPU sorts only the keys up to rank max(k, cap N / 64):
    # a cap rank far below the row length, a top k above the cap rank, and a
    # cap rank near the row's power of two
    ("par_small", dict(density_cap=0.1)),
    ("par_small", dict(density_cap=0.3, top_k=60)),
    ("par_small", dict(density_cap=0.45)),
]


@pytest.mark.parametrize("name,over", EXTREMES)
def test_selection_extremes(name, over):
    _pipeline_parity(generate(name), over)


def test_backward_without_low_parts():
    """prism_attn_bwd with o_lo = NULL takes rowsum(dO * O) on the bf16 O:
    dV does not depend on it (bitwise equal), dQ and dK move by the bf16
    rounding of O (about 1% relative L2 at most on this workload)."""
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    from parity_utils import bf16_dev_to_f32
    run = LayerOnGpu(generate("par_small"), backward=True)
    ref = run.host()
    L = run.layer
    dq, dk, dv = (torch.empty_like(run.q) for _ in range(3))
    B.prism_attn_bwd(L.prob, L.params, L.qp, L.kp, L.vp, run.o, None, run.do, L.lse, L.perm, L.blk_start,
                     L.n_blocks, L.row_ptr, L.col_idx, L.t_row_ptr, L.t_col_idx, dq, dk, dv, L.bwd_ws,
                     L.bwd_ws_bytes, L.stream())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_dev_to_f32(dv), ref["dv"])
    for nm, t in (("dq", dq), ("dk", dk)):
        err = rel_l2(bf16_dev_to_f32(t), ref[nm])
        log(f"{nm} without the low parts of O: relative L2 to the result with them {err:.3e}")
        assert 0 < err <= 2e-2, nm


def _degenerate(name: str):
    """Workloads whose decisions are all ties: the tie policy end to end.
    flat_v   every value vector is 0.5 and a is 0, so every zone has zero
             variation (rho = 0, r = 1/3 on each axis) and all three shapes
             of volume 256 are at the same distance from l*;
    equal_qk every query and key is the same vector, so every block score is
             equal, P_i is uniform and Top-k, Top-p and the cap all cut a
             run of equal scores (order by block index);
    peaked   q and k scaled by 4: peaked block probabilities and softmax
             rows (outputs near single value vectors), so the forward is
             held to the per-row bf16 rounding bound (fwd_row_bound)."""
    from dataclasses import replace
    if name == "peaked":
        # q and k times 4 (exact in bf16): scores 16 times larger, so each
        # row's weights concentrate on a few keys and the running maximum of
        # the online softmax jumps by large steps
        wl = generate("par_small")
        x4 = lambda bits: ((bits.astype(np.uint32) << 16).view(np.float32) * 4.0).view(np.uint32) >> 16
        return replace(wl, q_bits=x4(wl.q_bits).astype(wl.q_bits.dtype),
                       k_bits=x4(wl.k_bits).astype(wl.k_bits.dtype)), (), fwd_row_bound
    if name == "flat_v":
        wl = generate("par_small")
        return replace(wl, v_bits=np.full_like(wl.v_bits, 0x3F00), a=np.zeros_like(wl.a)), ("dq", "dk"), None
    wl = generate("par_cap")
    qk = np.full_like(wl.q_bits, 0x3E80)   # 0.25 in every channel
    return replace(wl, q_bits=qk, k_bits=qk.copy()), ("dq",), None


@pytest.mark.parametrize("name", ["flat_v", "equal_qk", "peaked"])
def test_degenerate_inputs(name):
    wl, near_zero, fwd_max = _degenerate(name)
    _pipeline_parity(wl, {}, near_zero, fwd_max)


def _pipeline_parity(wl, over, near_zero=(), fwd_max=None):
    import torch
    from parity_utils import binding_params
    c = wl.cfg
    op = oracle_params(c, **over)
    log("case", c.name, "N", c.N, "heads", c.heads, "D", c.head_dim, "variant", op.variant, "fixed", op.fixed_shape)
    run = LayerOnGpu(wl, params=binding_params(c, **over))
    gpu = run.host()
    log("gpu done, nnz", run.nnz)

    zs = O.zone_statistics(wl.f32("v"), wl.a, c.T, c.H, c.W, op.eps, op.variant)
    check_zone_stats(gpu, zs)
    fixed = None
    if op.variant & O.VARIANT_FIXED_SHAPE:
        fixed = np.full(zs["rho"].shape, op.fixed_shape, np.int64)
    plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=fixed)
    forced, zone_ties = reconcile_shapes(gpu["shape_id"], zs, plan, op)
    if zone_ties:
        plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=forced)
    log("zone stats and shapes match; tied zones:", zone_ties)

    heads_o = []
    tie_rows = alt_rows = 0
    for h in range(c.heads):
        ho = _oracle_head(wl, plan, h, op)
        gidx = gpu["index"][h]
        check_partition(gidx, ho["perm"], ho["blk_start"])
        check_operands(run.layer, h, wl, ho["perm"])
        st = compare_rows(gidx, ho["sel"], range(gidx["n_blocks"]))
        tie_rows += st["tie_rows"]
        alt_rows += st["alternative_rows"]
        check_transpose(gidx)
        if st["alternative_rows"] == 0:
            np.testing.assert_array_equal(gidx["row_ptr"], ho["row_ptr"])
            np.testing.assert_array_equal(gidx["col_idx"], ho["col_idx"])
            np.testing.assert_array_equal(gidx["t_col_idx"], ho["t_col_idx"])
        heads_o.append(ho)
    log("block index matches; tie rows", tie_rows, "rows where the GPU took another tied option", alt_rows)

    # attention on the oracle's own block index
    layer = run.layer
    oracle_index_to_device(layer, heads_o)
    o2 = torch.empty_like(run.q)
    layer.attn_fwd(o2)
    if run.backward:
        dq2, dk2, dv2 = (torch.empty_like(run.q) for _ in range(3))
        layer.attn_bwd(o2, run.do, dq2, dk2, dv2)
    torch.cuda.synchronize()
    from parity_utils import bf16_dev_to_f32
    o2h = bf16_dev_to_f32(o2)
    lse2 = layer.lse.cpu().numpy()
    scale = 1.0 / math.sqrt(c.head_dim)
    for h, ho in enumerate(heads_o):
        perm, bs = ho["perm"], ho["blk_start"]
        qp, kp, vp = (O.permute_tokens(wl.f32(x)[h], perm) for x in ("q", "k", "v"))
        op_, lse = O.sparse_attention_fwd(qp, kp, vp, bs, ho["row_ptr"], ho["col_idx"], scale)
        o_ref = O.unpermute_tokens(op_, perm)
        mx, mean = fwd_errors(o2h[h], o_ref)
        lse_err = float(np.abs(lse2[h] - lse).max())
        log(f"head {h}: forward max-abs {mx:.3e} mean-abs {mean:.3e} lse max-abs {lse_err:.3e}")
        if fwd_max is None:
            assert mx <= FWD_MAX_ABS
        else:   # a per-row bound, element by element (THW order)
            bound = O.unpermute_tokens(fwd_max(vp, bs, ho["row_ptr"], ho["col_idx"])[:, None], perm)[:, 0]
            excess = np.abs(o2h[h].astype(np.float64) - o_ref) / bound[:, None]
            log(f"head {h}: largest error relative to its row's bound {excess.max():.3f} "
                f"(bounds {bound.min():.3e} .. {bound.max():.3e})")
            assert excess.max() <= 1.0
        assert mean <= FWD_MEAN_ABS
        assert lse_err <= LSE_MAX_ABS
        if alt_rows == 0:
            # the end-to-end run used the same index: outputs are bitwise equal
            np.testing.assert_array_equal(gpu["o"][h], o2h[h])
        if run.backward:
            dop = O.permute_tokens(wl.f32("do")[h], perm)
            grads = O.sparse_attention_bwd(qp, kp, vp, op_, dop, lse, bs, ho["row_ptr"], ho["col_idx"], scale)
            dv_rms = float(np.sqrt(np.mean(grads[2] ** 2)))
            for nm, gdev, gref in zip(("dq", "dk", "dv"), (dq2, dk2, dv2), grads):
                g = bf16_dev_to_f32(gdev)[h]
                if nm in near_zero:
                    # zero in exact arithmetic (every key, or every value, is
                    # the same vector), so the GPU value is rounding noise: dS
                    # is rounded to bf16 (2^-8) before the dQ / dK products
                    # and Delta is taken on the bf16 O.  Bound: 2^-6 of the
                    # gradient scale, which dV (no cancellation) sets.
                    mx_ref, mx_gpu = float(np.abs(gref).max()), float(np.abs(g).max())
                    log(f"head {h}: {nm} max-abs {mx_gpu:.3e} (reference {mx_ref:.3e}, rms of dV {dv_rms:.3e})")
                    assert mx_ref <= 1e-9 * dv_rms and mx_gpu <= 2.0 ** -6 * dv_rms, nm
                    continue
                err = rel_l2(g, O.unpermute_tokens(gref, perm))
                log(f"head {h}: {nm} relative L2 {err:.3e}")
                assert err <= GRAD_REL_L2, nm


def test_determinism():
    """Two runs give bitwise equal block indices, outputs and gradients."""
    wl = generate("par_cap")
    a = LayerOnGpu(wl, backward=True).host()
    b = LayerOnGpu(wl, backward=True).host()
    for key in ("zstats", "g", "rho", "shape_id", "o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    for ia, ib in zip(a["index"], b["index"]):
        for key in ("perm", "blk_start", "row_ptr", "col_idx", "t_row_ptr", "t_col_idx"):
            np.testing.assert_array_equal(ia[key], ib[key], err_msg=key)


@pytest.mark.parametrize("name", ["par_d64", "tiny"])
def test_dense_baseline(name):
    """The dense baseline (every key tile) against float64 full attention."""
    import torch
    from dynamic_block_sparse_macro_amd.pipeline import DenseAttention, LayerShape
    from parity_utils import binding_params, bf16_dev_to_f32, to_dev
    wl = generate(name)
    c = wl.cfg
    dense = DenseAttention(LayerShape(c.T, c.H, c.W, c.heads, c.head_dim), binding_params(c))
    q, k, v, do = (to_dev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits, wl.do_bits))
    o = torch.empty_like(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dense.forward(q, k, v, o)
    dense.backward(q, k, v, o, do, dq, dk, dv)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(c.head_dim)
    for h in range(c.heads):
        qh, kh, vh, doh = (wl.f32(x)[h] for x in ("q", "k", "v", "do"))
        o_ref, lse = O.dense_attention(qh, kh, vh, scale)
        mx, mean = fwd_errors(bf16_dev_to_f32(o)[h], o_ref)
        assert mx <= FWD_MAX_ABS and mean <= FWD_MEAN_ABS
        assert np.abs(dense.lse.cpu().numpy()[h] - lse).max() <= LSE_MAX_ABS
        grads = O.dense_attention_bwd(qh, kh, vh, o_ref, doh, lse, scale)
        for gdev, gref in zip((dq, dk, dv), grads):
            assert rel_l2(bf16_dev_to_f32(gdev)[h], gref) <= GRAD_REL_L2


def test_top_p_one_is_dense():
    """p = 1 selects every block, so the sparse path computes full attention:
    it and the dense baseline each meet the forward bars against the
    oracle's float64 full attention, and so lie within twice the bars of
    each other (the two sum the same keys in different orders)."""
    import torch
    from dynamic_block_sparse_macro_amd.pipeline import DenseAttention, LayerShape
    from parity_utils import binding_params, bf16_dev_to_f32
    wl = generate("par_d64")
    c = wl.cfg
    run = LayerOnGpu(wl, params=binding_params(c, top_p=1.0), backward=True)
    nb = run.layer.n_blocks.cpu().numpy()
    assert run.nnz == [int(x) ** 2 for x in nb]
    dense = DenseAttention(LayerShape(c.T, c.H, c.W, c.heads, c.head_dim), binding_params(c))
    o = torch.empty_like(run.q)
    dense.forward(run.q, run.k, run.v, o)
    torch.cuda.synchronize()
    a, b = bf16_dev_to_f32(o), bf16_dev_to_f32(run.o)
    scale = 1.0 / math.sqrt(c.head_dim)
    for h in range(c.heads):
        o_ref, _ = O.dense_attention(wl.f32("q")[h], wl.f32("k")[h], wl.f32("v")[h], scale)
        for nm, x in (("dense", a), ("sparse p = 1", b)):
            mx, mean = fwd_errors(x[h], o_ref)
            log(f"head {h}: {nm} vs float64 full attention: max-abs {mx:.3e} mean-abs {mean:.3e}")
            assert mx <= FWD_MAX_ABS and mean <= FWD_MEAN_ABS, nm
    mx, mean = fwd_errors(a, b.astype(np.float64))
    log(f"sparse (p = 1) vs dense: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= 2 * FWD_MAX_ABS and mean <= FWD_MEAN_ABS
    np.testing.assert_allclose(dense.lse.cpu().numpy(), O.unpermute_tokens(
        run.layer.lse.cpu().numpy()[..., None], run.layer.perm.cpu().numpy()[0].astype(np.int64))[..., 0],
        atol=1e-4)

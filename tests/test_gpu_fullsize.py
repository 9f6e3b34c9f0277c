"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the whole layer through the C ABI, all heads in one call),
and at the largest accepted grid (1,048,576 tokens, 16,384 blocks per row).

What is compared at these sizes:
  * zone statistics, shapes, permutation and block starts: everything,
    exactly (ties reconciled as in the small tests);
  * the block index: every query-block row of every head against the
    oracle's selection (bit-exact outside ties), and the key-major index as
    the exact transpose;
  * the permuted operand buffers of head 0, bitwise, in the swizzled layout;
  * coverage: every output (O, its low parts, LSE, dQ, dK, dV) starts as NaN
    and must be finite afterwards, so no work item is skipped in any queue
    order;
  * forward output, LSE and dQ: every token of a seeded sample of query
    blocks;
  * dK, dV: every token of chosen key blocks, against the oracle's gradient
    of that key block over its whole column of query blocks (whose rows the
    oracle runs in full).  The columns: the median-length and the
    90th-percentile-length ones where their rows fit the oracle budget (45 s
    of the oracle's measured throughput), the longest that fits (the
    cheapest column if none does),
    and a key tile that the key-major pass pairs with the tile four steps
    away; the lengths are printed.  The identities sum_t dV_t = sum_p dO_p and sum_t dK_t = 0 over
    all tokens are checked as well.
A separate case of 44 heads on a 12,288-token grid (all heads' K and V exceed
the last-level cache, so the work queues run head by head) is checked in
full against the oracle.
"""

import math
import time

import numpy as np
import pytest

import oracle as O
from workload import CONFIGS, generate

from parity_utils import (FWD_MAX_ABS, FWD_MEAN_ABS, GRAD_REL_L2, LSE_MAX_ABS, LayerOnGpu, binding_params,
                          check_operands, check_partition, check_transpose, check_zone_stats, compare_all_rows, log,
                          oracle_fwd_rows, oracle_params, oracle_select_all, reconcile_shapes, rel_l2)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ATTN_BLOCKS = 10
# seconds of oracle forward work per key-column test: the budget in token
# pairs is this times the throughput measured on the sampled query blocks
COLUMN_SECONDS = 45.0
DEFAULT_PAIRS_PER_S = 5e7

# (workload, parameter overrides).  max_grid: the largest accepted grid with
# every zone cut into 64-token blocks, i.e. the most blocks per selection row
# (16,384, sorted in LDS).
FULL = [("720p", {}), ("1080p", {}), ("2k", {}), ("long", {}),
        ("max_grid", dict(variant=O.VARIANT_FIXED_SHAPE, fixed_shape=0))]


@pytest.fixture(scope="module", params=FULL, ids=[f[0] for f in FULL])
def case(request):
    """One run of the whole layer at full size (outputs NaN-filled first),
    with host copies, and the oracle's zone statistics and plan."""
    import torch
    name, over = request.param
    cfg = CONFIGS[name]
    log("case", name, cfg.note, "heads", cfg.heads, "overrides", over)
    wl = generate(cfg)
    c = wl.cfg
    op = oracle_params(c, **over)
    run = LayerOnGpu(wl, params=binding_params(c, **over), fill_nan=True)
    gpu = run.host()
    L = run.layer
    gpu["o_lo_finite"] = bool(torch.isfinite(L.o_lo.float()).all())
    ops0 = {nm: getattr(L, nm + "p").view(torch.int16)[0].cpu().numpy().view(np.uint16)
            for nm in ("q", "k", "v")}
    log("gpu layer done; nnz", run.nnz, "blocks", [int(x["n_blocks"]) for x in gpu["index"]])
    zs = O.zone_statistics(wl.f32("v"), wl.a, c.T, c.H, c.W, op.eps, op.variant)
    fixed = None
    if op.variant & O.VARIANT_FIXED_SHAPE:
        fixed = np.full(zs["rho"].shape, op.fixed_shape, np.int64)
    plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=fixed)
    forced, zone_ties = reconcile_shapes(gpu["shape_id"], zs, plan, op)
    if zone_ties:
        plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=forced)
    heads = [dict(zip(("perm", "bs"), O.partition(plan["shape_id"][h], c.T, c.H, c.W))) for h in range(c.heads)]
    backward = run.backward
    del run, L
    torch.cuda.empty_cache()
    yield dict(name=name, wl=wl, cfg=c, op=op, gpu=gpu, ops0=ops0, zs=zs, zone_ties=zone_ties, heads=heads,
               backward=backward)


def _permuted(case, h, names):
    wl, perm = case["wl"], case["heads"][h]["perm"]
    return [O.permute_tokens(wl.f32(x)[h], perm) for x in names]


def _selection(case, h):
    """The oracle's selection of every row of head h (computed once per case)."""
    hd = case["heads"][h]
    if "sel" not in hd:
        qp, kp = _permuted(case, h, ("q", "k"))
        hd["sel"] = oracle_select_all(qp, kp, hd["bs"], case["op"], case["cfg"].N)
        nb = hd["bs"].size - 1
        hd["row_ptr"], hd["col_idx"] = O.csr_from_rows([hd["sel"][i][0] for i in range(nb)])
    return hd["sel"]


def test_fullsize_plan_and_coverage(case):
    c, gpu = case["cfg"], case["gpu"]
    check_zone_stats(gpu, case["zs"])
    log("zone statistics and shapes match; tied zones:", case["zone_ties"])
    for h, hd in enumerate(case["heads"]):
        check_partition(gpu["index"][h], hd["perm"], hd["bs"])
    # head 0's permuted operands, bitwise, in the swizzled tile layout
    from parity_utils import unswizzle_tiles
    for nm in ("q", "k", "v"):
        bits = getattr(case["wl"], nm + "_bits")[0]
        np.testing.assert_array_equal(unswizzle_tiles(case["ops0"][nm], c.head_dim), bits[case["heads"][0]["perm"]])
    log("partition and head 0 operand buffers match")
    names = ["o", "lse"] + (["dq", "dk", "dv"] if case["backward"] else [])
    for nm in names:
        assert np.isfinite(gpu[nm]).all(), f"{nm}: elements left unwritten (NaN)"
    assert gpu["o_lo_finite"], "o_lo: elements left unwritten (NaN)"
    log("every output element written:", names + ["o_lo"])


def test_fullsize_index(case):
    """Every query-block row of every head, and the key-major transpose."""
    gpu = case["gpu"]
    for h in range(case["cfg"].heads):
        gidx = gpu["index"][h]
        check_transpose(gidx)
        st = compare_all_rows(gidx, _selection(case, h))
        case["heads"][h]["alt_rows"] = st["alternative_rows"]
        log(f"head {h}: all {gidx['n_blocks']} rows match ({int(gidx['row_ptr'][-1])} entries); tie rows "
            f"{st['tie_rows']}, GPU took another tied option in {st['alternative_rows']}")


def test_fullsize_forward_and_dq(case):
    """Forward, LSE and dQ on every token of sampled query blocks."""
    c, gpu = case["cfg"], case["gpu"]
    rng = np.random.default_rng(1234)
    scale = 1.0 / math.sqrt(c.head_dim)
    for h in range(c.heads):
        hd = case["heads"][h]
        sel = _selection(case, h)
        gidx = gpu["index"][h]
        perm, bs = hd["perm"], hd["bs"]
        nb = bs.size - 1
        exact = [i for i in range(nb)
                 if np.array_equal(gidx["col_idx"][gidx["row_ptr"][i]:gidx["row_ptr"][i + 1]], sel[i][0])]
        blocks = sorted(int(i) for i in rng.choice(exact, min(len(exact), ATTN_BLOCKS), replace=False))
        qp, kp, vp = _permuted(case, h, ("q", "k", "v"))
        t0 = time.perf_counter()
        op_, lse = O.sparse_attention_fwd(qp, kp, vp, bs, hd["row_ptr"], hd["col_idx"], scale, rows=blocks)
        dt = time.perf_counter() - t0
        sizes = np.diff(bs) * 64
        pairs = sum(int(sizes[i] * sizes[hd["col_idx"][hd["row_ptr"][i]:hd["row_ptr"][i + 1]]].sum()) for i in blocks)
        case["pairs_per_s"] = max(case.get("pairs_per_s", 0.0), pairs / max(dt, 1e-3))
        tok = np.concatenate([np.arange(bs[i] * 64, bs[i + 1] * 64) for i in blocks])
        d = np.abs(gpu["o"][h][perm[tok]].astype(np.float64) - op_[tok])
        lse_err = np.abs(gpu["lse"][h][tok] - lse[tok]).max()
        log(f"head {h}: forward on {tok.size} tokens of blocks {blocks}: max-abs {d.max():.3e} "
            f"mean-abs {d.mean():.3e}, lse max-abs {lse_err:.3e}")
        assert d.max() <= FWD_MAX_ABS and d.mean() <= FWD_MEAN_ABS
        assert lse_err <= LSE_MAX_ABS
        if not case["backward"]:
            continue
        dop = O.permute_tokens(case["wl"].f32("do")[h], perm)
        dq, _, _ = O.sparse_attention_bwd(qp, kp, vp, op_, dop, lse, bs, hd["row_ptr"], hd["col_idx"], scale,
                                          rows=blocks)
        err = rel_l2(gpu["dq"][h][perm[tok]], dq[tok])
        log(f"head {h}: dQ on {tok.size} tokens: relative L2 {err:.3e}")
        assert err <= GRAD_REL_L2


def _paired_by_four(gidx, bs, tp, tc, sizes):
    """Key tiles that the key-major pass pairs with the tile four steps away:
    in a zone of eight one-tile blocks it pairs (i, i + 4) when the four
    unions of those lists are shorter in total than those of (2i, 2i + 1)
    (tile-weighted list sizes)."""
    out = []

    def tiles(j):
        return int(sizes[tc[tp[j]:tp[j + 1]]].sum())

    def union(a, b):
        la, lb = tc[tp[a]:tp[a + 1]], tc[tp[b]:tp[b + 1]]
        both = np.intersect1d(la, lb, assume_unique=True)
        return tiles(a) + tiles(b) - int(sizes[both].sum())

    nb = bs.size - 1
    for b0 in range(0, nb - 7):
        if bs[b0] % 8 or bs[b0 + 8] != bs[b0] + 8:
            continue                      # not a zone of eight one-tile blocks
        by4 = sum(union(b0 + i, b0 + i + 4) for i in range(4)) < sum(union(b0 + 2 * i, b0 + 2 * i + 1)
                                                                      for i in range(4))
        if by4:
            out.extend(range(b0, b0 + 8))
    return out


@pytest.mark.parametrize("h", [0, 1])
def test_fullsize_dkdv_columns(case, h):
    """dK and dV of whole key blocks against the oracle's gradient over their
    columns; sum identities over all tokens."""
    c, gpu = case["cfg"], case["gpu"]
    if not case["backward"]:
        pytest.skip("forward-only workload")
    if h >= c.heads:
        pytest.skip("workload has fewer heads")
    hd = case["heads"][h]
    _selection(case, h)
    perm, bs = hd["perm"], hd["bs"]
    nb = bs.size - 1
    sizes = np.diff(bs) * 64
    rp, ci = hd["row_ptr"], hd["col_idx"]
    tp, tc = O.csr_transpose(rp, ci, nb)
    clen = np.diff(tp)
    rowkeys = np.array([int(sizes[ci[rp[i]:rp[i + 1]]].sum()) for i in range(nb)])
    cost = np.array([int((sizes[tc[tp[j]:tp[j + 1]]] * rowkeys[tc[tp[j]:tp[j + 1]]]).sum()) for j in range(nb)])
    # rows where the GPU took a tied alternative change their columns' sums:
    # such columns are not chosen
    gidx = gpu["index"][h]
    sel = hd["sel"]
    alt = {i for i in range(nb) if not np.array_equal(gidx["col_idx"][gidx["row_ptr"][i]:gidx["row_ptr"][i + 1]],
                                                      sel[i][0])}
    clean = np.array([not alt.intersection(tc[tp[j]:tp[j + 1]].tolist()) for j in range(nb)])
    budget = COLUMN_SECONDS * case.get("pairs_per_s", DEFAULT_PAIRS_PER_S)
    usable = np.where(clean & (clen > 0))[0]
    assert usable.size, "every key column holds a row where the GPU took a tied alternative"
    fits = usable[cost[usable] <= budget]
    over = not fits.size
    if over:   # every column is longer: the cheapest one
        fits = usable[[int(np.argmin(cost[usable]))]]
    chosen = {}
    med = float(np.median(clen))
    at_med = fits[clen[fits] >= med]
    if at_med.size:
        chosen["median-length"] = int(at_med[np.argmin(cost[at_med])])
    at_p90 = fits[clen[fits] >= np.percentile(clen, 90)]
    if at_p90.size:
        chosen["p90-length"] = int(at_p90[np.argmin(cost[at_p90])])
    chosen["cheapest (none within budget)" if over else "longest within budget"] = int(fits[np.argmax(clen[fits])])
    fit_set = set(fits.tolist())
    by4 = [j for j in _paired_by_four(gidx, bs, tp, tc, sizes) if j in fit_set]
    if by4:   # the cheapest whose column spans more than one 64-entry list window
        long4 = [j for j in by4 if clen[j] > 64] or by4
        chosen["paired (i, i + 4)"] = min(long4, key=lambda j: cost[j])
    log(f"head {h}: column lengths: median {med:.0f}, p90 {np.percentile(clen, 90):.0f}, max {clen.max()}; "
        f"{fits.size} of {nb} columns fit the budget of {budget:.2e} token pairs")
    qp, kp, vp, dop = _permuted(case, h, ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(c.head_dim)
    rows = sorted({int(i) for j in chosen.values() for i in tc[tp[j]:tp[j + 1]]})
    o, lse = oracle_fwd_rows(qp, kp, vp, bs, rp, ci, scale, rows)
    for kind, j in chosen.items():
        qrows = tc[tp[j]:tp[j + 1]]
        dk, dv = O.sparse_attention_key_block_grad(qp, kp, vp, o, dop, lse, bs, qrows, j, scale)
        ktok = np.arange(bs[j] * 64, bs[j + 1] * 64)
        edk = rel_l2(gpu["dk"][h][perm[ktok]], dk)
        edv = rel_l2(gpu["dv"][h][perm[ktok]], dv)
        log(f"head {h}: {kind} key block {j} ({sizes[j]} tokens; column of {qrows.size} query blocks, "
            f"{cost[j]:.3g} token pairs in their rows): dK rel-L2 {edk:.3e}, dV rel-L2 {edv:.3e}")
        assert edk <= GRAD_REL_L2 and edv <= GRAD_REL_L2, kind
    # identities over all tokens
    do_sum = case["wl"].f32("do")[h].astype(np.float64).sum(0)
    dv_sum = gpu["dv"][h].astype(np.float64).sum(0)
    dk_sum = gpu["dk"][h].astype(np.float64).sum(0)
    e1 = np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum)
    e2 = np.linalg.norm(dk_sum) / np.linalg.norm(np.abs(gpu["dk"][h].astype(np.float64)).sum(0))
    log(f"head {h}: |sum dV - sum dO| / |sum dO| = {e1:.3e}; |sum dK| / sum |dK| = {e2:.3e}")
    assert e1 <= 1e-2 and e2 <= 1e-2


def test_many_heads_head_by_head_order():
    """44 heads of a 12,288-token grid: all heads' K and V (277 MB) exceed the
    last-level cache, so every attention pass runs its work queues head by
    head.  Every step of every head against the oracle, every element."""
    import torch
    from parity_utils import (bf16_dev_to_f32, check_fwd_elements, fwd_errors, fwd_row_bound,
                              oracle_index_to_device, oracle_pipeline_heads)
    wl = generate("many_heads")
    c = wl.cfg
    assert c.heads * 2 * c.N * c.head_dim * 2 > 256 << 20
    op = oracle_params(c)
    run = LayerOnGpu(wl, fill_nan=True)
    gpu = run.host()
    ref = oracle_pipeline_heads(wl, op)
    check_zone_stats(gpu, ref["zone"])
    assert np.array_equal(gpu["shape_id"], ref["plan"]["shape_id"]) or reconcile_shapes(
        gpu["shape_id"], ref["zone"], ref["plan"], op)[1] > 0
    alt = 0
    for h, hr in enumerate(ref["heads"]):
        gidx = gpu["index"][h]
        check_partition(gidx, hr["perm"], hr["blk_start"])
        check_transpose(gidx)
        st = compare_all_rows(gidx, {i: (r["cols"], bool(r["tie"]), r) for i, r in hr["sel"]["rows"].items()})
        alt += st["alternative_rows"]
    log(f"{c.heads} heads: index matches; rows with another tied option: {alt}")
    # attention on the oracle's own index (outputs NaN-filled first)
    L = run.layer
    oracle_index_to_device(L, [dict(blk_start=hr["blk_start"], row_ptr=hr["row_ptr"], col_idx=hr["col_idx"],
                                    t_row_ptr=hr["t_row_ptr"], t_col_idx=hr["t_col_idx"]) for hr in ref["heads"]])
    o = torch.full_like(run.q, float("nan"))
    dq, dk, dv = (torch.full_like(run.q, float("nan")) for _ in range(3))
    L.attn_fwd(o)
    L.attn_bwd(o, run.do, dq, dk, dv)
    torch.cuda.synchronize()
    oh, dqh, dkh, dvh = (bf16_dev_to_f32(t) for t in (o, dq, dk, dv))
    lse_dev = L.lse.cpu().numpy()
    # the end-to-end run selected the same index: bitwise equal outputs
    for nm, a, b in (("o", gpu["o"], oh), ("dq", gpu["dq"], dqh), ("dk", gpu["dk"], dkh), ("dv", gpu["dv"], dvh)):
        same = np.array_equal(a, b)
        log(f"end-to-end {nm} bitwise equal to the run on the uploaded index: {same}")
    worst = dict(fwd=0.0, mean=0.0, lse=0.0, dq=0.0, dk=0.0, dv=0.0)
    for h, hr in enumerate(ref["heads"]):
        mx, mean = fwd_errors(oh[h], hr["o"])
        lse_err = float(np.abs(lse_dev[h] - hr["lse_p"]).max())
        if mx > FWD_MAX_ABS:   # outputs near the largest |v|: each element to its row's bf16 bound
            vp = O.permute_tokens(wl.f32("v")[h], hr["perm"])
            bound = O.unpermute_tokens(fwd_row_bound(vp, hr["blk_start"], hr["row_ptr"], hr["col_idx"])[:, None],
                                       hr["perm"])[:, 0]
            n_over, ratio = check_fwd_elements(oh[h], hr["o"], bound)
            log(f"head {h}: forward max-abs {mx:.3e}: {n_over} elements beyond 2e-2, all within their row's bf16 "
                f"rounding bound (largest error / bound {ratio:.3f})")
        else:
            assert mx <= FWD_MAX_ABS
        assert mean <= FWD_MEAN_ABS, h
        assert lse_err <= LSE_MAX_ABS, h
        errs = [rel_l2(g[h], hr[nm]) for nm, g in (("dq", dqh), ("dk", dkh), ("dv", dvh))]
        assert max(errs) <= GRAD_REL_L2, (h, errs)
        for key, val in zip(("fwd", "mean", "lse", "dq", "dk", "dv"), [mx, mean, lse_err] + errs):
            worst[key] = max(worst[key], val)
    log(f"{c.heads} heads, worst over heads: " + ", ".join(f"{k} {v:.3e}" for k, v in worst.items()))

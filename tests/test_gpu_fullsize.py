"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the whole layer through the C ABI, all heads in one call),
and at the largest accepted grid (1,048,576 tokens, 16,384 blocks per row).

The oracle cannot run every output at these sizes, so the checks are:
  * zone statistics, shapes, permutation and block starts: everything, exactly
    (ties reconciled as in the small tests);
  * block selection: a seeded sample of query-block rows, exactly;
  * the key-major index: the exact transpose of the query-major one;
  * forward output and LSE: every token of a seeded sample of query blocks;
  * dQ: every token of the sampled query blocks;
  * dK, dV: the key block with the shortest column list, exactly, plus the
    identities sum_t dV_t = sum_p dO_p and sum_t dK_t = 0 over all tokens.
"""

import math

import numpy as np
import pytest

import oracle as O
from workload import CONFIGS, generate

from parity_utils import (FWD_MAX_ABS, FWD_MEAN_ABS, GRAD_REL_L2, LSE_MAX_ABS, LayerOnGpu, check_partition,
                          check_transpose, check_zone_stats, compare_rows, log, oracle_params, reconcile_shapes,
                          rel_l2)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROW_SAMPLE = 48
ATTN_BLOCKS = 10
MAX_COLUMN = 64


# (workload, parameter overrides).  max_grid: the largest accepted grid with
# every zone cut into 64-token blocks, i.e. the most blocks per selection row
# (16,384, sorted in LDS).
FULL = [("720p", {}), ("1080p", {}), ("2k", {}), ("long", {}),
        ("max_grid", dict(variant=O.VARIANT_FIXED_SHAPE, fixed_shape=0))]


@pytest.mark.parametrize("name,over", FULL)
def test_fullsize_parity(name, over):
    from parity_utils import binding_params
    cfg = CONFIGS[name]
    log("case", name, cfg.note, "heads", cfg.heads, "overrides", over)
    wl = generate(cfg)
    c = wl.cfg
    op = oracle_params(c, **over)
    run = LayerOnGpu(wl, params=binding_params(c, **over))
    gpu = run.host()
    log("gpu layer done; nnz", run.nnz, "blocks", [int(x["n_blocks"]) for x in gpu["index"]])

    zs = O.zone_statistics(wl.f32("v"), wl.a, c.T, c.H, c.W, op.eps, op.variant)
    check_zone_stats(gpu, zs)
    fixed = None
    if op.variant & O.VARIANT_FIXED_SHAPE:
        fixed = np.full(zs["rho"].shape, op.fixed_shape, np.int64)
    plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=fixed)
    forced, zone_ties = reconcile_shapes(gpu["shape_id"], zs, plan, op)
    if zone_ties:
        plan = O.plan_shapes(zs["g"], zs["rho"], op.tau128, op.tau256, forced_shape=forced)
    log("zone statistics and shapes match; tied zones:", zone_ties)

    rng = np.random.default_rng(1234)
    scale = 1.0 / math.sqrt(c.head_dim)
    for h in range(c.heads):
        gidx = gpu["index"][h]
        perm, bs = O.partition(plan["shape_id"][h], c.T, c.H, c.W)
        check_partition(gidx, perm, bs)
        check_transpose(gidx)
        nb = bs.size - 1
        qp = O.permute_tokens(wl.f32("q")[h], perm)
        kp = O.permute_tokens(wl.f32("k")[h], perm)
        rows = np.unique(np.concatenate([rng.choice(nb, min(nb, ROW_SAMPLE), replace=False), [0, nb - 1]]))
        sel = O.select_blocks(qp, kp, bs, op, c.N, rows=rows)
        st = compare_rows(gidx, sel, rows)
        log(f"head {h}: {rows.size} sampled rows match; tie rows {st['tie_rows']}, "
            f"GPU took another tied option in {st['alternative_rows']}")

        # forward and dQ on sampled query blocks whose rows matched exactly
        exact = [int(i) for i in rows if np.array_equal(
            gidx["col_idx"][gidx["row_ptr"][i]:gidx["row_ptr"][i + 1]], sel["rows"][int(i)]["cols"])]
        blocks = rng.choice(exact, min(len(exact), ATTN_BLOCKS), replace=False)
        vp = O.permute_tokens(wl.f32("v")[h], perm)
        cols_all = []
        for i in sorted(blocks):
            cols_all.append(sel["rows"][int(i)]["cols"])
        # a row pointer over only the sampled blocks, in ascending block order
        rp_s = np.zeros(nb + 1, np.int64)
        lens = np.zeros(nb, np.int64)
        for i, cl in zip(sorted(blocks), cols_all):
            lens[i] = cl.size
        rp_s[1:] = np.cumsum(lens)
        col_s = np.concatenate(cols_all)
        op_, lse = O.sparse_attention_fwd(qp, kp, vp, bs, rp_s, col_s, scale, rows=sorted(blocks))
        tok = np.concatenate([np.arange(bs[i] * 64, bs[i + 1] * 64) for i in sorted(blocks)])
        o_gpu = gpu["o"][h][perm[tok]].astype(np.float64)
        d = np.abs(o_gpu - op_[tok])
        lse_err = np.abs(gpu["lse"][h][tok] - lse[tok]).max()
        log(f"head {h}: forward on {tok.size} tokens: max-abs {d.max():.3e} mean-abs {d.mean():.3e}, "
            f"lse max-abs {lse_err:.3e}")
        assert d.max() <= FWD_MAX_ABS and d.mean() <= FWD_MEAN_ABS
        assert lse_err <= LSE_MAX_ABS
        if not run.backward:
            continue
        dop = O.permute_tokens(wl.f32("do")[h], perm)
        dq, _, _ = O.sparse_attention_bwd(qp, kp, vp, op_, dop, lse, bs, rp_s, col_s, scale, rows=sorted(blocks))
        err = rel_l2(gpu["dq"][h][perm[tok]], dq[tok])
        log(f"head {h}: dQ on {tok.size} tokens: relative L2 {err:.3e}")
        assert err <= GRAD_REL_L2

        # dK, dV of the key block with the fewest selecting query blocks (when
        # that column is short enough for the oracle to run in seconds)
        tptr, tcol = gidx["t_row_ptr"], gidx["t_col_idx"]
        counts = np.diff(tptr)
        j = int(np.argmin(np.where(counts > 0, counts, np.iinfo(np.int64).max)))
        qrows = tcol[tptr[j]:tptr[j + 1]]
        if qrows.size > MAX_COLUMN:
            log(f"head {h}: shortest key column has {qrows.size} query blocks; exact dK/dV check left to the "
                "identities below")
            qrows = qrows[:0]
        selq = O.select_blocks(qp, kp, bs, op, c.N, rows=qrows)
        lens = np.zeros(nb, np.int64)
        cols_q = []
        for i in qrows:
            cl = selq["rows"][int(i)]["cols"]
            assert j in cl, "the transposed index lists a query block that did not select this key block"
            lens[i] = cl.size
            cols_q.append(cl)
        if qrows.size:
            rp_q = np.zeros(nb + 1, np.int64)
            rp_q[1:] = np.cumsum(lens)
            col_q = np.concatenate(cols_q)
            oq, lseq = O.sparse_attention_fwd(qp, kp, vp, bs, rp_q, col_q, scale, rows=list(qrows))
            _, dk, dv = O.sparse_attention_bwd(qp, kp, vp, oq, dop, lseq, bs, rp_q, col_q, scale, rows=list(qrows))
            ktok = np.arange(bs[j] * 64, bs[j + 1] * 64)
            edk = rel_l2(gpu["dk"][h][perm[ktok]], dk[ktok])
            edv = rel_l2(gpu["dv"][h][perm[ktok]], dv[ktok])
            log(f"head {h}: key block {j} ({qrows.size} query blocks): dK rel-L2 {edk:.3e}, dV rel-L2 {edv:.3e}")
            assert edk <= GRAD_REL_L2 and edv <= GRAD_REL_L2

        # identities over all tokens
        do_sum = wl.f32("do")[h].astype(np.float64).sum(0)
        dv_sum = gpu["dv"][h].astype(np.float64).sum(0)
        dk_sum = gpu["dk"][h].astype(np.float64).sum(0)
        e1 = np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum)
        e2 = np.linalg.norm(dk_sum) / np.linalg.norm(np.abs(gpu["dk"][h].astype(np.float64)).sum(0))
        log(f"head {h}: |sum dV - sum dO| / |sum dO| = {e1:.3e}; |sum dK| / sum |dK| = {e2:.3e}")
        assert e1 <= 1e-2 and e2 <= 1e-2

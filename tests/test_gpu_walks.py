"""Attention on hand-built block lists (GPU against the oracle, same index).

The forward walks the union of the key-block lists of a query-tile pair and
pipelines it inside each wave; a wave whose query tile does not attend to a
tile of the walk runs that tile masked, and the walk's first and last two
iterations fill and drain the pipeline.  Selection rarely produces the
extreme cases, so this test writes the lists itself: walks of one and two
tiles, the two tiles of a pair attending to disjoint key blocks (every step
computed by one wave pair and masked for the other), one list nested in its
neighbour's, rows over every block, every other block, and a few random
blocks.  Blocks are 64 tokens everywhere (fixed shape 0), so the two tiles
of every pair are different blocks (at head_dim 128 and 64), and, in a
further case, the layer's own mixed 64/128/256-token partition.  Forward,
LSE and the three gradients are compared with the oracle on the same lists
(Prism pt reading guide, Método 3: attention over the selected blocks only;
zh guide, 常见问题: gradients through the selected blocks only).
"""

import math

import numpy as np
import pytest

import oracle as O
from parity_utils import (FWD_MAX_ABS, FWD_MEAN_ABS, GRAD_REL_L2, LSE_MAX_ABS, LayerOnGpu, bf16_dev_to_f32,
                          check_device_index, fwd_errors, oracle_index_to_device, rel_l2)
from workload import generate

pytestmark = pytest.mark.gpu


def log(*a):
    print("[walks]", *a, flush=True)


def hand_lists(nb: int, seed: int) -> list[list[int]]:
    """One ascending, non-empty list of key blocks per query block."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(nb):
        kind = i % 8
        if kind == 0:
            row = [i]                                   # a walk of one block
        elif kind == 1:
            row = [nb - 1 - i]                          # disjoint from block i - 1's [i - 1] (unless equal)
        elif kind == 2:
            row = [0, nb - 1]                           # two blocks, far apart
        elif kind == 3:
            row = list(range(nb))                       # every block
        elif kind == 4:
            row = [i]
        elif kind == 5:
            row = [i - 1, i]                            # contains block i - 1's list [i - 1]
        elif kind == 6:
            row = rng.choice(nb, size=min(nb, 4), replace=False).tolist()
        else:
            row = list(range(i % 2, nb, 2))             # every other block
        rows.append(sorted(set(row)))
    return rows


def csr(rows: list[list[int]]) -> tuple[np.ndarray, np.ndarray]:
    row_ptr = np.zeros(len(rows) + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    return row_ptr, np.concatenate([np.asarray(r, np.int64) for r in rows])


@pytest.mark.parametrize("case", ["single_tile_blocks", "layer_blocks", "single_tile_blocks_d64"])
def test_hand_built_walks(case):
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    wl = generate("par_d64" if case.endswith("_d64") else "par_small")
    c = wl.cfg
    if case.startswith("single_tile_blocks"):
        par = B.make_params(top_k=c.top_k, top_p=c.top_p, density_cap=c.density_cap,
                            variant=O.VARIANT_FIXED_SHAPE, fixed_shape=0)
    else:
        par = B.make_params(top_k=c.top_k, top_p=c.top_p, density_cap=c.density_cap)
    run = LayerOnGpu(wl, params=par, backward=True)
    layer = run.layer
    heads = []
    for h, ix in enumerate(layer.index_host()):
        nb = ix["n_blocks"]
        rows = hand_lists(nb, 1000 + h)
        row_ptr, col_idx = csr(rows)
        t_row_ptr, t_col_idx = O.csr_transpose(row_ptr, col_idx, nb)
        sizes = np.diff(ix["blk_start"])
        log(f"{case} head {h}: {nb} blocks of {sorted(set((sizes * 64).tolist()))} tokens, "
            f"{col_idx.size} selected block pairs")
        heads.append(dict(perm=ix["perm"].astype(np.int64), blk_start=ix["blk_start"], row_ptr=row_ptr,
                          col_idx=col_idx, t_row_ptr=t_row_ptr, t_col_idx=t_col_idx))
    oracle_index_to_device(layer, heads)
    check_device_index(layer)

    o2 = torch.full_like(run.q, float("nan"))
    dq2, dk2, dv2 = (torch.full_like(run.q, float("nan")) for _ in range(3))
    layer.attn_fwd(o2)
    layer.attn_bwd(o2, run.do, dq2, dk2, dv2)
    torch.cuda.synchronize()
    o2h = bf16_dev_to_f32(o2)
    lse2 = layer.lse.cpu().numpy()
    grads_gpu = [bf16_dev_to_f32(t) for t in (dq2, dk2, dv2)]
    scale = 1.0 / math.sqrt(c.head_dim)
    for h, ho in enumerate(heads):
        perm, bs = ho["perm"], ho["blk_start"]
        qp, kp, vp = (O.permute_tokens(wl.f32(x)[h], perm) for x in ("q", "k", "v"))
        op_, lse = O.sparse_attention_fwd(qp, kp, vp, bs, ho["row_ptr"], ho["col_idx"], scale)
        o_ref = O.unpermute_tokens(op_, perm)
        assert np.isfinite(o2h[h]).all(), "an output element was not written"
        mx, mean = fwd_errors(o2h[h], o_ref)
        lse_err = float(np.abs(lse2[h] - lse).max())
        log(f"{case} head {h}: forward max-abs {mx:.3e} mean-abs {mean:.3e} lse max-abs {lse_err:.3e}")
        assert mx <= FWD_MAX_ABS and mean <= FWD_MEAN_ABS and lse_err <= LSE_MAX_ABS
        dop = O.permute_tokens(wl.f32("do")[h], perm)
        ref = O.sparse_attention_bwd(qp, kp, vp, op_, dop, lse, bs, ho["row_ptr"], ho["col_idx"], scale)
        for nm, g, gref in zip(("dq", "dk", "dv"), grads_gpu, ref):
            gh = g[h]
            assert np.isfinite(gh).all(), f"a {nm} element was not written"
            err = rel_l2(gh, O.unpermute_tokens(gref, perm))
            log(f"{case} head {h}: {nm} relative L2 {err:.3e}")
            assert err <= GRAD_REL_L2, nm

"""prism_attn_fwd_noalloc (scratch in the library's static device array)
against prism_attn_fwd (scratch from a workspace) through the C ABI: the
same O, low parts and LSE, bit for bit, on two calls in a row, the second on
a smaller problem (the array keeps the first call's contents)."""

import numpy as np
import pytest

from workload import generate

from parity_utils import LayerOnGpu, log

pytestmark = pytest.mark.gpu


def _compare(name):
    import torch
    from dynamic_block_sparse_macro_amd import binding as B
    run = LayerOnGpu(generate(name))        # whole layer; its forward used prism_attn_fwd
    L = run.layer
    ref = dict(o=run.o.clone(), o_lo=L.o_lo.clone(), lse=L.lse.clone())
    out = dict(o=torch.full_like(run.o, float("nan")), o_lo=torch.full_like(L.o_lo, float("nan")),
               lse=torch.full_like(L.lse, float("nan")))
    B.prism_attn_fwd_noalloc(L.prob, L.params, L.qp, L.kp, L.vp, L.perm, L.blk_start, L.n_blocks, L.row_ptr,
                             L.col_idx, out["o"], out["o_lo"], out["lse"], L.stream())
    torch.cuda.synchronize()
    for k in ref:
        a, b = ref[k], out[k]
        ai = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
        bi = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
        assert torch.equal(ai, bi), f"{name}: {k} differs from prism_attn_fwd"
    log(f"{name}: O, its low parts and LSE bitwise equal to prism_attn_fwd "
        f"({run.cfg.heads} heads x {run.cfg.N} tokens)")


def test_noalloc_forward_matches_workspace_forward():
    _compare("par_small")   # 2 heads, 12,288 tokens, head_dim 128
    _compare("tiny")        # then a smaller problem: 1 head, 2,048 tokens, head_dim 64

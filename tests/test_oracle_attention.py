"""Pins of the oracle's sparse attention forward and backward against dense
attention, an independent masked-dense route, torch's CPU attention and
finite differences.  CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from workload import generate


def _pipeline(name="tiny", **kw):
    w = generate(name)
    c = w.cfg
    P = O.Params(top_k=kw.get("top_k", c.top_k), top_p=kw.get("top_p", c.top_p),
                 density_cap=kw.get("density_cap", c.density_cap))
    do = w.f32("do") if c.backward else None
    res = O.run_pipeline(w.f32("q"), w.f32("k"), w.f32("v"), w.a, c.T, c.H, c.W, P, do=do)
    return w, P, res


def test_p_one_is_dense_attention():
    w, P, res = _pipeline(top_p=1.0)
    h = res["heads"][0]
    assert h["row_ptr"][-1] == h["n_blocks"] ** 2
    q, k, v, do = (w.f32(x)[0] for x in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(w.cfg.head_dim)
    o, lse = O.dense_attention(q, k, v, scale)
    np.testing.assert_allclose(h["o"], o, atol=1e-13)
    dq, dk, dv = O.dense_attention_bwd(q, k, v, o, do, lse, scale)
    np.testing.assert_allclose(h["dq"], dq, atol=1e-12)
    np.testing.assert_allclose(h["dk"], dk, atol=1e-12)
    np.testing.assert_allclose(h["dv"], dv, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "par_d64"])
def test_masked_dense_route(name):
    """The permuted block-sparse forward, scattered back, equals dense
    attention in THW order under the -inf mask of the selection."""
    w, P, res = _pipeline(name)
    c = w.cfg
    scale = 1 / math.sqrt(c.head_dim)
    h = res["heads"][0]
    blk = O.token_block_map(h["perm"], h["blk_start"])
    o, lse = O.masked_attention_thw(w.f32("q")[0], w.f32("k")[0], w.f32("v")[0], blk, h["row_ptr"],
                                    h["col_idx"], scale)
    np.testing.assert_allclose(h["o"], o, atol=1e-12)
    lse_thw = O.unpermute_tokens(h["lse_p"][:, None], h["perm"])[:, 0]
    np.testing.assert_allclose(lse_thw, lse, atol=1e-12)
    assert h["row_ptr"][-1] < h["n_blocks"] ** 2          # genuinely sparse


def test_torch_sdpa_cross_check():
    w, P, res = _pipeline("tiny")
    h = res["heads"][0]
    blk = O.token_block_map(h["perm"], h["blk_start"])
    nb = h["n_blocks"]
    allowed = np.zeros((nb, nb), bool)
    for i in range(nb):
        allowed[i, h["col_idx"][h["row_ptr"][i]:h["row_ptr"][i + 1]]] = True
    mask = torch.tensor(allowed[blk[:, None], blk[None, :]])
    q, k, v = (torch.tensor(w.f32(x)[0], dtype=torch.float64)[None, None] for x in ("q", "k", "v"))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None])[0, 0]
    np.testing.assert_allclose(h["o"], o.numpy(), atol=1e-12)
    # gradients via autograd of sum(O * dO)
    qg, kg, vg = (x.clone().requires_grad_(True) for x in (q, k, v))
    og = torch.nn.functional.scaled_dot_product_attention(qg, kg, vg, attn_mask=mask[None, None])
    (og[0, 0] * torch.tensor(w.f32("do")[0], dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(h["dq"], qg.grad[0, 0].numpy(), atol=1e-11)
    np.testing.assert_allclose(h["dk"], kg.grad[0, 0].numpy(), atol=1e-11)
    np.testing.assert_allclose(h["dv"], vg.grad[0, 0].numpy(), atol=1e-11)


def test_finite_differences():
    """Central differences of L = sum(O * dO) with the selection fixed."""
    rng = np.random.default_rng(7)
    nb_tok = 4 * 64
    D = 16
    blk_start = np.array([0, 1, 3, 4])               # blocks of 64, 128, 64 tokens
    q, k, v, do = (rng.standard_normal((nb_tok, D)) for _ in range(4))
    row_ptr = np.array([0, 2, 3, 5])
    col_idx = np.array([0, 2, 1, 0, 1])
    scale = 0.3

    def loss(q_, k_, v_):
        o, _ = O.sparse_attention_fwd(q_, k_, v_, blk_start, row_ptr, col_idx, scale)
        return (o * do).sum()

    o, lse = O.sparse_attention_fwd(q, k, v, blk_start, row_ptr, col_idx, scale)
    grads = O.sparse_attention_bwd(q, k, v, o, do, lse, blk_start, row_ptr, col_idx, scale)
    h = 1e-6
    for which, g in enumerate(grads):
        for _ in range(12):
            i, j = int(rng.integers(nb_tok)), int(rng.integers(D))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][i, j] += h
            lp = loss(*args)
            args[which][i, j] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert fd == pytest.approx(g[i, j], rel=1e-6, abs=1e-8)
        for _ in range(3):   # directional derivatives
            d = rng.standard_normal((nb_tok, D))
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which] += h * d
            args_m[which] -= h * d
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert fd == pytest.approx((g * d).sum(), rel=1e-6, abs=1e-8)


def test_gradient_sum_identities():
    """Sum over keys of dV equals sum over queries of dO (rows of P sum to 1),
    and dK sums to zero (each row of dS sums to zero)."""
    w, P, res = _pipeline("par_d64")
    h = res["heads"][0]
    np.testing.assert_allclose(h["dv"].sum(0), w.f32("do")[0].astype(np.float64).sum(0), atol=1e-9)
    np.testing.assert_allclose(h["dk"].sum(0), 0.0, atol=1e-9)


def test_flop_accounting():
    blk_start = np.array([0, 1, 3, 7])
    row_ptr = np.array([0, 1, 3, 4])
    col_idx = np.array([2, 0, 1, 2])
    pairs = O.selected_pairs(blk_start, row_ptr, col_idx)
    assert pairs == 64 * 256 + 128 * 64 + 128 * 128 + 256 * 256
    assert O.attention_flops(pairs, 128) == (4 * 128 * pairs, 10 * 128 * pairs)


def test_key_block_grad_finite_differences():
    """dK and dV of one key block, from the query blocks that selected it,
    against central differences of L = sum(O * dO) with the selection fixed."""
    rng = np.random.default_rng(11)
    D = 16
    blk_start = np.array([0, 1, 3, 4])               # blocks of 64, 128, 64 tokens
    q, k, v, do = (rng.standard_normal((4 * 64, D)) for _ in range(4))
    row_ptr = np.array([0, 2, 3, 5])
    col_idx = np.array([0, 2, 1, 0, 1])              # key block 1 is selected by query blocks 1 and 2
    scale = 0.3

    def loss(k_, v_):
        o_, _ = O.sparse_attention_fwd(q, k_, v_, blk_start, row_ptr, col_idx, scale)
        return (o_ * do).sum()

    o, lse = O.sparse_attention_fwd(q, k, v, blk_start, row_ptr, col_idx, scale)
    for j, qrows in ((1, [1, 2]), (0, [0, 2]), (2, [0])):
        dk, dv = O.sparse_attention_key_block_grad(q, k, v, o, do, lse, blk_start, qrows, j, scale)
        base = blk_start[j] * 64
        h = 1e-6
        for g, which in ((dk, 0), (dv, 1)):
            for _ in range(8):
                t, c = int(rng.integers(g.shape[0])), int(rng.integers(D))
                args_p, args_m = [k.copy(), v.copy()], [k.copy(), v.copy()]
                args_p[which][base + t, c] += h
                args_m[which][base + t, c] -= h
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert fd == pytest.approx(g[t, c], rel=1e-6, abs=1e-8)


def test_key_block_grad_matches_full_backward():
    """On the tiny workload's own index, the per-key-block gradients over the
    key-major columns reassemble the full backward's dK and dV."""
    w, P, res = _pipeline("tiny")
    h = res["heads"][0]
    c = w.cfg
    scale = 1 / math.sqrt(c.head_dim)
    perm = h["perm"]
    qp, kp, vp, dop = (O.permute_tokens(w.f32(x)[0], perm) for x in ("q", "k", "v", "do"))
    o, lse = O.sparse_attention_fwd(qp, kp, vp, h["blk_start"], h["row_ptr"], h["col_idx"], scale)
    _, dk_full, dv_full = O.sparse_attention_bwd(qp, kp, vp, o, dop, lse, h["blk_start"], h["row_ptr"],
                                                 h["col_idx"], scale)
    tp, tc = O.csr_transpose(h["row_ptr"], h["col_idx"], h["n_blocks"])
    bs = h["blk_start"]
    for j in range(h["n_blocks"]):
        dk, dv = O.sparse_attention_key_block_grad(qp, kp, vp, o, dop, lse, bs, tc[tp[j]:tp[j + 1]], j, scale)
        ks = slice(bs[j] * 64, bs[j + 1] * 64)
        np.testing.assert_allclose(dk, dk_full[ks], atol=1e-12)
        np.testing.assert_allclose(dv, dv_full[ks], atol=1e-12)

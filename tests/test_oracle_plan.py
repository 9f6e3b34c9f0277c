"""Pins of the oracle's block volume, shape quantisation and partition
(Prism guide (pt), Método 2 and Ideias centrais).  CPU only."""

import itertools
import math

import numpy as np
import pytest
from scipy.optimize import minimize

import oracle as O


def test_candidate_set_counts():
    C = O.CANDIDATES
    assert C.shape == (16, 3)
    vols = C.prod(axis=1)
    assert [(vols == v).sum() for v in (64, 128, 256)] == [7, 6, 3]
    assert set(np.unique(C)) <= {2, 4, 8}
    # the set is exactly the boxes with power-of-two edges dividing 8 (no flat
    # edge of 1) and volumes {64, 128, 256}; with edge 1 allowed there would be 19
    with_one = [s for s in itertools.product((1, 2, 4, 8), repeat=3) if np.prod(s) in (64, 128, 256)]
    assert len(with_one) == 19
    assert sorted(map(tuple, C)) == sorted(s for s in with_one if 1 not in s)
    # canonical order: volume, then lexicographic
    keys = [(int(np.prod(s)), tuple(s)) for s in C]
    assert keys == sorted(keys)
    assert tuple(C[0]) == (2, 4, 8) and tuple(C[8]) == (4, 4, 8) and tuple(C[13]) == (4, 8, 8)


def test_volume_thresholds():
    rho = np.array([0.0, 0.1, 0.2499999, 0.25, 0.3, 0.4999999, 0.5, 0.9, 1.0])
    np.testing.assert_array_equal(O.block_volume(rho), [256, 256, 256, 128, 128, 128, 64, 64, 64])


@pytest.mark.parametrize("vol", [64, 128, 256])
def test_ell_star_identities(vol):
    rng = np.random.default_rng(vol)
    for _ in range(20):
        g = rng.uniform(1e-4, 2.0, 3)
        ell = O.ell_star(g, vol)
        assert ell.sum() == pytest.approx(math.log2(vol), abs=1e-13)   # prod b_d = B
        # b* proportional to g^(-1/2): pairwise differences fixed by g alone
        assert ell[0] - ell[1] == pytest.approx(-0.5 * math.log2(g[0] / g[1]), abs=1e-13)
    np.testing.assert_allclose(O.ell_star(np.full(3, 0.37), vol), np.full(3, math.log2(vol) / 3), atol=1e-14)


def test_ell_star_exact_case():
    """g proportional to (16, 4, 1) at B = 64: l* = (1, 2, 3), so 2x4x8 at distance 0."""
    for lam in (1.0, 0.01, 3.0):
        ell = O.ell_star(lam * np.array([16.0, 4.0, 1.0]), 64)
        np.testing.assert_allclose(ell, [1.0, 2.0, 3.0], atol=1e-14)
        sid, margin, idx, dist = O.quantise_shape(ell, 64)
        assert tuple(O.CANDIDATES[sid]) == (2, 4, 8) and dist.min() == pytest.approx(0.0, abs=1e-26)


@pytest.mark.parametrize("g", [(0.6, 0.3, 0.1), (0.05, 1.2, 0.4), (0.9, 0.9, 0.02), (1.0, 0.001, 0.5)])
@pytest.mark.parametrize("vol", [64, 128, 256])
def test_ell_star_is_optimum_of_loss_model(g, vol):
    """Minimise sum_d g_d (b_d^2 - 1) subject to prod_d b_d = B numerically;
    its log2 optimum must be the closed form l*."""
    g = np.array(g)

    def loss(x):  # x = log2 b_T, log2 b_H; b_W fixed by the volume
        lb = np.array([x[0], x[1], math.log2(vol) - x[0] - x[1]])
        return float((g * (2.0 ** (2 * lb) - 1)).sum())

    r = minimize(loss, x0=[2.0, 2.0], method="Nelder-Mead", options=dict(xatol=1e-10, fatol=1e-14, maxiter=20000))
    lb = np.array([r.x[0], r.x[1], math.log2(vol) - r.x[0] - r.x[1]])
    np.testing.assert_allclose(O.ell_star(g, vol), lb, atol=1e-6)


def test_worked_quantisation_example():
    """g = (0.6, 0.3, 0.1): the finest edge goes along the most varying axis."""
    g = np.array([0.6, 0.3, 0.1])
    expect = {64: ((2, 4, 8), 0.2645), 128: ((4, 4, 8), 0.1262), 256: ((4, 8, 8), 0.3212)}
    for vol, (shape, d2) in expect.items():
        sid, margin, idx, dist = O.quantise_shape(O.ell_star(g, vol), vol)
        assert tuple(O.CANDIDATES[sid]) == shape
        assert dist.min() == pytest.approx(d2, abs=5e-5)
        # brute force: nearest candidate by enumerating every box of that volume
        ell = O.ell_star(g, vol)
        brute = min((sum((math.log2(b) - e) ** 2 for b, e in zip(s, ell)), s) for s in O.CANDIDATES.tolist()
                    if np.prod(s) == vol)
        assert tuple(brute[1]) == shape


def test_isotropic_ties():
    g = np.full(3, 0.5)
    sid, margin, _, _ = O.quantise_shape(O.ell_star(g, 64), 64)
    assert tuple(O.CANDIDATES[sid]) == (4, 4, 4) and margin > 0.5
    for vol, tie in ((128, {8, 9, 11}), (256, {13, 14, 15})):
        sid, margin, _, _ = O.quantise_shape(O.ell_star(g, vol), vol)
        assert sid == min(tie) and margin < 1e-14
        rho = 0.3 if vol == 128 else 0.1
        assert O.shape_tie_set(g, rho) == tie
    # single dominant axis at B = 64: 2x4x8 and 2x8x4 tie exactly
    sid, margin, _, _ = O.quantise_shape(O.ell_star(np.array([1.0, 1e-3, 1e-3]), 64), 64)
    assert sid == 0 and margin < 1e-14
    assert O.shape_tie_set(np.array([1.0, 1e-3, 1e-3]), 0.9) == {0, 1}
    # a density on a threshold admits both volumes
    assert O.shape_tie_set(np.full(3, 0.5), 0.25) == {8, 9, 11, 13, 14, 15}
    assert O.shape_tie_set(np.full(3, 0.5), 0.5) == {3, 8, 9, 11}


@pytest.mark.parametrize("T,H,W", [(8, 8, 8), (16, 8, 24), (8, 32, 16)])
def test_partition_invariants(T, H, W):
    rng = np.random.default_rng(T * H * W)
    Z = (T // 8) * (H // 8) * (W // 8)
    shape_id = rng.integers(0, 16, Z)
    perm, blk_start = O.partition(shape_id, T, H, W)
    N = T * H * W
    assert np.array_equal(np.sort(perm), np.arange(N))                    # bijection
    sizes = np.diff(blk_start) * 64
    assert sizes.sum() == N and set(sizes) <= {64, 128, 256}              # multiples of 64 tokens
    assert len(sizes) == sum(512 // O.CANDIDATE_VOLUMES[s] for s in shape_id)
    t, rem = np.divmod(perm, H * W)
    h, w = np.divmod(rem, W)
    b = 0
    for m in range(Z):
        bt, bh, bw = O.CANDIDATES[shape_id[m]]
        for _ in range(512 // (bt * bh * bw)):
            s = slice(blk_start[b] * 64, blk_start[b + 1] * 64)
            # every block is a b_T x b_H x b_W box inside one zone, raster ordered
            assert np.ptp(t[s]) == bt - 1 and np.ptp(h[s]) == bh - 1 and np.ptp(w[s]) == bw - 1
            zone = ((t[s] // 8) * (H // 8) + h[s] // 8) * (W // 8) + w[s] // 8
            assert (zone == m).all()
            assert (np.diff(perm[s]) > 0).all()
            b += 1
    x = rng.standard_normal((2, N, 3))
    assert np.array_equal(O.unpermute_tokens(O.permute_tokens(x, perm), perm), x)


def test_plan_on_workload_margins():
    from workload import generate
    w = generate("par_small")
    c = w.cfg
    zs = O.zone_statistics(w.f32("v"), w.a, c.T, c.H, c.W)
    plan = O.plan_shapes(zs["g"], zs["rho"])
    assert (O.CANDIDATE_VOLUMES[plan["shape_id"]] == plan["vol"]).all()
    assert len(set(plan["vol"].ravel())) >= 2

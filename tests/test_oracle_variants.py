"""Pins of the oracle's variant switches: the ablation baselines of the Prism
write-ups (fixed block shapes, Top-k-only and Top-p-only selection,
video-only and audio-only guidance; sd114.wiki post, 测试结果) and the
max(rho, a-bar) density reading.  CPU only."""

import numpy as np
import pytest

import oracle as O
from workload import CONFIGS, generate


def _row(rng, nb, spread=2.0):
    s = rng.standard_normal(nb) * spread
    return s, O.block_probabilities(s), rng.choice([64, 128, 256], nb)


def test_topk_only_is_the_k_best_scores():
    rng = np.random.default_rng(10)
    for _ in range(200):
        nb = int(rng.integers(1, 50))
        s, P, sizes = _row(rng, nb)
        k = int(rng.integers(1, 12))
        r = O.select_row(s, P, sizes, k, 0.9, 1.0, 10 ** 6, O.VARIANT_TOPK_ONLY)
        assert r["L"] == min(k, nb)
        # brute force: every selected score beats every rejected one
        chosen = set(r["cols"].tolist())
        rest = [j for j in range(nb) if j not in chosen]
        if rest:
            assert min(s[list(chosen)]) >= max(s[rest])


def test_topp_only_is_the_smallest_nucleus():
    """Top-p alone: the fewest blocks whose probability reaches p (brute
    force over subset sizes), at least one block."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        nb = int(rng.integers(1, 40))
        s, P, sizes = _row(rng, nb, spread=float(rng.uniform(0.1, 4)))
        p = float(rng.uniform(0.01, 0.99))
        r = O.select_row(s, P, sizes, 7, p, 1.0, 10 ** 6, O.VARIANT_TOPP_ONLY)
        best = np.sort(P)[::-1]
        need = next(n for n in range(1, nb + 1) if best[:n].sum() >= p - 1e-12)
        assert r["L"] == need
        assert P[r["cols"]].sum() >= p - 1e-12


def test_default_is_union_of_the_two_variants():
    """Without a cap the method's S_i is the union of the Top-k-only and the
    Top-p-only selections (the hybrid rule of Prism guide (pt), Método 3)."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        nb = int(rng.integers(1, 50))
        s, P, sizes = _row(rng, nb, spread=float(rng.uniform(0.1, 4)))
        k = int(rng.integers(1, 10))
        p = float(rng.uniform(0.05, 0.99))
        a = O.select_row(s, P, sizes, k, p, 1.0, 10 ** 6, O.VARIANT_TOPK_ONLY)["cols"]
        b = O.select_row(s, P, sizes, k, p, 1.0, 10 ** 6, O.VARIANT_TOPP_ONLY)["cols"]
        u = O.select_row(s, P, sizes, k, p, 1.0, 10 ** 6)["cols"]
        np.testing.assert_array_equal(u, np.union1d(a, b))


def test_topp_only_respects_the_cap():
    rng = np.random.default_rng(13)
    for _ in range(100):
        nb = int(rng.integers(2, 40))
        s, P, sizes = _row(rng, nb, spread=0.3)
        N = int(sizes.sum())
        cap = float(rng.uniform(0.05, 0.5))
        r = O.select_row(s, P, sizes, 3, 0.99, cap, N, O.VARIANT_TOPP_ONLY)
        assert r["L"] >= 1
        if r["L"] > 1:
            assert sizes[r["order"][:r["L"]]].sum() <= np.floor(cap * N)


def _zone_inputs(seed=0):
    cfg = CONFIGS["tiny"]
    wl = generate(cfg)
    return cfg, wl.f32("v"), wl.a


def test_visual_only_equals_silent_audio():
    """Dropping the audio term is the same as feeding an all-zero A2V map."""
    cfg, v, a = _zone_inputs()
    vis = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6, O.VARIANT_VISUAL_ONLY)
    silent = O.zone_statistics(v, None, cfg.T, cfg.H, cfg.W, 1e-6)
    np.testing.assert_array_equal(vis["g"], silent["g"])
    np.testing.assert_array_equal(vis["rho"], silent["rho"])


def test_audio_only_ignores_the_video():
    """With audio-only guidance g does not depend on V: scaling V or
    replacing it by noise leaves g unchanged, and every head sees the same
    g; g - eps lies in [0, 1] (a-bar and v-hat are both in [0, 1])."""
    cfg, v, a = _zone_inputs()
    rng = np.random.default_rng(5)
    g1 = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6, O.VARIANT_AUDIO_ONLY)["g"]
    g2 = O.zone_statistics(rng.standard_normal(v.shape), a, cfg.T, cfg.H, cfg.W, 1e-6, O.VARIANT_AUDIO_ONLY)["g"]
    np.testing.assert_array_equal(g1, g2)
    np.testing.assert_array_equal(g1, np.broadcast_to(g1[:1], g1.shape))
    assert (g1 - 1e-6 >= 0).all() and (g1 - 1e-6 <= 1 + 1e-12).all()
    full = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6)["g"]
    vis = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6, O.VARIANT_VISUAL_ONLY)["g"]
    # the composite indicator is the sum of the two single-signal terms
    np.testing.assert_allclose(full - 1e-6, (vis - 1e-6) + (g1 - 1e-6), rtol=1e-14, atol=1e-15)


def test_rho_max_audio():
    """rho' = max(rho, a-bar): never below rho, equal where the audio is
    weaker, and 1 in the zone with the strongest audio coupling."""
    cfg, v, a = _zone_inputs()
    base = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6)
    mx = O.zone_statistics(v, a, cfg.T, cfg.H, cfg.W, 1e-6, O.VARIANT_RHO_MAX_AUDIO)
    assert (mx["rho"] >= base["rho"]).all()
    weaker = base["abar"][None, :] <= base["rho"]
    np.testing.assert_array_equal(mx["rho"][weaker], base["rho"][weaker])
    assert np.allclose(mx["rho"][:, int(np.argmax(base["abar"]))], 1.0)
    np.testing.assert_array_equal(mx["g"], base["g"])


@pytest.mark.parametrize("sid", [0, 5, 15])
def test_fixed_shape_tiles_every_zone_alike(sid):
    """A fixed block shape gives N / volume blocks, each exactly one
    bt x bh x bw box of the video."""
    cfg = CONFIGS["tiny"]
    wl = generate(cfg)
    params = O.Params(variant=O.VARIANT_FIXED_SHAPE, fixed_shape=sid, top_k=cfg.top_k, top_p=cfg.top_p)
    res = O.run_pipeline(wl.f32("q"), wl.f32("k"), wl.f32("v"), wl.a, cfg.T, cfg.H, cfg.W, params,
                         attention=False)
    assert (res["plan"]["shape_id"] == sid).all()
    vol = int(O.CANDIDATE_VOLUMES[sid])
    bt, bh, bw = (int(x) for x in O.CANDIDATES[sid])
    for hr in res["heads"]:
        bs = hr["blk_start"]
        assert bs.size - 1 == cfg.N // vol
        assert (np.diff(bs) * 64 == vol).all()
        for b in range(bs.size - 1):
            toks = hr["perm"][bs[b] * 64:bs[b + 1] * 64]
            t, rem = np.divmod(toks, cfg.H * cfg.W)
            hh, ww = np.divmod(rem, cfg.W)
            for coord, edge in ((t, bt), (hh, bh), (ww, bw)):
                assert coord.max() - coord.min() == edge - 1 and coord.min() % edge == 0


def test_rho_max_closed_form():
    """max(rho, a-bar) on three zones along W whose densities and couplings
    are known exactly: V varies along T with amplitudes 1, 1/2, 0 (so
    E = E0 (1, 1/4, 0) and rho = (1, 1/4, 0)); the zone means of a are
    1/8, 3/8, 5/8 (a-bar = 0, 1/2, 1, min-max).  rho' takes rho in zone 0
    and a-bar in zones 1 and 2: (1, 1/2, 1)."""
    T, H, W, D = 8, 8, 24, 4
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    amp = np.array([1.0, 0.5, 0.0])[w // 8]
    field = amp * np.cos(np.pi * (t + 0.5) / 8)                   # along T only
    u = np.array([1.0, -2.0, 0.5, 3.0])
    v = (field.reshape(-1)[:, None] * u[None, :])[None]           # [1][N][D]
    a = (np.array([0.125, 0.375, 0.625])[w // 8] + 0.01 * np.cos(np.pi * (h + 0.5) / 8)).reshape(-1)
    base = O.zone_statistics(v, a, T, H, W, 1e-6)
    np.testing.assert_allclose(base["rho"][0], [1.0, 0.25, 0.0], atol=1e-15)
    np.testing.assert_allclose(base["abar"], [0.0, 0.5, 1.0], atol=1e-14)
    mx = O.zone_statistics(v, a, T, H, W, 1e-6, O.VARIANT_RHO_MAX_AUDIO)
    np.testing.assert_allclose(mx["rho"][0], [1.0, 0.5, 1.0], atol=1e-14)
    # the volumes follow the raised density (tau128 = 0.4, tau256 = 0.2):
    # 64 everywhere, where rho alone gives 64, 128, 256
    shapes = O.candidate_shapes()
    vol = lambda rho: [int(np.prod(shapes[s])) for s in O.plan_shapes(mx["g"], rho, 0.4, 0.2)["shape_id"][0]]
    assert vol(mx["rho"]) == [64, 64, 64]
    assert vol(base["rho"]) == [64, 128, 256]

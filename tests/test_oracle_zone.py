"""Pins of the oracle's zone statistics (Prism guide (pt), Método 1) against
closed forms on hand-built zones.  CPU only."""

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _field(T, H, W, D, fT, fH, fW, alpha, beta, gamma, rng):
    """v_c(t,h,w) = alpha fT(t%8) u_c + beta fH(h%8) w_c + gamma fW(w%8) z_c + const_c."""
    u, w, z, c0 = (rng.standard_normal(D) for _ in range(4))
    t, h, ww = np.meshgrid(np.arange(T) % 8, np.arange(H) % 8, np.arange(W) % 8, indexing="ij")
    v = (alpha * fT(t)[..., None] * u + beta * fH(h)[..., None] * w + gamma * fW(ww)[..., None] * z + c0)
    return v.reshape(1, T * H * W, D), (u, w, z)


def _popvar(f):
    x = f(np.arange(8.0))
    return ((x - x.mean()) ** 2).mean()


def test_population_variance_constants():
    # Var(tau) over tau = 0..7 is (8^2 - 1) / 12 = 5.25; Var of the half-shifted cosine is 1/2.
    assert _popvar(lambda i: i) == pytest.approx(5.25, abs=1e-15)
    assert _popvar(lambda i: np.cos(np.pi * (i + 0.5) / 8)) == pytest.approx(0.5, abs=1e-15)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_video_variance_closed_form(D):
    """sigma^2_v,d = coef_d^2 Var(f_d) |dir_d|^2 / D for a separable field."""
    rng = np.random.default_rng(D)
    fT = lambda i: i.astype(float)
    fH = lambda i: np.cos(np.pi * (i + 0.5) / 8)
    fW = lambda i: (i.astype(float) - 3.5) ** 2
    alpha, beta, gamma = 0.7, 1.9, 0.3
    v, (u, w, z) = _field(8, 16, 8, D, fT, fH, fW, alpha, beta, gamma, rng)
    sv2 = O.video_variation(v, 8, 16, 8)[0]
    expect = np.array([alpha ** 2 * _popvar(fT) * (u @ u) / D,
                       beta ** 2 * _popvar(fH) * (w @ w) / D,
                       gamma ** 2 * _popvar(fW) * (z @ z) / D])
    assert sv2.shape == (2, 3)
    for m in range(2):
        np.testing.assert_allclose(sv2[m], expect, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_single_axis_field_gives_unit_ratio(axis):
    rng = np.random.default_rng(axis)
    f = lambda i: np.sin(i * 0.9) + 0.1 * i
    zero = lambda i: np.zeros_like(i, dtype=float)
    fs = [zero, zero, zero]
    fs[axis] = f
    v, _ = _field(8, 8, 8, 32, *fs, 1.3, 1.3, 1.3, rng)
    zs = O.zone_statistics(v, None, 8, 8, 8)
    e = np.zeros(3)
    e[axis] = 1.0
    np.testing.assert_allclose(zs["r"][0, 0], e, atol=1e-14)


def test_constant_zone_gives_thirds_and_zero_density():
    v = np.ones((1, 512, 8)) * 0.25
    zs = O.zone_statistics(v, None, 8, 8, 8)
    np.testing.assert_array_equal(zs["r"][0, 0], np.full(3, 1 / 3))
    assert zs["rho"][0, 0] == 0.0
    assert zs["g"][0, 0] == pytest.approx(np.full(3, 1 / 3 + 1e-6), abs=1e-16)


def test_zone_order_and_layout():
    """Zone m = (z_t * H/8 + z_h) * W/8 + z_w; each zone gets exactly its 512 tokens."""
    T, H, W = 16, 8, 24
    x = np.arange(T * H * W, dtype=float).reshape(1, -1, 1)
    z = O.to_zones(x, T, H, W)[0, ..., 0]
    assert z.shape == (6, 8, 8, 8)
    for m in range(6):
        mt, rem = divmod(m, 3)
        mh, mw = divmod(rem, 3)
        for (a, b, c) in [(0, 0, 0), (7, 3, 5), (2, 6, 1)]:
            t, h, w = mt * 8 + a, mh * 8 + b, mw * 8 + c
            assert z[m, a, b, c] == (t * H + h) * W + w


def test_audio_terms_closed_forms():
    T, H, W = 8, 8, 24  # three zones along W
    N = T * H * W
    zone_vals = np.array([0.1, 0.35, 0.6])
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    a = zone_vals[w // 8] + 0.01 * np.cos(np.pi * ((h % 8) + 0.5) / 8)   # varies along H only
    abar, vhat, mu_a, sa2 = O.audio_terms(a.reshape(-1), T, H, W)
    np.testing.assert_allclose(abar, [0.0, 0.5, 1.0], atol=1e-15)
    np.testing.assert_allclose(vhat, np.tile([0.0, 1.0, 0.0], (3, 1)), atol=1e-15)
    np.testing.assert_allclose(sa2[:, 1], 0.01 ** 2 * 0.5, rtol=1e-12)
    # flat map: no coupling anywhere
    abar0, vhat0, _, _ = O.audio_terms(np.full(N, 0.3), T, H, W)
    np.testing.assert_array_equal(abar0, 0.0)
    np.testing.assert_array_equal(vhat0, 1 / 3)
    # absent map behaves as zero
    abar1, _, _, _ = O.audio_terms(None, T, H, W)
    np.testing.assert_array_equal(abar1, 0.0)


def test_a2v_norm_integer_cases():
    """Rows that are Pythagorean quadruples (and their permutations, signs
    and zero padding) have integer norms; a zero row has norm 0."""
    rows = [(1, 2, 2, 3), (2, 3, 6, 7), (1, 4, 8, 9), (2, 6, 9, 11), (4, 4, 7, 9), (6, 6, 7, 11)]
    h = np.zeros((len(rows) + 1, 64))
    rng = np.random.default_rng(0)
    for i, (x, y, z, _) in enumerate(rows):
        pos = rng.choice(64, 3, replace=False)
        h[i, pos] = np.array([x, -y, z]) * rng.choice([-1, 1])
    got = O.a2v_norms(h)
    np.testing.assert_array_equal(got[:-1], [r[3] for r in rows])
    assert got[-1] == 0.0


def test_a2v_norm_matches_generator():
    from workload import generate
    w = generate("tiny")
    np.testing.assert_allclose(O.a2v_norms(w.h_hat), w.a, rtol=3e-7)


def test_indicator_sums():
    """sum_d r = sum_d v-hat = 1, hence sum_d g = 1 + a-bar + 3 eps."""
    from workload import generate
    w = generate("par_d64")
    c = w.cfg
    zs = O.zone_statistics(w.f32("v"), w.a, c.T, c.H, c.W, eps=1e-6)
    np.testing.assert_allclose(zs["r"].sum(-1), 1.0, atol=1e-15)
    np.testing.assert_allclose(zs["vhat"].sum(-1), 1.0, atol=1e-15)
    np.testing.assert_allclose(zs["g"].sum(-1), 1.0 + zs["abar"][None, :] + 3e-6, atol=1e-14)
    assert zs["rho"].max() == 1.0 and (zs["rho"] >= 0).all()


def test_density_is_relative_total_variance():
    sv2 = np.array([[[1.0, 2.0, 1.0], [0.5, 0.25, 0.25], [0.1, 0.1, 0.1999]]])
    rho = O.information_density(sv2)
    np.testing.assert_allclose(rho, [[1.0, 0.25, 0.0999750]], rtol=1e-15)

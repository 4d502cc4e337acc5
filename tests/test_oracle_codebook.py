"""Pins of the oracle's rotation and Lloyd-Max codebook against closed forms, an independent
quadrature, a textbook limit and a KS test of the Beta coordinate model. CPU only."""
import math

import numpy as np
import pytest
from numpy.polynomial import legendre
from scipy import integrate, special, stats

from oracle import tq_oracle as O
from tests.conftest import read_golden

DS = (8, 64, 128, 256)


# --------------------------------------------------------------------------- Hadamard / rotation
@pytest.mark.parametrize("d", [2, 4, 8, 16, 64, 128, 256])
def test_hadamard_orthogonal_exact(d):
    H = O.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))


@pytest.mark.parametrize("d", [8, 64, 256])
def test_hadamard_natural_order_closed_form(d):
    # Sylvester natural order: H[i, j] = (-1)^popcount(i & j)
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(O.hadamard(d), np.where(pc % 2 == 0, 1.0, -1.0))


def _butterfly(x):
    # independent fast transform (in-place radix-2), natural order
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    h = 1
    while h < d:
        x = x.reshape(*x.shape[:-1], d // (2 * h), 2, h)
        a, b = x[..., 0, :].copy(), x[..., 1, :].copy()
        x[..., 0, :], x[..., 1, :] = a + b, a - b
        x = x.reshape(*x.shape[:-3], d)
        h *= 2
    return x


@pytest.mark.parametrize("d", DS)
def test_dense_equals_butterfly_on_integers(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(17, d)).astype(np.float64)
    s = O.head_signs(11, 0, d)
    # both routes: exact integer transform, then one division by the same fp64 sqrt(d)
    assert np.array_equal(O.rotate(x, s), _butterfly(x * s) / math.sqrt(d))


@pytest.mark.parametrize("d", DS)
def test_rotation_round_trip(d):
    rng = np.random.default_rng(1 + d)
    s = O.head_signs(3, 1, d)
    xi = rng.integers(-64, 64, size=(9, d)).astype(np.float64)
    # H H = d I: s ⊙ H(H(x ⊙ s))/d is exact for small integers
    assert np.array_equal(s * _butterfly(_butterfly(xi * s)) / d, xi)
    x = rng.standard_normal((33, d))
    back = O.unrotate(O.rotate(x, s), s)
    assert np.max(np.abs(back - x)) < 8 * np.finfo(float).eps * np.max(np.abs(x)) * math.log2(d)


@pytest.mark.parametrize("d", DS)
def test_rotated_unit_vector_coordinates_follow_beta_model(d):
    """[AB] §2 TurboQuant / [SI]: y = WHT(u ⊙ s)/sqrt(d) of a unit vector is Beta((d-1)/2,(d-1)/2)
    on [-1,1]; for a uniformly random u this is exact, checked by KS per pooled coordinates."""
    rng = np.random.default_rng(100 + d)
    n = max(4000, 200000 // d)
    x = rng.standard_normal((n, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = O.rotate(u, O.head_signs(5, 2, d))
    for j in (0, d // 2, d - 1):
        p = stats.kstest(y[:, j], lambda v: O.coord_cdf(v, d)).pvalue
        assert p > 1e-4, (d, j, p)


@pytest.mark.parametrize("d", [8, 64, 256])
def test_cdf_matches_independent_quadrature(d):
    for x in (-0.7, -0.1, 0.0, 0.05, 0.3, 0.9):
        q, _ = integrate.quad(lambda v: O.coord_pdf(v, d), -1.0, x, epsabs=1e-14, epsrel=1e-12, limit=200)
        assert abs(q - O.coord_cdf(x, d)) < 1e-11


# --------------------------------------------------------------------------- Lloyd-Max
def _gl_cell_moments(lo, hi, d, n_panels=64, n_nodes=24):
    """Independent composite Gauss-Legendre moments of (1-x^2)^alpha on [lo, hi] (unnormalised)."""
    al = (d - 3) / 2.0
    xg, wg = legendre.leggauss(n_nodes)
    edges = np.linspace(lo, hi, n_panels + 1)
    m0 = m1 = 0.0
    for a, b in zip(edges[:-1], edges[1:]):
        xs = 0.5 * (b - a) * xg + 0.5 * (a + b)
        f = np.maximum((1 - xs) * (1 + xs), 0.0) ** al
        m0 += 0.5 * (b - a) * np.sum(wg * f)
        m1 += 0.5 * (b - a) * np.sum(wg * xs * f)
    return m0, m1


@pytest.mark.parametrize("d", DS)
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6])
def test_lloyd_max_centroid_and_midpoint_conditions(d, b):
    t, c = O.lloyd_max(d, b)
    L = 1 << b
    assert t.shape == (L - 1,) and c.shape == (L,)
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    # symmetry and the zero threshold
    assert np.array_equal(c, -c[::-1])
    assert np.array_equal(t, -t[::-1])
    assert t[L // 2 - 1] == 0.0
    # midpoint condition, exactly as stored
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))
    # centroid condition, by an independent quadrature on every positive cell
    edges = np.concatenate(([-1.0], t, [1.0]))
    for i in range(L // 2, L):
        m0, m1 = _gl_cell_moments(edges[i], edges[i + 1], d)
        assert abs(m1 / m0 - c[i]) <= 1e-12 * max(1.0, abs(c[i])) + 1e-13, (d, b, i)


@pytest.mark.parametrize("d", [4, 8, 64, 128, 256, 1024])
def test_lloyd_max_one_bit_closed_form(d):
    al = (d - 3) / 2.0
    _, c = O.lloyd_max(d, 1)
    want = 1.0 / ((al + 1.0) * special.beta(0.5, al + 1.0))   # E|X| for the coordinate density
    assert abs(c[1] - want) < 1e-14 and c[0] == -c[1]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_lloyd_max_uniform_special_case(b):
    # d = 3: the coordinate density is uniform on [-1, 1] (Archimedes), whose Lloyd-Max quantiser
    # is the uniform quantiser with cells of width 2/L.
    t, c = O.lloyd_max(3, b)
    L = 1 << b
    assert np.allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-14)
    assert np.allclose(t, -1 + 2 * np.arange(1, L) / L, atol=1e-14)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_mse_decreases_with_bits_and_matches_monte_carlo(d):
    mses = [O.codebook_mse(d, *O.lloyd_max(d, b)) for b in range(1, 7)]
    assert all(a > b for a, b in zip(mses, mses[1:]))
    # Monte Carlo of the per-coordinate MSE at b = 3
    rng = np.random.default_rng(d)
    x = rng.standard_normal((20000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    t, c = O.lloyd_max(d, 3)
    y = O.rotate(u, O.head_signs(1, 0, d))
    mc = np.mean((y - c[O.quantise(y, t)]) ** 2)
    assert abs(mc - mses[2]) < 0.02 * mses[2]


def _gaussian_lloyd_max(L):
    """Independent Lloyd iteration for N(0,1) (library normal cdf/pdf)."""
    c = stats.norm.ppf((np.arange(L) + 0.5) / L)
    for _ in range(20000):
        t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        mass = stats.norm.cdf(t[1:]) - stats.norm.cdf(t[:-1])
        c_new = (stats.norm.pdf(t[:-1]) - stats.norm.pdf(t[1:])) / mass
        if np.max(np.abs(c_new - c)) < 1e-13:
            c = c_new
            break
        c = c_new
    return 0.5 * (c[:-1] + c[1:]), c


def test_large_d_tends_to_gaussian_lloyd_max_textbook():
    d = 1 << 16
    rows = read_golden("gaussian_lloyd_max_max1960.txt")
    for r in rows:
        L, kind, vals = int(r[0]), r[1], np.array([float(v) for v in r[2:]])
        t, c = O.lloyd_max(d, int(math.log2(L)))
        ours = (c if kind == "out" else t)[-len(vals):] * math.sqrt(d)
        # table has 4 significant digits; finite-d correction is O(1/d)
        assert np.allclose(ours, vals, rtol=1.5e-3, atol=1e-3), (L, kind, ours, vals)
        tg, cg = _gaussian_lloyd_max(L)
        ref = (cg if kind == "out" else tg)[-len(vals):]
        assert np.allclose(ours, ref, rtol=2e-4, atol=2e-4)


def test_sqrt_d_scaled_codebook_trend_to_gaussian():
    _, cg = _gaussian_lloyd_max(16)
    errs = [np.max(np.abs(O.lloyd_max(d, 4)[1] * math.sqrt(d) - cg)) for d in (64, 256, 1024, 4096)]
    assert all(a > b for a, b in zip(errs, errs[1:]))

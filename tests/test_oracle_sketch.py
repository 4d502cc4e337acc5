"""Pins of the 1-bit QJL sketch of the TurboQuant key path (oracle/tq_oracle.py ``sketch``,
``encode``).

Page: "Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2 "TurboQuant"
(the sketch of the WHT-domain residual e = y - ŷ) and "SpectralQuant" (sign(S e) inside the
asymmetric estimator).  The sketch is σ = [S e >= 0] on the exact residual, sign(0) = +1; a bit is
flagged when |S e| < 1e-6.  The expected values below are written out by hand or computed by an
independent route (the Sylvester matrix built by its recursion, exactly rounded sums), never by the
oracle's own matrix routines."""
import math

import numpy as np

from oracle import tq_oracle as O


def test_sketch_of_a_small_case_written_out():
    S = np.array([[1.0, -2.0, 0.5], [0.0, 1.0, 1.0], [0.0, 0.0, 0.0], [3.0, 0.0, 0.0]])
    e = np.array([[2.0 ** -8, 2.0 ** -9, 2.0 ** -6], [0.0, -2.0 ** -7, 2.0 ** -20]])
    r = O.sketch(e, S)
    want_z = np.array([[2.0 ** -8 - 2.0 ** -8 + 2.0 ** -7, 2.0 ** -9 + 2.0 ** -6, 0.0, 3 * 2.0 ** -8],
                       [2.0 ** -6 + 2.0 ** -21, -2.0 ** -7 + 2.0 ** -20, 0.0, 0.0]])
    assert np.array_equal(r["z"], want_z)
    assert r["sigma"].tolist() == [[True, True, True, True], [True, False, True, True]]   # sign(0) = +1
    # 2^-20 < 1e-6 < 2^-19: only exact zeros are flagged here
    assert r["sflag"].tolist() == [[False, False, True, False], [False, False, True, True]]


def test_sketch_takes_the_exact_residual():
    """Two residual coordinates 3e-6 apart that share one half-precision value (fp16 spacing of
    2^14 e near 164 is 1/8, i.e. 7.6e-6 in e): z = e0 - e1 = -3e-6 is outside the flag band, so the
    bit is 0; a projection of a rounded residual would see z = 0 and store 1."""
    S = np.array([[1.0, -1.0]])
    e = np.array([[0.01, 0.010003]])
    r = O.sketch(e, S)
    assert r["z"][0, 0] == 0.01 - 0.010003
    assert r["sigma"].tolist() == [[False]] and r["sflag"].tolist() == [[False]]
    assert np.float16(0.01 * 2 ** 14) == np.float16(0.010003 * 2 ** 14)       # the trap is real


def _sylvester(d):
    h = [[1]]
    while len(h) < d:
        h = [row + row for row in h] + [row + [-v for v in row] for row in h]
    return h


def test_encoded_sketch_by_brute_force_at_d8():
    """d = 8, m = 16 (so a transposed S cannot fit): every step written out with Python loops and
    exactly rounded sums: u = x/||x||, y = H(u ⊙ s)/sqrt(8), idx by a linear count, e = y - c[idx],
    z_i = Σ_k S_ik e_k."""
    d, b, m = 8, 2, 16
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(21, 0, d)
    S = O.gaussian_matrix(21, 0, m, d).astype(np.float64)
    H = _sylvester(d)
    x = np.random.default_rng(5).standard_normal((60, d))
    r = O.encode(x, s, t, c, S)
    checked = 0
    for v in range(x.shape[0]):
        n = math.sqrt(math.fsum(a * a for a in x[v]))
        u = [a / n for a in x[v]]
        y = [math.fsum(H[j][k] * s[k] * u[k] for k in range(d)) / math.sqrt(d) for j in range(d)]
        idx = [sum(1 for ti in t if ti <= yj) for yj in y]
        e = [y[j] - c[idx[j]] for j in range(d)]
        assert idx == r["idx"][v].tolist()
        assert np.allclose(r["e"][v], e, rtol=0, atol=1e-15)
        z = [math.fsum(S[i][k] * e[k] for k in range(d)) for i in range(m)]
        for i in range(m):
            if abs(z[i]) > 1e-12:
                assert r["sigma"][v, i] == (z[i] >= 0.0)
                checked += 1
        assert r["r16"][v] == np.float16(math.sqrt(math.fsum(a * a for a in e)))
    assert checked > 0.99 * x.shape[0] * m


def test_flags_are_the_decisions_within_the_tolerance():
    d, b, m = 128, 3, 64
    t, c = O.lloyd_max(d, b)
    s, S = O.head_signs(3, 0, d), O.gaussian_matrix(3, 0, m, d).astype(np.float64)
    r = O.encode(np.random.default_rng(7).standard_normal((4000, d)), s, t, c, S)
    z = r["z"]
    assert np.array_equal(r["sflag"], np.abs(z) < 1e-6)
    # z ~ N(0, ||e||^2): the band holds about 2e-6 · density(0) of the bits
    dens = 1.0 / (math.sqrt(2 * math.pi) * float(np.sqrt(np.mean(np.sum(r["e"] ** 2, axis=1)))))
    assert r["sflag"].mean() < 20 * 2e-6 * dens + 1e-4
    # any perturbation of z within the tolerance changes only flagged bits
    rng = np.random.default_rng(8)
    zp = z + rng.uniform(-1e-6, 1e-6, z.shape) * 0.999
    changed = (zp >= 0) != r["sigma"]
    assert not (changed & ~r["sflag"]).any()

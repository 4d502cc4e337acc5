"""Pins of the oracle's randomized Hadamard (RHT) QJL sketch and of the QJL decode correction.
CPU only.

[AB] §2 TurboQuant: b = sign(WHT(e ⊙ s2)) for a fixed sign vector s2, and the correction
Δŷ = sqrt(pi/2)/d · ||e|| · s2 ⊙ WHT(b) added at decode.  The oracle writes the sketch as the matrix
S = H diag(s2) (m = d) and the correction as sqrt(pi/2)/m · ||e|| · S^T (2σ - 1), the form shared
with the Gaussian sketch; these tests tie that form to the pages' one."""
import math

import numpy as np
from scipy import stats

from oracle import tq_oracle as O


def _sylvester(d):
    """H[i][j] = (-1)^popcount(i & j), written out independently of the oracle and of scipy."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 1, -1.0, 1.0)


def test_fwht_is_the_sylvester_matrix():
    rng = np.random.default_rng(0)
    for d in (8, 64, 256):
        v = rng.standard_normal((5, d))
        assert np.allclose(O.fwht(v), v @ _sylvester(d), rtol=0, atol=1e-11)


def test_rht_matrix_is_hadamard_times_second_signs():
    for d in (64, 128, 256):
        S = O.rht_matrix(77, 3, d).astype(np.float64)
        assert set(np.unique(S)) <= {-1.0, 1.0}
        assert np.array_equal(S @ S.T, d * np.eye(d))                      # orthogonal, scale d
        s2 = O.rht_signs(77, 3, d)
        assert np.array_equal(S, _sylvester(d) * s2[None, :])
        e = np.random.default_rng(d).standard_normal((4, d))
        assert np.allclose(e @ S.T, O.fwht(e * s2), rtol=0, atol=1e-11)    # S e = WHT(e ⊙ s2)


def test_rht_signs_balanced_and_distinct_from_rotation_signs():
    d = 4096
    s2, s1 = O.rht_signs(9, 0, d), O.rht_signs(9, 0, d)
    assert np.array_equal(s2, s1)                                          # deterministic
    assert stats.binomtest(int((s2 > 0).sum()), d, 0.5).pvalue > 1e-4
    agree = int((s2 == O.head_signs(9, 0, d)).sum())                        # tag 3 vs tag 1
    assert stats.binomtest(agree, d, 0.5).pvalue > 1e-4
    assert not np.array_equal(O.rht_signs(9, 1, 64), O.rht_signs(9, 0, 64))


def test_encode_sketch_is_sign_of_wht_of_signed_residual():
    d, b = 128, 3
    t, c = O.lloyd_max(d, b)
    s, S = O.head_signs(5, 0, d), O.rht_matrix(5, 0, d)
    x = np.random.default_rng(1).standard_normal((200, d))
    r = O.encode(x, s, t, c, S)
    z = O.fwht(r["e"] * O.rht_signs(5, 0, d))
    assert np.array_equal(r["sigma"], z >= 0.0)
    assert np.allclose(r["z"], z, rtol=0, atol=1e-12)


def test_correction_closed_form_on_a_hadamard_column():
    """e = α s2 ⊙ h_j (h_j a column of H): S e = α d δ_j, so every sign bit is +1 (sign(0) = +1),
    S^T 1 = s2 ⊙ H 1 = d s2_0 δ_0, and Δŷ = sqrt(pi/2) α sqrt(d) s2_0 δ_0."""
    d, alpha, j = 64, 0.25, 37
    S = O.rht_matrix(11, 2, d).astype(np.float64)
    s2 = O.rht_signs(11, 2, d)
    e = alpha * s2 * _sylvester(d)[:, j]
    z = S @ e
    assert z[j] == alpha * d and np.count_nonzero(z) == 1
    sigma = (z >= 0.0)[None, :]
    corr = O.qjl_correction(sigma, np.array([np.linalg.norm(e)]), S)[0]
    want = np.zeros(d)
    want[0] = math.sqrt(math.pi / 2) * alpha * math.sqrt(d) * s2[0]
    assert np.allclose(corr, want, rtol=1e-14, atol=1e-14)


def test_correction_norm_identity_and_error_reduction():
    """For S = H diag(s2), ||S^T b||² = d ||b||² = d², so ||Δŷ||² = (pi/2) ||e||² exactly; and with
    <Δŷ, e> ≈ ||e||² (half-normal |z_i|), the corrected residual e - Δŷ carries about (pi/2 - 1)
    of the uncorrected squared error."""
    d, b = 128, 2
    t, c = O.lloyd_max(d, b)
    s, S = O.head_signs(21, 0, d), O.rht_matrix(21, 0, d)
    x = np.random.default_rng(4).standard_normal((3000, d))
    r = O.encode(x, s, t, c, S)
    e = r["e"]
    en = np.linalg.norm(e, axis=1)
    corr = O.qjl_correction(r["sigma"], en, S)
    assert np.allclose(np.sum(corr * corr, axis=1), math.pi / 2 * en ** 2, rtol=1e-12)
    ratio = np.sum((e - corr) ** 2) / np.sum(e * e)
    assert abs(ratio - (math.pi / 2 - 1)) < 0.03, ratio
    # the decode with the correction lands closer to the input direction than the MSE decode
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    plain = O.decode(r["idx"], np.ones(len(x)), s, c)
    fixed = O.decode(r["idx"], np.ones(len(x)), s, c, corr)
    assert np.sum((fixed - u) ** 2) < 0.7 * np.sum((plain - u) ** 2)


def test_rht_score_estimate_nearly_unbiased_over_second_signs():
    """Over independent s2, the RHT estimate of <q, e> centres on the truth (the rows of H diag(s2)
    are Rademacher vectors, so unbiasedness holds up to the normal approximation of S_i·e)."""
    d, T = 128, 3000
    rng = np.random.default_rng(8)
    q = rng.standard_normal(d)
    e = rng.standard_normal(d) * 0.1 + 0.05 * q
    est = np.array([O.qjl_estimate(q, e, O.rht_matrix(5000 + k, 0, d)) for k in range(T)])
    truth = float(q @ e)
    sd = est.std(ddof=1)
    assert abs(est.mean() - truth) < 4 * sd / math.sqrt(T) + 0.02 * abs(truth), (est.mean(), truth)

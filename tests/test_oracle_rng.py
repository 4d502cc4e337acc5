"""Pins of the oracle's random state (SplitMix64 + Box-Muller) against published definitions
and distributional facts. CPU only."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import tq_oracle as O
from tests.conftest import read_golden


def test_splitmix64_reference_outputs():
    # SplitMix64 reference sequence from state 0 (tests/golden/splitmix64_state0.txt).
    want = [int(r[0], 16) for r in read_golden("splitmix64_state0.txt")]
    got = O.words(0, len(want)).tolist()
    assert got == want


def test_vectorised_mix_matches_scalar():
    key = O.stream_key(12345, O.TAG_GAUSS, 7)
    w = O.words(key, 257).tolist()
    state = key
    for i in range(257):
        state = (state + O.GAMMA) & ((1 << 64) - 1)
        assert w[i] == O.mix64(state)


def test_stream_keys_distinct():
    keys = {O.stream_key(s, t, h) for s in (0, 1, 2**63 + 5) for t in (1, 2, 3) for h in range(64)}
    assert len(keys) == 3 * 3 * 64


def test_signs_balanced_and_deterministic():
    s = np.concatenate([O.head_signs(4001, h, 256) for h in range(64)])
    assert set(np.unique(s)) == {-1.0, 1.0}
    # mean of 16384 fair signs: |mean| < 5 sigma
    assert abs(s.mean()) < 5.0 / math.sqrt(s.size)
    assert np.array_equal(O.head_signs(4001, 3, 256), O.head_signs(4001, 3, 256))
    assert not np.array_equal(O.head_signs(4001, 3, 256), O.head_signs(4001, 4, 256))
    assert not np.array_equal(O.head_signs(4001, 3, 256), O.head_signs(4002, 3, 256))
    # signs of a shorter table are a prefix of a longer one (counter-based)
    assert np.array_equal(O.head_signs(9, 1, 64), O.head_signs(9, 1, 256)[:64])


def test_gaussian_moments_and_ks():
    g = np.concatenate([O.gaussian_matrix(3001, h, 128, 128).ravel() for h in range(4)]).astype(np.float64)
    n = g.size
    assert abs(g.mean()) < 5 / math.sqrt(n)
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    kurt = stats.kurtosis(g, fisher=False)
    assert abs(kurt - 3.0) < 5 * math.sqrt(24.0 / n)
    assert stats.kstest(g, "norm").pvalue > 1e-3
    assert g.dtype == np.float64


def test_gaussian_is_fp16_and_prefix_stable():
    a = O.gaussian_matrix(5, 2, 32, 64)
    assert a.dtype == np.float16
    b = O.gaussian_matrix(5, 2, 64, 64)
    # row-major counter: the first 32 rows of an m=64 table equal the m=32 table
    assert np.array_equal(a, b[:32])


def test_box_muller_first_element_by_hand():
    key = O.stream_key(77, O.TAG_GAUSS, 0)
    w0, w1 = O.words(key, 2).tolist()
    u1 = ((w0 >> 11) + 1) * 2.0 ** -53
    u2 = (w1 >> 11) * 2.0 ** -53
    g = np.float16(math.sqrt(-2 * math.log(u1)) * math.cos(2 * math.pi * u2))
    assert O.gaussian_matrix(77, 0, 1, 1)[0, 0] == g

"""Pins of the oracle's encode/decode/pack/score/attention/KL steps. CPU only.

Each test targets a mistake that would otherwise go unnoticed: an off-by-one in the search (the bug
class reported in [AB] §2), a wrong bit order, a dropped or mis-scaled QJL term, a transposed S, a
wrong softmax axis."""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

from oracle import tq_oracle as O
from tests.conftest import read_golden


def _binary_search(t, y):
    """Textbook lower-bound style binary search for #{i: t_i <= y} (independent of numpy)."""
    lo, hi = 0, len(t)
    while lo < hi:
        mid = (lo + hi) // 2
        if t[mid] <= y:
            lo = mid + 1
        else:
            hi = mid
    return lo


@pytest.mark.parametrize("b", range(1, 9))
def test_search_equals_linear_count_at_and_around_every_threshold(b):
    t, c = O.lloyd_max(64, b) if b <= 6 else (np.sort(np.random.default_rng(b).uniform(-.5, .5, (1 << b) - 1)), None)
    probes = [0.0, 1.0, -1.0, 0.5, -0.5, np.nextafter(0, 1), np.nextafter(0, -1)]
    for ti in t:
        probes += [ti, np.nextafter(ti, np.inf), np.nextafter(ti, -np.inf)]
    probes = np.array(probes)
    idx = O.quantise(probes, t)
    lin = np.array([int(np.sum(t <= y)) for y in probes])
    bs = np.array([_binary_search(t, y) for y in probes])
    assert np.array_equal(idx, lin) and np.array_equal(idx, bs)
    # ties go to the upper cell; y = 0 lands in cell L/2
    for i, ti in enumerate(t):
        assert O.quantise(np.array([ti]), t)[0] == i + 1
    if c is not None:   # real (symmetric) codebooks have t_{L/2} = 0
        assert O.quantise(np.array([0.0]), t)[0] == (1 << b) // 2


def test_zero_vector_encodes_to_middle_cell_and_decodes_to_zero():
    d, b = 64, 4
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(1, 0, d)
    r = O.encode(np.zeros((2, d)), s, t, c)
    assert np.all(r["idx"] == 8) and np.all(r["flag"]) and np.all(r["n16"] == 0)
    assert np.all(O.decode(r["idx"], r["n16"], s, c) == 0)


@pytest.mark.parametrize("b", [1, 2])
def test_brute_force_product_codebook_d8(b):
    """d = 8: the scalar decisions pick the L2-nearest of all (2^b)^8 product codewords, and the
    decoded vector is the nearest codeword-image to u (rotation is orthogonal)."""
    d = 8
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(21, 0, d)
    code = np.array(list(itertools.product(range(1 << b), repeat=d)))
    words = c[code]                                              # ((2^b)^8, 8)
    rng = np.random.default_rng(b)
    x = rng.standard_normal((12, d))
    r = O.encode(x, s, t, c)
    for k in range(len(x)):
        dist = np.sum((words - r["y"][k]) ** 2, axis=1)
        best = code[np.argmin(dist)]
        assert np.array_equal(best, r["idx"][k])
        u = x[k] / np.linalg.norm(x[k])
        imgs = O.unrotate(words, s)
        assert np.argmin(np.sum((imgs - u) ** 2, axis=1)) == np.argmin(dist)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_brute_force_scalar_argmin_d8(b):
    d = 8
    t, c = O.lloyd_max(d, b)
    rng = np.random.default_rng(7 + b)
    x = rng.standard_normal((500, d))
    r = O.encode(x, O.head_signs(2, 0, d), t, c)
    am = np.argmin(np.abs(r["y"][..., None] - c[None, None, :]), axis=-1)
    assert np.array_equal(am, r["idx"])


@pytest.mark.parametrize("b", [1, 3, 6])
def test_boundary_distance_equals_brute_force_minimum(b):
    t, _ = O.lloyd_max(64, b)
    y = np.concatenate([np.random.default_rng(b).uniform(-1, 1, 5000), t, t + 1e-9, t - 1e-9, [-1.0, 1.0, 0.0]])
    brute = np.min(np.abs(y[:, None] - t[None, :]), axis=1)
    assert np.array_equal(O.boundary_distance(y, t), brute)


def test_flags_mark_exactly_the_near_boundary_coordinates():
    d, b = 64, 3
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(1, 0, d)
    x = np.random.default_rng(0).standard_normal((400, d))
    r = O.encode(x, s, t, c)
    d_min = np.min(np.abs(r["y"][..., None] - t), axis=-1)
    assert np.array_equal(r["flag"], d_min < 1e-6)


def test_encode_norm_and_reconstruction_error():
    d, b = 128, 4
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(2001, 3, d)
    x = np.random.default_rng(5).standard_normal((3000, d)) * 3.0
    r = O.encode(x, s, t, c)
    n = np.linalg.norm(x, axis=1)
    assert np.array_equal(r["n16"], n.astype(np.float16))
    xh = O.decode(r["idx"], r["n16"], s, c)
    rel = np.sum((xh - x) ** 2) / np.sum(x ** 2)
    assert abs(rel - d * O.codebook_mse(d, t, c)) < 0.05 * d * O.codebook_mse(d, t, c)
    # per-token cosine at b=2 near the figure [AB] §4 quotes for TQ-KV (0.953; different regimes):
    # parity unpinned, order-of-magnitude sanity only
    t2, c2 = O.lloyd_max(d, 2)
    r2 = O.encode(x, s, t2, c2)
    xh2 = O.decode(r2["idx"], r2["n16"], s, c2)
    cos = np.mean(np.sum(xh2 * x, 1) / np.linalg.norm(xh2, axis=1) / n)
    assert 0.9 < cos < 0.97


def test_encode_is_scale_invariant_except_the_norm():
    d, b = 64, 3
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(8, 0, d)
    x = np.random.default_rng(1).standard_normal((50, d))
    r1, r2 = O.encode(x, s, t, c), O.encode(4.0 * x, s, t, c)   # power of two: exact scaling
    assert np.array_equal(r1["idx"], r2["idx"])
    assert np.array_equal(r2["n16"].astype(np.float64), 4.0 * r1["n16"].astype(np.float64))


def test_pack_bits_closed_form_and_round_trip():
    # values 0..7 at 3 bits each: the 24-bit little-endian integer is sum_j j << 3j
    v = np.arange(8)[None, :]
    packed = O.pack_bits(v, 3)
    want = sum(j << (3 * j) for j in range(8))
    assert packed.tolist() == [[want & 0xFF, (want >> 8) & 0xFF, (want >> 16) & 0xFF]]
    rng = np.random.default_rng(0)
    for b in range(1, 9):
        vals = rng.integers(0, 1 << b, size=(7, 128))
        pk = O.pack_bits(vals, b)
        assert pk.shape == (7, 128 * b // 8)
        assert np.array_equal(O.unpack_bits(pk, b, 128), vals)
        # LSB-first: value j occupies bits [j b, (j+1) b) of the integer formed by the bytes
        big = int.from_bytes(pk[0].tobytes(), "little")
        assert all(((big >> (j * b)) & ((1 << b) - 1)) == vals[0, j] for j in range(128))


def test_storage_matches_pages_and_layout():
    for d, b, bits in ((int(r[0]), int(r[1]), int(r[2])) for r in read_golden("storage_bits_per_token.txt")):
        assert O.layout(d, b, 0, 1, 1)["idx_bytes_per_vec"] * 8 == bits
    for d, b, m in ((64, 4, 0), (128, 4, 0), (128, 3, 128), (256, 6, 256)):
        lay = O.layout(d, b, m, 3, 1000)
        per_vec = lay["idx_bytes_per_vec"] + lay["sketch_bytes_per_vec"] + 2 + (2 if m else 0)
        assert per_vec == d * b // 8 + m // 8 + 2 + 2 * (m > 0)
        for k in ("off_idx", "off_sketch", "off_norm", "off_rnorm", "total_bytes"):
            assert lay[k] % 256 == 0
        assert lay["total_bytes"] >= 3000 * per_vec


def test_pack_tensor_round_trip():
    d, b, m, ns, nt = 64, 3, 32, 2, 37
    t, c = O.lloyd_max(d, b)
    rng = np.random.default_rng(3)
    encs = []
    for st in range(ns):
        s = O.head_signs(9, st, d)
        S = O.gaussian_matrix(9, st, m, d)
        encs.append(O.encode(rng.standard_normal((nt, d)), s, t, c, S))
    buf = O.pack_tensor(d, b, m, ns, nt, encs)
    back = O.unpack_tensor(buf, d, b, m, ns, nt)
    for e, r in zip(encs, back):
        assert np.array_equal(e["idx"], r["idx"]) and np.array_equal(e["sigma"], r["sigma"])
        assert np.array_equal(e["n16"], r["n16"]) and np.array_equal(e["r16"], r["r16"])


def test_scores_without_qjl_equal_dot_with_decoded_keys():
    d, b = 128, 3
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(3001, 0, d)
    rng = np.random.default_rng(11)
    k = rng.standard_normal((300, d))
    q = rng.standard_normal((7, d))
    r = O.encode(k, s, t, c)
    est = O.scores(q, r, s, c)
    ref = q @ O.decode(r["idx"], r["n16"], s, c).T
    assert np.max(np.abs(est - ref)) < 1e-12 * np.max(np.abs(ref))


def test_qjl_scores_reduce_error_on_average_and_use_every_term():
    d, b, m = 128, 2, 256
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(5, 1, d)
    S = O.gaussian_matrix(5, 1, m, d)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((2000, d))
    q = rng.standard_normal((4, d))
    r = O.encode(k, s, t, c, S)
    exact = q @ k.T
    e_mse = np.mean((O.scores(q, r, s, c) - exact) ** 2)
    e_qjl = np.mean((O.scores(q, r, s, c, S) - exact) ** 2)
    base = O.scores(q, r, s, c)
    # the QJL estimate is unbiased, the MSE-only one is biased towards zero (shrinkage)
    slope_mse = np.sum(base * exact) / np.sum(exact * exact)
    slope_qjl = np.sum(O.scores(q, r, s, c, S) * exact) / np.sum(exact * exact)
    assert slope_mse < 0.93 and abs(slope_qjl - 1.0) < 0.02
    assert e_qjl < 4 * e_mse  # the correction adds variance but stays the same order


def test_qjl_estimator_unbiased_and_variance_closed_form():
    """[AB] §2 / [SI] abstract: for Gaussian S the 1-bit estimate of <q,e> is unbiased, with variance
    ((pi/2)||q||²||e||² - <q,e>²)/m.  T independent seeds; z-test on the mean, chi2 on the variance."""
    d, m, T = 16, 24, 6000                     # m != d so a transposed S would fail the shapes
    rng = np.random.default_rng(42)
    q = rng.standard_normal(d)
    e = rng.standard_normal(d) * 0.1 + 0.05 * q
    est = np.array([O.qjl_estimate(q, e, O.gaussian_matrix(1000 + k, 0, m, d)) for k in range(T)])
    truth = float(q @ e)
    var = (math.pi / 2 * (q @ q) * (e @ e) - truth ** 2) / m
    z = (est.mean() - truth) / math.sqrt(var / T)
    assert abs(z) < 4.0, z
    chi = (T - 1) * est.var(ddof=1) / var
    lo, hi = stats.chi2.ppf([1e-4, 1 - 1e-4], T - 1)
    assert lo < chi < hi


def test_attention_rotated_equals_dense():
    d, b, m = 64, 4, 64
    t, c = O.lloyd_max(d, b)
    sk, sv = O.head_signs(4001, 2, d), O.head_signs(4002, 2, d)
    S = O.gaussian_matrix(4001, 2, m, d)
    rng = np.random.default_rng(4)
    K, V, Q = rng.standard_normal((500, d)), rng.standard_normal((500, d)), rng.standard_normal((4, d))
    rk, rv = O.encode(K, sk, t, c, S), O.encode(V, sv, t, c)
    sc = O.scores(Q, rk, sk, c, S)
    dense = O.attention_dense(sc, O.decode(rv["idx"], rv["n16"], sv, c), 1 / math.sqrt(d))
    rot = O.attention_rotated(sc, rv, sv, c, 1 / math.sqrt(d))
    assert np.max(np.abs(dense - rot)) < 1e-12 * np.max(np.abs(dense))
    # softmax normalises over tokens: weights sum to one per query
    w = O.softmax(sc / math.sqrt(d))
    assert np.allclose(w.sum(axis=1), 1.0)


def test_kl_matches_library_entropy():
    rng = np.random.default_rng(9)
    p = rng.dirichlet(np.ones(50), size=3)
    q = rng.dirichlet(np.ones(50), size=3)
    assert np.allclose(O.kl_divergence(p, q), [stats.entropy(a, b) for a, b in zip(p, q)], rtol=1e-12)
    assert np.all(O.kl_divergence(p, p) == 0)


def test_bf16_bits_exact():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, -65504.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)     # these values are exact in bf16 or truncate
    back = O.bf16_bits_to_f64(bits)
    assert np.array_equal(back, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    assert back[0] == 1.0 and back[1] == -2.5

"""Pins of the SpectralQuant oracle (CPU only): the Gaussian Lloyd-Max codebook against Max's
table and closed forms, calibration against the pages' statements (participation ratio, spectral
gap, water-filling, storage), and the codec against the Gaussian rate-distortion of its own
allocation.  Pages: "Ablation, Statistical Inference, and Validation for KV-Cache Compression",
§2 "SpectralQuant", §3.2, §6, §7."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import sq_oracle as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _max_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "gaussian_lloyd_max_max1960.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        rows[(int(f[0]), f[1])] = [float(v) for v in f[2:]]
    return rows


def test_gauss_codebook_matches_max_1960_table():
    for (levels, kind), vals in _max_table().items():
        t, c = Q.gauss_lloyd_max(int(math.log2(levels)))
        ours = (t if kind == "thr" else c)[len(t if kind == "thr" else c) // 2:]
        if kind == "thr":
            ours = ours[1:]                           # the table lists the positive thresholds
        assert len(ours) == len(vals)
        for o, v in zip(ours, vals):
            # one unit of the table's 4th significant digit (its last digit is not always rounded
            # correctly: 0.50055 is printed as 0.5006)
            unit = 10.0 ** (math.floor(math.log10(abs(v))) - 3)
            assert abs(o - v) <= unit, (levels, kind, o, v)


def test_gauss_codebook_closed_forms_and_conditions():
    t, c = Q.gauss_lloyd_max(1)
    assert np.array_equal(t, [0.0]) and np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-15)
    assert abs(Q.gauss_codebook_mse(1) - (1 - 2 / math.pi)) < 1e-14
    prev = np.inf
    for b in range(2, 9):
        t, c = Q.gauss_lloyd_max(b)
        assert np.all(np.diff(c) > 0) and np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0, rtol=0)
        assert np.allclose(c, -c[::-1], atol=1e-15)
        edges = np.concatenate(([-np.inf], t, [np.inf]))
        if b <= 4:   # centroid condition and the distortion by independent quadrature
            mean = [integrate.quad(lambda x: x * stats.norm.pdf(x), edges[i], edges[i + 1])[0]
                    / (stats.norm.cdf(edges[i + 1]) - stats.norm.cdf(edges[i])) for i in range(len(c))]
            assert np.max(np.abs(np.array(mean) - c)) < 1e-10
            mse = sum(integrate.quad(lambda x, ci=ci: (x - ci) ** 2 * stats.norm.pdf(x), edges[i], edges[i + 1],
                                     epsabs=1e-14)[0] for i, ci in enumerate(c))
            assert abs(mse - Q.gauss_codebook_mse(b)) < 1e-10
        d_b = Q.gauss_codebook_mse(b)
        assert d_b < prev
        prev = d_b
    # high-rate limit (Panter-Dite): D(b) -> (sqrt(3) pi / 2) 4^-b
    assert abs(Q.gauss_codebook_mse(8) / (math.sqrt(3) * math.pi / 2 * 4.0 ** -8) - 1) < 0.02


def test_participation_ratio_closed_forms():
    for r in (1, 4, 8, 100):
        assert Q.participation_ratio(np.concatenate((np.ones(r), np.zeros(128 - r)))) == r
    lam = 0.5 ** np.arange(128)                      # (Σ 2^-k)² / Σ 4^-k -> 4 / (4/3) = 3
    assert Q.participation_ratio(lam) == 3


def test_gap_criterion_trims_a_spurious_dimension_and_the_cap_applies():
    # [AB] §7: a ninth eigenvalue ~200x below the eighth lifts the participation ratio to 9; the gap
    # criterion (gamma = 10) trims it back to the 8 signal dimensions.
    lam = np.concatenate((np.linspace(1.0, 0.8, 8), [0.005], np.full(119, 0.004)))
    assert Q.participation_ratio(lam) == 9
    assert Q.effective_dim(lam, gamma=10.0) == 8
    assert Q.effective_dim(lam, gamma=0.0) == 9
    assert Q.effective_dim(lam, gamma=10.0, d_eff_max=4) == 4
    # [AB] §7: the exponentially decaying rank-4 spectrum (ratio 8) gives a participation ratio of 3
    # (15²/85 = 2.65); a cap of 4 cannot raise it, the cap only trims
    steep = np.concatenate(([8.0, 4.0, 2.0, 1.0], np.full(124, 1e-4)))
    assert Q.participation_ratio(steep) == 3
    assert Q.effective_dim(steep, gamma=10.0, d_eff_max=4) == 3


def test_block_power_iteration_finds_the_top_eigenvectors():
    rng = np.random.default_rng(4)
    d, k = 64, 6
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.concatenate((np.linspace(5, 3, k), np.linspace(0.5, 0.01, d - k)))
    C = (V * lam) @ V.T
    w, U = Q.block_power_iteration(C, k, seed=1)
    we, Ue = Q.eigenbasis(C)
    assert np.allclose(w, lam[:k], rtol=1e-10)
    assert np.allclose(w, we[:k], rtol=1e-10)
    assert np.allclose(U, Ue[:, :k], atol=1e-8)          # both canonically signed
    assert np.allclose(Ue.T @ Ue, np.eye(d), atol=1e-12)
    assert np.allclose(C @ Ue, Ue * we, atol=1e-10)
    piv = np.argmax(np.abs(Ue), axis=0)
    assert np.all(Ue[piv, np.arange(d)] > 0)


def _best_allocation(lam, total, b_tail, b_max=8):
    best = None
    def rec(k, left, cur):
        nonlocal best
        if k == len(lam):
            if left == 0:
                val = sum(l * 4.0 ** -b for l, b in zip(lam, cur))
                if best is None or val < best[0] - 1e-15:
                    best = (val, list(cur))
            return
        for b in range(b_tail, b_max + 1):
            if b <= left:
                rec(k + 1, left - b, cur + [b])
    rec(0, total, [])
    return best


def test_waterfill_is_uniform_at_ratio_at_most_4_and_optimal_otherwise():
    rng = np.random.default_rng(7)
    for trial in range(200):
        k = int(rng.integers(1, 9))
        lam = rng.uniform(1.0, 4.0, k)
        lam[0] = 4.0 if trial % 2 else lam[0]            # include the ratio-exactly-4 boundary
        lam[-1] = 1.0
        b = int(rng.integers(2, 7))
        assert np.array_equal(Q.waterfill(lam, b * k, 2), np.full(k, b)), (lam, b)
    # the lowrank_steep regime: ratio 8 within d_eff = 4, water-filling does activate
    lam = np.array([8.0, 4.0, 2.0, 1.0])
    for b in (3, 4, 5):
        bits = Q.waterfill(lam, 4 * b, 2)
        assert bits.sum() == 4 * b and not np.all(bits == b)
        val = float(np.sum(lam * 4.0 ** -bits))
        assert abs(val - _best_allocation(list(lam), 4 * b, 2)[0]) < 1e-15
    for trial in range(30):
        lam = np.sort(rng.exponential(1.0, 4) * 50)[::-1]
        bits = Q.waterfill(lam, 16, 2)
        assert abs(float(np.sum(lam * 4.0 ** -bits)) - _best_allocation(list(lam), 16, 2)[0]) < 1e-12


def test_storage_bits_match_the_pages():
    for line in open(os.path.join(GOLDEN, "sq_storage_bits.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, d_eff, b_sem, b_tail, sq_bits, tq_bits = map(int, line.split())
        assert Q.storage_bits(d, d_eff, b_sem, b_tail) == sq_bits
        assert b_sem * d == tq_bits
    # a calibrated model on rank-8 data carries exactly those bits
    rng = np.random.default_rng(2)
    V, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    x = (rng.standard_normal((4096, 8)) * np.linspace(1.0, 0.8, 8)) @ V[:, :8].T
    x += 0.03 * rng.standard_normal(x.shape)
    for b in (2, 3):
        m = Q.calibrate(x, b, 2)
        assert m["d_eff"] == 8 and int(m["bits"].sum()) == Q.storage_bits(128, 8, b, 2)
        assert Q.record_bytes([m["bits"]]) == 4 * ((int(m["bits"].sum()) + 31) // 32)


def _gaussian_data(rng, lam, n):
    d = len(lam)
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return (rng.standard_normal((n, d)) * np.sqrt(lam)) @ V.T


@pytest.mark.parametrize("water", [False, True])
def test_codec_distortion_is_the_gaussian_rate_distortion_of_its_allocation(water):
    # For x ~ N(0, C) calibrated on many tokens, z_k ~ N(0, λ_k) and E‖x - x̂‖² = Σ_k λ_k D(b_k).
    rng = np.random.default_rng(11)
    d = 64
    lam = np.concatenate((8.0 * 0.7 ** np.arange(6), np.full(d - 6, 0.05)))
    x = _gaussian_data(rng, lam, 60000)
    m = Q.calibrate(x[:40000], 4, 2, water=water, gamma=0.0, d_eff_max=6)
    assert m["d_eff"] == 6
    test = x[40000:]
    r = Q.encode(test, m)
    xh = Q.decode(r["idx"], m)
    mse = float(np.mean(np.sum((xh - test) ** 2, axis=1)))
    model = sum(m["lam"][k] * Q.gauss_codebook_mse(int(m["bits"][k])) for k in range(d))
    assert abs(mse / model - 1) < 0.03, (mse, model)


def test_index_is_the_nearest_centroid_and_records_round_trip():
    rng = np.random.default_rng(5)
    d = 64
    x = _gaussian_data(rng, np.linspace(3, 0.1, d), 3000)
    m = Q.calibrate(x[:2000], 3, 1, water=True, gamma=0.0)
    r = Q.encode(x[2000:], m)
    for k in range(d):
        _, c = Q.gauss_lloyd_max(int(m["bits"][k]))
        nearest = np.argmin(np.abs(r["u"][:, k, None] - c[None, :]), axis=1)
        assert np.array_equal(nearest, r["idx"][:, k])
    rb = Q.record_bytes([m["bits"]])
    rec = Q.pack(r["idx"], m["bits"], rb)
    assert rec.shape == (1000, rb)
    assert np.array_equal(Q.unpack(rec, m["bits"]), r["idx"])
    # closed form: fields 5 (3 bits), 2 (2 bits), 1 (1 bit) -> 0b1_10_101 = 0x35
    assert Q.pack(np.array([[5, 2, 1]]), np.array([3, 2, 1]), 4).tolist() == [[0x35, 0, 0, 0]]


def test_scores_and_attention_equal_the_dense_products_of_the_decoded_cache():
    rng = np.random.default_rng(6)
    d = 64
    k = _gaussian_data(rng, np.linspace(2, 0.2, d), 700)
    v = _gaussian_data(rng, np.linspace(1, 0.5, d), 700)
    mk, mv = Q.calibrate(k[:500], 4, 2), Q.calibrate(v[:500], 3, 2)
    rk, rv = Q.encode(k[500:], mk), Q.encode(v[500:], mv)
    q = rng.standard_normal((5, d))
    kh, vh = Q.decode(rk["idx"], mk), Q.decode(rv["idx"], mv)
    sc = Q.scores(q, rk["idx"], mk)
    assert np.allclose(sc, q @ kh.T, rtol=1e-12, atol=1e-12)
    out = Q.attention(sc, rv["idx"], mv, 0.125)
    s = sc * 0.125
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(out, p @ vh, rtol=1e-12, atol=1e-12)


def test_scores_use_the_stored_tail():
    """Reading of the printed estimator <q_Z, z_k>, which sums the semantic dimensions only: the
    record stores the tail too (§3.2: 8 bits on 4 semantic dimensions plus 2 bits on the other 124
    make 280 bits per token, tests/golden/sq_storage_bits.txt), and eq. (1) runs on the
    reconstructed K, so the score takes every stored dimension: exactly <q, K̂>.  Dropping the tail
    leaves out <q_tail, ẑ_tail>, which is an unbiased part of <q, k> the record does hold: here the
    semantic-only form errs several times more against the exact q.k."""
    rng = np.random.default_rng(16)
    d = 64
    spec = np.concatenate([np.full(4, 4.0), np.full(d - 4, 0.3)])   # 4 strong dimensions, a real tail
    k = _gaussian_data(rng, spec, 4500)
    mk = Q.calibrate(k[:500], 4, 2)
    de = mk["d_eff"]
    assert 0 < de < d and np.all(mk["bits"][de:] == 2)
    rk = Q.encode(k[500:], mk)
    q = rng.standard_normal((8, d))
    full = Q.scores(q, rk["idx"], mk)
    z_hat = Q.dequantise(rk["idx"], mk)
    qz = q @ mk["U"]
    semantic = qz[:, :de] @ z_hat[:, :de].T
    tail = qz[:, de:] @ z_hat[:, de:].T
    assert np.allclose(full, semantic + tail, rtol=1e-12, atol=1e-12)
    assert np.allclose(full, q @ Q.decode(rk["idx"], mk).T, rtol=1e-12, atol=1e-12)
    exact = q @ k[500:].T
    e_full = np.mean((full - exact) ** 2)
    e_sem = np.mean((semantic - exact) ** 2)
    assert e_sem > 5 * e_full, (e_sem, e_full)


def test_covariance_is_not_centred():
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert np.allclose(Q.covariance(x), np.array([[5.0, 7.0], [7.0, 10.0]]))


def test_index_counts_thresholds_with_ties_to_the_upper_cell():
    d = 8
    for b in (1, 2, 3, 8):
        t, _ = Q.gauss_lloyd_max(b)
        model = {"U": np.eye(d), "sigma": np.full(d, 2.0), "bits": np.full(d, b)}
        sel = t[np.linspace(0, len(t) - 1, d).astype(int)]
        for x, want in ((2.0 * sel, None), (2.0 * sel - 1e-9 * (1.0 + np.abs(sel)), -1)):
            idx = Q.encode(x[None, :], model)["idx"][0]
            expect = np.array([np.sum(t <= v / 2.0) for v in x])
            assert np.array_equal(idx, expect)
            pos = np.searchsorted(t, sel)
            assert np.array_equal(idx, pos + 1 if want is None else pos)


# ---- the selective QJL sketch (SQU-QKV) --------------------------------------------------------

def _sq_model_with_sketch(d=64, d_eff=16, m=32, seed=5, head=1, rng_seed=3):
    rng = np.random.default_rng(rng_seed)
    lam = np.concatenate((np.linspace(3.2, 2.8, d_eff), np.full(d - d_eff, 0.05)))
    x = _gaussian_data(rng, lam, 3000)
    model = Q.calibrate(x[:2000], 3, 2, gamma=0.0, d_eff_max=d_eff)
    assert model["d_eff"] == d_eff
    return Q.with_sketch(model, m, seed, head), x[2000:]


def test_sketch_matrix_definition():
    from oracle import tq_oracle as O
    S = Q.sketch_matrix(77, 3, 16, 64)
    assert S.shape == (16, 64) and set(np.unique(S)) == {-1.0, 1.0}
    w = O.words(O.stream_key(77, 4, 3), 16 * 64)
    assert S[2, 5] == (-1.0 if int(w[2 * 64 + 5]) >> 63 else 1.0)
    assert abs(S.mean()) < 0.1
    assert not np.array_equal(S[0], O.head_signs(77, 3, 64))       # a different tag
    model, _ = _sq_model_with_sketch()
    assert np.array_equal(model["S"], Q.sketch_matrix(5, 1, 32, 64)[:, :16])


def test_sketch_bits_and_norm_written_out():
    model, x = _sq_model_with_sketch()
    r = Q.encode(x[:5], model)
    zh = Q.dequantise(r["idx"], model)
    for t in range(5):
        e = [r["z"][t, k] - zh[t, k] for k in range(16)]
        for i in range(32):
            zi = sum(model["S"][i, k] * e[k] for k in range(16))
            assert r["sigma_bits"][t, i] == (1 if zi >= 0 else 0)
        assert r["r16"][t] == np.float16(math.sqrt(sum(v * v for v in e)))


def test_selective_qjl_estimate_is_close_to_unbiased():
    # over random ±1 sketches the correction estimates <q_Z, e_z> on the semantic dimensions (exactly
    # so for Gaussian sketches; a ±1 sketch on 32 dimensions is within a few per cent)
    model, x = _sq_model_with_sketch(d_eff=32, m=64)
    q = np.random.default_rng(8).standard_normal((1, 64))
    r0 = Q.encode(x[:1], model)
    target = float((q @ model["U"])[0, :32] @ r0["e"][0])
    nosk = {k: v for k, v in model.items() if k not in ("m", "S")}
    base = Q.scores(q, r0["idx"], nosk)[0, 0]
    est = []
    for seed in range(20000):
        ms = Q.with_sketch(model, 64, 1000 + seed, 0)
        sk = Q.sketch_of(r0["z"], r0["idx"], ms)
        est.append(Q.scores(q, r0["idx"], ms, sk["sigma_bits"], sk["r16"])[0, 0] - base)
    est = np.array(est)
    se = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - target) < 3 * se + 0.03 * abs(target), (est.mean(), target, se)


def test_sketch_records_round_trip_and_m0_is_unchanged():
    model, x = _sq_model_with_sketch()
    r = Q.encode(x[:40], model)
    rb = Q.record_bytes([model["bits"]], 32)
    assert rb == 4 * ((int(model["bits"].sum()) + 32 + 16 + 31) // 32)
    rec = Q.pack(r["idx"], model["bits"], rb, r["sigma_bits"], r["r16"])
    idx, sig, r16 = Q.unpack(rec, model["bits"], 32)
    assert np.array_equal(idx, r["idx"]) and np.array_equal(sig, r["sigma_bits"]) and np.array_equal(r16, r["r16"])
    plain = dict(model)
    plain["m"] = 0
    assert np.array_equal(Q.scores(x[:3], r["idx"], plain), Q.scores(x[:3], r["idx"], {k: v for k, v in model.items() if k not in ("m", "S")}))

"""Pins of the oracle's Plain-KV scheme (rotation = none): the Beta codebook applied to the
normalised vector itself ([AB] §4 "Surviving schemes": Plain-KV applies the Beta codebook without
WHT; comparable to TQ-KV where the Beta marginals hold, worse where channels are unequal). CPU only."""
import numpy as np

from oracle import tq_oracle as O


def test_plain_encode_is_the_codebook_on_the_unit_vector():
    d, b = 128, 3
    t, c = O.lloyd_max(d, b)
    x = np.random.default_rng(3).standard_normal((300, d))
    r = O.encode(x, None, t, c)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    assert np.array_equal(r["y"], u)
    # the index is the count of thresholds at or below each coordinate, written out directly
    idx = (u[:, :, None] >= t[None, None, :]).sum(axis=2)
    assert np.array_equal(r["idx"], idx)
    x_hat = O.decode(r["idx"], r["n16"], None, c)
    assert np.allclose(x_hat, r["n16"].astype(np.float64)[:, None] * c[idx], rtol=0, atol=0)


def test_plain_matches_tq_on_isotropic_vectors_and_loses_on_unequal_channels():
    d, b = 128, 3
    t, c = O.lloyd_max(d, b)
    s = O.head_signs(5, 0, d)
    rng = np.random.default_rng(9)
    iso = rng.standard_normal((3000, d))

    def err(x, signs):
        r = O.encode(x, signs, t, c)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        return float(np.mean(np.sum((O.decode(r["idx"], np.ones(len(x)), signs, c) - u) ** 2, axis=1)))

    e_plain, e_tq = err(iso, None), err(iso, s)
    assert abs(e_plain / e_tq - 1.0) < 0.05, (e_plain, e_tq)        # Beta marginals hold either way
    aniso = iso.copy()
    aniso[:, :4] *= 10.0                                            # four outlier channels
    assert err(aniso, None) > 2.0 * err(aniso, s)                   # the rotation spreads them


def test_plain_scores_and_attention_need_no_rotation():
    d, b = 64, 4
    t, c = O.lloyd_max(d, b)
    rng = np.random.default_rng(1)
    k, v, q = rng.standard_normal((200, d)), rng.standard_normal((200, d)), rng.standard_normal((3, d))
    rk, rv = O.encode(k, None, t, c), O.encode(v, None, t, c)
    k_hat, v_hat = O.decode(rk["idx"], rk["n16"], None, c), O.decode(rv["idx"], rv["n16"], None, c)
    sc = O.scores(q, rk, None, c)
    assert np.allclose(sc, q @ k_hat.T, rtol=1e-12, atol=1e-12)
    out = O.attention_rotated(sc, rv, None, c, 0.125)
    assert np.allclose(out, O.attention_dense(sc, v_hat, 0.125), rtol=1e-12, atol=1e-12)

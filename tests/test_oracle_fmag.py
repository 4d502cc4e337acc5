"""Pins of the Fmag oracle (CPU only): the transform against a written-out DFT and the real
synthesis formula, a single cosine in closed form, the min-max and phase quantisers' exact points
and error bounds, Parseval for the scores, and the record layout.  Page: "Fourier Magnitude KV Cache
Quantization" (forum thread), "Method"."""
import math

import numpy as np
import pytest

from oracle import fmag_oracle as F


def _dft(x):
    d = x.shape[-1]
    j = np.arange(d)
    return np.stack([np.sum(x * np.exp(-2j * math.pi * j * k / d), axis=-1) for k in range(d // 2 + 1)], axis=-1)


def _synth(X, d):
    j = np.arange(d)
    out = X[..., :1].real / d + ((-1.0) ** j) * X[..., d // 2:d // 2 + 1].real / d
    for k in range(1, d // 2):
        out = out + 2.0 / d * np.real(X[..., k:k + 1] * np.exp(2j * math.pi * j * k / d))
    return out


@pytest.mark.parametrize("d", [8, 16, 64])
def test_transform_is_the_written_out_dft_and_its_real_inverse(d):
    x = np.random.default_rng(d).standard_normal((7, d))
    X = F.rfft(x)
    assert np.allclose(X, _dft(x), atol=1e-12)
    Y = X + 0.3 * np.random.default_rng(1).standard_normal(X.shape) * (1 + 1j)
    Y[:, 0] = Y[:, 0].real
    Y[:, -1] = Y[:, -1].real
    assert np.allclose(F.irfft(Y, d), _synth(Y, d), atol=1e-12)


@pytest.mark.parametrize("p", [6, 8, 16])
def test_single_cosine_closed_form(p):
    d, b, k0, A, theta = 128, 4, 5, 1.7, 0.9
    j = np.arange(d)
    x = (A * np.cos(2 * math.pi * k0 * j / d + theta))[None, :]
    r = F.encode(x, b, p)
    assert abs(r["hi"][0] - A * d / 2) < 1e-10 and r["lo"][0] < 1e-10
    assert r["q"][0, k0] == 15 and np.all(np.delete(r["q"][0], k0) == 0)
    if p == F.PHASE_BF16:
        th = F.bf16_round(np.array([theta]))[0]
    else:
        step = 2 * math.pi / (1 << p)
        th = math.floor((theta + math.pi) / step + 0.5) * step - math.pi
    want = A * np.cos(2 * math.pi * k0 * j / d + th)
    assert np.allclose(F.decode(r, b, p, d)[0], want, atol=1e-9)


def test_min_max_quantiser_exact_points_and_bound():
    x = np.random.default_rng(3).standard_normal((50, 64))
    for b in (2, 3, 4):
        r = F.encode(x, b, 8)
        L = (1 << b) - 1
        mag_q = r["lo"][:, None] + r["q"] * (r["hi"] - r["lo"])[:, None] / L
        i_max, i_min = np.argmax(r["mag"], axis=1), np.argmin(r["mag"], axis=1)
        rows = np.arange(50)
        assert np.allclose(mag_q[rows, i_max], r["hi"], rtol=1e-15)
        assert np.allclose(mag_q[rows, i_min], r["lo"], rtol=1e-15)
        assert np.all(np.abs(mag_q - r["mag"]) <= (r["hi"] - r["lo"])[:, None] / (2 * L) * (1 + 1e-12))
        assert np.all((r["q"] >= 0) & (r["q"] <= L))


@pytest.mark.parametrize("p", [6, 8])
def test_phase_levels_and_bound(p):
    P = 1 << p
    step = 2 * math.pi / P
    x = np.random.default_rng(4).standard_normal((40, 64))
    r = F.encode(x, 4, p)
    ph_q = F.phase_values(r, p)
    err = np.angle(np.exp(1j * (ph_q - r["phase"])))
    assert np.all(np.abs(err) <= step / 2 * (1 + 1e-9))
    # real bins: DC of a positive-mean vector sits on the 0 level, a negative one on -π
    pos = F.encode(np.full((1, 16), 2.0), 4, p)
    neg = F.encode(np.full((1, 16), -2.0), 4, p)
    assert pos["pidx"][0, 0] == P // 2 and neg["pidx"][0, 0] == 0
    assert F.phase_values(pos, p)[0, 0] == 0.0
    # off-level phases go to the nearer level: a quarter step above level 5 -> 5, three quarters -> 6
    k0, d = 3, 32
    j = np.arange(d)
    for frac, want in ((0.25, 5), (0.75, 6)):
        ph = -math.pi + (5 + frac) * step
        r2 = F.encode(np.cos(2 * math.pi * k0 * j / d + ph)[None, :], 4, p)
        assert r2["pidx"][0, k0] == want


def test_bf16_phase_rounding():
    assert F.bf16_round(np.array([math.pi]))[0] == 3.140625
    assert F.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0          # tie to even
    assert F.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    x = np.random.default_rng(5).standard_normal((10, 64))
    r = F.encode(x, 4, F.PHASE_BF16)
    assert np.all(np.abs(r["pbf"] - r["phase"]) <= np.abs(r["phase"]) * 2 ** -8 + 1e-300)


def test_reconstruction_error_is_parseval_of_the_spectrum_error():
    d = 128
    x = np.random.default_rng(6).standard_normal((20, d))
    r = F.encode(x, 3, 6)
    Xq = F.spectrum(r, 3, 6)
    w = np.full(d // 2 + 1, 2.0)
    w[0] = w[-1] = 1.0
    lhs = np.sum((F.decode(r, 3, 6, d) - x) ** 2, axis=1)
    rhs = np.sum(w * np.abs(Xq - r["X"]) ** 2, axis=1) / d
    assert np.allclose(lhs, rhs, rtol=1e-10)


def test_scores_equal_the_frequency_domain_sum():
    d = 64
    rng = np.random.default_rng(7)
    x, q = rng.standard_normal((30, d)), rng.standard_normal((4, d))
    r = F.encode(x, 4, 8)
    Q, Xq = F.rfft(q), F.spectrum(r, 4, 8)
    w = np.full(d // 2 + 1, 2.0)
    w[0] = w[-1] = 1.0
    freq = (Q.real * w) @ Xq.real.T / d + (Q.imag * w) @ Xq.imag.T / d
    assert np.allclose(F.scores(q, r, 4, 8, d), freq, atol=1e-10)
    out = F.attention(F.scores(q, r, 4, 8, d), r, 4, 8, d, 0.125)
    assert out.shape == (4, d)


@pytest.mark.parametrize("b,p", [(4, 8), (3, 6), (2, 16), (4, 16)])
def test_record_round_trip_and_layout(b, p):
    d = 64
    x = np.random.default_rng(8).standard_normal((9, d))
    r = F.encode(x, b, p)
    w = F.pack(r, b, p, d)
    assert w.shape == (9, F.record_words(d, b, p))
    u = F.unpack(w, b, p, d)
    assert np.array_equal(u["q"], r["q"])
    assert np.array_equal(u["lo"], r["lo"].astype(np.float32).astype(np.float64))
    if p == F.PHASE_BF16:
        assert np.array_equal(u["pbf"], r["pbf"])
    else:
        assert np.array_equal(u["pidx"], r["pidx"])
    # the first field is the DC magnitude index, LSB first
    assert (w[:, 0] & ((1 << b) - 1)).tolist() == r["q"][:, 0].tolist()


@pytest.mark.parametrize("b,p", [(4, 8), (3, 16)])
def test_attention_pins(b, p):
    """softmax(scale·ŝ) @ x̂ ("Method": attention runs on the reconstructed cache): a single token
    returns its reconstruction; equal scores give the mean; one dominant score gives its token; and
    by linearity of the inverse FFT the result equals irfft of the weighted spectra."""
    d = 64
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, d))
    r = F.encode(x, b, p)
    xh = F.decode(r, b, p, d)
    one = {k: (v[:1] if isinstance(v, np.ndarray) and v.shape[:1] == (40,) else v) for k, v in r.items()}
    assert np.allclose(F.attention(np.array([[3.7]]), one, b, p, d, 0.125), xh[:1], rtol=0, atol=1e-12)
    assert np.allclose(F.attention(np.zeros((2, 40)), r, b, p, d, 1.0), np.tile(xh.mean(axis=0), (2, 1)),
                       rtol=0, atol=1e-12)
    s = np.zeros((1, 40))
    s[0, 17] = 1e4
    assert np.allclose(F.attention(s, r, b, p, d, 1.0)[0], xh[17], rtol=0, atol=1e-12)
    sc = rng.standard_normal((3, 40)) * 4
    w = np.exp(0.5 * sc - (0.5 * sc).max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    freq = np.fft.irfft(w @ F.spectrum(r, b, p), n=d)
    assert np.allclose(F.attention(sc, r, b, p, d, 0.5), freq, rtol=0, atol=1e-12)

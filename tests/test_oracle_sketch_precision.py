"""Pins of the sketch's half-precision residual (oracle/tq_oracle.py ``sketch_input``, ``sketch``).

The projection takes ê = fp16(2^14 e)/2^14, round to nearest with ties to even: the IEEE 754
binary16 format (1 sign, 5 exponent, 10 fraction bits, subnormal spacing 2^-24).  The expected
values below are written out from that format, not computed by the oracle's own routine; the
flag band is checked by brute force against every perturbation of the residual within the
tolerance.  Page: "Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2
"TurboQuant" (the 1-bit sketch of the WHT-domain residual)."""
import numpy as np

from oracle import tq_oracle as O

K = 2.0 ** -14          # one unit of the scaled residual


def test_half_precision_residual_written_out():
    # (2^14 e, 2^14 ê)
    cases = [
        (1 + 2 ** -11, 1.0),                         # tie between 1 (even) and 1 + 2^-10 (odd)
        (1 + 3 * 2 ** -11, 1 + 2 ** -9),             # tie between 1 + 2^-10 (odd) and 1 + 2^-9 (even)
        (-(1 + 2 ** -11 + 2 ** -20), -(1 + 2 ** -10)),   # just past the tie: away from 1
        (3.0, 3.0),                                  # representable: unchanged
        (1000.3, 1000.5),                            # spacing 1/2 in [512, 1024)
        (2047.5, 2048.0),                            # spacing 1 in [1024, 2048): tie to even 2048
        (16383.9, 16384.0),                          # spacing 8 in [8192, 16384)
        (2 ** -25, 0.0),                             # half the least subnormal: tie to even 0
        (3 * 2 ** -25, 2 ** -23),                    # tie between 2^-24 (odd) and 2^-23 (even)
        (1.4 * 2 ** -24, 2 ** -24),
        (0.0, 0.0),
    ]
    e = np.array([c[0] for c in cases]) * K
    want = np.array([c[1] for c in cases]) * K
    assert np.array_equal(O.sketch_input(e), want)


def test_sketch_of_a_small_case_written_out():
    S = np.array([[1.0, -2.0, 0.5], [0.0, 1.0, 1.0], [0.0, 0.0, 0.0]])
    e = np.array([[1 + 2 ** -11, 3.0, 1 + 3 * 2 ** -11]]) * K
    r = O.sketch(e, S)
    # ê = (1, 3, 1 + 2^-9) 2^-14
    assert np.array_equal(r["z"], np.array([[-4.5 + 2 ** -10, 4 + 2 ** -9, 0.0]]) * K)
    assert r["sigma"].tolist() == [[False, True, True]]                   # sign(0) = +1
    # coordinates 0 and 2 sit on rounding midpoints (step 2^-10 each), coordinate 1 is representable:
    # band_i = 1e-6 + (|S_i0| + |S_i2|) 2^-10 2^-14
    band = 1e-6 + np.array([1 * 2 ** -10 + 0.5 * 2 ** -10, 1 * 2 ** -10, 0.0]) * K
    assert r["sflag"].tolist() == [list(np.abs(r["z"][0]) < band)]


def test_flag_band_covers_every_perturbation_within_the_tolerance():
    d, b, m = 128, 3, 64
    t, c = O.lloyd_max(d, b)
    s, S = O.head_signs(3, 0, d), O.gaussian_matrix(3, 0, m, d).astype(np.float64)
    x = np.random.default_rng(7).standard_normal((600, d))
    r = O.encode(x, s, t, c, S)
    e = r["e"]
    tol = O.FLAG_TOL
    rng = np.random.default_rng(8)
    v = e / K
    h = v.astype(np.float16)
    hv = h.astype(np.float64)
    lo = np.where(hv <= v, hv, np.nextafter(h, np.float16(-np.inf)).astype(np.float64))
    hi = np.where(hv >= v, hv, np.nextafter(h, np.float16(np.inf)).astype(np.float64))
    mid = 0.5 * (lo + hi)
    flips = 0
    for trial in range(12):
        if trial % 2 == 0:
            ep = e + rng.uniform(-tol, tol, e.shape) * 0.999
        else:   # push every coordinate within reach of its midpoint to the other side
            cross = np.abs(v - mid) < tol / K * 0.999
            vp = np.where(cross, mid - np.sign(v - mid) * 1e-9, v)
            ep = vp * K
        assert np.all(np.abs(ep - e) <= tol)
        sp = O.sketch(ep, S)["sigma"]
        changed = sp != r["sigma"]
        assert not (changed & ~r["sflag"]).any()
        flips += int(changed.sum())
    assert flips > 0                       # the perturbations do reach flagged decisions
    assert r["sflag"].mean() < 2e-3        # and the band stays narrow


def test_sketch_bits_differ_from_the_exact_residual_only_near_zero():
    d, b, m = 128, 4, 128
    t, c = O.lloyd_max(d, b)
    s, S = O.head_signs(4, 1, d), O.gaussian_matrix(4, 1, m, d).astype(np.float64)
    r = O.encode(np.random.default_rng(9).standard_normal((500, d)), s, t, c, S)
    z_exact = r["e"] @ S.T
    # |ê - e| <= 2^-11 |e| coordinate-wise, so the two projections differ by at most 2^-11 Σ|S||e|
    bound = 2.0 ** -11 * (np.abs(r["e"]) @ np.abs(S).T)
    assert np.all(np.abs(r["z"] - z_exact) <= bound)
    assert not ((z_exact >= 0) != r["sigma"])[np.abs(z_exact) > bound].any()

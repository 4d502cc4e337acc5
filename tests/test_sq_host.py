"""SpectralQuant host side, no GPU: the library's Gaussian codebooks and calibration (covariance,
eigenbasis, effective dimension, bit allocation) against the oracle, and argument validation
before any device call.  Pages: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", §2 "SpectralQuant", §6, §7."""
import ctypes
import os

import numpy as np
import pytest

from oracle import sq_oracle as Q
from synth import inputs as I

T = pytest.importorskip("kv_cache_transform_amd")
from kv_cache_transform_amd import _lib  # noqa: E402


def _lib_or_fail():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtq.so is not built (run python -m kv_cache_transform_amd.build)")
    return _lib.lib()


@pytest.mark.parametrize("b", range(1, 9))
def test_host_gaussian_codebook_matches_oracle(b):
    _lib_or_fail()
    h = T.sq_host_codebook(b)
    t, c = Q.gauss_lloyd_max(b)
    # the library finishes with Newton steps, the oracle with plain Lloyd sweeps, whose contraction
    # at 256 levels is slow enough to stop ~4e-11 short of the fixed point; both meet the centroid
    # condition to ~1e-13
    assert np.max(np.abs(h["centroids"] - c)) < 1e-10
    assert np.max(np.abs(h["thresholds"] - t)) < 1e-10


REGIMES = {
    # name: (spectrum, noise, gamma, d_eff_max)
    "lowrank_aligned": ([1.0] * 8, 0.05, 10.0, 0),
    "lowrank_steep": ([1.0, 0.5, 0.25, 0.125], 0.02, 10.0, 4),
    "lowrank_flat": (list(np.linspace(1.0, 0.7, 8)), 0.0, 10.0, 8),
    "isotropic": ([], 1.0, 10.0, 0),
}


def _regime(name, d, n, seed):
    spec, noise, gamma, cap = REGIMES[name]
    if not spec:
        x = I.gaussian((2, n, d), seed, dtype=torch_float32())
    else:
        x = I.low_rank(2, n, d, spec, noise, seed, seed + 1, dtype=torch_float32())
    return x.numpy().astype(np.float32), gamma, cap


def torch_float32():
    import torch
    return torch.float32


@pytest.mark.parametrize("name", list(REGIMES))
@pytest.mark.parametrize("water", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_calibration_matches_oracle(name, water, d):
    _lib_or_fail()
    x, gamma, cap = _regime(name, d, 512, 17)
    got = T.SQCodec.calibrate_host(x, 4, 2, waterfill=water, gamma=gamma, d_eff_max=cap)
    for h in range(x.shape[0]):
        m = Q.calibrate(x[h].astype(np.float64), 4, 2, water=water, gamma=gamma, d_eff_max=cap)
        lam = m["lam"]
        assert np.allclose(got["lam"][h], lam, rtol=1e-9, atol=1e-12 * lam[0])
        assert got["d_eff"][h] == m["d_eff"]
        assert np.array_equal(got["bits"][h], m["bits"])
        # eigenvectors agree where the eigenvalue is separated from its neighbours (an exactly
        # degenerate eigenspace has no unique basis); both are canonically signed
        gap = np.minimum(np.abs(np.diff(lam, prepend=np.inf)), np.abs(np.diff(lam, append=-np.inf)))
        ok = gap > 1e-6 * lam[0]
        assert ok[: m["d_eff"]].all() and ok.sum() >= min(8, d)
        assert np.max(np.abs(got["basis"][h][:, ok] - m["U"][:, ok])) < 1e-7


def test_calibration_regimes_give_the_expected_effective_dimension():
    _lib_or_fail()
    x, _, _ = _regime("lowrank_aligned", 128, 512, 3)
    assert list(T.SQCodec.calibrate_host(x, 3, 2)["d_eff"]) == [8, 8]
    x, _, _ = _regime("lowrank_steep", 128, 512, 3)
    # the participation ratio of the 1 : 1/2 : 1/4 : 1/8 spectrum rounds to 3 ([AB] §7)
    assert list(T.SQCodec.calibrate_host(x, 3, 2, d_eff_max=4)["d_eff"]) == [3, 3]


def test_sq_entry_points_validate_before_any_device_call():
    L = _lib_or_fail()
    P = _lib.SqParams
    x = np.zeros((1, 4, 64), dtype=np.float32)
    out = np.zeros(64 * 64, dtype=np.float64)
    for p in (P(48, 1, 4, 2, 0, 0, 10.0), P(64, 0, 4, 2, 0, 0, 10.0), P(64, 1, 9, 2, 0, 0, 10.0),
              P(64, 1, 2, 3, 0, 0, 10.0), P(64, 1, 4, 0, 0, 0, 10.0), P(64, 1, 4, 2, 0, -1, 10.0)):
        assert L.tq_sq_calibrate(ctypes.byref(p), x.ctypes.data, 4, out.ctypes.data, None, None, None) == _lib.TQ_EINVAL
    p = P(64, 1, 4, 2, 0, 0, 10.0)
    assert L.tq_sq_calibrate(ctypes.byref(p), None, 4, None, None, None, None) == _lib.TQ_EINVAL
    assert L.tq_sq_calibrate(ctypes.byref(p), x.ctypes.data, 0, None, None, None, None) == _lib.TQ_EINVAL
    basis = np.eye(64).ravel()
    lam = np.ones(64)
    h = ctypes.c_void_p()
    for bits in (np.zeros(64, np.int32), np.full(64, 9, np.int32)):
        assert L.tq_sq_create(ctypes.byref(p), basis.ctypes.data, lam.ctypes.data, bits.ctypes.data,
                              None, ctypes.byref(h)) == _lib.TQ_EINVAL
    bad = lam.copy()
    bad[3] = np.nan
    assert L.tq_sq_create(ctypes.byref(p), basis.ctypes.data, bad.ctypes.data, np.full(64, 4, np.int32).ctypes.data,
                          None, ctypes.byref(h)) == _lib.TQ_EINVAL
    p256 = P(256, 1, 4, 2, 0, 0, 10.0)
    assert L.tq_sq_create(ctypes.byref(p256), np.eye(256).ravel().ctypes.data, np.ones(256).ctypes.data,
                          np.full(256, 4, np.int32).ctypes.data, None, ctypes.byref(h)) == _lib.TQ_EINVAL
    # the selective sketch: m in {16, 32, 48, 64}, d_eff given and in 1..d; more than 32 is unsupported
    four = np.full(64, 4, np.int32)
    for m, de, want in ((20, 8, _lib.TQ_EINVAL), (64, None, _lib.TQ_EINVAL), (32, 0, _lib.TQ_EINVAL),
                        (16, 65, _lib.TQ_EINVAL), (64, 33, _lib.TQ_EUNSUPPORTED), (80, 8, _lib.TQ_EINVAL)):
        ps = P(64, 1, 4, 2, 0, 0, 10.0, m, 7)
        dv = None if de is None else np.array([de], np.int32)
        assert L.tq_sq_create(ctypes.byref(ps), basis.ctypes.data, lam.ctypes.data, four.ctypes.data,
                              None if dv is None else dv.ctypes.data, ctypes.byref(h)) == want, (m, de)
    assert h.value is None
    assert L.tq_sq_encode(None, None, _lib.TQ_BF16, 1, 1, None, None) == _lib.TQ_EINVAL
    assert L.tq_sq_decode(None, None, 1, 1, None, _lib.TQ_F32, None) == _lib.TQ_EINVAL
    assert L.tq_sq_host_codebook(0, None, None) == _lib.TQ_EINVAL
    assert L.tq_sq_host_codebook(9, None, None) == _lib.TQ_EINVAL
    rb = ctypes.c_int64()
    assert L.tq_sq_record_bytes(None, ctypes.byref(rb)) == _lib.TQ_EINVAL

"""C-ABI checks that need no GPU: the library loads, exports every symbol include/tq.h declares,
computes the packed layout and host tables exactly like the oracle, and rejects bad arguments
before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import tq_oracle as O
from tests.conftest import ROOT

T = pytest.importorskip("kv_cache_transform_amd")
from kv_cache_transform_amd import _lib  # noqa: E402


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtq.so is not built (run python -m kv_cache_transform_amd.build)")
    return _lib.lib()


def test_exports_every_declared_symbol():
    L = _lib_or_skip()
    declared = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            declared |= set(re.findall(r"\b(tq_[a-z_]+)\s*\(", open(os.path.join(ROOT, "include", h)).read()))
    assert declared == set(_lib.EXPORTS) | set(_lib.SQ_EXPORTS) | set(_lib.FMAG_EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


@pytest.mark.parametrize("d,b,m", [(64, 4, 0), (128, 3, 128), (128, 4, 32), (256, 6, 256), (256, 1, 64)])
def test_layout_matches_oracle(d, b, m):
    _lib_or_skip()
    for S, N in ((1, 1), (3, 1000), (32, 32768), (0, 5)):
        got = T.get_layout(T.Codec(d, b, m, 1, 0), S, N)
        assert got == O.layout(d, b, m, S, N)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6])
def test_host_codebook_matches_oracle(d, b):
    _lib_or_skip()
    h = T.host_tables(T.Codec(d, b, 0, 1, 7))
    t, c = O.lloyd_max(d, b)
    assert np.max(np.abs(h["centroids"] - c) / np.abs(c)) < 1e-11
    assert np.max(np.abs(h["thresholds"] - t)) < 1e-12
    # fp32 device thresholds: at most a handful may round differently (values within 1e-11 of an
    # fp32 midpoint); count them
    diff = np.sum(h["thresholds"].astype(np.float32) != t.astype(np.float32))
    assert diff <= 1


@pytest.mark.parametrize("seed,head,d,m", [(4001, 0, 128, 128), (4001, 7, 128, 128), (5001, 3, 256, 256),
                                         (2**63 + 11, 2, 64, 32)])
def test_host_signs_and_S_match_oracle_exactly(seed, head, d, m):
    _lib_or_skip()
    h = T.host_tables(T.Codec(d, 2, m, head + 1, seed), head)
    assert np.array_equal(h["signs"], O.head_signs(seed, head, d).astype(np.float32))
    assert np.array_equal(h["S"], O.gaussian_matrix(seed, head, m, d).astype(np.float32))


@pytest.mark.parametrize("seed,head,d", [(4001, 0, 128), (77, 5, 64), (2**63 + 3, 1, 256)])
def test_host_rht_sketch_matches_oracle_exactly(seed, head, d):
    _lib_or_skip()
    h = T.host_tables(T.Codec(d, 3, d, head + 1, seed, sketch=_lib.TQ_SKETCH_RHT), head)
    assert np.array_equal(h["signs"], O.head_signs(seed, head, d).astype(np.float32))
    assert np.array_equal(h["S"], O.rht_matrix(seed, head, d).astype(np.float32))


def test_status_strings():
    _lib_or_skip()
    for s in (0, -1, -2, -3, -4, -5):
        assert _lib.status_string(s)
    assert _lib.status_string(-99) == "unknown status"


def _p(d=128, b=4, m=0, H=1, seed=0, sketch=0, rotation=0):
    return ctypes.byref(_lib.Params(d, b, m, H, seed, sketch, rotation))


def test_argument_validation_before_any_gpu_call():
    L = _lib_or_skip()
    lay = _lib.Layout()
    bad = [(_p(d=96), "d"), (_p(d=32), "d"), (_p(b=0), "b"), (_p(b=9), "b"), (_p(m=48), "m%32"),
           (_p(m=256, d=128), "m>d"), (_p(H=0), "n_heads"), (_p(m=128, sketch=2), "sketch kind"),
           (_p(m=64, sketch=1), "RHT needs m = d"), (_p(sketch=-1), "sketch kind"), (_p(rotation=2), "rotation")]
    for p, why in bad:
        assert L.tq_get_layout(p, 1, 1, ctypes.byref(lay)) == _lib.TQ_EINVAL, why
        assert L.tq_encode(p, ctypes.c_void_p(16), 1, 1, 1, ctypes.c_void_p(16), None) == _lib.TQ_EINVAL, why
    p = _p()
    assert L.tq_get_layout(None, 1, 1, ctypes.byref(lay)) == _lib.TQ_EINVAL
    assert L.tq_get_layout(p, -1, 1, ctypes.byref(lay)) == _lib.TQ_EINVAL
    # null pointers, bad dtype, misaligned pointers: rejected on the host
    assert L.tq_encode(p, None, 1, 2, 2, ctypes.c_void_p(16), None) == _lib.TQ_EINVAL
    assert L.tq_encode(p, ctypes.c_void_p(16), 7, 2, 2, ctypes.c_void_p(16), None) == _lib.TQ_EINVAL
    assert L.tq_encode(p, ctypes.c_void_p(18), 1, 2, 2, ctypes.c_void_p(16), None) == _lib.TQ_EALIGN
    assert L.tq_decode(p, ctypes.c_void_p(16), 2, 2, ctypes.c_void_p(20), 0, None) == _lib.TQ_EALIGN
    # appends must land inside the capacity
    x16, b16 = ctypes.c_void_p(16), ctypes.c_void_p(16)
    assert L.tq_encode_append(p, x16, 1, 2, 5, b16, 10, 6, None) == _lib.TQ_EINVAL      # 6 + 5 > 10
    assert L.tq_encode_append(p, x16, 1, 2, 5, b16, 10, -1, None) == _lib.TQ_EINVAL
    assert L.tq_encode_append(p, x16, 1, 2, -1, b16, 10, 0, None) == _lib.TQ_EINVAL
    assert L.tq_encode_append(p, x16, 1, 2, 0, b16, 10, 10, None) == _lib.TQ_OK          # empty append
    # the corrected decode needs a sketch
    assert L.tq_decode_qjl(p, ctypes.c_void_p(16), 2, 2, ctypes.c_void_p(16), 0, None) == _lib.TQ_EINVAL
    assert L.tq_decode_qjl(_p(m=128), ctypes.c_void_p(16), 2, 2, ctypes.c_void_p(20), 0, None) == _lib.TQ_EALIGN
    # empty inputs are a valid no-op
    assert L.tq_encode(p, None, 1, 0, 5, None, None) == _lib.TQ_OK
    # the one-launch key + value encode: both parameter sets, pointers, dtype and alignment on the host
    pkv = _p(m=128)
    assert L.tq_encode_kv(pkv, _p(b=0), x16, x16, 1, 2, 2, b16, b16, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(None, p, x16, x16, 1, 2, 2, b16, b16, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(pkv, p, x16, None, 1, 2, 2, b16, b16, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(pkv, p, x16, x16, 1, 2, 2, b16, None, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(pkv, p, x16, x16, 7, 2, 2, b16, b16, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(pkv, p, x16, x16, 1, -1, 2, b16, b16, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv(pkv, p, x16, ctypes.c_void_p(24), 1, 2, 2, b16, b16, None) == _lib.TQ_EALIGN
    assert L.tq_encode_kv(pkv, p, None, None, 1, 0, 5, None, None, None) == _lib.TQ_OK
    assert L.tq_encode_kv(pkv, p, None, None, 1, 3, 0, None, None, None) == _lib.TQ_OK
    assert L.tq_encode_kv_append(pkv, p, x16, x16, 1, 2, 5, b16, b16, 10, 6, None) == _lib.TQ_EINVAL   # 6 + 5 > 10
    assert L.tq_encode_kv_append(pkv, p, x16, x16, 1, 2, 5, b16, b16, 10, -1, None) == _lib.TQ_EINVAL
    assert L.tq_encode_kv_append(pkv, p, x16, x16, 1, 2, 0, b16, b16, 10, 10, None) == _lib.TQ_OK  # empty append
    assert L.tq_decode(p, None, 3, 0, None, 0, None) == _lib.TQ_OK
    # scores: workspace too small, too many queries
    pk = _p(m=128)
    ws = L.tq_scores_workspace_bytes(pk, 2, 32)
    assert ws > 0
    v = ctypes.c_void_p(256)
    assert L.tq_qk_scores(pk, v, 1, 32, v, 2, 10, v, v, ws - 1, None) == _lib.TQ_EWORKSPACE
    assert L.tq_qk_scores(pk, v, 1, 257, v, 2, 10, v, v, ws, None) == _lib.TQ_EINVAL
    # attention cross-argument rules
    pv = _p(m=0, H=8)
    pk8 = _p(m=128, H=8)
    wsa = L.tq_attention_workspace_bytes(pk8, 2, 32, 8, 1000)
    call = lambda pk_, pv_, hq, hkv, n, scale=0.0, wsb=wsa: L.tq_decode_attention(
        pk_, pv_, v, 1, 2, hq, hkv, v, v, n, ctypes.c_float(scale), v, 1, v, wsb, None)
    assert call(pk8, _p(m=128, H=8), 32, 8, 1000) == _lib.TQ_EINVAL   # QJL on V
    assert call(pk8, _p(d=64, H=8), 32, 8, 1000) == _lib.TQ_EINVAL    # d mismatch
    assert call(pk8, pv, 30, 8, 1000) == _lib.TQ_EINVAL               # heads not divisible
    assert call(pk8, pv, 32 * 17, 32, 1000) == _lib.TQ_EINVAL         # group > 16 (and n_heads)
    assert call(pk8, _p(H=4), 32, 8, 1000) == _lib.TQ_EINVAL          # n_heads != n_kv_heads
    assert call(pk8, pv, 32, 8, 0) == _lib.TQ_EINVAL                  # empty cache
    assert call(pk8, pv, 32, 8, 1000, scale=-1.0) == _lib.TQ_EINVAL
    assert call(pk8, pv, 32, 8, 1000, wsb=wsa - 1) == _lib.TQ_EWORKSPACE
    # a stream's planes are addressed with 32-bit offsets: at d = 128, b = 4 (64-byte index rows)
    # the index plane must stay below 2^32 - 2^16 bytes, i.e. at most 67107840 tokens
    big = (2**32 - 2**16) // 64 + 1
    wsb = L.tq_attention_workspace_bytes(pk8, 2, 32, 8, big)
    assert wsb > wsa
    assert call(pk8, pv, 32, 8, big, wsb=wsb) == _lib.TQ_EUNSUPPORTED
    assert call(pk8, pv, 32, 8, big, wsb=wsb - 1) == _lib.TQ_EWORKSPACE   # the workspace is checked first


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "kv_cache_transform_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.replace("no oracle", ""), f


def test_fmag_record_size_and_validation():
    L = _lib_or_skip()
    from oracle import fmag_oracle as FO
    for d, b, p in ((128, 4, 8), (128, 4, 16), (64, 3, 6), (64, 8, 8), (128, 1, 1)):
        assert T.FmagCodec(d, b, p).record_bytes == 4 * FO.record_words(d, b, p)
    n = ctypes.c_int64()
    for d, b, p in ((256, 4, 8), (128, 0, 8), (128, 9, 8), (128, 4, 0), (128, 4, 9), (128, 4, 12)):
        prm = _lib.FmagParams(d, b, p)
        assert L.tq_fmag_record_bytes(ctypes.byref(prm), ctypes.byref(n)) == _lib.TQ_EINVAL
        assert L.tq_fmag_encode(ctypes.byref(prm), None, _lib.TQ_BF16, 1, 1, None, None) == _lib.TQ_EINVAL
    prm = _lib.FmagParams(128, 4, 8)
    assert L.tq_fmag_encode(ctypes.byref(prm), None, _lib.TQ_F32, 1, 1, None, None) == _lib.TQ_EUNSUPPORTED
    assert L.tq_fmag_encode(ctypes.byref(prm), None, _lib.TQ_BF16, 1, 0, None, None) == _lib.TQ_OK
    assert L.tq_fmag_decode(ctypes.byref(prm), None, 1, 1, None, _lib.TQ_F32, None) == _lib.TQ_EINVAL


def test_fmag_attention_validates_before_any_device_call():
    """tq_fmag_decode_attention checks its arguments on the host: bad params, mismatched head sizes,
    a query-head count that is not a multiple of the kv heads or more than 16 per kv head, unsupported
    dtypes, a negative or non-finite scale, missing or misaligned pointers, a short workspace."""
    L = _lib_or_skip()
    P = _lib.FmagParams
    pk, pv, p64, bad = P(128, 4, 8), P(128, 3, 16), P(64, 4, 8), P(128, 9, 8)
    r = lambda a, b, hq=8, hkv=2, qd=_lib.TQ_F32, od=_lib.TQ_F32, sc=0.0, q=None, o=None, ws=None, wsb=0, N=16, k=None, v=None: \
        L.tq_fmag_decode_attention(ctypes.byref(a), ctypes.byref(b), q, qd, 1, hq, hkv, k, v, N, None,
                                   ctypes.c_float(sc), o, od, ws, wsb, None)
    assert r(bad, pv) == _lib.TQ_EINVAL
    assert r(pk, p64) == _lib.TQ_EINVAL                       # head sizes differ
    assert r(pk, pv, hq=6, hkv=4) == _lib.TQ_EINVAL           # not a multiple
    assert r(pk, pv, hq=34, hkv=2) == _lib.TQ_EINVAL          # 17 query heads per kv head
    assert r(pk, pv, qd=_lib.TQ_F16) == _lib.TQ_EUNSUPPORTED
    assert r(pk, pv, sc=-1.0) == _lib.TQ_EINVAL
    assert r(pk, pv, sc=float("nan")) == _lib.TQ_EINVAL
    assert r(pk, pv) == _lib.TQ_EINVAL                        # NULL q, out, workspace
    buf = (ctypes.c_uint8 * 4096)()
    base = ctypes.addressof(buf)
    a16 = (base + 15) // 16 * 16
    assert r(pk, pv, q=a16 + 4, o=a16, ws=a16, wsb=64, k=a16, v=a16) == _lib.TQ_EALIGN
    need = L.tq_fmag_attention_workspace_bytes(ctypes.byref(pk), 1, 8, 2, 16)
    assert need > 0
    assert r(pk, pv, q=a16, o=a16, ws=a16, wsb=need - 1, k=a16, v=a16) == _lib.TQ_EWORKSPACE
    assert L.tq_fmag_attention_workspace_bytes(ctypes.byref(bad), 1, 8, 2, 16) == 0

"""GPU tests of tq_encode_kv, the one-launch encode of the keys and values of the same tokens.

Its records must be byte-identical to two separate tq_encode calls (the fused kernel runs the
single-tensor arithmetic step for step); the separate encodes are themselves checked against the
oracle elsewhere, and one case here checks the fused records against the oracle directly.  Cases
cover the Gaussian sketch with full and partial sketch words, the randomized Hadamard sketch, keys
without a sketch, d = 64 and 128, b = 1..4, ragged token counts, streams split over many blocks,
different head counts for K and V, and the configurations that fall back to two launches (fp32
input, d = 256, a value sketch)."""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from oracle import tq_oracle as O
from synth import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    T._lib.lib()
    yield


def _zeros(c, x):
    # zero-filled, so the alignment padding between the record planes compares equal too
    return torch.zeros(T.get_layout(c, x.shape[0], x.shape[1])["total_bytes"], dtype=torch.uint8, device=DEV)


def _both(ck, cv, k, v):
    pk, pv = T.encode_kv(ck, cv, k, v, out_k=_zeros(ck, k), out_v=_zeros(cv, v))
    rk, rv = T.encode(ck, k, out=_zeros(ck, k)), T.encode(cv, v, out=_zeros(cv, v))
    torch.cuda.synchronize()
    return pk.cpu().numpy(), pv.cpu().numpy(), rk.cpu().numpy(), rv.cpu().numpy()


# (d, b, m_K, sketch, n_streams, n_tokens, heads K, heads V, dtype)
CASES = [
    (128, 4, 128, 0, 5, 1000, 3, 3, torch.bfloat16),     # the benchmark's codec pair, ragged tail
    (128, 3, 128, 0, 4, 777, 2, 2, torch.bfloat16),
    (128, 2, 64, 0, 3, 513, 3, 3, torch.bfloat16),       # partial sketch words (16 bits per part)
    (128, 4, 32, 0, 2, 300, 1, 1, torch.bfloat16),
    (128, 4, 128, 1, 3, 600, 3, 3, torch.bfloat16),      # randomized Hadamard sketch
    (128, 4, 0, 0, 4, 1000, 2, 2, torch.bfloat16),       # no key sketch
    (128, 1, 0, 0, 2, 257, 1, 1, torch.bfloat16),
    (64, 4, 64, 0, 3, 1000, 3, 3, torch.bfloat16),
    (64, 3, 32, 0, 2, 129, 2, 2, torch.bfloat16),
    (128, 4, 128, 0, 6, 1000, 3, 2, torch.bfloat16),     # K and V with different head counts
    (128, 4, 128, 0, 2, 100000, 2, 2, torch.bfloat16),   # two streams over many blocks each
    (128, 4, 128, 0, 3, 1, 3, 3, torch.bfloat16),        # one token
    (128, 4, 128, 0, 3, 17, 3, 3, torch.bfloat16),
    (128, 4, 128, 0, 3, 500, 3, 3, torch.float32),       # fp32 input: two launches
    (256, 3, 256, 0, 2, 300, 2, 2, torch.bfloat16),      # d = 256: two launches
]


@pytest.mark.parametrize("d,b,m,sk,S,N,hk,hv,dt", CASES)
def test_encode_kv_equals_two_encodes(d, b, m, sk, S, N, hk, hv, dt):
    print(f"encode_kv d={d} b={b} m={m} sketch={sk} S={S} N={N} heads {hk}/{hv} {dt}", flush=True)
    ck, cv = T.Codec(d, b, m, hk, 7001 + d + b, sketch=sk), T.Codec(d, b, 0, hv, 7002 + d + b)
    k = I.gaussian((S, N, d), 31 + N, device=DEV, dtype=dt)
    v = I.gaussian((S, N, d), 32 + N, device=DEV, dtype=dt)
    pk, pv, rk, rv = _both(ck, cv, k, v)
    assert pk.shape == rk.shape and pv.shape == rv.shape
    lk, lv = T.get_layout(ck, S, N), T.get_layout(cv, S, N)
    assert np.array_equal(pk[: lk["total_bytes"]], rk[: lk["total_bytes"]]), "key records differ"
    assert np.array_equal(pv[: lv["total_bytes"]], rv[: lv["total_bytes"]]), "value records differ"


def test_encode_kv_with_a_value_sketch_falls_back_to_two_launches():
    ck, cv = T.Codec(128, 4, 128, 2, 7101), T.Codec(128, 4, 32, 2, 7102)
    k = I.gaussian((2, 400, 128), 41, device=DEV, dtype=torch.bfloat16)
    v = I.gaussian((2, 400, 128), 42, device=DEV, dtype=torch.bfloat16)
    pk, pv, rk, rv = _both(ck, cv, k, v)
    assert np.array_equal(pk, rk) and np.array_equal(pv, rv)


def test_encode_kv_against_the_oracle():
    """the fused records of the benchmark's codec pair (K b = 4 + QJL m = 128, V b = 4) on RoPE-rotated
    keys and values, checked against the oracle itself"""
    S, N, H = 3, 700, 3
    ck, cv = T.Codec(128, 4, 128, H, 7201), T.Codec(128, 4, 0, H, 7202)
    k = I.rope_gaussian(S, N, 128, 7201, device=DEV)
    v = I.rope_gaussian(S, N, 128, 7202, device=DEV)
    pk, pv = T.encode_kv(ck, cv, k, v)
    torch.cuda.synchronize()
    for c, x, buf, seed in ((ck, k, pk, 7201), (cv, v, pv, 7202)):
        tb = P.Tables(128, 4, c.m, H, seed)
        st = P.check_encode(tb, O.bf16_bits_to_f64(I.bf16_bits(x)), buf.cpu().numpy())
        print(f"m={c.m}: flagged {st['flagged']}, index mismatches {st['idx_mismatch']}, sketch flagged "
              f"{st['sketch_flagged']}, sketch mismatches {st['sketch_mismatch']}")


def test_encode_kv_is_deterministic_and_validates():
    ck, cv = T.Codec(128, 4, 128, 2, 7301), T.Codec(128, 4, 0, 2, 7302)
    k = I.gaussian((2, 333, 128), 51, device=DEV, dtype=torch.bfloat16)
    v = I.gaussian((2, 333, 128), 52, device=DEV, dtype=torch.bfloat16)
    a = [t.cpu().numpy() for t in T.encode_kv(ck, cv, k, v, out_k=_zeros(ck, k), out_v=_zeros(cv, v))]
    b = [t.cpu().numpy() for t in T.encode_kv(ck, cv, k, v, out_k=_zeros(ck, k), out_v=_zeros(cv, v))]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        T.encode_kv(ck, cv, k, v[:, :300].contiguous())
    with pytest.raises(ValueError):
        T.encode_kv(ck, cv, k, v.float())


@pytest.mark.parametrize("m,sk,n_new,t0,cap", [(128, 0, 1, 999, 1000), (128, 0, 17, 300, 1000), (128, 1, 40, 0, 64),
                                               (0, 0, 1, 0, 1), (64, 0, 33, 100, 200)])
def test_encode_kv_append_equals_two_appends(m, sk, n_new, t0, cap):
    """the decode step's append of new keys and values into caches of a given capacity, in one launch:
    the same bytes as two tq_encode_append calls (the rest of the caches untouched)"""
    print(f"encode_kv_append m={m} sketch={sk} n_new={n_new} t0={t0} capacity={cap}", flush=True)
    S, H = 4, 2
    ck, cv = T.Codec(128, 4, m, H, 7401, sketch=sk), T.Codec(128, 4, 0, H, 7402)
    k = I.gaussian((S, n_new, 128), 61 + n_new, device=DEV, dtype=torch.bfloat16)
    v = I.gaussian((S, n_new, 128), 62 + n_new, device=DEV, dtype=torch.bfloat16)
    zc = lambda c: torch.zeros(T.get_layout(c, S, cap)["total_bytes"], dtype=torch.uint8, device=DEV)
    fk, fv = T.encode_kv_append(ck, cv, k, v, zc(ck), zc(cv), cap, t0)
    rk, rv = T.encode_append(ck, k, zc(ck), cap, t0), T.encode_append(cv, v, zc(cv), cap, t0)
    torch.cuda.synchronize()
    assert torch.equal(fk, rk) and torch.equal(fv, rv)

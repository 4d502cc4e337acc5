"""GPU parity of the SpectralQuant and Fourier-magnitude paths at the benchmark's full shape (K and V
[16·8, 131072, 128] bf16, RoPE-rotated Gaussian), in the launch configuration the benchmark times:
the HIP path runs over the whole tensors, the oracles check token ranges (start, middle, ragged end)
of a few streams and whole attention rows (SpectralQuant and Fmag caches).  Tolerances as in
test_gpu_sq.py and test_gpu_fmag.py."""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from oracle import fmag_oracle as F
from oracle import sq_oracle as Q
from oracle import tq_oracle as O
from synth import inputs as I
from tests import test_gpu_fmag as GF

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, HQ, HKV, N, D = 16, 32, 8, 131072, 128


@pytest.fixture(scope="module")
def kv():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    T._lib.lib()
    K = I.rope_gaussian(B * HKV, N, D, 4001, device=DEV)
    V = I.rope_gaussian(B * HKV, N, D, 4002, device=DEV)
    yield K, V
    del K, V
    torch.cuda.empty_cache()


def _f64(x):
    return O.bf16_bits_to_f64(I.bf16_bits(x))


RANGES = [(0, 256), (N // 2 - 128, N // 2 + 128), (N - 256, N)]
STREAMS = [0, 61, 127]


@pytest.mark.timeout(900)
def test_sq_full_shape_encode_decode_attention(kv):
    K, V = kv
    ck = T.SQCodec.calibrate(K[:HKV, :512].float(), 4, 2, device=0)
    cv = T.SQCodec.calibrate(V[:HKV, :512].float(), 4, 2, device=0)
    mk = [Q.calibrate(_f64(K[h, :512]), 4, 2) for h in range(HKV)]
    mv = [Q.calibrate(_f64(V[h, :512]), 4, 2) for h in range(HKV)]
    pk, pv = ck.encode(K), cv.encode(V)
    xh = ck.decode(pk, B * HKV, N, torch.float32)
    torch.cuda.synchronize()
    rb = ck.record_bytes
    flagged = 0
    for st in STREAMS:
        m = mk[st % HKV]
        for a, b in RANGES:
            x64 = _f64(K[st, a:b])
            rec = pk[(st * N + a) * rb:(st * N + b) * rb].cpu().numpy().reshape(b - a, rb)
            ig = Q.unpack(rec, m["bits"])
            r = Q.encode(x64, m)
            band = 4e-6 + 2.0 ** -19 * (np.abs(x64) @ np.abs(m["U"])) / m["sigma"]
            flag = Q.boundary_distance(r["u"], m) < band
            assert not ((ig != r["idx"]) & ~flag).any(), (st, a)
            flagged += int(flag.sum())
            want = Q.decode(ig, m)
            got = xh[st, a:b].cpu().numpy()
            assert np.linalg.norm(got - want) <= 1e-5 * np.linalg.norm(want), (st, a)
    del xh
    # whole attention rows over the full context
    q = I.cfg4_queries(B, HQ, D, N, 4003, device=DEV)
    out = T.sq_decode_attention(ck, cv, q, pk, pv, HKV, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    q64 = _f64(q)
    for b, h in ((0, 0), (9, 21)):
        hk = h // (HQ // HKV)
        st = b * HKV + hk
        ik = Q.unpack(pk[st * N * rb:(st + 1) * N * rb].cpu().numpy().reshape(N, rb), mk[hk]["bits"])
        rbv = cv.record_bytes
        iv = Q.unpack(pv[st * N * rbv:(st + 1) * N * rbv].cpu().numpy().reshape(N, rbv), mv[hk]["bits"])
        sc = Q.scores(q64[b, h][None, :], ik, mk[hk])
        want = Q.attention(sc, iv, mv[hk], 1.0 / np.sqrt(D))[0]
        assert np.linalg.norm(got[b, h] - want) <= 2e-3 * np.linalg.norm(want), (b, h)
    print(f"SQ full shape: flagged {flagged} in the sampled ranges")


@pytest.mark.timeout(900)
def test_fmag_full_shape_encode_decode_scores_attention(kv):
    K, V = kv
    codec = T.FmagCodec(D, 4, 8)
    packed = codec.encode(K)
    xh = codec.decode(packed, B * HKV, N, torch.float32)
    torch.cuda.synchronize()
    W = F.record_words(D, 4, 8)
    for st in STREAMS:
        for a, b in RANGES:
            sub = K[st:st + 1, a:b].contiguous()
            words = packed[(st * N + a) * W * 4:(st * N + b) * W * 4]
            recs, _, _ = GF._check(codec, sub, words)
            want = F.decode(recs[0], 4, 8, D)
            got = xh[st, a:b].cpu().numpy()
            assert np.linalg.norm(got - want) <= 1e-5 * np.linalg.norm(want), (st, a)
    # scores of 32 queries of one stream over its last 4096 tokens
    st, a = 77, N - 4096
    sub = packed[(st * N + a) * W * 4:(st * N + N) * W * 4]
    q = torch.randn(1, 32, D, generator=torch.Generator(device=DEV).manual_seed(105), device=DEV)
    sc = codec.qk_scores(q, sub, 4096).cpu().numpy()[0]
    rec = F.unpack(sub.cpu().numpy().view(np.uint32).reshape(4096, W), 4, 8, D)
    want = F.scores(q.cpu().numpy()[0].astype(np.float64), rec, 4, 8, D)
    rel = np.linalg.norm(sc - want, axis=1) / np.linalg.norm(want, axis=1)
    assert rel.max() < 2e-3
    # whole attention rows over the full context, K and V both Fmag caches (the benchmark's launch)
    pv = codec.encode(V)
    qa = I.cfg4_queries(B, HQ, D, N, 4003, device=DEV)
    out = T.fmag_decode_attention(codec, codec, qa, packed, pv, HKV, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    q64 = _f64(qa)
    for b, h in ((0, 0), (9, 21), (15, 31)):
        stq = b * HKV + h // (HQ // HKV)
        rk = F.unpack(packed[stq * N * W * 4:(stq + 1) * N * W * 4].cpu().numpy().view(np.uint32).reshape(N, W), 4, 8, D)
        rv = F.unpack(pv[stq * N * W * 4:(stq + 1) * N * W * 4].cpu().numpy().view(np.uint32).reshape(N, W), 4, 8, D)
        scr = F.scores(q64[b, h][None, :], rk, 4, 8, D)
        want = F.attention(scr, rv, 4, 8, D, 1.0 / np.sqrt(D))[0]
        assert np.linalg.norm(got[b, h] - want) <= 2e-3 * np.linalg.norm(want), (b, h)

"""GPU parity of the Fourier-magnitude codec (through the C ABI) against the Fmag oracle.

Tolerances.  The kernel's spectrum comes from fp16 products of the exact (power-of-two scaled) input
with the DFT matrix as an fp16 hi + lo pair, accumulated in fp32: its error is below
e_X = 2^-18 Σ_j |x_j| per coefficient.  So
  * lo and hi within e_X of the oracle's;
  * magnitude indices equal except where the oracle's (|X| - lo)/(hi - lo)·(2^b - 1) lies within
    (2^b - 1)·3 e_X/(hi - lo) + 1e-5 of a rounding point;
  * phase fields equal except where the oracle's phase lies within e_X/|X_k| + 1e-6 rad (about the
    error of an fp32 atan2 of coefficients that far off) of a rounding point, or at ±π;
  * records word-identical to the oracle's packing of the GPU's own fields;
  * fp32 decode within 1e-5 relative L2 per stream of the oracle's decode of the GPU's records;
  * scores within 2e-3 relative L2 per (stream, query) row.
Page: "Fourier Magnitude KV Cache Quantization" (forum thread), "Method"."""
import math

import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from oracle import fmag_oracle as F
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


def _f64(x):
    return O.bf16_bits_to_f64(I.bf16_bits(x))


def _data(kind, S, N, d, seed):
    if kind == "gauss":
        return I.gaussian((S, N, d), seed, device=DEV)
    if kind == "rope":
        return I.rope_gaussian(S, N, d, seed, device=DEV)
    return I.student_t(S, N, d, 3, seed, device=DEV)


def _check(codec, x, packed):
    S, N, d = x.shape
    b, p = codec.b, codec.p
    W = F.record_words(d, b, p)
    words = packed.cpu().numpy()[: S * N * W * 4].view(np.uint32).reshape(S, N, W)
    x64 = _f64(x)
    recs, flagged, mism = [], 0, 0
    for st in range(S):
        g = F.unpack(words[st], b, p, d)
        assert np.array_equal(words[st], F.pack({**g, "pbf": g["pbf"]}, b, p, d)), "record layout or padding"
        o = F.encode(x64[st], b, p)
        ex = 2.0 ** -18 * np.abs(x64[st]).sum(axis=1)
        assert np.all(np.abs(g["lo"] - o["lo"]) <= ex) and np.all(np.abs(g["hi"] - o["hi"]) <= ex)
        L = (1 << b) - 1
        span = np.maximum(o["hi"] - o["lo"], 1e-300)
        mflag = F.magnitude_flags(o, 1e-5) | (np.abs(o["t"] - np.floor(o["t"]) - 0.5) < (L * 3 * ex / span)[:, None])
        pband = ex[:, None] / np.maximum(o["mag"], 1e-300) + 1e-6
        if p == F.PHASE_BF16:
            f = np.abs(o["phase"])
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(f, 1e-300))) - 7)
            dist = np.abs(f / ulp - np.floor(f / ulp) - 0.5) * ulp
            pflag = (dist < pband) | (np.abs(f - math.pi) < pband) | (o["mag"] <= 10 * ex[:, None])
            pdiff = g["pbf"] != o["pbf"]
        else:
            u = (o["phase"] + math.pi) / (2 * math.pi) * (1 << p)
            pflag = (np.abs(u - np.floor(u) - 0.5) < pband * (1 << p) / (2 * math.pi)) | (o["mag"] <= 10 * ex[:, None])
            pdiff = g["pidx"] != o["pidx"]
        qdiff = g["q"] != o["q"]
        assert not (qdiff & ~mflag).any(), (st, np.argwhere(qdiff & ~mflag)[:5])
        assert not (pdiff & ~pflag).any(), (st, np.argwhere(pdiff & ~pflag)[:5], o["phase"][pdiff & ~pflag][:5])
        flagged += int(mflag.sum() + pflag.sum())
        mism += int(qdiff.sum() + pdiff.sum())
        recs.append(g)
    return recs, flagged, mism


@pytest.mark.parametrize("d,b,p,kind", [
    (128, 4, 8, "rope"), (128, 4, 16, "gauss"), (128, 3, 6, "gauss"), (64, 4, 8, "gauss"),
    (64, 2, 16, "tdist"), (128, 8, 8, "tdist"), (64, 1, 1, "gauss"), (128, 5, 3, "rope"),
])
def test_fmag_encode_decode_scores_parity(d, b, p, kind):
    S, N = 3, 1000
    codec = T.FmagCodec(d, b, p)
    x = _data(kind, S, N, d, 41)
    packed = codec.encode(x)
    torch.cuda.synchronize()
    recs, flagged, mism = _check(codec, x, packed)
    print(f"fmag d={d} b={b} p={p} {kind}: flagged {flagged}, mismatched {mism}")
    xh = codec.decode(packed, S, N, torch.float32).cpu().numpy()
    xb = _f64(codec.decode(packed, S, N, torch.bfloat16))
    for st in range(S):
        want = F.decode(recs[st], b, p, d)
        rel = np.linalg.norm(xh[st] - want) / np.linalg.norm(want)
        assert rel < 1e-5, (st, rel)
        assert np.all(np.abs(xb[st] - want) <= np.abs(want) * 2.0 ** -8 + 1e-5 * np.abs(want).max())
    q = torch.randn(S, 19, d, generator=torch.Generator(device=DEV).manual_seed(9), device=DEV)
    sc = codec.qk_scores(q, packed, N).cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    for st in range(S):
        want = F.scores(q64[st], recs[st], b, p, d)
        rel = np.linalg.norm(sc[st] - want, axis=1) / np.linalg.norm(want, axis=1)
        assert rel.max() < 2e-3, (st, rel.max())


@pytest.mark.parametrize("N", [1, 15, 17])
def test_fmag_short_streams_and_zero_vectors(N):
    codec = T.FmagCodec(128, 4, 8)
    x = _data("gauss", 2, N, 128, 7)
    x[1, 0] = 0            # a zero vector: lo = hi = 0, every field 0 or the phase of +0
    packed = codec.encode(x)
    torch.cuda.synchronize()
    recs, _, _ = _check(codec, x, packed)
    xh = codec.decode(packed, 2, N).cpu().numpy()
    assert np.all(xh[1, 0] == 0.0)
    for st in range(2):
        want = F.decode(recs[st], 4, 8, 128)
        assert np.linalg.norm(xh[st] - want) <= 1e-5 * np.linalg.norm(want)


def test_fmag_leaves_other_bytes_and_rejects_fp32():
    codec = T.FmagCodec(64, 4, 8)
    x = _data("gauss", 2, 40, 64, 3)
    rb = codec.record_bytes
    buf = torch.full((2 * 40 * rb + 256,), 0xA5, dtype=torch.uint8, device=DEV)
    codec.encode(x, buf)
    torch.cuda.synchronize()
    assert torch.all(buf[2 * 40 * rb:] == 0xA5)
    with pytest.raises(T.TQError):
        codec.encode(x.float())


@pytest.mark.parametrize("batch,hq,hkv,N,d,kind,bpk,bpv,lens,out_dtype", [
    (2, 8, 2, 1000, 128, "rope", (4, 8), (4, 8), None, torch.float32),
    (1, 4, 4, 777, 64, "gauss", (3, 6), (4, 16), None, torch.bfloat16),
    (2, 16, 1, 300, 128, "tdist", (4, 16), (2, 3), None, torch.float32),
    (3, 8, 2, 600, 128, "gauss", (8, 16), (8, 16), [600, 1, 0], torch.float32),   # 51-word records
    (2, 4, 2, 2500, 64, "rope", (1, 1), (5, 8), [2500, 1234], torch.float32),
])
def test_fmag_decode_attention(batch, hq, hkv, N, d, kind, bpk, bpv, lens, out_dtype):
    """Attention rows from the GPU's own records against softmax(scale·ŝ) @ x̂ of the oracle:
    within 2e-3 relative L2 per row (a bf16 output against the oracle rounded to bf16)."""
    S, G = batch * hkv, hq // hkv
    ck, cv = T.FmagCodec(d, *bpk), T.FmagCodec(d, *bpv)
    K = _data(kind, S, N, d, 51)
    V = _data(kind, S, N, d, 52)
    pk, pv = ck.encode(K), cv.encode(V)
    q = torch.randn(batch, hq, d, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = T.fmag_decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=out_dtype, lengths=lt)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    Wk, Wv = F.record_words(d, *bpk), F.record_words(d, *bpv)
    wk = pk.cpu().numpy()[: S * N * Wk * 4].view(np.uint32).reshape(S, N, Wk)
    wv = pv.cpu().numpy()[: S * N * Wv * 4].view(np.uint32).reshape(S, N, Wv)
    rows, wants = [], []
    for b in range(batch):
        n_b = N if lens is None else lens[b]
        for h in range(hq):
            st = b * hkv + h // G
            if n_b == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            rk = F.unpack(wk[st, :n_b], *bpk, d)
            rv = F.unpack(wv[st, :n_b], *bpv, d)
            sc = F.scores(q64[b, h][None, :], rk, *bpk, d)
            wants.append(F.attention(sc, rv, *bpv, d, 1.0 / math.sqrt(d))[0])
            rows.append(got[b, h])
    r = P.check_attention_rows(np.array(rows), np.array(wants), out_dtype == torch.bfloat16)
    print(f"fmag attention worst row rel L2 {r['worst']:.2e} ({r['worst_unrounded']:.2e} against the unrounded oracle)")


def test_fmag_attention_validates_arguments():
    ck, c2 = T.FmagCodec(64, 4, 8), T.FmagCodec(128, 4, 8)
    q = torch.randn(1, 4, 64, generator=torch.Generator(device=DEV).manual_seed(183), device=DEV)
    pk = ck.encode(_data("gauss", 2, 32, 64, 1))
    with pytest.raises(T.TQError):          # K and V head sizes differ
        T.fmag_decode_attention(ck, c2, q, pk, pk, 2, 32)
    with pytest.raises(T.TQError):          # more than 16 query heads per kv head
        T.fmag_decode_attention(ck, ck, torch.zeros(1, 34, 64, device=DEV), pk, pk, 2, 32)


@pytest.mark.parametrize("N", [0, 1, 33])
def test_fmag_attention_short_caches(N):
    """An empty cache gives zero rows; one token returns its reconstruction; a ragged chunk."""
    ck = T.FmagCodec(128, 4, 8)
    B, Hq, Hkv = 2, 8, 2
    K = _data("gauss", B * Hkv, max(N, 1), 128, 61)[:, :N].contiguous()
    V = _data("gauss", B * Hkv, max(N, 1), 128, 62)[:, :N].contiguous()
    pk = ck.encode(K) if N else torch.zeros(16, dtype=torch.uint8, device=DEV)
    pv = ck.encode(V) if N else torch.zeros(16, dtype=torch.uint8, device=DEV)
    q = torch.randn(B, Hq, 128, generator=torch.Generator(device=DEV).manual_seed(4), device=DEV)
    out = T.fmag_decode_attention(ck, ck, q, pk, pv, Hkv, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if N == 0:
        assert np.all(got == 0.0)
        return
    W = F.record_words(128, 4, 8)
    wv = pv.cpu().numpy()[: B * Hkv * N * W * 4].view(np.uint32).reshape(B * Hkv, N, W)
    wk = pk.cpu().numpy()[: B * Hkv * N * W * 4].view(np.uint32).reshape(B * Hkv, N, W)
    q64 = q.cpu().numpy().astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            st = b * Hkv + h // (Hq // Hkv)
            rk, rv = F.unpack(wk[st], 4, 8, 128), F.unpack(wv[st], 4, 8, 128)
            want = F.attention(F.scores(q64[b, h][None, :], rk, 4, 8, 128), rv, 4, 8, 128, 1.0 / math.sqrt(128))[0]
            assert np.linalg.norm(got[b, h] - want) <= 2e-3 * np.linalg.norm(want), (b, h)

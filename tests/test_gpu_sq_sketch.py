"""GPU parity of SpectralQuant's selective QJL sketch (SQU-QKV: m sign bits of S e_z on the semantic
residual and the residual's fp16 norm, and the sketch term of the scores and the attention) through the
C ABI, against the SQ oracle.

Tolerances.  Indices as in the plain SpectralQuant tests.  The oracle's sketch is computed from the
GPU's own indices, so a flagged index moves both sides' residual alike.  The kernel's z_k carries at
most ε_k = 4e-6·σ_k + 2^-19 Σ_j |U_jk x_j| (the index band in z units); σ_k c is formed in fp32, and
S e_z comes from fp16 hi + lo halves of the scaled residual with fp32 accumulation.  So
  * sketch bits equal except where |(S e_z)_i| < Σ_{k<d_eff} ε_k + 2^-18 ||e_z||_1;
  * r16 within one fp16 step of the oracle's fp16 norm;
  * records word-identical to the oracle's packing of the GPU's own fields;
  * decode unchanged by the sketch (1e-5 relative L2 per stream);
  * scores and attention outputs within 2e-3 relative L2 per row.
Page: "Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2 "SpectralQuant"
(SQU-QKV), §6."""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from oracle import sq_oracle as Q
from oracle import tq_oracle as O
from synth import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SEED = 0x5EED


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    T._lib.lib()
    yield


def _f64(x):
    return O.bf16_bits_to_f64(I.bf16_bits(x))


REGIMES = {
    "lowrank_aligned": ([1.0] * 8, 0.05),
    "lowrank_steep": ([1.0, 0.5, 0.25, 0.125], 0.05),
    "isotropic": (None, 1.0),
    "fattail": ("t", 0.0),
}


def _tokens(regime, S, N, d, seed, n_heads):
    spec, noise = REGIMES[regime]
    if spec is None:
        return I.gaussian((S, N, d), seed, device=DEV)
    if spec == "t":
        return I.student_t(S, N, d, 3, seed, device=DEV)
    return I.low_rank(S, N, d, spec, noise, seed, 77, n_heads=n_heads, device=DEV)


def _codec(regime, d, b, b_tail, H, m, cap, seed, water=False):
    xc = _tokens(regime, H, 512, d, seed + 1000, H)
    codec = T.SQCodec.calibrate(xc.float(), b, b_tail, waterfill=water, d_eff_max=cap, device=0, m=m, seed=SEED)
    xc64 = _f64(xc)
    models = []
    for h in range(H):
        base = Q.calibrate(xc64[h], b, b_tail, water=water, d_eff_max=cap)
        assert np.array_equal(codec.bits[h], base["bits"]) and codec.d_eff[h] == base["d_eff"]
        models.append(Q.with_sketch(base, m, SEED, h))
    return codec, models


def _check_encode(codec, models, x, packed):
    """-> per stream the GPU's (indices, sketch bits, r16); asserts the tolerances above."""
    S, N, d = x.shape
    m = codec.m
    x64 = _f64(x)
    rb = codec.record_bytes
    assert rb == Q.record_bytes([mm["bits"] for mm in models], m)
    rec = packed.cpu().numpy()[: S * N * rb].reshape(S, N, rb)
    out, flagged, mism = [], 0, 0
    for st in range(S):
        md = models[st % codec.n_heads]
        ig, sg, rg = Q.unpack(rec[st], md["bits"], m)
        assert np.array_equal(rec[st], Q.pack(ig, md["bits"], rb, sg, rg)), "record layout or padding"
        r = Q.encode(x64[st], md)
        eps = 4e-6 * md["sigma"] + 2.0 ** -19 * (np.abs(x64[st]) @ np.abs(md["U"]))
        band = eps / md["sigma"]
        iflag = Q.boundary_distance(r["u"], md) < band
        assert not ((ig != r["idx"]) & ~iflag).any(), st
        k = Q.sketch_of(r["z"], ig, md)                         # the oracle's sketch of the GPU's indices
        de = md["d_eff"]
        zband = eps[:, :de].sum(axis=1) + 2.0 ** -18 * np.abs(k["e"]).sum(axis=1)
        sflag = np.abs(k["zs"]) < zband[:, None]
        sdiff = sg != k["sigma_bits"]
        assert not (sdiff & ~sflag).any(), (st, np.argwhere(sdiff & ~sflag)[:5])
        want16 = np.asarray(k["r16"], dtype=np.float16)
        got16 = np.asarray(rg, dtype=np.float16)
        step = np.spacing(want16.astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got16.astype(np.float64) - want16.astype(np.float64)) <= step), st
        flagged += int(iflag.sum() + sflag.sum())
        mism += int((ig != r["idx"]).sum() + sdiff.sum())
        out.append((ig, sg, rg))
    return out, flagged, mism


@pytest.mark.parametrize("regime,d,b,b_tail,m,cap,water", [
    ("lowrank_aligned", 128, 2, 1, 64, 0, False),
    ("lowrank_aligned", 128, 4, 2, 32, 0, False),
    ("lowrank_steep", 64, 3, 1, 16, 0, False),
    ("isotropic", 128, 3, 2, 48, 32, False),
    ("fattail", 128, 4, 2, 64, 24, True),
    ("isotropic", 64, 2, 2, 64, 32, False),
    ("lowrank_aligned", 128, 8, 8, 64, 0, False),
])
def test_sq_sketch_encode_decode_scores_parity(regime, d, b, b_tail, m, cap, water):
    S, H, N = 3, 2, 1000                                         # 63 tiles of 16, a ragged last tile
    codec, models = _codec(regime, d, b, b_tail, H, m, cap, 11, water)
    x = _tokens(regime, S, N, d, 11, H)
    packed = codec.encode(x)
    torch.cuda.synchronize()
    fields, flagged, mism = _check_encode(codec, models, x, packed)
    print(f"sketch {regime} d={d} b={b}/{b_tail} m={m}: flagged {flagged}, mismatched {mism}")
    xh = codec.decode(packed, S, N, torch.float32).cpu().numpy()
    for st in range(S):
        want = Q.decode(fields[st][0], models[st % H])
        assert np.linalg.norm(xh[st] - want) <= 1e-5 * np.linalg.norm(want), st
    nq = 17
    q = torch.randn(S, nq, d, generator=torch.Generator(device=DEV).manual_seed(5), device=DEV)
    sc = codec.qk_scores(q, packed, N).cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    for st in range(S):
        ig, sg, rg = fields[st]
        want = Q.scores(q64[st], ig, models[st % H], sg, rg)
        rel = np.linalg.norm(sc[st] - want, axis=1) / np.linalg.norm(want, axis=1)
        assert rel.max() < 2e-3, (st, rel.max())
        if b <= 4:   # the correction is really there: without it the scores are further off
            plain = Q.scores(q64[st], ig, models[st % H] | {"m": 0})
            assert np.linalg.norm(sc[st] - plain) > 10 * np.linalg.norm(sc[st] - want)


@pytest.mark.parametrize("N", [1, 15, 17])
def test_sq_sketch_short_streams(N):
    codec, models = _codec("lowrank_aligned", 128, 2, 1, 3, 64, 0, 12)
    x = _tokens("lowrank_aligned", 4, N, 128, 12, 3)
    packed = codec.encode(x)
    torch.cuda.synchronize()
    fields, _, _ = _check_encode(codec, models, x, packed)
    q = torch.randn(4, 3, 128, generator=torch.Generator(device=DEV).manual_seed(1200 + N), device=DEV,
                    dtype=torch.bfloat16)
    sc = codec.qk_scores(q, packed, N).cpu().numpy()
    q64 = _f64(q)
    for st in range(4):
        ig, sg, rg = fields[st]
        want = Q.scores(q64[st], ig, models[st % 3], sg, rg)
        assert np.linalg.norm(sc[st] - want) <= 2e-3 * np.linalg.norm(want)


@pytest.mark.parametrize("batch,hq,hkv,N,d,regime,bk,bv,m,mv,lens", [
    # key records of every prefetch size: about 1.6, 4.6 and 8.6 bits per dimension at d = 128, 2.6 and
    # 5 at d = 64; a value codec with a sketch of its own (unused by the attention); an empty row
    (2, 8, 2, 1000, 128, "lowrank_aligned", (2, 1), (4, 2), 64, 0, None),
    (2, 4, 2, 700, 128, "lowrank_aligned", (4, 4), (4, 2), 32, 0, [700, 333]),
    (1, 8, 1, 500, 128, "lowrank_aligned", (8, 8), (4, 2), 64, 0, None),
    (2, 4, 2, 900, 64, "lowrank_steep", (3, 1), (3, 1), 16, 16, None),
    (2, 4, 1, 400, 64, "lowrank_steep", (5, 4), (3, 2), 48, 0, [400, 0]),
])
def test_sq_sketch_decode_attention(batch, hq, hkv, N, d, regime, bk, bv, m, mv, lens):
    S, G = batch * hkv, hq // hkv
    ck, mk = _codec(regime, d, bk[0], bk[1], hkv, m, 0, 21)
    if mv:
        cv, mvs = _codec(regime, d, bv[0], bv[1], hkv, mv, 0, 22)
    else:
        xc = _tokens(regime, hkv, 512, d, 1022, hkv)
        cv = T.SQCodec.calibrate(xc.float(), bv[0], bv[1], device=0)
        mvs = [Q.calibrate(_f64(xc)[h], bv[0], bv[1]) for h in range(hkv)]
    K = _tokens(regime, S, N, d, 31, hkv)
    V = _tokens(regime, S, N, d, 32, hkv)
    pk, pv = ck.encode(K), cv.encode(V)
    q = torch.randn(batch, hq, d, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = T.sq_decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=torch.float32, lengths=lt)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    rk = pk.cpu().numpy()[: S * N * ck.record_bytes].reshape(S, N, ck.record_bytes)
    rv = pv.cpu().numpy()[: S * N * cv.record_bytes].reshape(S, N, cv.record_bytes)
    print(f"key record {ck.record_bytes // 4} words, value record {cv.record_bytes // 4} words")
    worst = 0.0
    for b in range(batch):
        n_b = N if lens is None else lens[b]
        for h in range(hq):
            hk = h // G
            st = b * hkv + hk
            if n_b == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            ik, sk, r16 = Q.unpack(rk[st, :n_b], mk[hk]["bits"], m)
            iv = Q.unpack(rv[st, :n_b], mvs[hk]["bits"], mv)
            iv = iv[0] if mv else iv
            sc = Q.scores(q64[b, h][None, :], ik, mk[hk], sk, r16)
            want = Q.attention(sc, iv, mvs[hk], 1.0 / np.sqrt(d))[0]
            worst = max(worst, np.linalg.norm(got[b, h] - want) / np.linalg.norm(want))
    print(f"sq sketch attention worst row rel {worst:.2e}")
    assert worst < 2e-3

"""GPU parity of the SpectralQuant path (through the C ABI) against the SQ oracle.

Both sides calibrate independently from the same calibration tokens (the library's Jacobi
eigensolver and Newton codebooks against the oracle's numpy eigh and Lloyd sweeps), then encode the
same bf16 tokens.  Tolerances:
  * indices bit-exact except where the oracle's u_k = z_k/σ_k lies within the flag band of a
    threshold: 4e-6 + 2^-19 Σ_j |U_jk x_j| / σ_k.  The kernel forms z_k from fp16 products of the
    exact (power-of-two scaled) input with U as an fp16 hi + lo pair (U to about 2^-22 relative) and
    accumulates 2d products in fp32; the search grid maps u to an fp32 cell coordinate (about
    2^-23·16 in u);
  * records byte-identical to the oracle's packing of the GPU's own indices (padding bits zero);
  * fp32 decode within 1e-5 relative L2 per stream of the oracle's decode of the GPU's indices;
    bf16 decode within one bf16 rounding;
  * scores within 2e-3 relative L2 per (stream, query) row.
Pages: "Ablation, Statistical Inference, and Validation for KV-Cache Compression", §2
"SpectralQuant", §6, §7."""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from oracle import sq_oracle as Q
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


REGIMES = {
    # name: (spectrum, noise)
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


def _case(regime, d, b, b_tail, water, S, H, N, cap=0, seed=11):
    xc = _tokens(regime, H, 512, d, seed + 1000, H)             # calibration tokens, one set per head
    x = _tokens(regime, S, N, d, seed, H)
    codec = T.SQCodec.calibrate(xc.float(), b, b_tail, waterfill=water, d_eff_max=cap, device=0)
    xc64 = _f64(xc)
    models = [Q.calibrate(xc64[h], b, b_tail, water=water, d_eff_max=cap) for h in range(H)]
    for h in range(H):
        assert np.array_equal(codec.bits[h], models[h]["bits"])
    return codec, models, x


def _check_encode(codec, models, x, packed):
    S, N, d = x.shape
    x64 = _f64(x)
    rb = codec.record_bytes
    rec = packed.cpu().numpy()[: S * N * rb].reshape(S, N, rb)
    idx_gpu = []
    flagged = mism = 0
    for st in range(S):
        m = models[st % codec.n_heads]
        assert rb == Q.record_bytes([mm["bits"] for mm in models])
        ig = Q.unpack(rec[st], m["bits"])
        assert np.array_equal(rec[st], Q.pack(ig, m["bits"], rb)), "record layout or padding"
        r = Q.encode(x64[st], m)
        band = 4e-6 + 2.0 ** -19 * (np.abs(x64[st]) @ np.abs(m["U"])) / m["sigma"]
        flag = Q.boundary_distance(r["u"], m) < band
        bad = (ig != r["idx"]) & ~flag
        assert not bad.any(), (st, np.argwhere(bad)[:5], r["u"][bad][:5])
        flagged += int(flag.sum())
        mism += int((ig != r["idx"]).sum())
        idx_gpu.append(ig)
    return idx_gpu, flagged, mism


@pytest.mark.parametrize("regime,d,b,b_tail,water,cap", [
    ("lowrank_aligned", 128, 4, 2, False, 0),
    ("lowrank_aligned", 64, 3, 1, False, 0),
    ("lowrank_steep", 128, 6, 2, True, 4),
    ("isotropic", 128, 3, 2, False, 0),
    ("isotropic", 64, 8, 8, False, 0),
    ("fattail", 128, 2, 1, True, 0),
    ("lowrank_aligned", 128, 8, 1, True, 0),
])
def test_sq_encode_decode_scores_parity(regime, d, b, b_tail, water, cap):
    S, H, N = 3, 2, 1000                                         # 63 tiles of 16, a ragged last tile
    codec, models, x = _case(regime, d, b, b_tail, water, S, H, N, cap)
    packed = codec.encode(x)
    torch.cuda.synchronize()
    idx, flagged, mism = _check_encode(codec, models, x, packed)
    print(f"{regime} d={d} b={b}/{b_tail} water={water}: flagged {flagged}, mismatched {mism}")
    # decode from the GPU's own records
    xh = codec.decode(packed, S, N, torch.float32).cpu().numpy()
    xb = codec.decode(packed, S, N, torch.bfloat16)
    xb64 = _f64(xb)
    for st in range(S):
        want = Q.decode(idx[st], models[st % H])
        rel = np.linalg.norm(xh[st] - want) / np.linalg.norm(want)
        assert rel < 1e-5, (st, rel)
        tol = np.abs(want) * 2.0 ** -8 + 1e-30
        assert np.all(np.abs(xb64[st] - want) <= tol + 2e-6 * np.abs(want).max())
    # scores
    nq = 17
    q = torch.randn(S, nq, d, generator=torch.Generator(device=DEV).manual_seed(5), device=DEV)
    sc = codec.qk_scores(q, packed, N).cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    for st in range(S):
        want = Q.scores(q64[st], idx[st], models[st % H])
        rel = np.linalg.norm(sc[st] - want, axis=1) / np.linalg.norm(want, axis=1)
        assert rel.max() < 2e-3, (st, rel.max())


@pytest.mark.parametrize("N", [1, 15, 16, 17, 33])
def test_sq_short_and_ragged_streams(N):
    codec, models, x = _case("lowrank_aligned", 128, 4, 2, False, 5, 3, N)
    packed = codec.encode(x)
    torch.cuda.synchronize()
    idx, _, _ = _check_encode(codec, models, x, packed)
    xh = codec.decode(packed, 5, N, torch.float32).cpu().numpy()
    for st in range(5):
        want = Q.decode(idx[st], models[st % 3])
        assert np.linalg.norm(xh[st] - want) <= 1e-5 * np.linalg.norm(want)
    q = torch.randn(5, 3, 128, generator=torch.Generator(device=DEV).manual_seed(140), device=DEV,
                    dtype=torch.bfloat16)
    sc = codec.qk_scores(q, packed, N).cpu().numpy()
    q64 = _f64(q)
    for st in range(5):
        want = Q.scores(q64[st], idx[st], models[st % 3])
        assert np.linalg.norm(sc[st] - want) <= 2e-3 * np.linalg.norm(want)


def test_sq_encode_leaves_other_bytes_and_handles_empty_input():
    codec, models, x = _case("lowrank_aligned", 64, 4, 2, False, 2, 2, 40)
    rb = codec.record_bytes
    buf = torch.full((2 * 40 * rb + 256,), 0xA5, dtype=torch.uint8, device=DEV)
    codec.encode(x, buf)
    torch.cuda.synchronize()
    assert torch.all(buf[2 * 40 * rb:] == 0xA5)
    empty = torch.empty(2, 0, 64, dtype=torch.bfloat16, device=DEV)
    codec.encode(empty, buf)
    codec.decode(buf, 2, 0)
    torch.cuda.synchronize()


def test_sq_many_queries_and_fp32_queries():
    codec, models, x = _case("isotropic", 64, 4, 2, False, 2, 1, 300)
    packed = codec.encode(x)
    idx, _, _ = _check_encode(codec, models, x, packed)
    for nq in (1, 256):
        q = torch.randn(2, nq, 64, generator=torch.Generator(device=DEV).manual_seed(160 + nq), device=DEV)
        sc = codec.qk_scores(q, packed, 300).cpu().numpy()
        q64 = q.cpu().numpy().astype(np.float64)
        for st in range(2):
            want = Q.scores(q64[st], idx[st], models[0])
            rel = np.linalg.norm(sc[st] - want, axis=1) / np.linalg.norm(want, axis=1)
            assert rel.max() < 2e-3


def test_sq_rejects_unsupported_inputs():
    codec, _, x = _case("isotropic", 64, 4, 2, False, 1, 1, 16)
    with pytest.raises(T.TQError) as e:
        codec.encode(x.float())
    assert e.value.status == T._lib.TQ_EUNSUPPORTED
    with pytest.raises(T.TQError):
        codec.qk_scores(torch.zeros(1, 257, 64, device=DEV), codec.encode(x), 16)


def _sq_models(regime, d, b, b_tail, hkv, seed):
    xc = _tokens(regime, hkv, 512, d, seed + 1000, hkv)
    codec = T.SQCodec.calibrate(xc.float(), b, b_tail, device=0)
    xc64 = _f64(xc)
    return codec, [Q.calibrate(xc64[h], b, b_tail) for h in range(hkv)]


@pytest.mark.parametrize("batch,hq,hkv,N,d,regime,bk,bv,lens,out_dtype", [
    (2, 8, 2, 1000, 128, "lowrank_aligned", (4, 2), (4, 2), None, torch.float32),
    (1, 4, 4, 777, 64, "isotropic", (3, 2), (2, 1), None, torch.bfloat16),
    (2, 16, 1, 300, 128, "lowrank_steep", (5, 2), (3, 2), None, torch.float32),
    (3, 8, 2, 600, 128, "lowrank_aligned", (4, 2), (4, 2), [600, 1, 0], torch.float32),
    (2, 4, 2, 2500, 128, "isotropic", (6, 6), (6, 6), [2500, 1234], torch.float32),
    (1, 2, 1, 64, 64, "isotropic", (8, 8), (8, 8), None, torch.float32),
])
def test_sq_decode_attention(batch, hq, hkv, N, d, regime, bk, bv, lens, out_dtype):
    S, G = batch * hkv, hq // hkv
    ck, mk = _sq_models(regime, d, bk[0], bk[1], hkv, 21)
    cv, mv = _sq_models(regime, d, bv[0], bv[1], hkv, 22)
    K = _tokens(regime, S, N, d, 31, hkv)
    V = _tokens(regime, S, N, d, 32, hkv)
    pk, pv = ck.encode(K), cv.encode(V)
    q = torch.randn(batch, hq, d, generator=torch.Generator(device=DEV).manual_seed(3), device=DEV)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = T.sq_decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=out_dtype, lengths=lt)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    q64 = q.cpu().numpy().astype(np.float64)
    rk = pk.cpu().numpy()[: S * N * ck.record_bytes].reshape(S, N, ck.record_bytes)
    rv = pv.cpu().numpy()[: S * N * cv.record_bytes].reshape(S, N, cv.record_bytes)
    scale = 1.0 / np.sqrt(d)
    rows, wants = [], []
    for b in range(batch):
        n_b = N if lens is None else lens[b]
        for h in range(hq):
            hk = h // G
            st = b * hkv + hk
            if n_b == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            ik = Q.unpack(rk[st, :n_b], mk[hk]["bits"])
            iv = Q.unpack(rv[st, :n_b], mv[hk]["bits"])
            sc = Q.scores(q64[b, h][None, :], ik, mk[hk])
            wants.append(Q.attention(sc, iv, mv[hk], scale)[0])
            rows.append(got[b, h])
    r = P.check_attention_rows(np.array(rows), np.array(wants), out_dtype == torch.bfloat16)
    print(f"sq attention worst row rel L2 {r['worst']:.2e} ({r['worst_unrounded']:.2e} against the unrounded oracle)")


def test_sq_attention_validates_arguments():
    ck, _ = _sq_models("isotropic", 64, 4, 2, 2, 21)
    c1, _ = _sq_models("isotropic", 64, 4, 2, 1, 21)
    q = torch.randn(1, 4, 64, generator=torch.Generator(device=DEV).manual_seed(237), device=DEV)
    pk = ck.encode(_tokens("isotropic", 2, 32, 64, 1, 2))
    with pytest.raises(T.TQError):          # codec heads must equal n_kv_heads
        T.sq_decode_attention(ck, c1, q, pk, pk, 2, 32)
    with pytest.raises(T.TQError):          # more than 16 query heads per kv head
        T.sq_decode_attention(ck, ck, torch.zeros(1, 34, 64, device=DEV), pk, pk, 2, 32)

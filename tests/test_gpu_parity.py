"""GPU parity of the HIP path (through the C ABI) against the oracle, on seeded synthetic inputs
shaped like the five workloads, at sizes the oracle finishes in seconds (several tiles plus a ragged
tail), and edge cases.  Full-size runs live in test_gpu_fullsize.py."""
import math

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
    T._lib.lib()            # fail loudly if libtq.so is missing
    yield


def _enc(codec, x):
    buf = T.encode(codec, x)
    torch.cuda.synchronize()
    return buf.cpu().numpy()


def _x64(x):
    if x.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(I.bf16_bits(x))
    return x.detach().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------------------------
# encode / decode over the parameter space
MATRIX = ([(d, b, 0, torch.bfloat16) for d in (64, 128, 256) for b in range(1, 7)]
          + [(128, b, 0, torch.bfloat16) for b in (7, 8)]
          + [(d, b, m, torch.bfloat16) for d in (64, 128, 256) for b in (2, 3, 4) for m in (32, d)]
          + [(256, b, 128, torch.bfloat16) for b in (3, 4)]
          + [(d, 4, 0, torch.float32) for d in (64, 128, 256)] + [(64, 3, 64, torch.float32)])


@pytest.mark.parametrize("d,b,m,dt", MATRIX)
def test_encode_decode_parity(d, b, m, dt):
    S, N, H, seed = 3, 37, 2, 900 + d + b + m
    codec = T.Codec(d, b, m, H, seed)
    x = I.gaussian((S, N, d), seed, device=DEV, dtype=dt)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, H, seed)
    st = P.check_encode(tb, _x64(x), buf)
    recs = st["recs"]
    xh = T.decode(codec, torch.as_tensor(buf, device=DEV), S, N, torch.float32).cpu().numpy()
    P.check_decode_f32(tb, recs, list(range(S)), xh)
    xb = T.decode(codec, torch.as_tensor(buf, device=DEV), S, N, torch.bfloat16)
    P.check_decode_bf16(tb, recs, list(range(S)), O.bf16_bits_to_f64(I.bf16_bits(xb)))


@pytest.mark.parametrize("m,rht", [(0, 0), (128, 0), (128, 1)])
def test_encode_parity_across_vector_scales(m, rht):
    """Vectors scaled by 2^-60, 2^-20, 2^-8, 1 and 2^8 (squared norms from about 2^-113 to 2^23):
    the normalisation (hardware square root and reciprocal square root) keeps every decision
    within the bands and the norms within one fp16 step.  Powers of two keep the bf16 inputs exact;
    at 2^-20 the fp16 norm is subnormal, at 2^-60 it rounds to 0 on both sides (a zero decode)."""
    d, b, H, N = 128, 4, 2, 40
    codec = T.Codec(d, b, m, H, 77, sketch=rht)
    base = I.gaussian((5, N, d), 78, device=DEV, dtype=torch.float32)
    scale = torch.tensor([2.0 ** -60, 2.0 ** -20, 2.0 ** -8, 1.0, 2.0 ** 8], device=DEV).view(5, 1, 1)
    x = (base * scale).to(torch.bfloat16)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, H, 77, sketch=rht)
    st = P.check_encode(tb, _x64(x), buf)
    xh = T.decode(codec, torch.as_tensor(buf, device=DEV), 5, N, torch.float32).cpu().numpy()
    P.check_decode_f32(tb, st["recs"], list(range(5)), xh)


@pytest.mark.parametrize("d,b,m,dt,S,H,N", [(128, 4, 128, torch.bfloat16, 5, 3, 1000),
                                              (128, 3, 0, torch.bfloat16, 7, 16, 333),
                                              (64, 3, 64, torch.float32, 4, 3, 517)])
def test_encode_many_tiles_per_wave(d, b, m, dt, S, H, N):
    """Many tiles per wave and block, streams not a multiple of heads (and more heads than streams):
    every vector matches the oracle; repeated launches and a launch on a second stream give the
    same packed fields."""
    seed = 4242 + d + b + m + S
    codec = T.Codec(d, b, m, H, seed)
    x = I.gaussian((S, N, d), seed, device=DEV, dtype=dt)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, H, seed)
    P.check_encode(tb, _x64(x), buf)

    def planes(bb):      # the packed fields (the alignment padding between planes is never written)
        return O.unpack_tensor(bb, d, b, m, S, N)

    ref = planes(buf)

    def same(bb):
        for r, o in zip(ref, planes(bb)):
            for k in r:
                assert np.array_equal(r[k], o[k]), k

    for _ in range(2):
        same(_enc(codec, x))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = T.encode(codec, x)
    side.synchronize()
    same(out.cpu().numpy())


def test_cfg1_full_round_trip_and_determinism():
    """Single head, d=64, 4096 fp32 keys with per-channel std U[0.5,2]; b=4, no QJL."""
    w = I.CONFIGS["cfg1"]
    codec = T.Codec(w.d, w.b, 0, 1, w.seed_k)
    xh = I.per_channel_gaussian(4096, 64, 1)[None]
    x = torch.as_tensor(xh, device=DEV)
    buf = _enc(codec, x)
    assert np.array_equal(buf, _enc(codec, x)), "encode is not deterministic"
    tb = P.Tables(w.d, w.b, 0, 1, w.seed_k)
    st = P.check_encode(tb, xh.astype(np.float64), buf)
    print(f"cfg1: flagged={st['flagged']} idx_mismatch={st['idx_mismatch']} n16_1ulp={st['n16_1ulp']}")
    out = T.decode(codec, torch.as_tensor(buf, device=DEV), 1, 4096, torch.float32).cpu().numpy()
    err = P.check_decode_f32(tb, st["recs"], [0], out)
    print(f"cfg1: decode rel L2 vs oracle {err:.2e}")


def test_cfg2_reduced_outliers():
    w = I.CONFIGS["cfg2"]
    S, N = 4, 1000
    for seed in (w.seed_k, w.seed_v):
        codec = T.Codec(128, 4, 0, S, seed)
        x = I.outlier_gaussian(S, N, 128, 4, 10.0, seed, device=DEV)
        buf = _enc(codec, x)
        tb = P.Tables(128, 4, 0, S, seed)
        st = P.check_encode(tb, _x64(x), buf)
        out = T.decode(codec, torch.as_tensor(buf, device=DEV), S, N, torch.float32).cpu().numpy()
        P.check_decode_f32(tb, st["recs"], list(range(S)), out)


@pytest.mark.parametrize("b,m,nq", [(3, 128, 32), (4, 0, 20), (2, 64, 7)])
def test_cfg3_reduced_scores(b, m, nq):
    S, N, seed = 2, 3000, 3001
    codec = T.Codec(128, b, m, S, seed)
    k = I.gaussian((S, N, 128), seed, device=DEV)
    q = I.gaussian((S, nq, 128), seed + 17, device=DEV)
    buf = _enc(codec, k)
    tb = P.Tables(128, b, m, S, seed)
    st = P.check_encode(tb, _x64(k), buf)
    sc = T.qk_scores(codec, q, torch.as_tensor(buf, device=DEV), N).cpu().numpy()
    worst = P.check_scores(tb, st["recs"], list(range(S)), _x64(q), sc)
    print(f"scores b={b} m={m}: worst row rel L2 {worst:.2e}")


def _attention_case(batch, hq, hkv, N, d, b, m, out_dtype, seed=4001, scale=0.0, sketch=0, rotation=0):
    ck, cv = T.Codec(d, b, m, hkv, seed, sketch, rotation), T.Codec(d, b, 0, hkv, seed + 1)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    q = I.cfg4_queries(batch, hq, d, N, seed + 2, device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    out = T.decode_attention(ck, cv, q, pk, pv, hkv, N, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    tk, tv = P.Tables(d, b, m, hkv, seed, sketch, rotation), P.Tables(d, b, 0, hkv, seed + 1)
    rk = O.unpack_tensor(pk.cpu().numpy(), d, b, m, batch * hkv, N)
    rv = O.unpack_tensor(pv.cpu().numpy(), d, b, 0, batch * hkv, N)
    q64 = _x64(q)
    sc = scale if scale > 0 else 1.0 / math.sqrt(d)
    g = hq // hkv
    ref = np.zeros((batch, hq, d))
    for bi in range(batch):
        for h in range(hq):
            st = bi * hkv + h // g
            ref[bi, h] = P.oracle_attention_row(tk, tv, rk[st], rv[st], st, q64[bi, h], sc)
    got = out.float().cpu().numpy().astype(np.float64)
    return P.check_attention_rows(got, ref, out_dtype == torch.bfloat16)


@pytest.mark.parametrize("batch,hq,hkv,N,d,b,m", [
    (2, 8, 2, 5000, 128, 4, 128),      # cfg4 shape, reduced; several splits + ragged tail
    (1, 4, 4, 777, 128, 4, 0),         # MHA, no QJL
    (2, 16, 1, 2100, 64, 4, 64),       # d=64, 16 queries per kv head
    (1, 6, 2, 1500, 256, 3, 256),      # d=256, b=3
    (1, 2, 1, 33, 128, 2, 32),         # tiny cache
])
def test_decode_attention_reduced(batch, hq, hkv, N, d, b, m):
    r32 = _attention_case(batch, hq, hkv, N, d, b, m, torch.float32)
    rb = _attention_case(batch, hq, hkv, N, d, b, m, torch.bfloat16)
    print(f"attention {batch}x{hq}/{hkv} N={N} d={d} b={b} m={m}: worst row rel L2 f32 {r32['worst']:.2e},"
          f" bf16 {rb['worst']:.2e} against the rounded oracle ({rb['worst_unrounded']:.2e} unrounded,"
          f" rounding floor {rb['floor']:.2e})")


# shapes whose split count is a multiple of the 12 waves of a block, so every block covers one
# stream and the attention kernel runs the query prep itself (4-bit keys and values, d <= 128, at
# most 8 query heads per kv head)
@pytest.mark.parametrize("batch,hq,hkv,N,d,m,rot", [
    (2, 8, 2, 3072, 128, 128, 0),      # 12 splits of 256 tokens
    (2, 8, 2, 3000, 128, 128, 0),      # 12 splits, ragged last split
    (1, 8, 1, 6144, 128, 128, 0),      # one stream, 24 splits, 8 query heads per kv head
    (2, 4, 2, 3072, 64, 64, 0),        # d = 64
    (2, 4, 4, 3072, 128, 0, 0),        # no sketch, one query head per kv head
    (2, 8, 2, 3072, 128, 32, 0),       # m = 32
    (2, 8, 2, 3072, 128, 128, 1),      # Plain-KV keys (no rotation of the queries)
])
def test_decode_attention_in_kernel_query_prep(batch, hq, hkv, N, d, m, rot):
    print(f"attention with the in-kernel query prep {batch}x{hq}/{hkv} N={N} d={d} m={m} rotation={rot}", flush=True)
    r32 = _attention_case(batch, hq, hkv, N, d, 4, m, torch.float32, seed=4301 + N + m, rotation=rot)
    rb = _attention_case(batch, hq, hkv, N, d, 4, m, torch.bfloat16, seed=4301 + N + m, rotation=rot)
    print(f"  worst row rel L2 f32 {r32['worst']:.2e}, bf16 {rb['worst']:.2e} against the rounded oracle")


# ---------------------------------------------------------------------------------------------
# randomized Hadamard sketch (S = H diag(s2), m = d)
@pytest.mark.parametrize("d,b,dt", [(64, 3, torch.bfloat16), (128, 2, torch.bfloat16), (128, 4, torch.bfloat16),
                                    (256, 3, torch.bfloat16), (128, 3, torch.float32)])
def test_rht_encode_decode_scores_parity(d, b, dt):
    S, N, H, nq, seed = 3, 700, 2, 9, 6100 + d + b
    codec = T.Codec(d, b, d, H, seed, sketch=1)
    x = I.gaussian((S, N, d), seed, device=DEV, dtype=dt)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, d, H, seed, sketch=1)
    st = P.check_encode(tb, _x64(x), buf)
    out = T.decode(codec, torch.as_tensor(buf, device=DEV), S, N, torch.float32).cpu().numpy()
    P.check_decode_f32(tb, st["recs"], list(range(S)), out)
    q = I.gaussian((S, nq, d), seed + 5, device=DEV)
    sc = T.qk_scores(codec, q, torch.as_tensor(buf, device=DEV), N).cpu().numpy()
    worst = P.check_scores(tb, st["recs"], list(range(S)), _x64(q), sc)
    print(f"rht d={d} b={b}: flagged={st['flagged']} sketch_flagged={st['sketch_flagged']} scores row max {worst:.2e}")


@pytest.mark.parametrize("d,b,m,kind", [(128, 4, 128, 0), (64, 3, 64, 0), (256, 3, 128, 0), (128, 2, 32, 0),
                                         (128, 4, 128, 1), (64, 2, 64, 1), (128, 6, 96, 0),
                                         (256, 3, 256, 0), (256, 6, 256, 0)])
def test_decode_with_qjl_correction(d, b, m, kind):
    """tq_decode_qjl: n16 · s ⊙ H (c[idx] + sqrt(pi/2)/m · r16 · S^T (2σ - 1)) / sqrt(d), from the GPU's
    packed fields; fp32 within 1e-5 relative L2, bf16 within one rounding."""
    S, N, H, seed = 3, 530, 2, 7300 + d + b + m + kind
    codec = T.Codec(d, b, m, H, seed, kind)
    x = I.gaussian((S, N, d), seed, device=DEV)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, H, seed, kind)
    recs = O.unpack_tensor(buf, d, b, m, S, N)
    gbuf = torch.as_tensor(buf, device=DEV)
    out = T.decode(codec, gbuf, S, N, torch.float32, qjl=True).cpu().numpy()
    err = P.check_decode_f32(tb, recs, list(range(S)), out, qjl=True)
    xb = T.decode(codec, gbuf, S, N, torch.bfloat16, qjl=True)
    P.check_decode_bf16(tb, recs, list(range(S)), O.bf16_bits_to_f64(I.bf16_bits(xb)), qjl=True)
    # the correction brings the reconstruction closer to the input
    plain = T.decode(codec, gbuf, S, N, torch.float32).cpu().numpy()
    x64 = _x64(x)
    e_plain, e_corr = np.sum((plain - x64) ** 2), np.sum((out - x64) ** 2)
    print(f"qjl decode d={d} b={b} m={m} kind={kind}: rel L2 vs oracle {err:.2e}; error vs input "
          f"{e_corr / e_plain:.3f} of the MSE decode's")
    if kind == 1:
        assert e_corr < 0.75 * e_plain


def test_decode_with_qjl_correction_limits():
    x = I.gaussian((1, 40, 128), 3, device=DEV)
    buf = T.encode(T.Codec(128, 4, 0, 1, 3), x)
    with pytest.raises(T._lib.TQError):                       # no sketch to correct with
        T.decode(T.Codec(128, 4, 0, 1, 3), buf, 1, 40, qjl=True)


@pytest.mark.parametrize("batch,hq,hkv,N,d,b", [(2, 8, 2, 3000, 128, 4), (1, 4, 2, 900, 256, 3), (1, 8, 1, 500, 64, 4)])
def test_rht_decode_attention(batch, hq, hkv, N, d, b):
    r32 = _attention_case(batch, hq, hkv, N, d, b, d, torch.float32, sketch=1)
    rb = _attention_case(batch, hq, hkv, N, d, b, d, torch.bfloat16, sketch=1)
    print(f"rht attention d={d} b={b}: worst row rel L2 f32 {r32['worst']:.2e}, bf16 {rb['worst']:.2e}")


# ---------------------------------------------------------------------------------------------
# growing caches: appends at an offset, and attention over per-batch lengths
@pytest.mark.parametrize("d,b,m,kind,dt", [(128, 4, 128, 0, torch.bfloat16), (128, 3, 0, 0, torch.bfloat16),
                                           (64, 4, 64, 1, torch.bfloat16), (128, 4, 128, 0, torch.float32)])
def test_encode_append_equals_one_encode(d, b, m, kind, dt):
    S, cap, H, seed = 3, 1000, 3, 8800 + d + b + m + kind
    codec = T.Codec(d, b, m, H, seed, kind)
    x = I.gaussian((S, cap, d), seed, device=DEV, dtype=dt)
    whole = _enc(codec, x)
    lay = T.get_layout(codec, S, cap)
    buf = torch.full((lay["total_bytes"],), 0xA5, dtype=torch.uint8, device=DEV)
    cuts = [0, 300, 301, 717, 718, 1000]                      # tile-aligned and ragged offsets, 1-token steps
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        T.encode_append(codec, x[:, t0:t1].contiguous(), buf, cap, t0)
    torch.cuda.synchronize()
    got = O.unpack_tensor(buf.cpu().numpy(), d, b, m, S, cap)
    ref = O.unpack_tensor(whole, d, b, m, S, cap)
    for r, g in zip(ref, got):
        for k in r:
            assert np.array_equal(r[k], g[k]), k
    # an append writes only its own records: a fresh buffer keeps the fill outside [t0, t1)
    part = torch.full((lay["total_bytes"],), 0xA5, dtype=torch.uint8, device=DEV)
    T.encode_append(codec, x[:, 301:717].contiguous(), part, cap, 301)
    pb = part.cpu().numpy()
    ib = d * b // 8
    for st in range(S):
        lo, hi = lay["off_idx"] + (st * cap + 301) * ib, lay["off_idx"] + (st * cap + 717) * ib
        row0, row1 = lay["off_idx"] + st * cap * ib, lay["off_idx"] + (st + 1) * cap * ib
        assert np.all(pb[row0:lo] == 0xA5) and np.all(pb[hi:row1] == 0xA5)
        assert np.array_equal(pb[lo:hi], whole[lo:hi])
    tb = P.Tables(d, b, m, H, seed, kind)
    P.check_encode(tb, _x64(x[:1]), buf.cpu().numpy(), streams=[0], n_streams=S, n_tokens=cap)


@pytest.mark.parametrize("lens", [(3000, 37, 1999), (0, 513, 3000)])
def test_decode_attention_per_batch_lengths(lens):
    batch, hq, hkv, N, d, b, m, seed = 3, 8, 2, 3000, 128, 4, 128, 4101
    ck, cv = T.Codec(d, b, m, hkv, seed), T.Codec(d, b, 0, hkv, seed + 1)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    q = I.cfg4_queries(batch, hq, d, N, seed + 2, device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = T.decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=torch.float32, lengths=ln).cpu().numpy()
    tk, tv = P.Tables(d, b, m, hkv, seed), P.Tables(d, b, 0, hkv, seed + 1)
    rk = O.unpack_tensor(pk.cpu().numpy(), d, b, m, batch * hkv, N)
    rv = O.unpack_tensor(pv.cpu().numpy(), d, b, 0, batch * hkv, N)
    q64 = _x64(q)
    g = hq // hkv
    for bi in range(batch):
        L = lens[bi]
        for h in range(hq):
            if L == 0:
                assert np.all(out[bi, h] == 0.0)
                continue
            st = bi * hkv + h // g
            cut = lambda r: {k: v[:L] for k, v in r.items()}
            ref = P.oracle_attention_row(tk, tv, cut(rk[st]), cut(rv[st]), st, q64[bi, h], 1 / math.sqrt(d))
            assert P.rel_l2(out[bi, h], ref) <= 2e-3, (bi, h, L)


# ---------------------------------------------------------------------------------------------
# Plain-KV: the Beta codebook on the unrotated unit vector (rotation = none)
@pytest.mark.parametrize("d,b,m,kind,dt", [(128, 4, 0, 0, torch.bfloat16), (128, 3, 128, 0, torch.bfloat16),
                                           (64, 2, 64, 1, torch.bfloat16), (256, 5, 0, 0, torch.bfloat16),
                                           (128, 4, 32, 0, torch.float32)])
def test_plain_encode_decode_scores_parity(d, b, m, kind, dt):
    S, N, H, nq, seed = 2, 600, 2, 5, 9100 + d + b + m
    codec = T.Codec(d, b, m, H, seed, kind, rotation=1)
    x = I.gaussian((S, N, d), seed, device=DEV, dtype=dt)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, H, seed, kind, rotation=1)
    st = P.check_encode(tb, _x64(x), buf)
    gbuf = torch.as_tensor(buf, device=DEV)
    out = T.decode(codec, gbuf, S, N, torch.float32).cpu().numpy()
    P.check_decode_f32(tb, st["recs"], list(range(S)), out)
    if m:
        outq = T.decode(codec, gbuf, S, N, torch.float32, qjl=True).cpu().numpy()
        P.check_decode_f32(tb, st["recs"], list(range(S)), outq, qjl=True)
    q = I.gaussian((S, nq, d), seed + 3, device=DEV)
    sc = T.qk_scores(codec, q, gbuf, N).cpu().numpy()
    P.check_scores(tb, st["recs"], list(range(S)), _x64(q), sc)


@pytest.mark.parametrize("rk,rv", [(1, 1), (1, 0), (0, 1)])
def test_plain_decode_attention(rk, rv):
    batch, hq, hkv, N, d, b, m, seed = 2, 8, 2, 1500, 128, 4, 128, 9300
    ck, cv = T.Codec(d, b, m, hkv, seed, rotation=rk), T.Codec(d, b, 0, hkv, seed + 1, rotation=rv)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    q = I.cfg4_queries(batch, hq, d, N, seed + 2, device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    out = T.decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=torch.float32).cpu().numpy()
    tk, tv = P.Tables(d, b, m, hkv, seed, rotation=rk), P.Tables(d, b, 0, hkv, seed + 1, rotation=rv)
    rkk = O.unpack_tensor(pk.cpu().numpy(), d, b, m, batch * hkv, N)
    rvv = O.unpack_tensor(pv.cpu().numpy(), d, b, 0, batch * hkv, N)
    q64 = _x64(q)
    g = hq // hkv
    for bi in range(batch):
        for h in range(hq):
            st = bi * hkv + h // g
            ref = P.oracle_attention_row(tk, tv, rkk[st], rvv[st], st, q64[bi, h], 1 / math.sqrt(d))
            assert P.rel_l2(out[bi, h], ref) <= 2e-3, (bi, h)


def test_decode_attention_explicit_scale():
    _attention_case(1, 4, 2, 900, 128, 4, 128, torch.float32, scale=0.05)


@pytest.mark.parametrize("b", [2, 3, 5, 6])
@pytest.mark.parametrize("m", [0, 256])
def test_cfg5_reduced_heavy_tail(b, m):
    S, N, nq, seed = 2, 1200, 8, 5001
    codec = T.Codec(256, b, m, S, seed + b)
    k = I.student_t(S, N, 256, 3, seed, device=DEV)
    q = I.gaussian((S, nq, 256), seed + 99, device=DEV)
    buf = _enc(codec, k)
    tb = P.Tables(256, b, m, S, seed + b)
    st = P.check_encode(tb, _x64(k), buf)
    out = T.decode(codec, torch.as_tensor(buf, device=DEV), S, N, torch.float32).cpu().numpy()
    P.check_decode_f32(tb, st["recs"], list(range(S)), out)
    sc = T.qk_scores(codec, q, torch.as_tensor(buf, device=DEV), N).cpu().numpy()
    P.check_scores(tb, st["recs"], list(range(S)), _x64(q), sc)


# ---------------------------------------------------------------------------------------------
# short rows, cancelling scores, query scales, few-token attention
def _estimator_vectors(tb, rec, st):
    """w_t with ŝ(q, k_t) = <q, w_t>: the estimate is linear in q (q_rot = R q), so
    w_t = n16 · R^T (ŷ + sqrt(pi/2)/m · r16 · S^T(2σ - 1)), the QJL-corrected reconstruction."""
    h = tb.head(st)
    corr = O.qjl_correction(rec["sigma"], rec["r16"], tb.S[h]) if tb.m else None
    return O.decode(rec["idx"], rec["n16"], tb.s[h], tb.c, corr)


@pytest.mark.parametrize("N", [1, 2, 15, 17, 33])
@pytest.mark.parametrize("m", [0, 128])
def test_scores_short_rows_and_cancelling_scores(N, m):
    """Rows of a few tokens, where errors cannot average out.  Query 0 of every stream is made
    orthogonal (in fp64, then rounded to fp32) to the estimator vector of token 0, so its estimate
    cancels to ~1e-8 of |q| |w|: within a row of N >= 2 the row bar applies; alone (N = 1) the error
    is held to 2e-3 of |q| |w|, the scale of that inner product."""
    d, b, S, nq, seed = 128, 3, 3, 5, 7300 + N + m
    codec = T.Codec(d, b, m, S, seed)
    k = I.gaussian((S, N, d), seed, device=DEV)
    buf = _enc(codec, k)
    tb = P.Tables(d, b, m, S, seed)
    st = P.check_encode(tb, _x64(k), buf)
    q64 = np.random.default_rng(seed + 1).standard_normal((S, nq, d))
    for s_ in range(S):
        w0 = _estimator_vectors(tb, st["recs"][s_], s_)[0]
        q64[s_, 0] -= (q64[s_, 0] @ w0) / (w0 @ w0) * w0
    q = torch.tensor(q64, dtype=torch.float32, device=DEV)
    q64 = q.cpu().numpy().astype(np.float64)
    sc = T.qk_scores(codec, q, torch.as_tensor(buf, device=DEV), N).cpu().numpy()
    worst = 0.0
    for s_ in range(S):
        ref = P.oracle_scores(tb, st["recs"][s_], s_, q64[s_])
        w = _estimator_vectors(tb, st["recs"][s_], s_)
        assert abs(ref[0, 0]) < 1e-6 * np.linalg.norm(q64[s_, 0]) * np.linalg.norm(w[0])
        for i in range(nq):
            if N == 1 and i == 0:
                err = abs(sc[s_, 0, 0] - ref[0, 0]) / (np.linalg.norm(q64[s_, 0]) * np.linalg.norm(w[0]))
            else:
                err = P.rel_l2(sc[s_, i], ref[i])
            worst = max(worst, err)
            assert err <= 2e-3, (s_, i, err)
    print(f"short rows N={N} m={m}: worst {worst:.2e}")


@pytest.mark.parametrize("scale", [2.0 ** -30, 2.0 ** -12, 1.0, 2.0 ** 8])
def test_scores_across_query_scales(scale):
    """fp32 queries from 2^-30 to 2^8 times N(0,1): the per-row power of two keeps every operand in
    the fp16 range (no subnormal loss, no overflow)."""
    d, b, m, S, N, nq, seed = 128, 4, 128, 2, 40, 6, 7400
    codec = T.Codec(d, b, m, S, seed)
    k = I.gaussian((S, N, d), seed, device=DEV)
    buf = _enc(codec, k)
    tb = P.Tables(d, b, m, S, seed)
    st = P.check_encode(tb, _x64(k), buf)
    q = torch.tensor(np.random.default_rng(seed + 2).standard_normal((S, nq, d)) * scale, dtype=torch.float32,
                     device=DEV)
    sc = T.qk_scores(codec, q, torch.as_tensor(buf, device=DEV), N).cpu().numpy()
    worst = P.check_scores(tb, st["recs"], list(range(S)), _x64(q), sc)
    print(f"query scale {scale:.3g}: worst row rel L2 {worst:.2e}")


@pytest.mark.parametrize("N", [1, 2, 3])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_attention_few_tokens(N, out_dtype):
    r = _attention_case(2, 8, 2, N, 128, 4, 128, out_dtype, seed=4101 + N)
    print(f"attention over {N} tokens ({out_dtype}): worst row rel L2 {r['worst']:.2e}")


def _query_scale_case(scale, N, hq, b, seed=4201):
    d, m, batch, hkv = 128, 128, 1, 2
    ck, cv = T.Codec(d, b, m, hkv, seed), T.Codec(d, b, 0, hkv, seed + 1)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    q = torch.tensor(np.random.default_rng(seed).standard_normal((batch, hq, d)) * scale, dtype=torch.float32,
                     device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    out = T.decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tk, tv = P.Tables(d, b, m, hkv, seed), P.Tables(d, b, 0, hkv, seed + 1)
    rk = O.unpack_tensor(pk.cpu().numpy(), d, b, m, batch * hkv, N)
    rv = O.unpack_tensor(pv.cpu().numpy(), d, b, 0, batch * hkv, N)
    q64 = _x64(q)
    g = hq // hkv
    ref = np.array([[P.oracle_attention_row(tk, tv, rk[h // g], rv[h // g], h // g, q64[0, h], 1 / math.sqrt(d))
                     for h in range(hq)]])
    r = P.check_attention_rows(out.cpu().numpy(), ref, False)
    print(f"attention query scale {scale:.3g}, {hq} query heads over {hkv} kv heads, b = {b}, {N} tokens: "
          f"worst row rel L2 {r['worst']:.2e}")


@pytest.mark.parametrize("N", [700, 3072])        # 3072: the in-kernel query prep (12 splits per stream)
@pytest.mark.parametrize("scale", [2.0 ** -20, 2.0 ** 6])
def test_decode_attention_across_query_scales(scale, N):
    _query_scale_case(scale, N, 4, 4)


def test_decode_attention_zero_and_tiny_query_rows():
    """rows of one group with very different scales in the in-kernel query prep (3072 tokens: 12
    splits per stream): an all-zero row (uniform softmax: the mean of the decoded values), a row
    scaled by 2^-30 and a row scaled by 2^8 beside an ordinary one; each row takes its own power of
    two"""
    d, b, m, batch, hq, hkv, N, seed = 128, 4, 128, 1, 8, 2, 3072, 4281
    ck, cv = T.Codec(d, b, m, hkv, seed), T.Codec(d, b, 0, hkv, seed + 1)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    qn = np.random.default_rng(seed).standard_normal((batch, hq, d))
    qn[0, 0] = 0.0
    qn[0, 1] *= 2.0 ** -30
    qn[0, 2] *= 2.0 ** 8
    qn[0, 5] = 0.0                              # a zero row in the second group too
    q = torch.tensor(qn, dtype=torch.float32, device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    out = T.decode_attention(ck, cv, q, pk, pv, hkv, N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tk, tv = P.Tables(d, b, m, hkv, seed), P.Tables(d, b, 0, hkv, seed + 1)
    rk = O.unpack_tensor(pk.cpu().numpy(), d, b, m, batch * hkv, N)
    rv = O.unpack_tensor(pv.cpu().numpy(), d, b, 0, batch * hkv, N)
    g, q64 = hq // hkv, _x64(q)
    ref = np.array([[P.oracle_attention_row(tk, tv, rk[h // g], rv[h // g], h // g, q64[0, h], 1 / math.sqrt(d))
                     for h in range(hq)]])
    r = P.check_attention_rows(out.cpu().numpy(), ref, False)
    print(f"zero, 2^-30 and 2^8 query rows: worst row rel L2 {r['worst']:.2e}")


# more than 8 query heads per kv head: the sketch term's lo parts take their own MFMAs (no free
# query columns); b = 3 runs the geometry without the shared 4-bit tables
@pytest.mark.parametrize("hq,b", [(32, 4), (32, 3), (4, 3)])
def test_decode_attention_sharp_softmax_other_geometries(hq, b):
    _query_scale_case(2.0 ** 6, 1000, hq, b, seed=4251 + b)


# ---------------------------------------------------------------------------------------------
# edge cases
def test_zero_vectors_and_single_token():
    d, b = 128, 4
    codec = T.Codec(d, b, 128, 1, 3)
    x = torch.zeros(1, 1, d, dtype=torch.bfloat16, device=DEV)
    buf = _enc(codec, x)
    r = O.unpack_tensor(buf, d, b, 128, 1, 1)[0]
    assert np.all(r["idx"] == 8) and r["n16"][0] == 0 and r["r16"][0] >= 0
    out = T.decode(codec, torch.as_tensor(buf, device=DEV), 1, 1).cpu().numpy()
    assert np.all(out == 0)


@pytest.mark.parametrize("d,b,m", [(64, 1, 0), (128, 2, 0), (128, 3, 128), (128, 4, 128), (64, 4, 64)])
def test_encode_rotation_aligned_vectors(d, b, m):
    """Vectors whose rotation is exactly +-e_j (x = c * sign * s ⊙ H[:, j], so y_j = +-1 and the
    other coordinates are 0): the two ends of the quantiser's domain, and coordinates lying on the
    middle threshold (t = 0 of the symmetric codebook, flagged by the oracle).  Scales c are powers of
    two, so the bf16 inputs are exact."""
    seed = 77 + d + b + m
    codec = T.Codec(d, b, m, 1, seed)
    s = O.head_signs(seed, 0, d)
    Hm = O.hadamard(d)
    cols = np.arange(d)
    rows = []
    for c in (0.5, 4.0, 2.0 ** -10):
        for sign in (1.0, -1.0):
            rows.append(sign * c * (s[None, :] * Hm[:, cols].T))
    x64 = np.concatenate(rows, axis=0)[None]                  # [1, 6 d, d]
    x = torch.as_tensor(x64, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    assert np.array_equal(_x64(x), x64)
    buf = _enc(codec, x)
    tb = P.Tables(d, b, m, 1, seed)
    st = P.check_encode(tb, x64, buf)
    idx = st["recs"][0]["idx"]
    L = 1 << b
    y = np.stack([O.rotate(v / np.linalg.norm(v), s) for v in x64[0]])
    ends = np.abs(y) > 0.5
    assert ends.sum() == x64.shape[1]
    assert np.all(idx[ends & (y > 0)] == L - 1) and np.all(idx[ends & (y < 0)] == 0)
    xh = T.decode(codec, torch.as_tensor(buf, device=DEV), 1, x64.shape[1], torch.float32).cpu().numpy()
    P.check_decode_f32(tb, st["recs"], [0], xh)
    print(f"rotation-aligned d={d} b={b} m={m}: flagged {st['flagged']}, index mismatches {st['idx_mismatch']}")


def test_norm_above_fp16_range_is_inf():
    d = 64
    codec = T.Codec(d, 3, 0, 1, 5)
    x = torch.full((1, 2, d), 1.0e4, dtype=torch.float32, device=DEV)   # norm 8e4 > 65504
    buf = _enc(codec, x)
    r = O.unpack_tensor(buf, d, 3, 0, 1, 2)[0]
    assert np.all(np.isinf(r["n16"]))


def test_empty_inputs_are_noops():
    codec = T.Codec(128, 4, 0, 1, 0)
    x = torch.zeros(0, 5, 128, dtype=torch.bfloat16, device=DEV)
    T.encode(codec, x)
    torch.cuda.synchronize()


def test_misaligned_pointer_rejected():
    codec = T.Codec(64, 4, 0, 1, 0)
    x = torch.zeros(2 * 64 * 2 + 8, dtype=torch.bfloat16, device=DEV)
    xm = x[1:1 + 2 * 64].view(1, 2, 64)        # 2-byte offset
    with pytest.raises(T.TQError) as ei:
        T.encode(codec, xm)
    assert ei.value.status == T._lib.TQ_EALIGN


def test_unsupported_attention_combination():
    ck, cv = T.Codec(128, 4, 128, 2, 1), T.Codec(128, 2, 0, 2, 2)
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device=DEV)
    pk = torch.zeros(T.get_layout(ck, 2, 64)["total_bytes"], dtype=torch.uint8, device=DEV)
    pv = torch.zeros(T.get_layout(cv, 2, 64)["total_bytes"], dtype=torch.uint8, device=DEV)
    with pytest.raises(T.TQError) as ei:
        T.decode_attention(ck, cv, q, pk, pv, 2, 64)
    assert ei.value.status == T._lib.TQ_EUNSUPPORTED

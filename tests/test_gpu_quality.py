"""Quality of the HIP path on the pages' synthetic regimes ([AB] §2 "Error metric", eq. (2)), and a
statistical comparison of the HIP path with the oracle under different seeds ([AB] §5, which compares
two implementations with different random generators by a Kolmogorov-Smirnov test).

Metrics, for T = softmax(q Kᵀ/sqrt(d)) V on the exact bf16 cache and T̂ on the compressed one:
  relMSE_T = ||T - T̂||²_F / ||T||²_F;  d2 = sqrt((1 - cos(T, T̂))² + NF²), NF = relMSE_T/(1 + relMSE_T);
  relMSE_K: only K compressed (scores from tq_qk_scores, exact V); relMSE_V: only V compressed;
  ptcosine_K/V: mean over tokens of cos(k, k̂) with k̂ from tq_decode.
cos(T, T̂) is taken over the flattened outputs (the pages do not say per row or whole).
On the key path alone ([AB] §5 "Jensen's inequality", its Figure 2 and Table 2; [SI] abstract):
  KL = KL(softmax(q·k/sqrt d) || softmax(ŝ/sqrt d)) per query, ŝ the score estimates of tq_qk_scores;
  top-5 recall = |top5(q·k) ∩ top5(ŝ)| / 5 per query (the pages name the metric without defining it;
  this is the plain reading: the share of the five highest exact scores among the five highest
  estimates).
These are measurements with sanity bounds, not parity; parity lives in test_gpu_parity.py."""
import math

import numpy as np
import pytest
import torch
from scipy import stats

import kv_cache_transform_amd as T
from oracle import tq_oracle as O
from synth import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H, N, D, NQ = 4, 2048, 128, 16


def _f64(x):
    return O.bf16_bits_to_f64(I.bf16_bits(x))


def _softmax(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def _regime(name, seed):
    if name == "gaussian":
        return I.gaussian((H, N, D), seed, device=DEV), I.gaussian((H, N, D), seed + 1, device=DEV)
    if name == "outlier":
        return (I.outlier_gaussian(H, N, D, 4, 10.0, seed, device=DEV),
                I.outlier_gaussian(H, N, D, 4, 10.0, seed + 1, device=DEV))
    return I.student_t(H, N, D, 3, seed, device=DEV), I.student_t(H, N, D, 3, seed + 1, device=DEV)


def _metrics(K, V, q, b, m, kind, seed):
    ck, cv = T.Codec(D, b, m, H, seed, kind), T.Codec(D, b, 0, H, seed + 7)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    k64, v64, q64 = _f64(K), _f64(V), _f64(q)                      # [H,N,D], [H,N,D], [1,H*NQ,D]
    qh = q64[0].reshape(H, NQ, D)
    sc = 1.0 / math.sqrt(D)
    Tref = np.stack([_softmax(qh[h] @ k64[h].T * sc) @ v64[h] for h in range(H)])
    That = T.decode_attention(ck, cv, q, pk, pv, H, N, out_dtype=torch.float32).cpu().numpy()[0].reshape(H, NQ, D)
    s_hat = T.qk_scores(ck, q[0].reshape(H, NQ, D).contiguous(), pk, N).cpu().numpy()
    khat = T.decode(ck, pk, H, N, torch.float32).cpu().numpy()
    vhat = T.decode(cv, pv, H, N, torch.float32).cpu().numpy()
    TK = np.stack([_softmax(s_hat[h] * sc) @ v64[h] for h in range(H)])
    TV = np.stack([_softmax(qh[h] @ k64[h].T * sc) @ vhat[h] for h in range(H)])

    def rel(a, r):
        return float(np.sum((a - r) ** 2) / np.sum(r ** 2))

    def ptcos(a, r):
        num = np.sum(a * r, axis=-1)
        den = np.linalg.norm(a, axis=-1) * np.linalg.norm(r, axis=-1)
        return float(np.mean(num / np.maximum(den, 1e-300)))

    rT = rel(That, Tref)
    cos = float(np.sum(That * Tref) / (np.linalg.norm(That) * np.linalg.norm(Tref)))
    nf = rT / (1 + rT)
    per_query = np.sum((That - Tref) ** 2, axis=-1) / np.sum(Tref ** 2, axis=-1)
    return dict(relMSE_T=rT, d2=math.hypot(1 - cos, nf), relMSE_K=rel(TK, Tref), relMSE_V=rel(TV, Tref),
                ptcos_K=ptcos(khat, k64), ptcos_V=ptcos(vhat, v64), per_query=per_query.ravel())


@pytest.mark.parametrize("regime", ["gaussian", "outlier", "student_t"])
def test_quality_across_budgets_and_schemes(regime):
    K, V = _regime(regime, 600)
    q = I.gaussian((1, H * NQ, D), 609, device=DEV)
    rows = {}
    for b in (2, 3, 4):
        for m, kind, label in ((0, 0, "TQ-KV"), (D, 1, "TQ-QKV (RHT)")):
            r = _metrics(K, V, q, b, m, kind, 1000 + b)
            rows[(b, label)] = r
            print(f"{regime:9s} b={b} {label:13s} relMSE_T {r['relMSE_T']:.4f} d2 {r['d2']:.4f} "
                  f"relMSE_K {r['relMSE_K']:.4f} relMSE_V {r['relMSE_V']:.4f} "
                  f"ptcos_K {r['ptcos_K']:.4f} ptcos_V {r['ptcos_V']:.4f}")
            assert 0.0 <= r["d2"] <= math.sqrt(2.0)
    for label in ("TQ-KV", "TQ-QKV (RHT)"):
        e = [rows[(b, label)]["relMSE_T"] for b in (2, 3, 4)]
        assert e[0] > e[1] > e[2], (label, e)                    # more bits, less error
        c = [rows[(b, label)]["ptcos_V"] for b in (2, 3, 4)]
        assert c[0] < c[1] < c[2] and c[2] > 0.99, (label, c)


def test_hip_and_oracle_agree_in_distribution_with_different_seeds():
    """[AB] §5 style: the per-query relMSE_T of the HIP path (seeds A) and of the oracle (seeds B)
    come from the same distribution (two-sample KS test)."""
    Hs, Ns, nq, b = 48, 256, 4, 3        # many independent sign draws, few queries sharing each
    K = I.gaussian((Hs, Ns, D), 71, device=DEV)
    V = I.gaussian((Hs, Ns, D), 72, device=DEV)
    q = I.gaussian((1, Hs * nq, D), 73, device=DEV)
    k64, v64, q64 = _f64(K), _f64(V), _f64(q)[0].reshape(Hs, nq, D)
    sc = 1.0 / math.sqrt(D)
    Tref = np.stack([_softmax(q64[h] @ k64[h].T * sc) @ v64[h] for h in range(Hs)])
    ck, cv = T.Codec(D, b, 0, Hs, 11), T.Codec(D, b, 0, Hs, 12)
    pk, pv = T.encode(ck, K), T.encode(cv, V)
    gpu = T.decode_attention(ck, cv, q, pk, pv, Hs, Ns, out_dtype=torch.float32).cpu().numpy()[0].reshape(Hs, nq, D)
    def oracle(bits):
        t, c = O.lloyd_max(D, bits)
        out = []
        for h in range(Hs):
            sk, sv = O.head_signs(911, h, D), O.head_signs(912, h, D)
            rk, rv = O.encode(k64[h], sk, t, c), O.encode(v64[h], sv, t, c)
            out.append(O.attention_rotated(O.scores(q64[h], rk, sk, c), rv, sv, c, sc))
        return np.stack(out)

    def pq(a):
        return (np.sum((a - Tref) ** 2, axis=-1) / np.sum(Tref ** 2, axis=-1)).ravel()

    p = stats.ks_2samp(pq(gpu), pq(oracle(b))).pvalue
    p_off = stats.ks_2samp(pq(gpu), pq(oracle(b - 1))).pvalue     # the test can tell one bit apart
    print(f"KS HIP vs oracle (different seeds), per-query relMSE_T: p = {p:.3f}; against b-1: p = {p_off:.1e}")
    assert p > 1e-3 and p_off < 1e-6


def _regime4(name, seed, sub):
    """the four regimes of [AB] §8 named in the text (its Table 4 is missing): heavy-tailed, the flat
    rank-8 and the steep rank-4 (1 : 1/2 : 1/4 : 1/8) subspaces with noise std 0.05, isotropic"""
    if name == "isotropic":
        return I.gaussian((H, N, D), seed, device=DEV)
    if name == "fattail":
        return I.student_t(H, N, D, 3, seed, device=DEV)
    spec = {"lowrank_aligned": [1.0] * 8, "lowrank_steep": [1.0, 0.5, 0.25, 0.125]}[name]
    return I.low_rank(H, N, D, spec, 0.05, seed, sub, n_heads=H, device=DEV)


def _kl_top5(K, q, b, m, kind, seed):
    ck = T.Codec(D, b, m, H, seed, kind)
    pk = T.encode(ck, K)
    k64, q64 = _f64(K), _f64(q)[0].reshape(H, NQ, D)
    s_hat = T.qk_scores(ck, q[0].reshape(H, NQ, D).contiguous(), pk, N).cpu().numpy().astype(np.float64)
    sc = 1.0 / math.sqrt(D)
    kl, rec = [], []
    for h in range(H):
        ex = q64[h] @ k64[h].T
        kl.append(O.kl_divergence(_softmax(ex * sc), _softmax(s_hat[h] * sc)))
        top_ex, top_q = np.argsort(-ex, axis=1)[:, :5], np.argsort(-s_hat[h], axis=1)[:, :5]
        rec.append([len(set(a.tolist()) & set(c.tolist())) / 5.0 for a, c in zip(top_ex, top_q)])
    return float(np.mean(kl)), float(np.mean(rec))


@pytest.mark.parametrize("regime", ["fattail", "lowrank_aligned", "lowrank_steep", "isotropic"])
def test_kl_and_top5_recall_across_regimes(regime):
    K = _regime4(regime, 620, 91)
    q = I.gaussian((1, H * NQ, D), 629, device=DEV)
    res = {}
    for b in (2, 3, 4):
        for m, kind, label in ((0, 0, "TQ-KV"), (D, 1, "TQ-QKV (RHT)")):
            kl, rec = _kl_top5(K, q, b, m, kind, 1300 + b)
            res[(b, label)] = (kl, rec)
            print(f"{regime:15s} b={b} {label:13s} KL {kl:.5f} top-5 recall {rec:.3f}")
            assert kl >= 0.0 and 0.0 <= rec <= 1.0
    for label in ("TQ-KV", "TQ-QKV (RHT)"):
        kls = [res[(b, label)][0] for b in (2, 3, 4)]
        recs = [res[(b, label)][1] for b in (2, 3, 4)]
        assert kls[0] > kls[1] > kls[2], (label, kls)              # more bits, closer attention weights
        assert recs[2] > recs[0], (label, recs)                     # and more of the top-5 kept

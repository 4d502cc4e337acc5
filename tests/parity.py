"""Parity checks of the HIP path against the oracle (test infrastructure).

All oracle inputs are the exact input bytes handed to the GPU (copied back to the host); decode,
score and attention parity are computed by the oracle from the GPU's own packed bytes, so a
legitimately flagged encode decision cannot propagate.

Tolerances (the workload statement's, with the readings listed in the design doc):
  * packed indices bit-exact except coordinates the oracle flags within 1e-6 of a threshold;
    sketch bits exact except where the oracle flags them, |S e| < 1e-6 on the exact residual
    (recomputed from the GPU's indices where one differed);
  * n16 / r16 equal or one fp16 ulp apart (fp32 vs fp64 rounding before the fp16 rounding);
  * fp32 reconstructions within 1e-5 relative L2 per stream;
  * scores within 2e-3 relative L2 per (stream, query) row; attention within 2e-3 relative L2.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import tq_oracle as O


_CODEBOOKS = {}


def codebook(d, b):
    if (d, b) not in _CODEBOOKS:
        _CODEBOOKS[(d, b)] = O.lloyd_max(d, b)
    return _CODEBOOKS[(d, b)]


class Tables:
    def __init__(self, d, b, m, n_heads, seed, sketch=0, rotation=0):
        """sketch: 0 = Gaussian S (m x d), 1 = randomized Hadamard S = H diag(s2) (m = d);
        rotation: 0 = WHT with signs, 1 = none (the oracle's s = None)."""
        self.d, self.b, self.m, self.n_heads, self.seed, self.sketch = d, b, m, n_heads, seed, sketch
        self.t, self.c = codebook(d, b)
        self.s = [None if rotation == 1 else O.head_signs(seed, h, d) for h in range(n_heads)]
        if not m:
            self.S = None
        elif sketch == 1:
            assert m == d
            self.S = [O.rht_matrix(seed, h, d).astype(np.float64) for h in range(n_heads)]
        else:
            self.S = [O.gaussian_matrix(seed, h, m, d).astype(np.float64) for h in range(n_heads)]

    def head(self, st):
        return st % self.n_heads


def fp16_ulp_diff(a, b):
    a16 = np.asarray(a, dtype=np.float16).view(np.int16).astype(np.int32)
    b16 = np.asarray(b, dtype=np.float16).view(np.int16).astype(np.int32)
    # map sign-magnitude to a monotone integer line
    a16 = np.where(a16 < 0, -32768 - a16, a16)
    b16 = np.where(b16 < 0, -32768 - b16, b16)
    return np.abs(a16 - b16)


def check_encode(tb: Tables, x64: np.ndarray, buf: np.ndarray, streams=None, n_streams=None,
                 n_tokens=None, token_range=None) -> dict:
    """x64: [S_sel, n, d] fp64 inputs of the selected streams (tokens token_range = [t0, t1) of
    n_tokens, default all); buf: the GPU's packed bytes of the whole tensor."""
    N = n_tokens if n_tokens is not None else x64.shape[1]
    S_all = n_streams if n_streams is not None else x64.shape[0]
    streams = list(range(S_all)) if streams is None else list(streams)
    recs = O.unpack_tensor(buf, tb.d, tb.b, tb.m, S_all, N, streams, token_range)
    st_flag = st_mis = st_n16 = st_sflag = st_smis = st_r16 = 0
    for k, st in enumerate(streams):
        h = tb.head(st)
        S = tb.S[h] if tb.m else None
        o = O.encode(x64[k], tb.s[h], tb.t, tb.c, S)
        g = recs[k]
        mis = g["idx"] != o["idx"]
        bad = mis & ~o["flag"]
        assert not bad.any(), f"stream {st}: {int(bad.sum())} unflagged index mismatches"
        st_flag += int(o["flag"].sum())
        st_mis += int(mis.sum())
        nd = fp16_ulp_diff(g["n16"], o["n16"])
        assert nd.max(initial=0) <= 1, f"stream {st}: n16 differs by {nd.max()} ulp"
        st_n16 += int((nd == 1).sum())
        if tb.m:
            vmis = mis.any(axis=1)
            # recompute the sketch of vectors whose indices legitimately differ from the GPU's
            e = o["y"] - tb.c[g["idx"]]
            k = O.sketch(e, S)
            sig_ref = np.where(vmis[:, None], k["sigma"], o["sigma"])
            sflag = np.where(vmis[:, None], k["sflag"], o["sflag"])
            smis = g["sigma"] != sig_ref
            sb = smis & ~sflag
            assert not sb.any(), f"stream {st}: {int(sb.sum())} unflagged sketch-bit mismatches"
            st_sflag += int(sflag.sum())
            st_smis += int(smis.sum())
            r_ref = np.where(vmis, O.fp16_rne(np.sqrt(np.sum(e * e, axis=1))), o["r16"])
            rd = fp16_ulp_diff(g["r16"], r_ref)
            assert rd.max(initial=0) <= 1, f"stream {st}: r16 differs by {rd.max()} ulp"
            st_r16 += int((rd == 1).sum())
    return dict(flagged=st_flag, idx_mismatch=st_mis, n16_1ulp=st_n16, sketch_flagged=st_sflag,
                sketch_mismatch=st_smis, r16_1ulp=st_r16, recs=recs)


def oracle_decode(tb: Tables, recs, streams):
    return [O.decode(r["idx"], r["n16"], tb.s[tb.head(st)], tb.c) for r, st in zip(recs, streams)]


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def oracle_decode_qjl(tb, recs, streams):
    """Reconstruction with the QJL correction, from the GPU's indices, norms and sketch bits."""
    out = []
    for r, st in zip(recs, streams):
        h = tb.head(st)
        corr = O.qjl_correction(r["sigma"], r["r16"], tb.S[h])
        out.append(O.decode(r["idx"], r["n16"], tb.s[h], tb.c, corr))
    return out


def check_decode_f32(tb, recs, streams, xh_gpu: np.ndarray, tol=1e-5, qjl=False) -> float:
    ref = oracle_decode_qjl(tb, recs, streams) if qjl else oracle_decode(tb, recs, streams)
    worst = 0.0
    for k, r in enumerate(ref):
        e = rel_l2(xh_gpu[k], r)
        worst = max(worst, e)
        assert e <= tol, f"stream {streams[k]}: decode rel L2 {e:.3e} > {tol}"
    return worst


def check_decode_bf16(tb, recs, streams, xh_bf16_as_f64: np.ndarray, qjl=False) -> int:
    """Each bf16 output equals the oracle value rounded to bf16, or its neighbour (fp32 path)."""
    ref = oracle_decode_qjl(tb, recs, streams) if qjl else oracle_decode(tb, recs, streams)
    far = 0
    for k, r in enumerate(ref):
        ulp = np.maximum(np.abs(r), 1e-30) * 2.0 ** -8
        err = np.abs(xh_bf16_as_f64[k] - r)
        assert np.all(err <= 1.01 * ulp + 1e-7 * np.max(np.abs(r))), f"stream {streams[k]}: bf16 decode off"
        far += int(np.sum(err > 0.51 * ulp))
    return far


def oracle_scores(tb, rec, st, q64):
    h = tb.head(st)
    return O.scores(q64, rec, tb.s[h], tb.c, tb.S[h] if tb.m else None)


def check_scores(tb, recs, streams, q64_sel: np.ndarray, sc_gpu: np.ndarray, tol=2e-3) -> float:
    worst = 0.0
    for k, st in enumerate(streams):
        ref = oracle_scores(tb, recs[k], st, q64_sel[k])
        for i in range(ref.shape[0]):
            e = rel_l2(sc_gpu[k, i], ref[i])
            worst = max(worst, e)
            assert e <= tol, f"stream {st} query {i}: scores rel L2 {e:.3e} > {tol}"
    return worst


def oracle_attention_row(tk: Tables, tv: Tables, rec_k, rec_v, st, q64_row, scale):
    hk, hv = tk.head(st), tv.head(st)
    sc = O.scores(q64_row[None, :], rec_k, tk.s[hk], tk.c, tk.S[hk] if tk.m else None)
    return O.attention_rotated(sc, rec_v, tv.s[hv], tv.c, scale)[0]

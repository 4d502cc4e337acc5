"""Parity checks of the HIP path against the oracle (test infrastructure).

All oracle inputs are the exact input bytes handed to the GPU (copied back to the host); decode,
score and attention parity are computed by the oracle from the GPU's own packed bytes, so a
legitimately flagged encode decision cannot propagate.

Tolerances (the bars the codec's parity is held to, and the readings they rest on):
  * packed indices bit-exact except coordinates the oracle flags within 1e-6 of a threshold;
    sketch bits exact except where the oracle flags them, |S e| < 1e-6 on the exact residual
    (recomputed from the GPU's indices where one differed);
  * n16 / r16 equal or one fp16 ulp apart (fp32 vs fp64 rounding before the fp16 rounding);
  * fp32 reconstructions within 1e-5 relative L2 per stream;
  * scores within 2e-3 relative L2 per (stream, query) row; attention within 2e-3 relative L2 per
    row.  A bf16 output is held to the distance from the oracle to the set of values that round to
    it: element i contributes how far the oracle value lies outside the rounding interval of the
    output element (half-way to its bf16 neighbours), so the row passes iff it is the bf16 rounding
    of some row within 2e-3 of the oracle.  bf16 rounding alone moves a row by about 1.7e-3 relative
    L2 (up to 2.1e-3 over 500 Gaussian rows of 128), so the bar against the unrounded value would
    measure the output format, not the kernel; that distance is reported beside it.
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


def bf16_rne(x):
    """fp64 values rounded to the nearest bf16 (8 significant bits, ties to even), exactly: the
    quotient by the value's ulp is an exact fp64 integer-or-half, rounded half to even."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.ldexp(1.0, (e - 7).astype(np.int64))
    ulp = np.where(ax >= 2.0 ** -126, ulp, 2.0 ** -133)      # bf16 subnormal spacing below 2^-126
    return np.where(ax > 0, np.round(x / ulp) * ulp, x)


def bf16_interval(g):
    """For bf16 values g (held as fp64), the interval of reals that round to g: half-way to the bf16
    neighbours below and above (exact in fp64)."""
    g = np.asarray(g, dtype=np.float64)
    bits = (g.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    def val(b):
        return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    # neighbours along the bit pattern (sign-magnitude: step the magnitude)
    mag = bits & 0x7FFF
    sgn = bits & 0x8000
    up = val(sgn | np.minimum(mag + 1, 0x7F7F))                 # away from zero
    dn = np.where(mag > 0, val(sgn | np.maximum(mag - 1, 0)), -val(sgn | 1))   # toward zero (past 0: -tiny)
    a, b = 0.5 * (g + dn), 0.5 * (g + up)
    return np.minimum(a, b), np.maximum(a, b)


def check_attention_rows(got, ref, bf16: bool, tol=2e-3) -> dict:
    """Per-row relative L2 of attention outputs [..., d] against the oracle rows (bf16 outputs by the
    distance of the oracle to their rounding intervals, see the module docstring).  Returns the worst
    row against the bar, the worst plain distance to the oracle, and the worst bf16 rounding floor
    (the oracle rounded to bf16 against itself)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    if bf16:
        lo, hi = bf16_interval(got)
        dist = np.where(ref < lo, lo - ref, np.where(ref > hi, ref - hi, 0.0))
    else:
        dist = got - ref
    rows = [(float(np.linalg.norm(dist[i]) / max(np.linalg.norm(ref[i]), 1e-300)), rel_l2(got[i], ref[i]),
             rel_l2(bf16_rne(ref[i]), ref[i]) if bf16 else 0.0) for i in range(got.shape[0])]
    worst = max(r[0] for r in rows)
    assert worst <= tol, f"attention row rel L2 {worst:.3e} > {tol}"
    return dict(worst=worst, worst_unrounded=max(r[1] for r in rows), floor=max(r[2] for r in rows))

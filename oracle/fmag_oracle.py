"""fp64 CPU oracle of the Fourier-magnitude KV codec (Fmag).

TEST INFRASTRUCTURE ONLY. Like ``tq_oracle`` this is the plain, slow definition the HIP library is
checked against; only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it, and it shares no code with the product package.  fp64 throughout.

Source: "Fourier Magnitude KV Cache Quantization" (forum thread), the "Method" section of its first
post: take the FFT of each K/V vector along head_dim, quantise the magnitude spectrum to b bits
with min-max quantisation, keep the phase (at bf16, or at 8 or 6 bits in its "Fmag4+phase8b" and
"phase6b" variants), and reconstruct with the inverse FFT of mag_q·(cos φ + i sin φ).

Readings where the thread is silent (the plainest reading the rest supports):
  * The transform is the real FFT of the d real coordinates, X_k = Σ_j x_j e^{-2πi jk/d},
    k = 0..d/2 (the other bins are conjugates), inverted by the real inverse FFT.
  * Min-max is per vector over its d/2 + 1 magnitudes: lo = min, hi = max,
    q_k = floor((|X_k| - lo)/(hi - lo)·(2^b - 1) + 1/2) (q = 0 when hi = lo), decoded as
    lo + q·(hi - lo)/(2^b - 1); lo and hi are stored as fp32.
  * A p-bit phase takes the nearest of the 2^p angles -π + 2π i/2^p (ties up, index mod 2^p), so
    0 and ±π (the DC and Nyquist bins of a real vector) are levels.  p = 16 means the phase itself
    rounded to bf16.
  * A record holds the d/2 + 1 magnitude indices (b bits each), then the d/2 + 1 phase fields (p bits
    each), LSB first, padded to a word, then lo and hi.
"""
from __future__ import annotations

import math

import numpy as np

PHASE_BF16 = 16


def rfft(x: np.ndarray) -> np.ndarray:
    return np.fft.rfft(np.asarray(x, dtype=np.float64), axis=-1)


def irfft(X: np.ndarray, d: int) -> np.ndarray:
    return np.fft.irfft(X, n=d, axis=-1)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), through fp32 (exact for these fp64 inputs' uses)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def encode(x: np.ndarray, b: int, p: int) -> dict:
    """Rows of x -> magnitude indices q, phase fields (indices, or bf16 phases for p = 16), lo, hi."""
    X = rfft(x)
    mag = np.abs(X)
    ph = np.angle(X)                                   # (-π, π]
    lo = mag.min(axis=-1)
    hi = mag.max(axis=-1)
    L = (1 << b) - 1
    span = hi - lo
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(span[:, None] > 0, (mag - lo[:, None]) / span[:, None] * L, 0.0)
    q = np.floor(t + 0.5).astype(np.int64)
    if p == PHASE_BF16:
        pf = bf16_round(ph)
        pidx = None
    else:
        P = 1 << p
        pidx = np.floor((ph + math.pi) / (2.0 * math.pi) * P + 0.5).astype(np.int64) % P
        pf = None
    return {"X": X, "mag": mag, "phase": ph, "t": t, "q": q, "pidx": pidx, "pbf": pf, "lo": lo, "hi": hi}


def phase_values(rec: dict, p: int) -> np.ndarray:
    if p == PHASE_BF16:
        return rec["pbf"]
    return rec["pidx"] * (2.0 * math.pi / (1 << p)) - math.pi


def spectrum(rec: dict, b: int, p: int) -> np.ndarray:
    """X' = mag'·e^{iφ'} with mag' = lo + q (hi - lo)/(2^b - 1)."""
    L = (1 << b) - 1
    lo = np.asarray(rec["lo"], dtype=np.float64)[:, None]
    hi = np.asarray(rec["hi"], dtype=np.float64)[:, None]
    mag = lo + rec["q"] * (hi - lo) / L
    ph = phase_values(rec, p)
    return mag * np.cos(ph) + 1j * mag * np.sin(ph)


def decode(rec: dict, b: int, p: int, d: int) -> np.ndarray:
    return irfft(spectrum(rec, b, p), d)


def scores(q: np.ndarray, rec: dict, b: int, p: int, d: int) -> np.ndarray:
    """<q_i, x'_t> for every query row i and token t."""
    return np.asarray(q, dtype=np.float64) @ decode(rec, b, p, d).T


def attention(score_est: np.ndarray, rec_v: dict, b: int, p: int, d: int, scale: float) -> np.ndarray:
    s = score_est * scale
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=-1, keepdims=True)
    return w @ decode(rec_v, b, p, d)


# ---- flags: decisions within a band of a rounding boundary ---------------------------------------

def magnitude_flags(rec: dict, tol: float) -> np.ndarray:
    """|t - (k + 1/2)| < tol for the nearest half-integer."""
    t = rec["t"]
    return np.abs(t - np.floor(t) - 0.5) < tol


def phase_flags(rec: dict, p: int, tol: float) -> np.ndarray:
    ph = rec["phase"]
    if p == PHASE_BF16:
        # absolute distance to the nearest midpoint between two bf16 neighbours; ±π (a real bin whose
        # imaginary part is a signed zero) is flagged too
        f = np.abs(ph)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(f, 1e-300))) - 7)
        dist = np.abs(f / ulp - np.floor(f / ulp) - 0.5) * ulp
        return (dist < tol) | (np.abs(f - math.pi) < tol)
    u = (ph + math.pi) / (2.0 * math.pi) * (1 << p)
    return (np.abs(u - np.floor(u) - 0.5) < tol) | (np.abs(np.abs(ph) - math.pi) < tol)


# ---- records ---------------------------------------------------------------------------------------

def record_words(d: int, b: int, p: int) -> int:
    nb = d // 2 + 1
    return (nb * (b + p) + 31) // 32 + 2


def pack(rec: dict, b: int, p: int, d: int) -> np.ndarray:
    """uint32 words [n][record_words]: magnitude fields, phase fields (bf16 bit patterns for p = 16),
    then lo and hi as fp32."""
    nb = d // 2 + 1
    n = rec["q"].shape[0]
    W = record_words(d, b, p)
    bits = np.zeros((n, (W - 2) * 32), dtype=np.uint8)
    for k in range(nb):
        for i in range(b):
            bits[:, k * b + i] = (rec["q"][:, k] >> i) & 1
    if p == PHASE_BF16:
        pv = rec["pbf"].astype(np.float32).view(np.uint32) >> 16
    else:
        pv = rec["pidx"]
    for k in range(nb):
        for i in range(p):
            bits[:, nb * b + k * p + i] = (pv[:, k] >> i) & 1
    words = np.packbits(bits, axis=1, bitorder="little").view(np.uint32)
    lohi = np.stack([rec["lo"].astype(np.float32), rec["hi"].astype(np.float32)], axis=1).view(np.uint32)
    return np.concatenate([words, lohi], axis=1)


def unpack(words: np.ndarray, b: int, p: int, d: int) -> dict:
    nb = d // 2 + 1
    w = np.ascontiguousarray(words, dtype=np.uint32)
    bits = np.unpackbits(w[:, :-2].view(np.uint8), axis=1, bitorder="little").astype(np.int64)
    q = np.zeros((w.shape[0], nb), dtype=np.int64)
    pv = np.zeros((w.shape[0], nb), dtype=np.int64)
    for k in range(nb):
        for i in range(b):
            q[:, k] |= bits[:, k * b + i] << i
        for i in range(p):
            pv[:, k] |= bits[:, nb * b + k * p + i] << i
    lo = w[:, -2].view(np.float32).astype(np.float64)
    hi = w[:, -1].view(np.float32).astype(np.float64)
    rec = {"q": q, "lo": lo, "hi": hi, "pidx": None, "pbf": None}
    if p == PHASE_BF16:
        rec["pbf"] = (pv.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        rec["pidx"] = pv
    return rec

"""fp64 CPU oracle of SpectralQuant (SQ): a calibrated per-head eigenbasis, per-dimension bit
allocation and Gaussian Lloyd-Max scalar codebooks.

TEST INFRASTRUCTURE ONLY. Like ``tq_oracle`` this is the plain, slow definition the HIP library is
checked against; only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it, and it shares no code with the product package.  fp64 throughout.

Sources (cited by page title and section):
  [AB]  "Ablation, Statistical Inference, and Validation for KV-Cache Compression" (arXiv 2607.09683)
        §2 "SpectralQuant": empirical covariance of the calibration tokens C = XᵀX/n_cal, its
        top-d_eff eigenvectors (block power iteration), projection z = Uᵀk, a separate basis for V,
        d_eff = round(tr(C)²/‖C‖_F²), water-filling of Σ_k λ_k 4^(-b_k) under Σ_k b_k = B with
        b_k >= b_tail, tail dimensions at b_tail bits, the score <q_Z, ẑ> with q_Z = Uᵀq;
        §3.2 "Storage complexity": b_sem·d_eff + b_tail·(d - d_eff) bits per token;
        §6 "Water-filling": σ_k² are the projected calibration variances, B = b·d_eff, integer
        greedy allocation, uniform whenever σ_max²/σ_min² <= 4;
        §7 "Spectral gap criterion": trim d_eff at the first k with λ_{k-1}/λ_k > γ (γ = 10) and
        cap it at a known maximum; the Gaussian assumption behind the per-dimension codebooks.
  [MAX] J. Max, "Quantizing for minimum distortion", IRE Trans. IT-6 (1960): the Lloyd-Max
        quantiser of a unit Gaussian.

Readings where the pages are silent (the plainest reading the rest supports):
  * The basis is the full eigenbasis of C, eigenvalues descending; the first d_eff columns are the
    semantic dimensions (block power iteration converges to them; ``block_power_iteration`` below
    is the pages' method and is pinned to the library eigensolver), the remaining d - d_eff
    columns are the tail.  Each eigenvector is signed so its largest-magnitude entry is positive.
  * σ_k² = λ_k, the mean of z_k² over the calibration tokens (the second moment, as C is not
    centred), floored at 1e-12·λ_1.
  * Every dimension is quantised with the Gaussian Lloyd-Max codebook of its bit width, applied to
    u_k = z_k/σ_k; the index counts thresholds <= u_k (ties go up), like the TurboQuant codebook.
  * round() is round-half-up; d_eff >= 1; γ <= 0 disables the gap criterion; a cap of 0 means none.
  * Water-filling starts every semantic dimension at b_tail and gives one bit at a time to the
    largest λ_k 4^(-b_k) among dimensions below 8 bits, ties to the fewer bits, then the lower k.
    The uniform variant gives every semantic dimension b bits.
  * Records are the fields idx_0 .. idx_{d-1} in basis order, LSB first, at bit offsets
    Σ_{j<k} b_j; a record takes 4·ceil(max over heads of Σ_k b_k / 32) bytes.  No norm is stored.
  * The selective QJL sketch (SQU-QKV; §2 "SpectralQuant"): S ∈ {±1}^{m x d_eff} per head, entry
    (i, k) = -1 iff bit 63 of SplitMix64 word i·d + k of tag 4 (the first d_eff columns of an m x d
    table); e_z = z - ẑ over the semantic dimensions; sketch bit i = [(S e_z)_i >= 0]; ||e_z|| is stored
    as fp16.  The score adds sqrt(pi/2)/m · ||e_z|| · <S q_Z, 2σ - 1> with q_Z the semantic part of Uᵀq.
    A record with a sketch holds the index fields, then the m sketch bits, then the fp16 norm,
    padded to 4·ceil((max Σ_k b_k + m + 16)/32) bytes.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy import special

from oracle import tq_oracle as _T

B_MAX = 8
LAMBDA_FLOOR = 1e-12
TAG_SQ_SKETCH = 4


# ----------------------------------------------------------------------------------------------
# Gaussian Lloyd-Max codebook [MAX]: thresholds at midpoints, centroids at the cell means of N(0,1)
# ----------------------------------------------------------------------------------------------

def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper(x):
    """P(X >= x) for X ~ N(0,1), accurate in the tail."""
    return special.ndtr(-x)


@functools.lru_cache(maxsize=None)
def gauss_lloyd_max(b: int, tol: float = 1e-15, max_iter: int = 3_000_000):
    """(thresholds[L-1], centroids[L]) ascending for L = 2^b levels of a unit Gaussian.

    Lloyd iteration on the positive half (the quantiser is symmetric), started at the quantiles
    Φ^{-1}((K + k + 1/2)/L); the centroid of [lo, hi) is (φ(lo) - φ(hi)) / (P(X >= lo) - P(X >= hi)).
    The Gaussian is log-concave, so the fixed point is unique."""
    if not 1 <= b <= B_MAX:
        raise ValueError("b out of range")
    L = 1 << b
    K = L // 2
    c = special.ndtri((K + np.arange(K) + 0.5) / L)
    best, since_best = np.inf, 0
    for _ in range(max_iter):
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        c_new = (_phi(t[:-1]) - _phi(t[1:])) / (_upper(t[:-1]) - _upper(t[1:]))
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta <= tol:
            break
        if delta < best:
            best, since_best = delta, 0
        else:
            since_best += 1
            if since_best > 2000 and delta < 1e-12:
                break
    inner = 0.5 * (c[:-1] + c[1:])
    thresholds = np.concatenate((-inner[::-1], [0.0], inner))
    centroids = np.concatenate((-c[::-1], c))
    return thresholds, centroids


def gauss_codebook_mse(b: int) -> float:
    """E[(X - Q(X))²] for X ~ N(0,1) from the cell moments: mass, first moment φ(lo) - φ(hi) and
    second moment mass + lo φ(lo) - hi φ(hi)."""
    t, c = gauss_lloyd_max(b)
    lo = np.concatenate(([-np.inf], t))
    hi = np.concatenate((t, [np.inf]))
    mass = special.ndtr(hi) - special.ndtr(lo)
    xphi = lambda x: np.where(np.isfinite(x), x * _phi(np.where(np.isfinite(x), x, 0.0)), 0.0)
    m1 = _phi(lo) - _phi(hi)
    m2 = mass + xphi(lo) - xphi(hi)
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))


# ----------------------------------------------------------------------------------------------
# Calibration ([AB] §2 "SpectralQuant", §6, §7)
# ----------------------------------------------------------------------------------------------

def covariance(x_cal: np.ndarray) -> np.ndarray:
    """C = XᵀX / n_cal over the calibration tokens (rows), not centred."""
    x = np.asarray(x_cal, dtype=np.float64)
    return x.T @ x / x.shape[0]


def sign_canonical(V: np.ndarray) -> np.ndarray:
    """Flip each column so that its entry of largest magnitude (first such) is positive."""
    V = V.copy()
    piv = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[piv, np.arange(V.shape[1])])
    sgn[sgn == 0] = 1.0
    return V * sgn


def eigenbasis(C: np.ndarray):
    """(λ descending, U with the matching unit eigenvectors as columns, canonical signs)."""
    w, V = np.linalg.eigh(C)
    order = np.argsort(-w, kind="stable")
    return w[order], sign_canonical(V[:, order])


def block_power_iteration(C: np.ndarray, k: int, seed: int = 0, iters: int = 500):
    """The pages' route to the top-k eigenvectors: Q <- orth(C Q) from a random orthonormal block,
    then a Rayleigh-Ritz step on QᵀCQ.  Returns (λ[k] descending, U[d,k])."""
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((C.shape[0], k)))
    for _ in range(iters):
        Q, _ = np.linalg.qr(C @ Q)
    w, Y = np.linalg.eigh(Q.T @ C @ Q)
    order = np.argsort(-w, kind="stable")
    return w[order], sign_canonical(Q @ Y[:, order])


def participation_ratio(lam: np.ndarray) -> int:
    """round((Σλ)² / Σλ²), round half up."""
    lam = np.asarray(lam, dtype=np.float64)
    return int(math.floor(float(np.sum(lam)) ** 2 / float(np.sum(lam * lam)) + 0.5))


def effective_dim(lam: np.ndarray, gamma: float = 10.0, d_eff_max: int = 0) -> int:
    """Participation ratio, trimmed at the first spectral gap λ_{k-1}/λ_k > γ, capped, at least 1."""
    d_eff = min(max(participation_ratio(lam), 1), len(lam))
    if gamma > 0:
        for k in range(1, d_eff):             # 0-based: gap between λ[k-1] and λ[k]
            if lam[k] <= 0 or lam[k - 1] / lam[k] > gamma:
                d_eff = k
                break
    if d_eff_max > 0:
        d_eff = min(d_eff, d_eff_max)
    return max(d_eff, 1)


def waterfill(lam_sem: np.ndarray, total: int, b_tail: int, b_max: int = B_MAX) -> np.ndarray:
    """Integer greedy minimisation of Σ λ_k 4^(-b_k) with Σ b_k = total, b_tail <= b_k <= b_max."""
    bits = np.full(len(lam_sem), b_tail, dtype=np.int64)
    for _ in range(total - int(bits.sum())):
        best = None
        for k in range(len(lam_sem)):
            if bits[k] >= b_max:
                continue
            key = (lam_sem[k] * 4.0 ** (-int(bits[k])), -int(bits[k]), -k)
            if best is None or key > best[0]:
                best = (key, k)
        bits[best[1]] += 1
    return bits


def calibrate(x_cal: np.ndarray, b: int, b_tail: int, water: bool = False, gamma: float = 10.0,
              d_eff_max: int = 0) -> dict:
    """One head's SQ model from its calibration tokens x_cal[n_cal, d]."""
    if not 1 <= b_tail <= b <= B_MAX:
        raise ValueError("need 1 <= b_tail <= b <= 8")
    C = covariance(x_cal)
    lam, U = eigenbasis(C)
    d = len(lam)
    d_eff = effective_dim(lam, gamma, d_eff_max)
    lam_c = np.maximum(lam, LAMBDA_FLOOR * max(lam[0], 0.0))
    if lam[0] <= 0:
        lam_c = np.ones(d)
    bits = np.full(d, b_tail, dtype=np.int64)
    bits[:d_eff] = waterfill(lam_c[:d_eff], b * d_eff, b_tail) if water else b
    return {"U": U, "lam": lam, "sigma": np.sqrt(lam_c), "bits": bits, "d_eff": d_eff}


def sketch_matrix(seed: int, head: int, m: int, d: int) -> np.ndarray:
    """The m x d table of ±1 whose first d_eff columns are the selective QJL sketch of one head."""
    w = _T.words(_T.stream_key(seed, TAG_SQ_SKETCH, head), m * d)
    return np.where((w >> np.uint64(63)) == 1, -1.0, 1.0).reshape(m, d)


def with_sketch(model: dict, m: int, seed: int, head: int) -> dict:
    """The model with the selective QJL sketch of m rows on its semantic dimensions."""
    out = dict(model)
    d = model["U"].shape[0]
    out["m"] = m
    out["S"] = sketch_matrix(seed, head, m, d)[:, : model["d_eff"]]
    return out


def storage_bits(d: int, d_eff: int, b_sem: int, b_tail: int) -> int:
    """Bits per token of the uniform scheme ([AB] §3.2)."""
    return b_sem * d_eff + b_tail * (d - d_eff)


# ----------------------------------------------------------------------------------------------
# Encode / decode / scores / attention
# ----------------------------------------------------------------------------------------------

def project(x: np.ndarray, model: dict) -> np.ndarray:
    """z = Uᵀx for each row x."""
    return np.asarray(x, dtype=np.float64) @ model["U"]


def encode(x: np.ndarray, model: dict) -> dict:
    """Per token: z = Uᵀx, u_k = z_k/σ_k, idx_k = #{thresholds of the b_k-bit codebook <= u_k}; with
    a sketch also e_z, its sketch values S e_z, the bits σ and the fp16 norm r16."""
    z = project(x, model)
    u = z / model["sigma"]
    idx = np.zeros(u.shape, dtype=np.int64)
    for w in np.unique(model["bits"]):
        cols = model["bits"] == w
        t, _ = gauss_lloyd_max(int(w))
        idx[:, cols] = np.sum(u[:, cols, None] >= t[None, None, :], axis=2)
    out = {"z": z, "u": u, "idx": idx}
    if model.get("m"):
        out.update(sketch_of(z, idx, model))
    return out


def sketch_of(z: np.ndarray, idx: np.ndarray, model: dict) -> dict:
    """The selective QJL sketch of tokens with projections z and indices idx."""
    de = model["d_eff"]
    e = z[:, :de] - dequantise(idx, model)[:, :de]
    zs = e @ model["S"].T
    return {"e": e, "zs": zs, "sigma_bits": (zs >= 0).astype(np.int64),
            "r16": _T.fp16_rne(np.linalg.norm(e, axis=1))}


def dequantise(idx: np.ndarray, model: dict) -> np.ndarray:
    """ẑ_k = σ_k c_{b_k}[idx_k]."""
    zh = np.zeros(idx.shape, dtype=np.float64)
    for w in np.unique(model["bits"]):
        cols = model["bits"] == w
        _, c = gauss_lloyd_max(int(w))
        zh[:, cols] = c[idx[:, cols]]
    return zh * model["sigma"]


def decode(idx: np.ndarray, model: dict) -> np.ndarray:
    """x̂ = U ẑ."""
    return dequantise(idx, model) @ model["U"].T


def boundary_distance(u: np.ndarray, model: dict) -> np.ndarray:
    """|u_k - nearest threshold of its codebook| (inf for 1 level)."""
    out = np.full(u.shape, np.inf)
    for w in np.unique(model["bits"]):
        cols = model["bits"] == w
        t, _ = gauss_lloyd_max(int(w))
        out[:, cols] = np.min(np.abs(u[:, cols, None] - t[None, None, :]), axis=2)
    return out


def scores(q: np.ndarray, idx: np.ndarray, model: dict, sigma_bits=None, r16=None) -> np.ndarray:
    """ŝ[i, t] = <Uᵀq_i, ẑ_t> ([AB] §2 "SpectralQuant" with the tail included), plus with a sketch
    sqrt(pi/2)/m · r16_t · <S q_Z, 2σ_t - 1>."""
    qz = np.asarray(q, dtype=np.float64) @ model["U"]
    out = qz @ dequantise(idx, model).T
    if model.get("m"):
        p = qz[:, : model["d_eff"]] @ model["S"].T
        pm = 2.0 * np.asarray(sigma_bits, dtype=np.float64) - 1.0
        out = out + math.sqrt(math.pi / 2) / model["m"] * (p @ pm.T) * np.asarray(r16, dtype=np.float64)[None, :]
    return out


def attention(score_est: np.ndarray, idx_v: np.ndarray, model_v: dict, scale: float) -> np.ndarray:
    """softmax(scale·ŝ) over tokens, weights applied to ẑ_V in the V basis, then one U_V."""
    s = score_est * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return (p @ dequantise(idx_v, model_v)) @ model_v["U"].T


# ----------------------------------------------------------------------------------------------
# Packed records
# ----------------------------------------------------------------------------------------------

def record_bytes(bits_per_head: list, m: int = 0) -> int:
    """4·ceil(max_h Σ_k b_k / 32), or 4·ceil((max_h Σ_k b_k + m + 16)/32) with an m-bit sketch."""
    extra = m + 16 if m else 0
    return 4 * ((max(int(np.sum(bh)) for bh in bits_per_head) + extra + 31) // 32)


def pack(idx: np.ndarray, bits: np.ndarray, rec_bytes: int, sigma_bits=None, r16=None) -> np.ndarray:
    """Rows of indices -> uint8 records, field k LSB first at bit Σ_{j<k} b_j; then the sketch bits
    and the fp16 norm when given."""
    n, d = idx.shape
    out = np.zeros((n, rec_bytes * 8), dtype=np.uint8)
    pos = 0
    for k in range(d):
        for i in range(int(bits[k])):
            out[:, pos + i] = (idx[:, k] >> i) & 1
        pos += int(bits[k])
    if sigma_bits is not None:
        m = sigma_bits.shape[1]
        out[:, pos:pos + m] = sigma_bits
        h = np.asarray(r16, dtype=np.float16).view(np.uint16).astype(np.int64)
        for i in range(16):
            out[:, pos + m + i] = (h >> i) & 1
    return np.packbits(out, axis=1, bitorder="little")


def unpack(rec: np.ndarray, bits: np.ndarray, m: int = 0):
    """uint8 records -> indices (inverse of ``pack``); with m > 0 also (sketch bits, r16)."""
    allbits = np.unpackbits(np.asarray(rec, dtype=np.uint8), axis=1, bitorder="little").astype(np.int64)
    d = len(bits)
    idx = np.zeros((rec.shape[0], d), dtype=np.int64)
    pos = 0
    for k in range(d):
        for i in range(int(bits[k])):
            idx[:, k] |= allbits[:, pos + i] << i
        pos += int(bits[k])
    if not m:
        return idx
    sig = allbits[:, pos:pos + m].copy()
    h = np.zeros(rec.shape[0], dtype=np.int64)
    for i in range(16):
        h |= allbits[:, pos + m + i] << i
    return idx, sig, h.astype(np.uint16).view(np.float16).astype(np.float64)

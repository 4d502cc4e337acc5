"""fp64 CPU oracle of the TurboQuant-family KV-cache codec.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow definition the HIP library is checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it; the product package ``kv_cache_transform_amd`` never does, and the two share no
code (no kernels, headers, tables, constants or pre/post-processing).  Floating point is fp64
throughout unless a step says otherwise.

Sources (cited by page title and section):
  [AB]  "Ablation, Statistical Inference, and Validation for KV-Cache Compression" (arXiv 2607.09683)
        §2 Background: attention eq. (1); "TurboQuant" paragraph (per-head random signs,
        y = WHT(k ⊙ s)/sqrt(d), Beta((d-1)/2,(d-1)/2) coordinates, one analytical Lloyd-Max codebook
        shared by all coordinates, WHT-domain residual e = y - ŷ); "SpectralQuant" paragraph
        (the asymmetric 1-bit QJL score estimator <q,k̂> + sqrt(pi/2)/m ||e|| q^T S sign(S e));
        §3.2 "Storage complexity" (b·d bits per token); §2 end (binary-search off-by-one in
        quantise_scalar); §5 "Jensen's inequality" (QJL variance ∝ ||e||²/m).
  [SI]  "Statistical Inference and Quality Measures of KV Cache Quantisations Inspired by
        TurboQuant" (arXiv 2605.08114), abstract (Beta on the hypersphere; QJL variance inflated by
        pi/2; KL(p_ref || p_quant) over attention weights).
  [SM]  Steele, Lea, Flood, "Fast splittable pseudorandom number generators" (OOPSLA 2014):
        SplitMix64.  [BM] Box & Muller (1958): normal deviates from two uniforms.

Readings where the pages are silent (the plainest reading the rest supports):
  * WHT is the unnormalised Sylvester-ordered Hadamard matrix H (H_2n = [[H, H], [H, -H]]).
  * Codebook index = number of thresholds <= y (ties go to the upper cell), centroids ascending.
  * Vectors are normalised by their exact norm; the norm is stored as fp16 (round to nearest even).
  * QJL uses a seeded Gaussian S (m x d) on the WHT-domain residual, or the randomized Hadamard
    sketch S = H diag(s2) (m = d); sign(0) = +1.
  * Random signs and S come from SplitMix64 keyed by (seed, tag, head); Gaussians by Box-Muller.
  * The Gaussian S holds the fp16 roundings of its Box-Muller draws (the pages say only
    "Gaussian"; the estimator's unbiasedness is pinned with this table).  The sketch itself is the
    pages' sign(S e) on the exact fp64 residual e = y - c[idx].
"""
from __future__ import annotations

import math

import numpy as np
from scipy import linalg, special

# ----------------------------------------------------------------------------------------------
# Random state: SplitMix64 [SM], counter form.  word(key, i) = mix64(key + (i + 1) * GAMMA).
# ----------------------------------------------------------------------------------------------
GAMMA = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1
TAG_SIGNS = 1
TAG_GAUSS = 2
TAG_RHT = 3


def mix64(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2**64) [SM]."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def mix64_np(z: np.ndarray) -> np.ndarray:
    """Vectorised mix64 on uint64 arrays (numpy wraps modulo 2**64)."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, tag: int, head: int) -> int:
    """Key of the counter stream for one (seed, table tag, head)."""
    return mix64((seed & _M64) ^ mix64((tag << 40) | head))


def words(key: int, n: int) -> np.ndarray:
    """First n outputs of SplitMix64 started from state `key` (uint64 array)."""
    i = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + i * np.uint64(GAMMA)
    return mix64_np(state)


def head_signs(seed: int, head: int, d: int) -> np.ndarray:
    """Per-head random signs s in {-1,+1}^d ([AB] §2 TurboQuant): s_j = -1 iff bit 63 of word j."""
    w = words(stream_key(seed, TAG_SIGNS, head), d)
    return np.where((w >> np.uint64(63)) == 1, -1.0, 1.0)


def gaussian_matrix(seed: int, head: int, m: int, d: int) -> np.ndarray:
    """QJL projection S (m x d), i.i.d. N(0,1) rounded to fp16 (round-to-nearest-even; |g| < 8.6
    always fits), row-major element e uses words 2e and 2e+1: u1 = (w>>11 + 1)·2^-53 in (0,1],
    u2 = (w>>11)·2^-53 in [0,1), g = sqrt(-2 ln u1)·cos(2·pi·u2) in fp64 via libm (Python math) [BM].
    The pages fix only "Gaussian"; fp16 entries make S exactly representable in half precision."""
    n = m * d
    w = words(stream_key(seed, TAG_GAUSS, head), 2 * n)
    a = (w[0::2] >> np.uint64(11)).tolist()
    c = (w[1::2] >> np.uint64(11)).tolist()
    two_pi = 2.0 * math.pi
    out = np.empty(n, dtype=np.float64)
    sc = 2.0 ** -53
    for k in range(n):
        u1 = (a[k] + 1) * sc
        u2 = c[k] * sc
        out[k] = math.sqrt(-2.0 * math.log(u1)) * math.cos(two_pi * u2)
    return out.astype(np.float16).reshape(m, d)


def rht_signs(seed: int, head: int, d: int) -> np.ndarray:
    """Second sign vector s2 of the randomized Hadamard sketch ([AB] §2 TurboQuant: "a fixed sign
    vector s2"), drawn like the rotation signs but from tag 3."""
    w = words(stream_key(seed, TAG_RHT, head), d)
    return np.where((w >> np.uint64(63)) == 1, -1.0, 1.0)


def rht_matrix(seed: int, head: int, d: int) -> np.ndarray:
    """The randomized Hadamard sketch as a matrix: S = H diag(s2) (d x d, entries ±1), so that
    S e = WHT(e ⊙ s2) ([AB] §2 TurboQuant, b = sign(WHT(e ⊙ s2))) and the estimator of the Gaussian
    case applies with m = d.  fp16 holds ±1 exactly."""
    return (hadamard(d) * rht_signs(seed, head, d)[None, :]).astype(np.float16)


# ----------------------------------------------------------------------------------------------
# Codebook: Lloyd-Max for the coordinate density of a uniformly random unit vector in R^d,
# f(x) = (1 - x^2)^alpha / B(1/2, alpha + 1) on [-1, 1], alpha = (d - 3)/2  ([AB] §2 TurboQuant:
# Beta((d-1)/2, (d-1)/2) on the sphere; [SI] abstract).  Symmetric, so the positive half is solved.
# ----------------------------------------------------------------------------------------------

def beta_alpha(d: int) -> float:
    return (d - 3) / 2.0


def coord_cdf(x, d: int):
    """F(x) = I_{(1+x)/2}((d-1)/2, (d-1)/2)."""
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + np.asarray(x, dtype=np.float64)) / 2.0)


def coord_sf(x, d: int):
    """1 - F(x) = I_{(1-x)/2}((d-1)/2, (d-1)/2) (accurate in the upper tail)."""
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 - np.asarray(x, dtype=np.float64)) / 2.0)


def coord_pdf(x, d: int):
    al = beta_alpha(d)
    x = np.asarray(x, dtype=np.float64)
    return ((1.0 - x) * (1.0 + x)) ** al / special.beta(0.5, al + 1.0)


def first_moment(lo, hi, d: int):
    """∫_lo^hi x f(x) dx = [(1-lo²)^(α+1) - (1-hi²)^(α+1)] / (2(α+1) B(1/2, α+1))."""
    al = beta_alpha(d)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    g = lambda x: ((1.0 - x) * (1.0 + x)) ** (al + 1.0)
    return (g(lo) - g(hi)) / (2.0 * (al + 1.0) * special.beta(0.5, al + 1.0))


def upper_mass(lo, hi, d: int):
    """P(lo <= X < hi) for 0 <= lo < hi <= 1, from upper-tail values (no cancellation near 1)."""
    return coord_sf(lo, d) - coord_sf(hi, d)


def lloyd_max(d: int, b: int, tol: float = 1e-16, max_iter: int = 2_000_000):
    """Lloyd-Max codebook with L = 2^b levels.  Returns (thresholds[L-1], centroids[L]) ascending.

    Iteration (Lloyd): thresholds at midpoints of neighbouring centroids, centroids at the
    conditional mean of their cell, started from the quantiles F^-1((i+1/2)/L), until the largest
    centroid change is <= tol (or has stopped reaching new lows at rounding level).  The density is log-concave, so the fixed
    point is unique."""
    if d < 2:
        raise ValueError("d must be >= 2")
    if not 1 <= b <= 12:
        raise ValueError("b out of range")
    L = 1 << b
    K = L // 2
    a = (d - 1) / 2.0
    # quantile start, positive half: F(x) = (K + k + 1/2)/L  <=>  sf(x) = (K - k - 1/2)/L
    p_up = (K - np.arange(K) - 0.5) / L
    c = 1.0 - 2.0 * special.betaincinv(a, a, p_up)
    best, since_best = np.inf, 0
    for _ in range(max_iter):
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        c_new = first_moment(t[:-1], t[1:], d) / upper_mass(t[:-1], t[1:], d)
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta <= tol:
            break
        # Lloyd contracts slowly for many levels: keep going while the step still reaches new lows
        if delta < best:
            best, since_best = delta, 0
        else:
            since_best += 1
            if since_best > 2000 and delta < 1e-12:
                break
    t_inner = 0.5 * (c[:-1] + c[1:])
    thresholds = np.concatenate((-t_inner[::-1], [0.0], t_inner))
    centroids = np.concatenate((-c[::-1], c))
    return thresholds, centroids


def codebook_mse(d: int, thresholds: np.ndarray, centroids: np.ndarray) -> float:
    """E[(X - Q(X))^2] per coordinate, by the closed-form moments on each cell."""
    al = beta_alpha(d)
    edges = np.concatenate(([-1.0], thresholds, [1.0]))
    lo, hi = edges[:-1], edges[1:]
    mass = coord_cdf(hi, d) - coord_cdf(lo, d)
    m1 = first_moment(lo, hi, d)
    # second moment: E[X^2] over the cell via E[X^2] = 1/d overall and the identity
    # ∫ x^2 f = ∫ f - ∫ (1-x^2) f, with ∫_lo^hi (1-x^2)^(α+1) dx / B(1/2,α+1) a scaled beta mass
    a1 = (d + 1) / 2.0  # density of the d+2 sphere coordinate has alpha+1
    scale = special.beta(0.5, al + 2.0) / special.beta(0.5, al + 1.0)
    m_one_minus_x2 = scale * (special.betainc(a1, a1, (1 + hi) / 2) - special.betainc(a1, a1, (1 + lo) / 2))
    m2 = mass - m_one_minus_x2
    return float(np.sum(m2 - 2 * centroids * m1 + centroids ** 2 * mass))


# ----------------------------------------------------------------------------------------------
# Rotation: y = H (u ⊙ s) / sqrt(d), H the Sylvester Hadamard matrix ([AB] §2 TurboQuant).
# ----------------------------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    return linalg.hadamard(d).astype(np.float64)


def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis by radix-2 butterflies (natural
    order: the pair (j, j + h) of each stage becomes (a + b, a - b)); equals v @ H."""
    v = np.array(v, dtype=np.float64, copy=True)
    d = v.shape[-1]
    h = 1
    while h < d:
        w = v.reshape(v.shape[:-1] + (d // (2 * h), 2, h))
        a, b = w[..., 0, :].copy(), w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(v.shape)
        h *= 2
    return v


def rotate(u: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    """y = H (u ⊙ s) / sqrt(d); s = None is Plain-KV ([AB] §4: the Beta codebook without the WHT),
    y = u."""
    if s is None:
        return np.array(u, dtype=np.float64, copy=True)
    d = u.shape[-1]
    return (u * s) @ hadamard(d) / math.sqrt(d)          # H is symmetric


def unrotate(y: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    if s is None:
        return np.array(y, dtype=np.float64, copy=True)
    d = y.shape[-1]
    return s * (y @ hadamard(d)) / math.sqrt(d)


# ----------------------------------------------------------------------------------------------
# Encode / decode ([AB] §2 TurboQuant; [AB] §3.2 storage).
# ----------------------------------------------------------------------------------------------
FLAG_TOL = 1e-6


def fp16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 round-to-nearest-even (numpy converts directly, no double rounding)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def quantise(y: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """idx = #{i : t_i <= y} (linear count; ties to the upper cell)."""
    return np.searchsorted(thresholds, y, side="right").astype(np.int64)


def boundary_distance(y: np.ndarray, thresholds: np.ndarray, idx: np.ndarray | None = None) -> np.ndarray:
    """min_i |y - t_i| over the sorted thresholds: attained at a neighbour of the insertion point
    idx = #{t_i <= y}, i.e. at t[idx-1] or t[idx]."""
    if idx is None:
        idx = quantise(y, thresholds)
    tp = np.concatenate((thresholds, [np.inf]))
    lo = np.abs(y - tp[np.maximum(idx - 1, 0)])
    lo = np.where(idx > 0, lo, np.inf)
    hi = np.abs(tp[idx] - y)
    return np.minimum(lo, hi)


def sketch(e: np.ndarray, S: np.ndarray, tol: float = FLAG_TOL) -> dict:
    """1-bit sketch of residual rows e (N, d) ([AB] §2 TurboQuant: the sign sketch of the WHT-domain
    residual; SpectralQuant paragraph: sign(S e) in the asymmetric estimator): z = e Sᵀ in fp64,
    σ = [z >= 0] (sign(0) = +1), sflag = [|z| < tol] (decisions within the tolerance of zero)."""
    z = np.asarray(e, dtype=np.float64) @ np.asarray(S, dtype=np.float64).T
    return {"z": z, "sigma": z >= 0.0, "sflag": np.abs(z) < tol}


def encode(x: np.ndarray, s: np.ndarray, thresholds: np.ndarray, centroids: np.ndarray,
           S: np.ndarray | None = None) -> dict:
    """Encode rows of x (N, d) that share one RNG head.

    Returns idx (N,d), n16 (N,) fp16, flag (N,d) bool [|y - t_i| < 1e-6], y (N,d); with S (m x d)
    also e, r16 = fp16(||e||), z = S e, sigma (N,m) bool [z >= 0] and sflag (N,m) (``sketch``)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[:, None] > 0, x / safe[:, None], 0.0)
    y = rotate(u, s)
    idx = quantise(y, thresholds)
    out = {"idx": idx, "n16": fp16_rne(n), "flag": boundary_distance(y, thresholds, idx) < FLAG_TOL,
           "y": y, "norm": n}
    if S is not None:
        e = y - centroids[idx]
        out.update(e=e, r16=fp16_rne(np.sqrt(np.sum(e * e, axis=1))), **sketch(e, S))
    return out


def qjl_correction(sigma: np.ndarray, r16: np.ndarray, S: np.ndarray) -> np.ndarray:
    """WHT-domain QJL correction Δŷ = sqrt(pi/2)/m · ||e|| · S^T (2σ - 1) per row ([AB] §2
    TurboQuant: sqrt(pi/2)/d · ||e|| · s2 ⊙ WHT(b) for S = H diag(s2), m = d; the same form with
    the Gaussian S), with ||e|| the stored r16."""
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    return math.sqrt(math.pi / 2.0) / m * np.asarray(r16, dtype=np.float64)[:, None] * (pm @ S)


def decode(idx: np.ndarray, n16: np.ndarray, s: np.ndarray, centroids: np.ndarray,
           corr: np.ndarray | None = None) -> np.ndarray:
    """x̂ = n16 · s ⊙ (H (c[idx] + Δŷ)) / sqrt(d); Δŷ = corr (qjl_correction) or 0 for the MSE
    reconstruction."""
    y_hat = centroids[np.asarray(idx)]
    if corr is not None:
        y_hat = y_hat + corr
    return np.asarray(n16, dtype=np.float64)[:, None] * unrotate(y_hat, s)


# ----------------------------------------------------------------------------------------------
# Packed format: per vector a little-endian bit string, coordinate j at bits [j·b, (j+1)·b);
# sketch bit i = sigma_i LSB-first.  Planes [stream][token]: idx | sketch | n16 | r16, each plane
# starting on a 256-byte boundary ([AB] §3.2 counts b·d bits per token; norms are extra).
# ----------------------------------------------------------------------------------------------
PLANE_ALIGN = 256


def _align(x: int) -> int:
    return (x + PLANE_ALIGN - 1) // PLANE_ALIGN * PLANE_ALIGN


def layout(d: int, b: int, m: int, n_streams: int, n_tokens: int) -> dict:
    nv = n_streams * n_tokens
    ib, sb = d * b // 8, m // 8
    off_idx = 0
    off_sketch = _align(off_idx + nv * ib)
    off_norm = _align(off_sketch + nv * sb)
    off_rnorm = _align(off_norm + nv * 2)
    total = _align(off_rnorm + (nv * 2 if m > 0 else 0))
    return dict(idx_bytes_per_vec=ib, sketch_bytes_per_vec=sb, off_idx=off_idx,
                off_sketch=off_sketch, off_norm=off_norm, off_rnorm=off_rnorm, total_bytes=total)


def pack_bits(vals: np.ndarray, b: int) -> np.ndarray:
    """(N, n) integers < 2^b -> (N, n·b/8) bytes, value j at bits [j·b, (j+1)·b) LSB-first."""
    vals = np.asarray(vals, dtype=np.int64)
    N, n = vals.shape
    bits = ((vals[:, :, None] >> np.arange(b)[None, None, :]) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(N, n * b), axis=1, bitorder="little")


def unpack_bits(buf: np.ndarray, b: int, n: int) -> np.ndarray:
    buf = np.asarray(buf, dtype=np.uint8)
    bits = np.unpackbits(buf, axis=1, bitorder="little")[:, : n * b].reshape(buf.shape[0], n, b)
    return np.sum(bits.astype(np.int64) << np.arange(b)[None, None, :], axis=2)


def pack_tensor(d: int, b: int, m: int, n_streams: int, n_tokens: int, enc: list[dict]) -> np.ndarray:
    """Assemble the packed byte buffer from per-stream encode results (list over streams)."""
    lay = layout(d, b, m, n_streams, n_tokens)
    buf = np.zeros(lay["total_bytes"], dtype=np.uint8)
    ib, sb = lay["idx_bytes_per_vec"], lay["sketch_bytes_per_vec"]
    for st, r in enumerate(enc):
        v0 = st * n_tokens
        buf[lay["off_idx"] + v0 * ib: lay["off_idx"] + (v0 + n_tokens) * ib] = pack_bits(r["idx"], b).ravel()
        buf[lay["off_norm"] + 2 * v0: lay["off_norm"] + 2 * (v0 + n_tokens)] = \
            np.asarray(r["n16"], dtype=np.float16).view(np.uint8)
        if m > 0:
            buf[lay["off_sketch"] + v0 * sb: lay["off_sketch"] + (v0 + n_tokens) * sb] = \
                pack_bits(r["sigma"].astype(np.int64), 1).ravel()
            buf[lay["off_rnorm"] + 2 * v0: lay["off_rnorm"] + 2 * (v0 + n_tokens)] = \
                np.asarray(r["r16"], dtype=np.float16).view(np.uint8)
    return buf


def unpack_tensor(buf: np.ndarray, d: int, b: int, m: int, n_streams: int, n_tokens: int,
                  streams=None, token_range=None) -> list[dict]:
    """Read planes back (for the listed streams, optionally only tokens [t0, t1) of each):
    idx, n16, and with m>0 sigma, r16."""
    lay = layout(d, b, m, n_streams, n_tokens)
    buf = np.asarray(buf, dtype=np.uint8)
    ib, sb = lay["idx_bytes_per_vec"], lay["sketch_bytes_per_vec"]
    t0, t1 = (0, n_tokens) if token_range is None else token_range
    n = t1 - t0
    out = []
    for st in (range(n_streams) if streams is None else streams):
        v0 = st * n_tokens + t0
        r = {"idx": unpack_bits(buf[lay["off_idx"] + v0 * ib: lay["off_idx"] + (v0 + n) * ib]
                                .reshape(n, ib), b, d),
             "n16": buf[lay["off_norm"] + 2 * v0: lay["off_norm"] + 2 * (v0 + n)].view(np.float16)}
        if m > 0:
            r["sigma"] = unpack_bits(buf[lay["off_sketch"] + v0 * sb: lay["off_sketch"] + (v0 + n) * sb]
                                     .reshape(n, sb), 1, m).astype(bool)
            r["r16"] = buf[lay["off_rnorm"] + 2 * v0: lay["off_rnorm"] + 2 * (v0 + n)].view(np.float16)
        out.append(r)
    return out


# ----------------------------------------------------------------------------------------------
# Scores on compressed keys ([AB] §2 TurboQuant "QJL on K improves the attention score estimate";
# [AB] §2 SpectralQuant asymmetric estimator, here in the WHT domain with Gaussian S).
#   ŝ(q,k) = n16 · ( <q_rot, c[idx]> + sqrt(pi/2)/m · r16 · <S q_rot, 2σ - 1> ),  q_rot = H(q⊙s)/√d
# ----------------------------------------------------------------------------------------------

def query_rotate(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return rotate(np.asarray(q, dtype=np.float64), s)


def scores(q: np.ndarray, rec: dict, s: np.ndarray, centroids: np.ndarray,
           S: np.ndarray | None = None) -> np.ndarray:
    """Unscaled score estimates (n_q, N) of <q, k> for one stream's packed record `rec`."""
    q_rot = query_rotate(q, s)
    y_hat = centroids[np.asarray(rec["idx"])]
    n16 = np.asarray(rec["n16"], dtype=np.float64)
    base = q_rot @ y_hat.T
    if S is None:
        return base * n16[None, :]
    m = S.shape[0]
    p = q_rot @ np.asarray(S, dtype=np.float64).T                 # (n_q, m)
    pm = 2.0 * np.asarray(rec["sigma"], dtype=np.float64) - 1.0    # (N, m)
    r16 = np.asarray(rec["r16"], dtype=np.float64)
    corr = math.sqrt(math.pi / 2.0) / m * r16[None, :] * (p @ pm.T)
    return (base + corr) * n16[None, :]


def qjl_estimate(q: np.ndarray, e: np.ndarray, S: np.ndarray) -> float:
    """Plain QJL estimate of <q, e>: sqrt(pi/2)/m · ||e|| · <S q, sign(S e)> with sign(0)=+1."""
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    z = S @ e
    sgn = np.where(z >= 0.0, 1.0, -1.0)
    return math.sqrt(math.pi / 2.0) / m * float(np.linalg.norm(e)) * float((S @ q) @ sgn)


# ----------------------------------------------------------------------------------------------
# Attention T = softmax(Q K^T / sqrt(d)) V  ([AB] eq. (1)) over a compressed cache.
# ----------------------------------------------------------------------------------------------

def softmax(x: np.ndarray, axis=-1) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    x = x - np.max(x, axis=axis, keepdims=True)
    e = np.exp(x)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention_dense(score_est: np.ndarray, v_hat: np.ndarray, scale: float) -> np.ndarray:
    """softmax(score_est · scale) @ v_hat  for score_est (n_q, N), v_hat (N, d)."""
    return softmax(score_est * scale, axis=-1) @ v_hat


def attention_rotated(score_est: np.ndarray, rec_v: dict, s_v: np.ndarray, centroids_v: np.ndarray,
                      scale: float) -> np.ndarray:
    """Same quantity accumulated in the rotated domain, one inverse rotation at the end."""
    w = softmax(score_est * scale, axis=-1)
    acc = w @ (np.asarray(rec_v["n16"], dtype=np.float64)[:, None] * centroids_v[np.asarray(rec_v["idx"])])
    return unrotate(acc, s_v)


def kl_divergence(p_ref: np.ndarray, p_q: np.ndarray) -> np.ndarray:
    """KL(p_ref || p_q) along the last axis ([SI] abstract)."""
    p_ref = np.asarray(p_ref, dtype=np.float64)
    p_q = np.asarray(p_q, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p_ref > 0, p_ref * (np.log(p_ref) - np.log(p_q)), 0.0)
    return np.sum(t, axis=-1)


# ----------------------------------------------------------------------------------------------
# Input bytes -> fp64 (exact).
# ----------------------------------------------------------------------------------------------

def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)

"""Seeded synthetic workloads (inputs only: no step of the codec lives here).

Both sides of every check consume the same bytes produced here: the HIP library gets the device
tensor, the oracle gets a host copy of exactly those bytes.  Distributions follow the workload
descriptions (Gaussian with per-channel scales, Gaussian with outlier channels, RoPE-rotated
Gaussian, Student-t ν = 3 as the heavy-tailed "fattail" regime of "Ablation, Statistical Inference,
and Validation for KV-Cache Compression" §8).  Generation is chunked over streams to bound memory.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def per_channel_gaussian(n_tokens: int, d: int, seed: int) -> np.ndarray:
    """fp32 [n_tokens, d]: channel j ~ sigma_j N(0,1), sigma_j ~ U[0.5, 2] (numpy default_rng(seed))."""
    rng = np.random.default_rng(seed)
    sigma = rng.uniform(0.5, 2.0, size=d)
    return (rng.standard_normal((n_tokens, d)) * sigma).astype(np.float32)


def outlier_gaussian(n_heads: int, n_tokens: int, d: int, n_outliers: int, scale: float, seed: int,
                     device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """[n_heads, n_tokens, d] ~ N(0,1) with `n_outliers` distinct channels per head scaled by `scale`."""
    out = torch.empty(n_heads, n_tokens, d, dtype=dtype, device=device)
    rng = np.random.default_rng(seed)
    for h in range(n_heads):
        g = _gen(seed * 1000003 + h, device)
        x = torch.randn(n_tokens, d, generator=g, device=device, dtype=torch.float32)
        ch = torch.as_tensor(rng.choice(d, n_outliers, replace=False), device=device)
        x[:, ch] *= scale
        out[h] = x.to(dtype)
    return out


def gaussian(shape, seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty(*shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for i in range(shape[0]):
        g = _gen(seed * 1000003 + i, device)
        flat[i] = torch.randn(flat.shape[1], generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def rope_rotate_(x: torch.Tensor, positions: torch.Tensor) -> torch.Tensor:
    """In place: rotate interleaved pairs (2j, 2j+1) by theta = t * 10000^(-2j/d) (fp64 angles)."""
    d = x.shape[-1]
    j = torch.arange(d // 2, device=x.device, dtype=torch.float64)
    theta = positions.to(torch.float64)[:, None] * torch.pow(10000.0, -2.0 * j / d)[None, :]
    c, s = torch.cos(theta).to(torch.float32), torch.sin(theta).to(torch.float32)
    xe, xo = x[..., 0::2].to(torch.float32), x[..., 1::2].to(torch.float32)
    re = xe * c - xo * s
    ro = xe * s + xo * c
    x[..., 0::2] = re.to(x.dtype)
    x[..., 1::2] = ro.to(x.dtype)
    return x


def rope_gaussian(n_streams: int, n_tokens: int, d: int, seed: int, device="cpu",
                  dtype=torch.bfloat16, token_chunk: int = 32768) -> torch.Tensor:
    """[n_streams, n_tokens, d]: N(0,1) then rotated by position (same distribution, RoPE-like)."""
    out = torch.empty(n_streams, n_tokens, d, dtype=dtype, device=device)
    for s in range(n_streams):
        g = _gen(seed * 1000003 + s, device)
        for t0 in range(0, n_tokens, token_chunk):
            t1 = min(n_tokens, t0 + token_chunk)
            x = torch.randn(t1 - t0, d, generator=g, device=device, dtype=torch.float32)
            rope_rotate_(x, torch.arange(t0, t1, device=device))
            out[s, t0:t1] = x.to(dtype)
    return out


def student_t(n_streams: int, n_tokens: int, d: int, nu: int, seed: int, device="cpu",
              dtype=torch.bfloat16) -> torch.Tensor:
    """i.i.d. Student-t(nu) coordinates: Z / sqrt(chi2_nu / nu), chi2_nu a sum of nu squared normals."""
    out = torch.empty(n_streams, n_tokens, d, dtype=dtype, device=device)
    for s in range(n_streams):
        g = _gen(seed * 1000003 + s, device)
        z = torch.randn(n_tokens, d, generator=g, device=device, dtype=torch.float32)
        chi = torch.zeros_like(z)
        for _ in range(nu):
            w = torch.randn(n_tokens, d, generator=g, device=device, dtype=torch.float32)
            chi += w * w
        out[s] = (z / torch.sqrt(chi / nu)).to(dtype)
    return out


def low_rank(n_streams: int, n_tokens: int, d: int, spectrum, noise: float, seed: int, subspace_seed: int,
             n_heads: int | None = None, device="cpu", dtype=torch.bfloat16, exclude_seed: int | None = None
             ) -> torch.Tensor:
    """Tokens in a random rank-r subspace plus isotropic noise: x = B_h (g ⊙ sqrt(spectrum)) + noise·n,
    g, n ~ N(0, I), B_h a d x r orthonormal basis drawn per head h = stream % n_heads from
    `subspace_seed` (QR of a Gaussian matrix).  With `exclude_seed`, B_h is drawn inside the
    orthogonal complement of the basis that seed gives (K and V in orthogonal subspaces).  These are
    the structured regimes "lowrank", "lowrank_aligned", "lowrank_steep" and "lowrank_misalign" of
    "Ablation, Statistical Inference, and Validation for KV-Cache Compression", §8 (Table 4)."""
    spec = np.asarray(spectrum, dtype=np.float64)
    r = len(spec)
    n_heads = n_heads or n_streams
    bases = []
    for h in range(n_heads):
        rng = np.random.default_rng(subspace_seed * 7919 + h)
        if exclude_seed is None:
            B, _ = np.linalg.qr(rng.standard_normal((d, r)))
        else:
            E, _ = np.linalg.qr(np.random.default_rng(exclude_seed * 7919 + h).standard_normal((d, r)))
            M = rng.standard_normal((d, r))
            B, _ = np.linalg.qr(M - E @ (E.T @ M))
        bases.append(torch.from_numpy(B * np.sqrt(spec)[None, :]).float())
    out = torch.empty(n_streams, n_tokens, d, dtype=dtype, device=device)
    for s in range(n_streams):
        g = _gen(seed * 1000003 + s, device)
        z = torch.randn(n_tokens, r, generator=g, device=device, dtype=torch.float32)
        x = z @ bases[s % n_heads].to(device).T
        if noise > 0:
            x += noise * torch.randn(n_tokens, d, generator=g, device=device, dtype=torch.float32)
        out[s] = x.to(dtype)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Exact host copy of a bf16 tensor as uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------------------------
# The five workloads.  `scale` < 1 shrinks token counts (and heads) for parity tests.
# ---------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    b: int
    m: int
    seed_k: int
    seed_v: int


CONFIGS = {
    "cfg1": Workload("single head d=64, 4096 fp32 keys, per-channel std U[0.5,2]; b=4, no QJL", 64, 4, 0, 1001, 0),
    "cfg2": Workload("K,V bf16 32 heads x 32768 x d=128, 4 outlier channels x10; b=4", 128, 4, 0, 2001, 2002),
    "cfg3": Workload("K bf16 8 heads x 65536 x d=128 N(0,1); b=3 + QJL m=128; 32 queries/head", 128, 3, 128, 3001, 0),
    "cfg4": Workload("GQA decode attention: batch 16, 32 q / 8 kv heads, context 131072, d=128; "
                     "K b=4 + QJL m=128, V b=4; RoPE-rotated N(0,1)", 128, 4, 128, 4001, 4002),
    "cfg5": Workload("Student-t nu=3, d=256, 16 heads x 262144 tokens bf16; b in {2,3,5,6}, QJL m=256 on K",
                     256, 3, 0, 5001, 5002),
}


def cfg4_queries(batch: int, n_q_heads: int, d: int, position: int, seed: int, device="cpu") -> torch.Tensor:
    q = gaussian((batch, n_q_heads, d), seed, device=device, dtype=torch.float32)
    flat = q.view(-1, d)
    rope_rotate_(flat, torch.full((flat.shape[0],), position, device=device))
    return q.to(torch.bfloat16)

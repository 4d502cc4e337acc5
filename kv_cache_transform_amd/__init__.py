"""MI355X-native TurboQuant-family KV-cache codec (Python binding of libtq.so).

Every step of the path runs in the HIP kernels behind the C ABI (include/tq.h); this module only
marshals torch tensors (device memory) and the current HIP stream.  Sources: "Ablation, Statistical
Inference, and Validation for KV-Cache Compression" (arXiv 2607.09683), §2 TurboQuant.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import TQError, TQ_BF16, TQ_F32

__all__ = ["Codec", "TQError", "get_layout", "encode", "decode", "qk_scores", "decode_attention",
           "attention_workspace_bytes", "decode_attention_noalloc", "host_tables", "clear_cache", "SQCodec", "sq_host_codebook", "sq_decode_attention", "FmagCodec",
           "fmag_decode_attention"]

_DT = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}


@dataclass(frozen=True)
class Codec:
    """d: head_dim (64/128/256); b: codebook bits; m: QJL sketch rows (0 = none);
    n_heads: heads with distinct random state (stream st uses head st % n_heads); seed;
    sketch: 0 = Gaussian S, 1 = randomized Hadamard S = H diag(s2) (needs m = d);
    rotation: 0 = WHT with random signs (TurboQuant), 1 = none (Plain-KV)."""
    d: int
    b: int
    m: int = 0
    n_heads: int = 1
    seed: int = 0
    sketch: int = 0
    rotation: int = 0

    def params(self) -> _lib.Params:
        return _lib.Params(self.d, self.b, self.m, self.n_heads, self.seed & ((1 << 64) - 1), self.sketch,
                           self.rotation)


def _stream(device=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def get_layout(codec: Codec, n_streams: int, n_tokens: int) -> dict:
    lay = _lib.Layout()
    _lib.check(_lib.lib().tq_get_layout(ctypes.byref(codec.params()), n_streams, n_tokens, ctypes.byref(lay)),
               "tq_get_layout")
    return {f: getattr(lay, f) for f, _ in _lib.Layout._fields_}


def encode(codec: Codec, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """x: [n_streams, n_tokens, d] float32 or bfloat16 on the GPU -> packed uint8 buffer."""
    if x.dim() != 3 or x.shape[-1] != codec.d or not x.is_contiguous():
        raise ValueError("x must be a contiguous [n_streams, n_tokens, d] tensor")
    S, N, _ = x.shape
    lay = get_layout(codec, S, N)
    if out is None:
        out = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=x.device)
    elif out.numel() < lay["total_bytes"] or out.dtype != torch.uint8:
        raise ValueError("packed buffer too small")
    _lib.check(_lib.lib().tq_encode(ctypes.byref(codec.params()), _ptr(x), _DT[x.dtype], S, N, _ptr(out),
                                    _stream(x.device)), "tq_encode")
    return out


def encode_kv(ck: Codec, cv: Codec, k: torch.Tensor, v: torch.Tensor, out_k: torch.Tensor | None = None,
              out_v: torch.Tensor | None = None):
    """Keys and values of the same tokens (tq_encode_kv): k, v [n_streams, n_tokens, d] of one dtype
    on the GPU -> (packed K, packed V), the same bytes as encode(ck, k) and encode(cv, v)."""
    for x, c in ((k, ck), (v, cv)):
        if x.dim() != 3 or x.shape[-1] != c.d or not x.is_contiguous():
            raise ValueError("k and v must be contiguous [n_streams, n_tokens, d] tensors")
    if k.shape[:2] != v.shape[:2] or k.dtype != v.dtype:
        raise ValueError("k and v must have the same streams, tokens and dtype")
    S, N, _ = k.shape
    outs = []
    for c, o in ((ck, out_k), (cv, out_v)):
        need = get_layout(c, S, N)["total_bytes"]
        if o is None:
            o = torch.empty(need, dtype=torch.uint8, device=k.device)
        elif o.numel() < need or o.dtype != torch.uint8:
            raise ValueError("packed buffer too small")
        outs.append(o)
    _lib.check(_lib.lib().tq_encode_kv(ctypes.byref(ck.params()), ctypes.byref(cv.params()), _ptr(k), _ptr(v),
                                       _DT[k.dtype], S, N, _ptr(outs[0]), _ptr(outs[1]), _stream(k.device)),
               "tq_encode_kv")
    return outs[0], outs[1]


def encode_kv_append(ck: Codec, cv: Codec, k: torch.Tensor, v: torch.Tensor, packed_k: torch.Tensor,
                     packed_v: torch.Tensor, capacity: int, t0: int):
    """Keys and values of the same new tokens (tq_encode_kv_append): k, v [n_streams, n_new, d] into
    tokens [t0, t0 + n_new) of caches laid out for n_streams x capacity tokens."""
    for x, c in ((k, ck), (v, cv)):
        if x.dim() != 3 or x.shape[-1] != c.d or not x.is_contiguous():
            raise ValueError("k and v must be contiguous [n_streams, n_new, d] tensors")
    if k.shape[:2] != v.shape[:2] or k.dtype != v.dtype:
        raise ValueError("k and v must have the same streams, tokens and dtype")
    S, N, _ = k.shape
    for c, pb in ((ck, packed_k), (cv, packed_v)):
        if pb.dtype != torch.uint8 or pb.numel() < get_layout(c, S, capacity)["total_bytes"]:
            raise ValueError("packed buffer too small for the capacity")
    _lib.check(_lib.lib().tq_encode_kv_append(ctypes.byref(ck.params()), ctypes.byref(cv.params()), _ptr(k), _ptr(v),
                                              _DT[k.dtype], S, N, _ptr(packed_k), _ptr(packed_v), capacity, t0,
                                              _stream(k.device)), "tq_encode_kv_append")
    return packed_k, packed_v


def encode_append(codec: Codec, x: torch.Tensor, packed: torch.Tensor, capacity: int, t0: int) -> torch.Tensor:
    """x: [n_streams, n_new, d] -> tokens [t0, t0 + n_new) of `packed`, a buffer laid out for
    n_streams x capacity tokens (get_layout(codec, n_streams, capacity))."""
    if x.dim() != 3 or x.shape[-1] != codec.d or not x.is_contiguous():
        raise ValueError("x must be a contiguous [n_streams, n_new, d] tensor")
    S, N, _ = x.shape
    if packed.dtype != torch.uint8 or packed.numel() < get_layout(codec, S, capacity)["total_bytes"]:
        raise ValueError("packed buffer too small for the capacity")
    _lib.check(_lib.lib().tq_encode_append(ctypes.byref(codec.params()), _ptr(x), _DT[x.dtype], S, N, _ptr(packed),
                                           capacity, t0, _stream(x.device)), "tq_encode_append")
    return packed


def decode(codec: Codec, packed: torch.Tensor, n_streams: int, n_tokens: int,
           dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None, qjl: bool = False) -> torch.Tensor:
    """MSE reconstruction (tq_decode), or with qjl=True the reconstruction with the sketch
    correction added in the rotated domain (tq_decode_qjl; needs codec.m > 0)."""
    if out is None:
        out = torch.empty(n_streams, n_tokens, codec.d, dtype=dtype, device=packed.device)
    fn = _lib.lib().tq_decode_qjl if qjl else _lib.lib().tq_decode
    _lib.check(fn(ctypes.byref(codec.params()), _ptr(packed), n_streams, n_tokens, _ptr(out),
                  _DT[out.dtype], _stream(packed.device)), "tq_decode_qjl" if qjl else "tq_decode")
    return out


def qk_scores(codec: Codec, q: torch.Tensor, packed_k: torch.Tensor, n_tokens: int,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """q: [n_streams, n_q, d] -> unscaled score estimates [n_streams, n_q, n_tokens] (float32)."""
    S, nq, _ = q.shape
    ws_bytes = _lib.lib().tq_scores_workspace_bytes(ctypes.byref(codec.params()), S, nq)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(S, nq, n_tokens, dtype=torch.float32, device=q.device)
    _lib.check(_lib.lib().tq_qk_scores(ctypes.byref(codec.params()), _ptr(q), _DT[q.dtype], nq, _ptr(packed_k), S,
                                       n_tokens, _ptr(out), _ptr(workspace), workspace.numel(),
                                       _stream(q.device)), "tq_qk_scores")
    return out


def attention_workspace_bytes(ck: Codec, batch: int, n_q_heads: int, n_kv_heads: int, n_tokens: int) -> int:
    return int(_lib.lib().tq_attention_workspace_bytes(ctypes.byref(ck.params()), batch, n_q_heads, n_kv_heads,
                                                       n_tokens))


def decode_attention(ck: Codec, cv: Codec, q: torch.Tensor, packed_k: torch.Tensor, packed_v: torch.Tensor,
                     n_kv_heads: int, n_tokens: int, softmax_scale: float = 0.0,
                     out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, lengths: torch.Tensor | None = None) -> torch.Tensor:
    """q: [batch, n_q_heads, d] -> attention output [batch, n_q_heads, d] over the packed cache of
    n_tokens per stream; lengths (int32 [batch] on the GPU): valid tokens per batch element."""
    B, Hq, d = q.shape
    if workspace is None:
        workspace = torch.empty(max(attention_workspace_bytes(ck, B, Hq, n_kv_heads, n_tokens), 16),
                                dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() < B or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per batch element")
    _lib.check(_lib.lib().tq_decode_attention_varlen(
        ctypes.byref(ck.params()), ctypes.byref(cv.params()), _ptr(q), _DT[q.dtype], B, Hq, n_kv_heads,
        _ptr(packed_k), _ptr(packed_v), n_tokens, _ptr(lengths) if lengths is not None else None,
        ctypes.c_float(softmax_scale), _ptr(out), _DT[out.dtype],
        _ptr(workspace), workspace.numel(), _stream(q.device)), "tq_decode_attention_varlen")
    return out


def decode_attention_noalloc(ck: Codec, cv: Codec, q: torch.Tensor, packed_k: torch.Tensor,
                             packed_v: torch.Tensor, n_kv_heads: int, n_tokens: int, out: torch.Tensor,
                             softmax_scale: float = 0.0, lengths: torch.Tensor | None = None) -> torch.Tensor:
    """decode_attention into a caller-given `out`, with no device allocation anywhere: the workspace
    is the library's own per-device array (at most tq_attention_noalloc_max_bytes()), and the codec
    tables must already be resident (an earlier encode with the same codecs on this device)."""
    B, Hq, _ = q.shape
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() < B or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per batch element")
    _lib.check(_lib.lib().tq_decode_attention_noalloc(
        ctypes.byref(ck.params()), ctypes.byref(cv.params()), _ptr(q), _DT[q.dtype], B, Hq, n_kv_heads,
        _ptr(packed_k), _ptr(packed_v), n_tokens, _ptr(lengths) if lengths is not None else None,
        ctypes.c_float(softmax_scale), _ptr(out), _DT[out.dtype], _stream(q.device)), "tq_decode_attention_noalloc")
    return out


def host_tables(codec: Codec, head: int = 0) -> dict:
    """Host copies of the library's tables (thresholds, centroids in fp64; signs; S as float)."""
    import numpy as np
    L = 1 << codec.b
    thr = np.zeros(L - 1, dtype=np.float64)
    cen = np.zeros(L, dtype=np.float64)
    sg = np.zeros(codec.d, dtype=np.float32)
    S = np.zeros(max(codec.m, 1) * codec.d, dtype=np.float32)
    _lib.check(_lib.lib().tq_host_tables(ctypes.byref(codec.params()), head, thr.ctypes.data, cen.ctypes.data,
                                         sg.ctypes.data, S.ctypes.data), "tq_host_tables")
    return {"thresholds": thr, "centroids": cen, "signs": sg,
            "S": S[: codec.m * codec.d].reshape(codec.m, codec.d) if codec.m else None}


def clear_cache() -> None:
    _lib.lib().tq_clear_cache()


class SQCodec:
    """SpectralQuant codec (include/tq_sq.h): one calibrated eigenbasis per head, the semantic
    dimensions at b bits (or water-filled), the tail at b_tail bits, per-dimension Gaussian
    Lloyd-Max codebooks ("Ablation, Statistical Inference, and Validation for KV-Cache
    Compression", §2 "SpectralQuant", §6, §7).  Build with ``SQCodec.calibrate``; the device tables
    live on the device that was current then and are freed with the object.  m > 0 adds the
    selective QJL sketch of the semantic residual (SQU-QKV), keyed by ``seed``; it needs d_eff."""

    def __init__(self, d: int, n_heads: int, basis, lam, bits, d_eff=None, device=None, m: int = 0,
                 seed: int = 0):
        import numpy as np
        self.d, self.n_heads, self.m, self.seed = int(d), int(n_heads), int(m), int(seed)
        self.basis = np.ascontiguousarray(basis, dtype=np.float64).reshape(n_heads, d, d)
        self.lam = np.ascontiguousarray(lam, dtype=np.float64).reshape(n_heads, d)
        self.bits = np.ascontiguousarray(bits, dtype=np.int32).reshape(n_heads, d)
        self.d_eff = None if d_eff is None else np.ascontiguousarray(d_eff, dtype=np.int32).reshape(n_heads)
        self._h = None
        p = _lib.SqParams(self.d, self.n_heads, 1, 1, 0, 0, 0.0, self.m, self.seed)
        h = ctypes.c_void_p()
        de = self.d_eff.ctypes.data if self.d_eff is not None else None
        with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
            self.device = torch.cuda.current_device()
            _lib.check(_lib.lib().tq_sq_create(ctypes.byref(p), self.basis.ctypes.data, self.lam.ctypes.data,
                                               self.bits.ctypes.data, de, ctypes.byref(h)), "tq_sq_create")
        self._h = h
        rb = ctypes.c_int64()
        _lib.check(_lib.lib().tq_sq_record_bytes(self._h, ctypes.byref(rb)), "tq_sq_record_bytes")
        self.record_bytes = int(rb.value)

    @staticmethod
    def calibrate_host(x_cal, b: int, b_tail: int, waterfill: bool = False, gamma: float = 10.0,
                       d_eff_max: int = 0) -> dict:
        """x_cal: [n_heads, n_cal, d] float32 (host or device) -> the model arrays (host numpy)."""
        import numpy as np
        x = x_cal.detach().float().cpu().numpy() if isinstance(x_cal, torch.Tensor) else np.asarray(x_cal)
        x = np.ascontiguousarray(x, dtype=np.float32)
        H, n_cal, d = x.shape
        p = _lib.SqParams(d, H, b, b_tail, int(bool(waterfill)), d_eff_max, float(gamma), 0, 0)
        basis = np.zeros((H, d, d), dtype=np.float64)
        lam = np.zeros((H, d), dtype=np.float64)
        bits = np.zeros((H, d), dtype=np.int32)
        d_eff = np.zeros(H, dtype=np.int32)
        _lib.check(_lib.lib().tq_sq_calibrate(ctypes.byref(p), x.ctypes.data, n_cal, basis.ctypes.data,
                                              lam.ctypes.data, bits.ctypes.data, d_eff.ctypes.data),
                   "tq_sq_calibrate")
        return {"basis": basis, "lam": lam, "bits": bits, "d_eff": d_eff}

    @classmethod
    def calibrate(cls, x_cal, b: int, b_tail: int, waterfill: bool = False, gamma: float = 10.0,
                  d_eff_max: int = 0, device=None, m: int = 0, seed: int = 0) -> "SQCodec":
        md = cls.calibrate_host(x_cal, b, b_tail, waterfill, gamma, d_eff_max)
        H, d = md["lam"].shape
        return cls(d, H, md["basis"], md["lam"], md["bits"], md["d_eff"], device, m, seed)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h is None:
            return
        try:        # at interpreter exit the modules may already be gone: then the process frees it
            torch.cuda.synchronize(self.device)
            _lib.lib().tq_sq_destroy(h)
        except Exception:
            pass

    def encode(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """x: [n_streams, n_tokens, d] bfloat16 -> packed records (uint8, n_streams·n_tokens·record_bytes)."""
        if x.dim() != 3 or x.shape[-1] != self.d or not x.is_contiguous():
            raise ValueError("x must be a contiguous [n_streams, n_tokens, d] tensor")
        S, N, _ = x.shape
        need = S * N * self.record_bytes
        if out is None:
            out = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
        elif out.numel() < need or out.dtype != torch.uint8:
            raise ValueError("packed buffer too small")
        _lib.check(_lib.lib().tq_sq_encode(self._h, _ptr(x), _DT.get(x.dtype, -1), S, N, _ptr(out),
                                           _stream(x.device)), "tq_sq_encode")
        return out

    def decode(self, packed: torch.Tensor, n_streams: int, n_tokens: int, dtype: torch.dtype = torch.float32,
               out: torch.Tensor | None = None) -> torch.Tensor:
        if out is None:
            out = torch.empty(n_streams, n_tokens, self.d, dtype=dtype, device=packed.device)
        _lib.check(_lib.lib().tq_sq_decode(self._h, _ptr(packed), n_streams, n_tokens, _ptr(out),
                                           _DT[out.dtype], _stream(packed.device)), "tq_sq_decode")
        return out

    def qk_scores(self, q: torch.Tensor, packed_k: torch.Tensor, n_tokens: int, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
        """q: [n_streams, n_q, d] -> <Uᵀq, ẑ> as float32 [n_streams, n_q, n_tokens]."""
        S, nq, _ = q.shape
        ws = int(_lib.lib().tq_sq_scores_workspace_bytes(self._h, S, nq))
        if workspace is None:
            workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty(S, nq, n_tokens, dtype=torch.float32, device=q.device)
        _lib.check(_lib.lib().tq_sq_qk_scores(self._h, _ptr(q), _DT[q.dtype], nq, _ptr(packed_k), S, n_tokens,
                                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device)),
                   "tq_sq_qk_scores")
        return out


def sq_decode_attention(ck: SQCodec, cv: SQCodec, q: torch.Tensor, packed_k: torch.Tensor,
                        packed_v: torch.Tensor, n_kv_heads: int, n_tokens: int, softmax_scale: float = 0.0,
                        out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, lengths: torch.Tensor | None = None) -> torch.Tensor:
    """q: [batch, n_q_heads, d] -> attention output over SpectralQuant K/V caches (tq_sq_decode_attention)."""
    B, Hq, d = q.shape
    if workspace is None:
        ws = int(_lib.lib().tq_sq_attention_workspace_bytes(ck._h, B, Hq, n_kv_heads, n_tokens))
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() < B or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per batch element")
    _lib.check(_lib.lib().tq_sq_decode_attention(
        ck._h, cv._h, _ptr(q), _DT[q.dtype], B, Hq, n_kv_heads, _ptr(packed_k), _ptr(packed_v), n_tokens,
        _ptr(lengths) if lengths is not None else None, ctypes.c_float(softmax_scale), _ptr(out), _DT[out.dtype],
        _ptr(workspace), workspace.numel(), _stream(q.device)), "tq_sq_decode_attention")
    return out


def sq_host_codebook(b: int) -> dict:
    """The library's b-bit Gaussian Lloyd-Max codebook (host fp64)."""
    import numpy as np
    thr = np.zeros((1 << b) - 1, dtype=np.float64)
    cen = np.zeros(1 << b, dtype=np.float64)
    _lib.check(_lib.lib().tq_sq_host_codebook(b, thr.ctypes.data, cen.ctypes.data), "tq_sq_host_codebook")
    return {"thresholds": thr, "centroids": cen}


@dataclass(frozen=True)
class FmagCodec:
    """Fourier-magnitude codec (include/tq_fmag.h; "Fourier Magnitude KV Cache Quantization",
    "Method"): d = 64 or 128, b magnitude bits (1..8), p phase bits (1..8, or 16 for a bf16 phase)."""
    d: int
    b: int = 4
    p: int = 8

    def params(self) -> _lib.FmagParams:
        return _lib.FmagParams(self.d, self.b, self.p)

    @property
    def record_bytes(self) -> int:
        n = ctypes.c_int64()
        _lib.check(_lib.lib().tq_fmag_record_bytes(ctypes.byref(self.params()), ctypes.byref(n)), "tq_fmag_record_bytes")
        return int(n.value)

    def encode(self, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        if x.dim() != 3 or x.shape[-1] != self.d or not x.is_contiguous():
            raise ValueError("x must be a contiguous [n_streams, n_tokens, d] tensor")
        S, N, _ = x.shape
        need = S * N * self.record_bytes
        if out is None:
            out = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
        elif out.numel() < need or out.dtype != torch.uint8:
            raise ValueError("packed buffer too small")
        _lib.check(_lib.lib().tq_fmag_encode(ctypes.byref(self.params()), _ptr(x), _DT.get(x.dtype, -1), S, N,
                                             _ptr(out), _stream(x.device)), "tq_fmag_encode")
        return out

    def decode(self, packed: torch.Tensor, n_streams: int, n_tokens: int, dtype: torch.dtype = torch.float32,
               out: torch.Tensor | None = None) -> torch.Tensor:
        if out is None:
            out = torch.empty(n_streams, n_tokens, self.d, dtype=dtype, device=packed.device)
        _lib.check(_lib.lib().tq_fmag_decode(ctypes.byref(self.params()), _ptr(packed), n_streams, n_tokens, _ptr(out),
                                             _DT[out.dtype], _stream(packed.device)), "tq_fmag_decode")
        return out

    def qk_scores(self, q: torch.Tensor, packed: torch.Tensor, n_tokens: int, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
        S, nq, _ = q.shape
        ws = int(_lib.lib().tq_fmag_scores_workspace_bytes(ctypes.byref(self.params()), S, nq))
        if workspace is None:
            workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty(S, nq, n_tokens, dtype=torch.float32, device=q.device)
        _lib.check(_lib.lib().tq_fmag_qk_scores(ctypes.byref(self.params()), _ptr(q), _DT[q.dtype], nq, _ptr(packed),
                                                S, n_tokens, _ptr(out), _ptr(workspace), workspace.numel(),
                                                _stream(q.device)), "tq_fmag_qk_scores")
        return out


def fmag_decode_attention(ck: FmagCodec, cv: FmagCodec, q: torch.Tensor, packed_k: torch.Tensor,
                          packed_v: torch.Tensor, n_kv_heads: int, n_tokens: int, softmax_scale: float = 0.0,
                          out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, lengths: torch.Tensor | None = None) -> torch.Tensor:
    """q: [batch, n_q_heads, d] -> attention output over Fmag K/V caches (tq_fmag_decode_attention)."""
    B, Hq, d = q.shape
    pk, pv = ck.params(), cv.params()
    if workspace is None:
        ws = int(_lib.lib().tq_fmag_attention_workspace_bytes(ctypes.byref(pk), B, Hq, n_kv_heads, n_tokens))
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=q.device)
    if lengths is not None and (lengths.dtype != torch.int32 or lengths.numel() < B or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous int32 tensor with one entry per batch element")
    _lib.check(_lib.lib().tq_fmag_decode_attention(
        ctypes.byref(pk), ctypes.byref(pv), _ptr(q), _DT[q.dtype], B, Hq, n_kv_heads, _ptr(packed_k), _ptr(packed_v),
        n_tokens, _ptr(lengths) if lengths is not None else None, ctypes.c_float(softmax_scale), _ptr(out),
        _DT[out.dtype], _ptr(workspace), workspace.numel(), _stream(q.device)), "tq_fmag_decode_attention")
    return out

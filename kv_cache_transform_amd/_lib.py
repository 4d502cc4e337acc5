"""ctypes loader for libtq.so (the C ABI declared in include/tq.h, tq_sq.h and tq_fmag.h).

The library is required: there is no fallback implementation.  If libtq.so has not been built
(``python -m kv_cache_transform_amd.build``) every call raises."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_EWORKSPACE, TQ_EHIP = 0, -1, -2, -3, -4, -5
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_SKETCH_GAUSSIAN, TQ_SKETCH_RHT = 0, 1
TQ_ROTATION_WHT, TQ_ROTATION_NONE = 0, 1

# every symbol include/tq.h declares
EXPORTS = ("tq_get_layout", "tq_encode", "tq_encode_kv", "tq_encode_kv_append", "tq_encode_append", "tq_decode", "tq_decode_qjl", "tq_scores_workspace_bytes", "tq_qk_scores",
           "tq_attention_workspace_bytes", "tq_decode_attention", "tq_decode_attention_varlen",
           "tq_decode_attention_noalloc", "tq_attention_noalloc_max_bytes", "tq_host_tables",
           "tq_status_string",
           "tq_clear_cache")
# every symbol include/tq_sq.h declares
SQ_EXPORTS = ("tq_sq_calibrate", "tq_sq_create", "tq_sq_destroy", "tq_sq_record_bytes", "tq_sq_encode",
              "tq_sq_decode", "tq_sq_scores_workspace_bytes", "tq_sq_qk_scores", "tq_sq_attention_workspace_bytes",
              "tq_sq_decode_attention", "tq_sq_host_codebook")
# every symbol include/tq_fmag.h declares
FMAG_EXPORTS = ("tq_fmag_record_bytes", "tq_fmag_encode", "tq_fmag_decode", "tq_fmag_scores_workspace_bytes",
                "tq_fmag_qk_scores", "tq_fmag_attention_workspace_bytes", "tq_fmag_decode_attention")


class Params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("b", ctypes.c_int32), ("m", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("seed", ctypes.c_uint64), ("sketch", ctypes.c_int32),
                ("rotation", ctypes.c_int32)]


class SqParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("b", ctypes.c_int32),
                ("b_tail", ctypes.c_int32), ("waterfill", ctypes.c_int32), ("d_eff_max", ctypes.c_int32),
                ("gamma", ctypes.c_double), ("m", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class FmagParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("b", ctypes.c_int32), ("p", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("idx_bytes_per_vec", ctypes.c_int64), ("sketch_bytes_per_vec", ctypes.c_int64),
                ("off_idx", ctypes.c_int64), ("off_sketch", ctypes.c_int64), ("off_norm", ctypes.c_int64),
                ("off_rnorm", ctypes.c_int64), ("total_bytes", ctypes.c_int64)]


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_transform_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, VP, I32, SZ = ctypes.POINTER(Params), ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    Q = ctypes.POINTER(SqParams)
    FP = ctypes.POINTER(FmagParams)
    sig = {
        "tq_get_layout": (ctypes.c_int, [P, I64, I64, ctypes.POINTER(Layout)]),
        "tq_encode": (ctypes.c_int, [P, VP, ctypes.c_int, I64, I64, VP, VP]),
        "tq_encode_append": (ctypes.c_int, [P, VP, ctypes.c_int, I64, I64, VP, I64, I64, VP]),
        "tq_encode_kv": (ctypes.c_int, [P, P, VP, VP, ctypes.c_int, I64, I64, VP, VP, VP]),
        "tq_encode_kv_append": (ctypes.c_int, [P, P, VP, VP, ctypes.c_int, I64, I64, VP, VP, I64, I64, VP]),
        "tq_decode": (ctypes.c_int, [P, VP, I64, I64, VP, ctypes.c_int, VP]),
        "tq_decode_qjl": (ctypes.c_int, [P, VP, I64, I64, VP, ctypes.c_int, VP]),
        "tq_scores_workspace_bytes": (SZ, [P, I64, I64]),
        "tq_qk_scores": (ctypes.c_int, [P, VP, ctypes.c_int, I64, VP, I64, I64, VP, VP, SZ, VP]),
        "tq_attention_workspace_bytes": (SZ, [P, I32, I32, I32, I64]),
        "tq_decode_attention": (ctypes.c_int, [P, P, VP, ctypes.c_int, I32, I32, I32, VP, VP, I64,
                                               ctypes.c_float, VP, ctypes.c_int, VP, SZ, VP]),
        "tq_decode_attention_varlen": (ctypes.c_int, [P, P, VP, ctypes.c_int, I32, I32, I32, VP, VP, I64, VP,
                                                      ctypes.c_float, VP, ctypes.c_int, VP, SZ, VP]),
        "tq_decode_attention_noalloc": (ctypes.c_int, [P, P, VP, ctypes.c_int, I32, I32, I32, VP, VP, I64, VP,
                                                       ctypes.c_float, VP, ctypes.c_int, VP]),
        "tq_attention_noalloc_max_bytes": (SZ, []),
        "tq_host_tables": (ctypes.c_int, [P, I32, VP, VP, VP, VP]),
        "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tq_clear_cache": (None, []),
        "tq_sq_calibrate": (ctypes.c_int, [Q, VP, I64, VP, VP, VP, VP]),
        "tq_sq_create": (ctypes.c_int, [Q, VP, VP, VP, VP, ctypes.POINTER(VP)]),
        "tq_sq_destroy": (None, [VP]),
        "tq_sq_record_bytes": (ctypes.c_int, [VP, ctypes.POINTER(I64)]),
        "tq_sq_encode": (ctypes.c_int, [VP, VP, ctypes.c_int, I64, I64, VP, VP]),
        "tq_sq_decode": (ctypes.c_int, [VP, VP, I64, I64, VP, ctypes.c_int, VP]),
        "tq_sq_scores_workspace_bytes": (SZ, [VP, I64, I64]),
        "tq_sq_qk_scores": (ctypes.c_int, [VP, VP, ctypes.c_int, I64, VP, I64, I64, VP, VP, SZ, VP]),
        "tq_sq_host_codebook": (ctypes.c_int, [I32, VP, VP]),
        "tq_sq_attention_workspace_bytes": (SZ, [VP, I32, I32, I32, I64]),
        "tq_fmag_record_bytes": (ctypes.c_int, [FP, ctypes.POINTER(I64)]),
        "tq_fmag_encode": (ctypes.c_int, [FP, VP, ctypes.c_int, I64, I64, VP, VP]),
        "tq_fmag_decode": (ctypes.c_int, [FP, VP, I64, I64, VP, ctypes.c_int, VP]),
        "tq_fmag_scores_workspace_bytes": (SZ, [FP, I64, I64]),
        "tq_fmag_qk_scores": (ctypes.c_int, [FP, VP, ctypes.c_int, I64, VP, I64, I64, VP, VP, SZ, VP]),
        "tq_fmag_attention_workspace_bytes": (SZ, [FP, I32, I32, I32, I64]),
        "tq_fmag_decode_attention": (ctypes.c_int, [FP, FP, VP, ctypes.c_int, I32, I32, I32, VP, VP, I64, VP,
                                                    ctypes.c_float, VP, ctypes.c_int, VP, SZ, VP]),
        "tq_sq_decode_attention": (ctypes.c_int, [VP, VP, VP, ctypes.c_int, I32, I32, I32, VP, VP, I64, VP,
                                                  ctypes.c_float, VP, ctypes.c_int, VP, SZ, VP]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def check(status: int, what: str) -> None:
    if status != TQ_OK:
        raise TQError(status, what)

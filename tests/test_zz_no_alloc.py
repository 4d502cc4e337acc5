"""The allocation-free decode-attention entry point, tq_decode_attention_noalloc (include/tq.h),
through the C ABI: two calls in a row on the library's device array, the second smaller, against
tq_decode_attention_varlen with a caller workspace on the same inputs, and against the oracle; and
its limits (a problem above the array's size, codec tables not yet resident)."""
import math

import numpy as np
import pytest
import torch

import kv_cache_transform_amd as T
from kv_cache_transform_amd import _lib
from oracle import tq_oracle as O
from synth import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(batch, hq, hkv, N, d, b, m, seed, lens=None):
    ck, cv = T.Codec(d, b, m, hkv, seed), T.Codec(d, b, 0, hkv, seed + 1)
    K = I.rope_gaussian(batch * hkv, N, d, seed, device=DEV)
    V = I.rope_gaussian(batch * hkv, N, d, seed + 1, device=DEV)
    q = I.cfg4_queries(batch, hq, d, N, seed + 2, device=DEV)
    pk, pv = T.encode(ck, K), T.encode(cv, V)          # builds (and leaves resident) the codec tables
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    return dict(ck=ck, cv=cv, q=q, pk=pk, pv=pv, hkv=hkv, N=N, lt=lt, lens=lens)


def _oracle_rows(c, rows):
    ck, cv, d = c["ck"], c["cv"], c["q"].shape[-1]
    tk, tv = P.Tables(d, ck.b, ck.m, c["hkv"], ck.seed), P.Tables(d, cv.b, 0, c["hkv"], cv.seed)
    B, Hq = c["q"].shape[:2]
    rk = O.unpack_tensor(c["pk"].cpu().numpy(), d, ck.b, ck.m, B * c["hkv"], c["N"])
    rv = O.unpack_tensor(c["pv"].cpu().numpy(), d, cv.b, 0, B * c["hkv"], c["N"])
    q64 = O.bf16_bits_to_f64(I.bf16_bits(c["q"]))
    out = []
    for bi, h in rows:
        st = bi * c["hkv"] + h // (Hq // c["hkv"])
        L = c["N"] if c["lens"] is None else c["lens"][bi]
        cut = lambda r: {k: v[:L] for k, v in r.items()}
        out.append(P.oracle_attention_row(tk, tv, cut(rk[st]), cut(rv[st]), st, q64[bi, h], 1 / math.sqrt(d)))
    return np.array(out)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_the_workspace_entry_point_on_two_calls(out_dtype):
    big = _case(2, 8, 2, 5000, 128, 4, 128, 9101, lens=[5000, 3001])
    small = _case(1, 4, 1, 700, 128, 4, 128, 9201)
    outs = []
    for c in (big, small):            # back to back: the second call finds the first one's contents
        B, Hq, d = c["q"].shape
        out = torch.empty(B, Hq, d, dtype=out_dtype, device=DEV)
        T.decode_attention_noalloc(c["ck"], c["cv"], c["q"], c["pk"], c["pv"], c["hkv"], c["N"], out,
                                   lengths=c["lt"])
        outs.append(out)
    torch.cuda.synchronize()
    for c, out in zip((big, small), outs):
        ref = T.decode_attention(c["ck"], c["cv"], c["q"], c["pk"], c["pv"], c["hkv"], c["N"],
                                 out_dtype=out_dtype, lengths=c["lt"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref)            # the same kernels on the same inputs: bit-identical
        rows = [(0, 0), (0, 3), (c["q"].shape[0] - 1, c["q"].shape[1] - 1)]
        want = _oracle_rows(c, rows)
        got = np.array([out[bi, h].float().cpu().numpy() for bi, h in rows])
        r = P.check_attention_rows(got, want, out_dtype == torch.bfloat16)
        print(f"no-alloc attention N={c['N']}: worst row rel L2 {r['worst']:.2e}")


def test_noalloc_rejects_a_problem_above_the_array():
    # 4096 streams of one split each: 4096 x 16 x 128 x 4 B of partials alone exceed 32 MiB
    ck, cv = T.Codec(128, 4, 0, 8, 9301), T.Codec(128, 4, 0, 8, 9302)
    need = T.attention_workspace_bytes(ck, 512, 8, 8, 256)
    assert need > _lib.lib().tq_attention_noalloc_max_bytes()
    dummy = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    q = torch.zeros(512, 8, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(512, 8, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(T.TQError) as ei:
        T.decode_attention_noalloc(ck, cv, q, dummy, dummy, 8, 256, out)
    assert ei.value.status == _lib.TQ_EWORKSPACE


def test_noalloc_needs_resident_tables():
    ck, cv = T.Codec(128, 4, 0, 1, 987654321), T.Codec(128, 4, 0, 1, 987654322)   # never used before
    dummy = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(T.TQError) as ei:
        T.decode_attention_noalloc(ck, cv, q, dummy, dummy, 1, 16, out)
    assert ei.value.status == _lib.TQ_EUNSUPPORTED

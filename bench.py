"""Benchmark: encode & decode-attention throughput of the TurboQuant-family KV-cache codec on one
MI355X, in bf16-equivalent GB/s and as a fraction of the HBM roofline.

Workload (the configuration the metric is quoted on): fused GQA decode attention over a compressed
cache — batch 16, 32 query heads / 8 KV heads, context 131072, d = 128; K encoded with a 4-bit
WHT + Lloyd-Max codebook plus a 1-bit QJL sketch (m = 128), V with a 4-bit codebook; K and V are
seeded N(0,1) bf16 rotated RoPE-style by position; queries N(0,1) bf16 rotated at t = 131072.

One step = encode K and V (one launch) + decode-attention (split-K attention, which does the
query prep itself on this shape, then the split combine).
bf16-equivalent bytes of a step = (#K + #V vectors) x d x 2 B, counted once for the encode and
once for the attention pass over the cache.

Extra per-kernel lines (standalone decode of the V cache to bf16) are timed separately after the
headline step and reported under "kernels"; they are not part of `value`.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published (the sketch projection's operand type)

# HBM bytes per launch from two rocprofv3 counter runs of this benchmark (FETCH_SIZE, WRITE_SIZE,
# per dispatch), scaled by what the same counters read for the 1 GiB copy that copy_ceiling()
# times: 1 FETCH_SIZE unit = 2048 B, 1 WRITE_SIZE unit = 1024 B.  A figure is reported only while
# the kernel's sources are the ones it was measured on (sha256 of the .hip file + shared headers).
FETCH_UNIT_B, WRITE_UNIT_B = 2048, 1024
TRAFFIC = {
    "encode_kv": {"fetch": 4194704.0, "write": 2495027.78125, "src": "encode.hip",
        "sha": "992d71c591d2d8a443bf0051e0ef8e31966255a4ca7629b73e9250ddda24daac"},
    "encode_k": {"fetch": 2097505.5, "write": 1394656.375, "src": "encode.hip",
        "sha": "992d71c591d2d8a443bf0051e0ef8e31966255a4ca7629b73e9250ddda24daac"},
    "encode_v": {"fetch": 2111449.75, "write": 1091140.375, "src": "encode.hip",
        "sha": "992d71c591d2d8a443bf0051e0ef8e31966255a4ca7629b73e9250ddda24daac"},
    "decode_attention": {"fetch": 1232278.4375, "write": 6240.0, "src": "attention.hip",
        "sha": "57c6ef526353f7a450afd9a3dc46799f2fd1264f7a21d212250aa6aa4b42032f"},
    "decode_v_bf16": {"fetch": 550368.25, "write": 4194304.0, "src": "decode.hip",
        "sha": "b1ba67ba042266686af375dd30fa7fbae0fbf2bf933c7820de5b5978f1c26054"},
}
TRAFFIC["decode_attention_back_to_back"] = TRAFFIC["decode_attention"]
TRAFFIC_HEADERS_SHA = ("6643b4ed6d32e0cc4205551fb1ef8fab74077690c7d82ac29a903d73ebc0d666"   # common.hpp
                       "183fca10670edac7211b62d0d02df11d2a540416ee2b250c1d8ac7525a821db7")  # kernels.hpp


def _sha(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes(kernel: str):
    """calibrated HBM bytes per launch of `kernel`, or None if its sources changed since measured"""
    t = TRAFFIC.get(kernel)
    csrc = os.path.join(ROOT, "kv_cache_transform_amd", "csrc")
    if t is None or _sha(os.path.join(csrc, t["src"])) != t["sha"]:
        return None
    hdr = _sha(os.path.join(csrc, "common.hpp")) + _sha(os.path.join(csrc, "kernels.hpp"))
    if TRAFFIC_HEADERS_SHA is not None and hdr != TRAFFIC_HEADERS_SHA:
        return None
    return int(round(t["fetch"] * FETCH_UNIT_B + t["write"] * WRITE_UNIT_B))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--no-extra", action="store_true", help="skip the per-kernel lines of the other workloads")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the codec has no "
                  f"multi-GPU path (one GPU per process is all it runs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_transform_amd as T
    from synth import inputs as I

    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, Hq, Hkv, N, d = 16, 32, 8, args.context, 128
    ck = T.Codec(d, 4, 128, Hkv, 4001)
    cv = T.Codec(d, 4, 0, Hkv, 4002)
    streams = B * Hkv
    print(f"[bench] generating K,V bf16 [{streams},{N},{d}] on {dev}", file=sys.stderr, flush=True)
    K = I.rope_gaussian(streams, N, d, 4001, device=dev)
    V = I.rope_gaussian(streams, N, d, 4002, device=dev)
    q = I.cfg4_queries(B, Hq, d, N, 4003, device=dev)
    lk, lv = T.get_layout(ck, streams, N), T.get_layout(cv, streams, N)
    pk = torch.empty(lk["total_bytes"], dtype=torch.uint8, device=dev)
    pv = torch.empty(lv["total_bytes"], dtype=torch.uint8, device=dev)
    ws = torch.empty(T.attention_workspace_bytes(ck, B, Hq, Hkv, N), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # the step: keys and values encoded in one launch (tq_encode_kv: each wave takes a key group
    # and then the values of the same tokens), then decode-attention
    names = ("encode_kv", "decode_attention")
    ev = {n: [] for n in names}

    def step(record: bool):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if record else None
        if record:
            marks[0].record(stream)
        T.encode_kv(ck, cv, K, V, pk, pv)
        if record:
            marks[1].record(stream)
        T.decode_attention(ck, cv, q, pk, pv, Hkv, N, out=out, workspace=ws)
        if record:
            marks[2].record(stream)
            for i, n in enumerate(names):
                ev[n].append((marks[i], marks[i + 1]))

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    samples = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in names}
    kms = {n: sum(samples[n]) / len(samples[n]) for n in names}

    # algorithmic bytes per launch (what each kernel must move at minimum)
    nvec = streams * N
    k_rec = d * 4 // 8 + 128 // 8 + 2 + 2          # 84 B packed K per vector
    v_rec = d * 4 // 8 + 2                         # 66 B packed V per vector
    alg = {
        "encode_k": nvec * (2 * d + k_rec),
        "encode_v": nvec * (2 * d + v_rec),
        "decode_attention": nvec * (k_rec + v_rec) + 2 * B * Hq * d * 2,
    }
    alg["encode_kv"] = alg["encode_k"] + alg["encode_v"]
    bf16eq_step = 2 * nvec * d * 2 * 2             # K and V, encode pass + attention pass
    value = bf16eq_step / (ms_step * 1e-3) / 1e9
    value_single = bf16eq_step / 2 / (ms_step * 1e-3) / 1e9   # the cache's bf16 size once per step
    # each tensor's encode alone (tq_encode), 20 launches after one untimed, outside the step
    for n, c, x, pb in (("encode_k", ck, K, pk), ("encode_v", cv, V, pv)):
        T.encode(c, x, pb)
        torch.cuda.synchronize()
        pairs = []
        for _ in range(args.steps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            T.encode(c, x, pb)
            b_.record(stream)
            pairs.append((a_, b_))
        torch.cuda.synchronize()
        samples[n] = [a_.elapsed_time(b_) for a_, b_ in pairs]
        kms[n] = sum(samples[n]) / len(samples[n])
    T.encode_kv(ck, cv, K, V, pk, pv)     # the step's records again, for the parity sample below
    torch.cuda.synchronize()
    # decode-attention launched back to back (no encode between calls): the kernel in the power state
    # of its own load; the step's figure above is the one that counts
    pairs = []
    for _ in range(args.steps):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        T.decode_attention(ck, cv, q, pk, pv, Hkv, N, out=out, workspace=ws)
        b_.record(stream)
        pairs.append((a_, b_))
    torch.cuda.synchronize()
    samples["decode_attention_back_to_back"] = [a_.elapsed_time(b_) for a_, b_ in pairs]
    kms["decode_attention_back_to_back"] = sum(samples["decode_attention_back_to_back"]) / args.steps
    alg["decode_attention_back_to_back"] = alg["decode_attention"]
    kern = {}
    for n in ("encode_kv", "encode_k", "encode_v", "decode_attention", "decode_attention_back_to_back"):
        gbs = alg[n] / (kms[n] * 1e-3) / 1e9
        nb = (1 if n in ("encode_k", "encode_v") else 2) * nvec * d * 2
        bf = nb / (kms[n] * 1e-3) / 1e9
        kern[n] = {"ms": round(kms[n], 4), **_spread(samples[n]), "alg_bytes": alg[n], "achieved_GBs": round(gbs, 1),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bf16_equiv_GBs": round(bf, 1)}
        if n in ("encode_kv", "encode_k"):
            kern[n]["sketch_tflops"] = round(nvec * 2 * ck.m * d / (kms[n] * 1e-3) / 1e12, 2)

    # the CPU baseline's parity sample: the GPU's own records of the step's caches (taken now: the
    # extra lines below reuse the packed buffers)
    sample = None
    if not args.no_cpu_baseline:
        sample = _parity_sample(K[:1, :2048], V[:1, :2048], pk, pv, ck, cv, streams, N, d)

    # standalone decode of the V cache to bf16, timed apart from the step
    xh = torch.empty(streams, N, d, dtype=torch.bfloat16, device=dev)
    T.decode(cv, pv, streams, N, torch.bfloat16, out=xh)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        T.decode(cv, pv, streams, N, torch.bfloat16, out=xh)
    e1.record(stream)
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / 3
    dec_alg = nvec * (v_rec + 2 * d)
    kern["decode_v_bf16"] = {"ms": round(dms, 4), "alg_bytes": dec_alg,
                             "achieved_GBs": round(dec_alg / (dms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(dec_alg / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del xh

    if not args.no_extra:
        # a decode step on a growing cache: append one token to every stream of K (launch-bound), and
        # attention over per-batch lengths spread evenly from N/2 to N
        x1 = K[:, -1:].contiguous()
        T.encode_append(ck, x1, pk, N, N - 1)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            T.encode_append(ck, x1, pk, N, N - 1)
        e1.record(stream)
        torch.cuda.synchronize()
        kern["append_k_1_token"] = {"us": round(e0.elapsed_time(e1) / 20 * 1e3, 2), "vectors": streams}
        # the decode step's append of one key and one value per stream, in one launch
        v1 = V[:, -1:].contiguous()
        T.encode_kv_append(ck, cv, x1, v1, pk, pv, N, N - 1)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            T.encode_kv_append(ck, cv, x1, v1, pk, pv, N, N - 1)
        e1.record(stream)
        torch.cuda.synchronize()
        kern["append_kv_1_token"] = {"us": round(e0.elapsed_time(e1) / 20 * 1e3, 2), "vectors": 2 * streams}
        lens = torch.linspace(N // 2, N, B).to(torch.int32).to(dev)
        T.decode_attention(ck, cv, q, pk, pv, Hkv, N, out=out, workspace=ws, lengths=lens)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            T.decode_attention(ck, cv, q, pk, pv, Hkv, N, out=out, workspace=ws, lengths=lens)
        e1.record(stream)
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / 5
        valg = int(lens.sum().item()) * Hkv * (k_rec + v_rec) + 2 * B * Hq * d * 2
        kern["decode_attention_varlen"] = {"ms": round(vms, 4), "alg_bytes": valg,
                                           "achieved_GBs": round(valg / (vms * 1e-3) / 1e9, 1),
                                           "hbm_frac": round(valg / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

        # the same K encode with the randomized Hadamard sketch (S = H diag(s2), m = d = 128): the
        # sketch is one more 32-point transform of the residual, not a dense m x d product
        ck_rht = T.Codec(d, 4, 128, Hkv, 4001, sketch=1)
        T.encode(ck_rht, K, pk)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            T.encode(ck_rht, K, pk)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / 3
        kern["encode_k_rht"] = {"ms": round(rms, 4), "alg_bytes": alg["encode_k"],
                                "achieved_GBs": round(alg["encode_k"] / (rms * 1e-3) / 1e9, 1),
                                "hbm_frac": round(alg["encode_k"] / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # and its decode to bf16 with the sketch correction added (84 B in, 256 B out per key)
        xh = torch.empty(streams, N, d, dtype=torch.bfloat16, device=dev)
        T.decode(ck_rht, pk, streams, N, torch.bfloat16, out=xh, qjl=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            T.decode(ck_rht, pk, streams, N, torch.bfloat16, out=xh, qjl=True)
        e1.record(stream)
        torch.cuda.synchronize()
        qms = e0.elapsed_time(e1) / 3
        qalg = nvec * (k_rec + 2 * d)
        kern["decode_k_rht_qjl_bf16"] = {"ms": round(qms, 4), "alg_bytes": qalg,
                                         "achieved_GBs": round(qalg / (qms * 1e-3) / 1e9, 1),
                                         "hbm_frac": round(qalg / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del xh
        # the V encode without rotation (Plain-KV): the same quantiser on the unrotated unit vector
        cv_plain = T.Codec(d, 4, 0, Hkv, 4002, rotation=1)
        T.encode(cv_plain, V, pv)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            T.encode(cv_plain, V, pv)
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / 3
        kern["encode_v_plain"] = {"ms": round(pms, 4), "alg_bytes": alg["encode_v"],
                                  "achieved_GBs": round(alg["encode_v"] / (pms * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(alg["encode_v"] / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # SpectralQuant on the same K cache: one eigenbasis per kv head calibrated on that head's first
        # 512 tokens of batch element 0, semantic dimensions at 4 bits, the tail at 2 bits
        sq = T.SQCodec.calibrate(K[:Hkv, :512].float(), 4, 2, device=0)
        sq_alg = nvec * (2 * d + sq.record_bytes)
        sq.encode(K, pk)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            sq.encode(K, pk)
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / 3
        kern["sq_encode_k"] = {"ms": round(sms, 4), "alg_bytes": sq_alg, "record_bytes": sq.record_bytes,
                               "d_eff": [int(v) for v in sq.d_eff],
                               "achieved_GBs": round(sq_alg / (sms * 1e-3) / 1e9, 1),
                               "hbm_frac": round(sq_alg / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        xh = torch.empty(streams, N, d, dtype=torch.bfloat16, device=dev)
        sq.decode(pk, streams, N, torch.bfloat16, out=xh)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            sq.decode(pk, streams, N, torch.bfloat16, out=xh)
        e1.record(stream)
        torch.cuda.synchronize()
        sdm = e0.elapsed_time(e1) / 3
        kern["sq_decode_k_bf16"] = {"ms": round(sdm, 4), "alg_bytes": sq_alg,
                                    "achieved_GBs": round(sq_alg / (sdm * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(sq_alg / (sdm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del xh
        # SpectralQuant decode-attention over SQ K and V caches of the same shape (V calibrated the
        # same way), 32 query heads per batch element
        sqv = T.SQCodec.calibrate(V[:Hkv, :512].float(), 4, 2, device=0)
        sqv.encode(V, pv)
        sws = torch.empty(max(int(T._lib.lib().tq_sq_attention_workspace_bytes(sq._h, B, Hq, Hkv, N)), 16),
                          dtype=torch.uint8, device=dev)
        T.sq_decode_attention(sq, sqv, q, pk, pv, Hkv, N, out=out, workspace=sws)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            T.sq_decode_attention(sq, sqv, q, pk, pv, Hkv, N, out=out, workspace=sws)
        e1.record(stream)
        torch.cuda.synchronize()
        sam = e0.elapsed_time(e1) / 5
        sqa_alg = nvec * (sq.record_bytes + sqv.record_bytes) + 2 * B * Hq * d * 2
        kern["sq_decode_attention"] = {"ms": round(sam, 4), "alg_bytes": sqa_alg,
                                       "achieved_GBs": round(sqa_alg / (sam * 1e-3) / 1e9, 1),
                                       "hbm_frac": round(sqa_alg / (sam * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del sq, sqv, sws
        # the Fourier-magnitude codec on the same K cache: 4-bit magnitudes and 8-bit phases
        # ("Fmag4+phase8b"), 108-byte records
        fm = T.FmagCodec(d, 4, 8)
        fm_alg = nvec * (2 * d + fm.record_bytes)
        fpk = torch.empty(nvec * fm.record_bytes, dtype=torch.uint8, device=dev)
        fm.encode(K, fpk)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            fm.encode(K, fpk)
        e1.record(stream)
        torch.cuda.synchronize()
        fms = e0.elapsed_time(e1) / 3
        kern["fmag_encode_k"] = {"ms": round(fms, 4), "alg_bytes": fm_alg, "record_bytes": fm.record_bytes,
                                 "achieved_GBs": round(fm_alg / (fms * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(fm_alg / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        xh = torch.empty(streams, N, d, dtype=torch.bfloat16, device=dev)
        fm.decode(fpk, streams, N, torch.bfloat16, out=xh)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            fm.decode(fpk, streams, N, torch.bfloat16, out=xh)
        e1.record(stream)
        torch.cuda.synchronize()
        fdm = e0.elapsed_time(e1) / 3
        kern["fmag_decode_k_bf16"] = {"ms": round(fdm, 4), "alg_bytes": fm_alg,
                                      "achieved_GBs": round(fm_alg / (fdm * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(fm_alg / (fdm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del xh
        # Fmag decode-attention over Fmag K and V caches of the same shape, 32 query heads per batch
        fpv = torch.empty(nvec * fm.record_bytes, dtype=torch.uint8, device=dev)
        fm.encode(V, fpv)
        fws = torch.empty(max(int(T._lib.lib().tq_fmag_attention_workspace_bytes(
            ctypes.byref(fm.params()), B, Hq, Hkv, N)), 16), dtype=torch.uint8, device=dev)
        T.fmag_decode_attention(fm, fm, q, fpk, fpv, Hkv, N, out=out, workspace=fws)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            T.fmag_decode_attention(fm, fm, q, fpk, fpv, Hkv, N, out=out, workspace=fws)
        e1.record(stream)
        torch.cuda.synchronize()
        fam = e0.elapsed_time(e1) / 3
        fa_alg = nvec * 2 * fm.record_bytes + 2 * B * Hq * d * 2
        kern["fmag_decode_attention"] = {"ms": round(fam, 4), "alg_bytes": fa_alg,
                                         "achieved_GBs": round(fa_alg / (fam * 1e-3) / 1e9, 1),
                                         "hbm_frac": round(fa_alg / (fam * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del fpk, fpv, fws
    del K

    copy = copy_ceiling(torch, dev, stream)
    del V
    torch.cuda.empty_cache()
    extra = None if args.no_extra else other_workloads(torch, T, I, dev, stream)

    for n in kern:
        kern[n]["traffic_bytes"] = traffic_bytes(n)

    # roofline of the dominant kernel.  The sketch encode also carries a dense m x d contraction
    # (2 m d flop per key, one fp16 MFMA pass); its bound is whichever floor is longer: the
    # algorithmic bytes at the HBM peak or the flops at the fp16 MFMA peak.  Both rates are reported.
    dom = max(names, key=lambda n: kms[n])
    flops = nvec * 2 * ck.m * d if (dom in ("encode_k", "encode_kv") and ck.m > 0) else 0
    if flops and flops / (MFMA_F16_PEAK_TFLOPS * 1e12) > alg[dom] / (HBM_PEAK_GBS * 1e9):
        ach = flops / (kms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic_bytes(dom),
                "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg[dom], "avg_launch_ms": kern[dom]["ms"],
                "hbm_achieved_GBs": kern[dom]["achieved_GBs"], "hbm_frac": kern[dom]["hbm_frac"]}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["achieved_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kern[dom]["hbm_frac"], "traffic": traffic_bytes(dom),
                "alg_bytes_per_launch": alg[dom], "avg_launch_ms": kern[dom]["ms"]}
        if flops:
            ach = flops / (kms[dom] * 1e-3) / 1e12
            roof.update({"alg_flops_per_launch": flops, "mfma_achieved_TFLOPs": round(ach, 1),
                         "mfma_frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4)})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sample)

    line = {
        "metric": "encode & decode-attention bf16-equiv GB/s on 1 MI355X; % of HBM peak",
        "value": round(value, 1), "unit": "GB/s (bf16-equivalent)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate, fp16 MFMA operands",
        "data": "synthetic (seeded N(0,1) bf16, RoPE-rotated by position)",
        "config": {"workload": "GQA decode attention over a TQ-compressed cache: batch 16, 32 q / 8 kv heads, "
                               f"context {N}, d=128; K b=4 + QJL m=128, V b=4; step = encode K and V (one launch) + "
                               "decode-attention", "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "context": N, "d": d, "b_k": 4, "m_k": 128, "b_v": 4},
        "value_single_pass": round(value_single, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        "copy_ceiling": copy,
        "other_workloads": extra,
    }
    print(json.dumps(line))


_FLUSH = []


def _spread(ms: list) -> dict:
    """median and 10th / 90th percentiles of per-launch times (nearest rank)"""
    v = sorted(ms)
    at = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]
    return {"median_ms": round(at(0.5), 4), "p10_ms": round(at(0.1), 4), "p90_ms": round(at(0.9), 4)}


def _time(torch, stream, fn, reps: int = 20) -> list:
    """per-launch ms of fn() over reps launches on `stream` (after one untimed call); before every timed
    launch, outside its events, a 1 GiB buffer is read (a reduction: clean lines only, so no
    write-back lands in the timed launch) so that neither the L2s nor the 256 MB Infinity Cache
    still hold the launch's inputs (the smaller workloads would otherwise fit)"""
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.int32, device=torch.cuda.current_device()))
    fn()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        _FLUSH[0].sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _line(samples: list, alg_bytes: int) -> dict:
    """mean ms (the rate's basis), its spread, and the algorithmic rate"""
    ms = sum(samples) / len(samples)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), **_spread(samples), "alg_bytes": alg_bytes, "achieved_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def other_workloads(torch, T, I, dev, stream) -> dict:
    """Per-kernel lines (not part of `value`) for the other workload shapes: encode / decode of
    outlier-channel K,V (32 heads x 32768 x 128, b = 4), encode with a QJL sketch and q.k scores
    (8 heads x 65536 x 128, b = 3, m = 128, 32 queries per head), and heavy-tailed d = 256 vectors
    (16 heads x 262144, Student-t nu = 3, b = 3, with and without a sketch of m = 256); the sketch
    encodes also with the randomized Hadamard sketch (m = d).  Every timed launch starts from a
    flushed cache hierarchy (see _time)."""
    out = {}
    H, N, d = 32, 32768, 128
    x = I.outlier_gaussian(H, N, d, 4, 10.0, 2001, device=dev)
    c = T.Codec(d, 4, 0, H, 2001)
    pk = T.encode(c, x)
    xh = torch.empty(H, N, d, dtype=torch.bfloat16, device=dev)
    nv = H * N
    out["outlier K 32x32768x128 b4: encode"] = _line(_time(torch, stream, lambda: T.encode(c, x, pk)), nv * (256 + 66))
    out["outlier K 32x32768x128 b4: decode to bf16"] = _line(
        _time(torch, stream, lambda: T.decode(c, pk, H, N, torch.bfloat16, out=xh)), nv * (66 + 256))
    # its K and V (V: other outlier channels, own seed) encoded in one launch (tq_encode_kv)
    xv = I.outlier_gaussian(H, N, d, 4, 10.0, 2002, device=dev)
    cv = T.Codec(d, 4, 0, H, 2002)
    pv = T.encode(cv, xv)
    out["outlier K,V 32x32768x128 b4: encode K and V (one launch)"] = _line(
        _time(torch, stream, lambda: T.encode_kv(c, cv, x, xv, pk, pv)), 2 * nv * (256 + 66))
    del x, xv, pk, pv, xh

    H, N, d, nq = 8, 65536, 128, 32
    x = I.gaussian((H, N, d), 3001, device=dev)
    q = I.gaussian((H, nq, d), 3008, device=dev)
    c = T.Codec(d, 3, 128, H, 3001)
    pk = T.encode(c, x)
    sc = torch.empty(H, nq, N, dtype=torch.float32, device=dev)
    import ctypes
    ws = torch.empty(max(int(T._lib.lib().tq_scores_workspace_bytes(ctypes.byref(c.params()), H, nq)), 16),
                     dtype=torch.uint8, device=dev)
    nv = H * N
    out["gaussian K 8x65536x128 b3 m128: encode"] = _line(_time(torch, stream, lambda: T.encode(c, x, pk)),
                                                         nv * (256 + 48 + 16 + 4))
    out["gaussian K 8x65536x128 b3 m128: scores, 32 queries"] = _line(
        _time(torch, stream, lambda: T.qk_scores(c, q, pk, N, out=sc, workspace=ws)), nv * (48 + 16 + 4 + 4 * nq))
    c = T.Codec(d, 3, 128, H, 3001, sketch=1)
    out["gaussian K 8x65536x128 b3 RHT m128: encode"] = _line(_time(torch, stream, lambda: T.encode(c, x, pk)),
                                                             nv * (256 + 48 + 16 + 4))
    del x, q, pk, sc, ws

    H, N, d = 16, 262144, 256
    x = I.student_t(H, N, d, 3, 5001, device=dev)
    nv = H * N
    for m, kind in ((0, 0), (256, 0), (256, 1)):
        c = T.Codec(d, 3, m, H, 5004, sketch=kind)
        pk = T.encode(c, x)
        rec = 96 + m // 8 + 2 + (2 if m else 0)
        name = f"student-t K 16x262144x256 b3 {'RHT ' if kind else ''}m{m}: encode"
        out[name] = _line(_time(torch, stream, lambda: T.encode(c, x, pk)), nv * (512 + rec))
        if m == 0:
            xh = torch.empty(H, N, d, dtype=torch.bfloat16, device=dev)
            out["student-t K 16x262144x256 b3: decode to bf16"] = _line(
                _time(torch, stream, lambda: T.decode(c, pk, H, N, torch.bfloat16, out=xh)), nv * (rec + 512))
            del xh
        del pk
    del x
    _FLUSH.clear()
    torch.cuda.empty_cache()
    return out


def copy_ceiling(torch, dev, stream, n_bytes: int = 1 << 30, reps: int = 5):
    """Practical HBM ceiling: torch's device copy of an n_bytes buffer (read n_bytes + write n_bytes),
    timed with HIP events over `reps` launches.  Its hardware byte counters also calibrate the
    FETCH_SIZE / WRITE_SIZE figures of the codec kernels."""
    src = torch.empty(n_bytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"kernel": "torch copy_ of a 1 GiB bf16 buffer", "bytes_per_launch": 2 * n_bytes,
            "ms": round(ms, 4), "GBs": round(2 * n_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(2 * n_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle (unchanged) on the host cores, on bounded samples of every workload
# ---------------------------------------------------------------------------------------------
def _oracle_samples(name: str, seed: int):
    """Seeded host inputs of one workload's sample (the same recipes as the GPU inputs, generated on
    the CPU) and the codec parameters: returns (d, x, q, codecs)."""
    import numpy as np
    import torch

    from oracle import tq_oracle as O
    from synth import inputs as I

    def f64(t):
        return O.bf16_bits_to_f64(I.bf16_bits(t)) if t.dtype == torch.bfloat16 else t.double().numpy()

    if name == "1":
        return 64, I.per_channel_gaussian(4096, 64, 1).astype(np.float64), None, {"x": (4, 0, 1001)}
    if name == "2":
        return 128, f64(I.outlier_gaussian(1, 2048, 128, 4, 10.0, seed)[0]), None, {"x": (4, 0, 2001)}
    if name == "3":
        return (128, f64(I.gaussian((1, 2048, 128), seed)[0]), f64(I.gaussian((1, 32, 128), seed + 7)[0]),
                {"x": (3, 128, 3001)})
    if name == "4":
        kv = I.rope_gaussian(2, 2048, 128, seed)
        return (128, (f64(kv[0]), f64(kv[1])), f64(I.cfg4_queries(1, 4, 128, 131072, seed + 2)[0]),
                {"k": (4, 128, 4001), "v": (4, 0, 4002)})
    if name == "5":
        return (256, f64(I.student_t(1, 1024, 256, 3, seed)[0]), f64(I.gaussian((1, 64, 256), seed + 3)[0]),
                {"x": (3, 0, 5004), "xs": (3, 256, 5004)})
    raise ValueError(name)


def _oracle_ops(name: str, seed: int, min_s: float) -> dict:
    """Time the oracle's steps on one workload's sample: {op: [seconds per repetition, bf16-equivalent
    bytes per repetition]}.  Tables (codebook, signs, S) are built before the clock starts, as the
    library builds them once per parameter set."""
    import numpy as np

    from oracle import tq_oracle as O

    d, x, q, cod = _oracle_samples(name, seed)
    tabs = {}
    for key, (b, m, sd) in cod.items():
        t, c = O.lloyd_max(d, b)
        tabs[key] = (t, c, O.head_signs(sd, 0, d), O.gaussian_matrix(sd, 0, m, d).astype(np.float64) if m else None)

    def clock(fn, nbytes):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                return [el / reps, nbytes]

    out = {}
    if name == "4":
        (k, v), (tk, ck, sk, Sk), (tv, cv, sv, _) = x, tabs["k"], tabs["v"]
        n = k.shape[0]
        rk, rv = O.encode(k, sk, tk, ck, Sk), O.encode(v, sv, tv, cv)
        out["encode_k"] = clock(lambda: O.encode(k, sk, tk, ck, Sk), n * d * 2)
        out["encode_v"] = clock(lambda: O.encode(v, sv, tv, cv), n * d * 2)
        out["attention"] = clock(lambda: O.attention_rotated(O.scores(q, rk, sk, ck, Sk), rv, sv, cv,
                                                             1.0 / math.sqrt(d)), 2 * n * d * 2)
        return out
    n = x.shape[0]
    for key, (t, c, s, S) in tabs.items():
        tag = "" if len(tabs) == 1 else ("_m0" if S is None else f"_m{S.shape[0]}")
        r = O.encode(x, s, t, c, S)
        out["encode" + tag] = clock(lambda: O.encode(x, s, t, c, S), n * d * 2)
        if S is None:
            out["decode"] = clock(lambda: O.decode(r["idx"], r["n16"], s, c), n * d * 2)
        if q is not None:
            out["scores" + tag] = clock(lambda: O.scores(q, r, s, c, S), n * d * 2)
    return out


CPU_CONFIGS = {
    "1": "4096 x 64 fp32 per-channel Gaussian, b = 4 (the whole workload)",
    "2": "2048 of the 32 x 32768 x 128 outlier-channel tokens, b = 4",
    "3": "2048 of the 8 x 65536 x 128 Gaussian keys, b = 3 + QJL m = 128; 32 queries",
    "4": "2048 K and 2048 V tokens of one (batch, kv head) of the 16 x 8 x 131072 x 128 RoPE caches, "
         "K b = 4 + QJL m = 128, V b = 4; attention of its 4 query heads",
    "5": "1024 of the 16 x 262144 x 256 Student-t tokens, b = 3 with m = 0 and m = 256; 64 queries",
}


def _cpu_worker(args):
    """pool worker: every workload's oracle steps on one thread (BLAS, OpenMP and torch's own pool,
    whose idle threads would otherwise spin beside the other workers)"""
    seed, min_s = args
    import torch
    from threadpoolctl import threadpool_limits
    torch.set_num_threads(1)
    with threadpool_limits(1):
        return {name: _oracle_ops(name, seed, min_s) for name in CPU_CONFIGS}


def _cpu_model() -> str:
    import subprocess
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def _parity_sample(sample_k, sample_v, pk, pv, ck, cv, streams, N, d):
    """Flag and mismatch counts of the GPU's own packed bytes against the oracle on the CPU
    baseline's benchmark sample (stream 0, its first tokens): indices differ only at coordinates the
    oracle flags within 1e-6 of a threshold, sketch bits only where |S e| < 1e-6."""
    import numpy as np

    import kv_cache_transform_amd as T
    from oracle import tq_oracle as O
    from synth import inputs as I

    n = sample_k.shape[1]
    res = {"tokens": n}
    for tag, x, buf, c in (("k", sample_k, pk, ck), ("v", sample_v, pv, cv)):
        lay = T.get_layout(c, streams, N)
        ib, sb = d * c.b // 8, c.m // 8
        small = O.layout(d, c.b, c.m, 1, n)
        host = np.zeros(small["total_bytes"], dtype=np.uint8)
        host[:n * ib] = buf[lay["off_idx"]:lay["off_idx"] + n * ib].cpu().numpy()
        host[small["off_norm"]:small["off_norm"] + 2 * n] = buf[lay["off_norm"]:lay["off_norm"] + 2 * n].cpu().numpy()
        if c.m:
            host[small["off_sketch"]:small["off_sketch"] + n * sb] = \
                buf[lay["off_sketch"]:lay["off_sketch"] + n * sb].cpu().numpy()
            host[small["off_rnorm"]:small["off_rnorm"] + 2 * n] = \
                buf[lay["off_rnorm"]:lay["off_rnorm"] + 2 * n].cpu().numpy()
        g = O.unpack_tensor(host, d, c.b, c.m, 1, n)[0]
        t, cent = O.lloyd_max(d, c.b)
        S = O.gaussian_matrix(c.seed, 0, c.m, d).astype(np.float64) if c.m else None
        o = O.encode(O.bf16_bits_to_f64(I.bf16_bits(x[0])), O.head_signs(c.seed, 0, d), t, cent, S)
        mis = g["idx"] != o["idx"]
        res[f"{tag}_flagged"] = int(o["flag"].sum())
        res[f"{tag}_idx_mismatch"] = int(mis.sum())
        res[f"{tag}_idx_mismatch_unflagged"] = int((mis & ~o["flag"]).sum())
        if c.m:
            k = O.sketch(o["y"] - cent[g["idx"]], S)          # from the GPU's indices
            smis = g["sigma"] != k["sigma"]
            res[f"{tag}_sketch_flagged"] = int(k["sflag"].sum())
            res[f"{tag}_sketch_mismatch"] = int(smis.sum())
            res[f"{tag}_sketch_mismatch_unflagged"] = int((smis & ~k["sflag"]).sum())
    return res


def cpu_baseline(parity_sample: dict, min_s=0.3):
    """The oracle, unchanged, on the host cores: every workload's steps on a bounded sample (see
    CPU_CONFIGS), once on one core and once on all cores (a process pool, one BLAS thread per
    worker, each worker on its own seeded sample), as bf16-equivalent GB/s per step and workload.
    `value` is the all-core rate of the benchmark step's oracle steps (encode K, encode V, attention,
    with the bytes counted as the GPU value counts them)."""
    import multiprocessing as mp
    import statistics

    from threadpoolctl import threadpool_info, threadpool_limits

    t_all = time.perf_counter()
    n_cpu = os.cpu_count() or 1
    workers = max(1, min(n_cpu, 16))
    import torch
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    with threadpool_limits(1):
        one = {name: _oracle_ops(name, 11, min_s) for name in CPU_CONFIGS}
    torch.set_num_threads(torch_threads)
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(workers)
    try:
        runs = pool.map(_cpu_worker, [(101 + w, min_s) for w in range(workers)])
    finally:
        # close and wait, so that no worker outlives the benchmark
        pool.close()
        pool.join()

    def rate(sec, nbytes, k=1):
        return round(k * nbytes / sec / 1e9, 5)

    per = {}
    for name in CPU_CONFIGS:
        per[name] = {"sample": CPU_CONFIGS[name], "ops": {}}
        for op, (sec, nbytes) in one[name].items():
            med = statistics.median(r[name][op][0] for r in runs)
            per[name]["ops"][op] = {"one_core_GBs": rate(sec, nbytes), "all_cores_GBs": rate(med, nbytes, workers)}
    step_ops = ("encode_k", "encode_v", "attention")
    step_bytes = sum(one["4"][op][1] for op in step_ops)
    step_one = sum(one["4"][op][0] for op in step_ops)
    step_all = statistics.median(sum(r["4"][op][0] for op in step_ops) for r in runs)
    blas = sorted({f"{i.get('internal_api')} x{i.get('num_threads')}" for i in threadpool_info()
                   if i.get("user_api") == "blas"})
    return {"value": rate(step_all, step_bytes, workers), "unit": "GB/s (bf16-equivalent)", "cores": workers,
            "kind": "oracle",
            "sample": "benchmark step (encode K with QJL m = 128, encode V, attention) on " + CPU_CONFIGS["4"] +
                      f"; {workers} worker processes, each on its own seeded sample, one BLAS thread each",
            "one_core": {"value": rate(step_one, step_bytes), "cores": 1},
            "cpu_model": _cpu_model(), "os_cpu_count": n_cpu, "blas": blas,
            "per_workload": per,
            "parity_sample": parity_sample,
            "seconds": round(time.perf_counter() - t_all, 1)}


if __name__ == "__main__":
    main()

"""Benchmark: encode & decode-attention throughput of the TurboQuant-family KV-cache codec on one
MI355X, in bf16-equivalent GB/s and as a fraction of the HBM roofline.

Workload (the configuration the metric is quoted on): fused GQA decode attention over a compressed
cache — batch 16, 32 query heads / 8 KV heads, context 131072, d = 128; K encoded with a 4-bit
WHT + Lloyd-Max codebook plus a 1-bit QJL sketch (m = 128), V with a 4-bit codebook; K and V are
seeded N(0,1) bf16 rotated RoPE-style by position; queries N(0,1) bf16 rotated at t = 131072.

One step = encode K + encode V + decode-attention (query prep, split-K attention, combine).
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
    "encode_k": {"fetch": 2098036.3125, "write": 1396372.1875, "src": "encode.hip",
        "sha": "8a0903eabd6cacabcc36311aa6afbed04c33927a364972d4494d305cbd3cdc24"},
    "encode_v": {"fetch": 2103114.8125, "write": 1091211.78125, "src": "encode.hip",
        "sha": "8a0903eabd6cacabcc36311aa6afbed04c33927a364972d4494d305cbd3cdc24"},
    "decode_attention": {"fetch": 1229622.5625, "write": 4160.0, "src": "attention.hip",
        "sha": "5eaa6f22be6d97fd700da9ac46a3e41690d14c0314e54edf6993c26acab1c6d7"},
    "decode_v_bf16": {"fetch": 550394.375, "write": 4194304.0, "src": "decode.hip",
        "sha": "2add9ea1fa8cf5d1d37b9846a4505b28cdfa3553557c2e41c88d2f2cc96455e9"},
}
TRAFFIC_HEADERS_SHA = ("9241f7e7fc6398e3b61bd782d033f3beac2c8fe34392745cceb9f2f364e6409c"   # common.hpp
                       "4b7bff386ff4b44e581f4d585bec686d2e3a7033871a21ebe797ef96ebd8decf")  # kernels.hpp


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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--no-extra", action="store_true", help="skip the per-kernel lines of the other workloads")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the codec has no "
                  f"multi-GPU path in this build; run with --gpus 1", file=sys.stderr)
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

    names = ("encode_k", "encode_v", "decode_attention")
    ev = {n: [] for n in names}

    def step(record: bool):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            marks[0].record(stream)
        T.encode(ck, K, pk)
        if record:
            marks[1].record(stream)
        T.encode(cv, V, pv)
        if record:
            marks[2].record(stream)
        T.decode_attention(ck, cv, q, pk, pv, Hkv, N, out=out, workspace=ws)
        if record:
            marks[3].record(stream)
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
    kms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / len(ev[n]) for n in names}

    # algorithmic bytes per launch (what each kernel must move at minimum)
    nvec = streams * N
    k_rec = d * 4 // 8 + 128 // 8 + 2 + 2          # 84 B packed K per vector
    v_rec = d * 4 // 8 + 2                         # 66 B packed V per vector
    alg = {
        "encode_k": nvec * (2 * d + k_rec),
        "encode_v": nvec * (2 * d + v_rec),
        "decode_attention": nvec * (k_rec + v_rec) + 2 * B * Hq * d * 2,
    }
    bf16eq_step = 2 * nvec * d * 2 * 2             # K and V, encode pass + attention pass
    value = bf16eq_step / (ms_step * 1e-3) / 1e9
    kern = {}
    for n in names:
        gbs = alg[n] / (kms[n] * 1e-3) / 1e9
        bf = (2 * nvec * d * 2 if n == "decode_attention" else nvec * d * 2) / (kms[n] * 1e-3) / 1e9
        kern[n] = {"ms": round(kms[n], 4), "alg_bytes": alg[n], "achieved_GBs": round(gbs, 1),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bf16_equiv_GBs": round(bf, 1)}
    kern["encode_k"]["sketch_tflops"] = round(nvec * 2 * ck.m * d / (kms["encode_k"] * 1e-3) / 1e12, 2)

    # standalone decode of the V cache to bf16 (row a8), timed apart from the step
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
    sample_k, sample_v = K[:1, :2048].clone(), V[:1, :2048].clone()   # the CPU baseline's sample
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
    flops = nvec * 2 * ck.m * d if (dom == "encode_k" and ck.m > 0) else 0
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
        cpu = cpu_baseline(sample_k, sample_v, q, pk, pv, ck, cv, B, Hq, Hkv, N, d, args.cpu_seconds)

    line = {
        "metric": "encode & decode-attention bf16-equiv GB/s on 1 MI355X; % of HBM peak",
        "value": round(value, 1), "unit": "GB/s (bf16-equivalent)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate, fp16 MFMA operands",
        "data": "synthetic (seeded N(0,1) bf16, RoPE-rotated by position)",
        "config": {"workload": "GQA decode attention over a TQ-compressed cache: batch 16, 32 q / 8 kv heads, "
                               f"context {N}, d=128; K b=4 + QJL m=128, V b=4; step = encode K + encode V + "
                               "decode-attention", "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "context": N, "d": d, "b_k": 4, "m_k": 128, "b_v": 4},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        "copy_ceiling": copy,
        "other_workloads": extra,
    }
    print(json.dumps(line))


def _time(torch, stream, fn, reps: int = 5) -> float:
    """average ms of fn() over reps launches on `stream` (after one untimed call)"""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _line(ms: float, alg_bytes: int) -> dict:
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "alg_bytes": alg_bytes, "achieved_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def other_workloads(torch, T, I, dev, stream) -> dict:
    """Per-kernel lines (not part of `value`) for the other workload shapes: encode / decode of
    outlier-channel K,V (32 heads x 32768 x 128, b = 4), encode with a QJL sketch and q.k scores
    (8 heads x 65536 x 128, b = 3, m = 128, 32 queries per head), and heavy-tailed d = 256 vectors
    (16 heads x 262144, Student-t nu = 3, b = 3, with and without a sketch of m = 256); the sketch
    encodes also with the randomized Hadamard sketch (m = d)."""
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
    del x, pk, xh

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


def cpu_baseline(K, V, q, pk, pv, ck, cv, B, Hq, Hkv, N, d, budget_s):
    """The oracle (unchanged) timed on the host on a bounded sample of the same workload: encode
    of the first n_tok tokens of K and V of stream 0, then decode-attention of the 4 query heads of
    that stream over those tokens (the oracle's scores and rotated-domain attention of its own
    encoding).
    Rate scaled to bf16-equivalent GB/s like the GPU value."""
    import numpy as np
    import torch

    from oracle import tq_oracle as O
    from synth import inputs as I

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    n_tok = 2048
    kx = O.bf16_bits_to_f64(I.bf16_bits(K[0, :n_tok]))
    vx = O.bf16_bits_to_f64(I.bf16_bits(V[0, :n_tok]))
    q64 = O.bf16_bits_to_f64(I.bf16_bits(q[0, :Hq // Hkv]))
    t_k, c_k = O.lloyd_max(d, ck.b)
    t_v, c_v = O.lloyd_max(d, cv.b)
    s_k, s_v = O.head_signs(ck.seed, 0, d), O.head_signs(cv.seed, 0, d)
    S_k = O.gaussian_matrix(ck.seed, 0, ck.m, d)
    reps = 0
    t0 = time.perf_counter()
    while True:
        rk = O.encode(kx, s_k, t_k, c_k, S_k)
        rv = O.encode(vx, s_v, t_v, c_v)
        sc = O.scores(q64, rk, s_k, c_k, S_k)
        O.attention_rotated(sc, rv, s_v, c_v, 1.0 / math.sqrt(d))
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    bytes_bf16 = reps * (2 * n_tok * d * 2) * 2          # encode pass + attention pass, K and V
    return {"value": round(bytes_bf16 / el / 1e9, 4), "unit": "GB/s (bf16-equivalent)", "cores": threads,
            "kind": "oracle", "seconds": round(el, 2),
            "sample": f"stream 0: encode {n_tok} K (QJL) + {n_tok} V tokens, then attention of its "
                      f"{Hq // Hkv} query heads over them; {reps} repetitions"}


if __name__ == "__main__":
    main()

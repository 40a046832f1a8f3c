#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline]

A step is one fused forward (``attn_fwd``) over the whole batch of the
workload, inputs resident in HBM. The default workload is the causal prefill
(B=4, H=32, N=4096, d=128, bf16). Throughput counts mask-adjusted FLOPs: 4 d
per allowed (query, key) pair (QK^T and PV), nothing for the softmax.

Prints ONE JSON line with the metric, the per-launch roofline of the kernel
(HIP events on the launch stream over the timed region, against the MI355X
dense matrix peak of the arithmetic type) and the CPU float64 oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import torch

from tiled_attention_05_amd import _lib, flops
from tiled_attention_05_amd import inputs as I

METRIC = "attention fwd TFLOPS (mask-adjusted FLOPs) and % of MI355X MFMA peak"
# MI355X dense matrix peaks (256 CUs x 2.4 GHz): bf16 4096 FLOP/clk/CU, fp8 twice that, fp32 1/16 of bf16
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}
PEAK_MHZ = 2400.0   # the clock the published peaks assume
HOST_CORES = 16   # the host-CPU share of one GPU on the benchmark machines
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "tiled_attention_05_amd", "csrc")
# kernel sources whose hash keys the measured HBM traffic of a profile summary
KERNEL_SOURCES = {"bf16": ["attn_fwd_bf16.hip", "fwd_common.h", "common.h", "fwd_params.h"],
                  "varlen": ["attn_fwd_bf16.hip", "varlen.hip", "fwd_common.h", "common.h", "fwd_params.h"],
                  "decode": ["decode.hip", "fwd_common.h", "common.h"],
                  "bwd": ["bwd.hip", "fwd_common.h", "common.h"],
                  "fp8": ["fp8.hip", "fwd_common.h", "common.h", "fwd_params.h"],
                  "f32": ["attn_fwd_f32.hip", "fwd_common.h", "common.h", "fwd_params.h"]}
PROFILE_SUMMARY = {2: "profiles/fwd_bf16_causal_prefill_b4_h32_n4096_d128.md",
                   3: "profiles/fwd_bf16_gqa_window_b2_h32x8_n16384_w4096_d128.md",
                   4: "profiles/fwd_bf16_docs_softcap_alibi_b1_h16_n32768_d128.md",
                   5: "profiles/fwd_fp8_dense_b4_h16_n8192_d128.md",
                   6: "profiles/fwd_bf16_varlen_causal_t32768_h32x8_d128.md",
                   7: "profiles/decode_paged_b64_h32x8_d128_len1k-8k.md",
                   8: "profiles/bwd_bf16_causal_b4_h32_n4096_d128.md"}


def sources_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_profile(workload, kind):
    """HBM bytes per launch and the graphics clock (MHz) from the committed
    counter summary of this workload, if it was taken on the current kernel
    sources (else None for each)."""
    path = os.path.join(ROOT, PROFILE_SUMMARY.get(workload, "-"))
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    hm = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    if not hm or hm.group(1) != sources_hash(kind):
        return None, None
    tm = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    cm = re.search(r"sclk_mhz:\s*([0-9.]+)", text)
    return (int(tm.group(1)) if tm else None), (float(cm.group(1)) if cm else None)


def calibrate_copy(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}))


def mask_name(m):
    parts = [n for b, n in ((1, "causal"), (2, "window"), (4, "doc")) if m & b]
    return "+".join(parts) or "none"


def run_cpu_baseline(w, x, budget_s=15.0):
    """Oracle on whole heads of the same inputs until ~budget_s of wall time.
    Returns (summary, {(b, h): (O, LSE)} of the heads it computed)."""
    from oracle import attention as A
    threads = max(1, min(HOST_CORES, len(os.sched_getaffinity(0))))
    heads_all = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    order = heads_all[::max(1, len(heads_all) // 64)] + heads_all
    done, fl, t0 = [], 0, time.perf_counter()
    docs = x["doc_ids"]
    per_head = flops.attention_flops(1, 1, w.N, w.N, w.d, w.mask, w.window,
                                     None if docs is None else docs[:1])
    i = 0
    results = {}
    while time.perf_counter() - t0 < budget_s and i < len(order):
        batch = [hb for hb in order[i:i + threads] if hb not in done]
        i += threads
        if not batch:
            continue
        O, L = A.attention(x["q"], x["k"], x["v"], w.scale, w.mask, w.window, docs, w.softcap, x["slopes"],
                           heads=batch, threads=threads)
        for j, hb in enumerate(batch):
            results[hb] = (O[j], L[j])
        for b, h in batch:
            row = None if docs is None else docs[b:b + 1]
            fl += flops.attention_flops(1, 1, w.N, w.N, w.d, w.mask, w.window, row)
        done += batch
    dt = time.perf_counter() - t0
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} of {len(heads_all)} (batch, head) pairs, all {w.N} query rows each, "
                      f"float64 numpy, {dt:.1f} s wall",
            "seconds": round(dt, 2), "flops_per_head": per_head,
            "host": {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                     "pool_threads": threads, "blas_threads_per_job": 1}}, results


def parity_of_timed_output(w, o, lse, results):
    """The timed launches' output (the last one's O and LSE) against the oracle
    heads the CPU baseline computed: max-abs / mean-abs over O and max LSE
    error (bf16 / fp32 bars), or relative RMS (fp8 bar)."""
    import numpy as np
    heads = sorted(results)
    if not heads:
        return None
    og = torch.stack([o[b, h] for b, h in heads]).float().cpu().double().numpy()
    lg = torch.stack([lse[b, h] for b, h in heads]).cpu().double().numpy()
    O = np.stack([results[hb][0] for hb in heads])
    L = np.stack([results[hb][1] for hb in heads])
    fin = np.isfinite(L)
    out = {"heads": len(heads), "of": w.B * w.Hq, "rows": "all",
           "lse_max": float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0}
    if w.dtype == "fp8":
        per = np.sqrt(((og - O) ** 2).sum(axis=(1, 2)) / (O ** 2).sum(axis=(1, 2)))
        out.update({"relrms": float(np.linalg.norm(og - O) / np.linalg.norm(O)),
                    "relrms_head_max": float(per.max()), "bar": {"relrms": 5e-2}})
        out["ok"] = out["relrms"] <= 5e-2 and out["relrms_head_max"] <= 5e-2
    else:
        err = np.abs(og - O)
        out.update({"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                    "bar": {"max_abs": 2e-2, "mean_abs": 2e-3, "lse": 1e-3}})
        out["ok"] = out["max_abs"] <= 2e-2 and out["mean_abs"] <= 2e-3 and out["lse_max"] <= 1e-3
    return out


def bench_decode(w, args):
    """Paged decode (attn_decode_paged): HBM-bound, measured in GB/s of algorithmic bytes --
    every cached key and value row of every sequence read once, Q read and O written once."""
    lens = I.decode_lengths(w)
    q, kc, vc, bt, sl = (t.to("cuda") for t in I.decode_inputs(w.B, w.Hq, w.Hkv, w.d, lens, w.extra["block"],
                                                                 seed=w.k))
    splits = w.extra.get("splits", 4)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, device="cuda", dtype=torch.float32)
    ws = torch.empty(_lib.attn_decode_workspace_floats(w.B, w.Hq, w.d, splits), device="cuda",
                     dtype=torch.float32)

    def step():
        _lib.decode_paged(q, kc, vc, bt, sl, scale=w.scale, num_splits=splits, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_kernel = evs[0].elapsed_time(evs[-1]) / args.steps
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    n_keys = sum(lens)
    nbytes = n_keys * w.Hkv * 2 * w.d * 2 + 2 * q.numel() * 2 + lse.numel() * 4 + sl.numel() * 4 + \
        sum(-(-n // w.extra["block"]) for n in lens) * 4
    fl = 4 * w.d * n_keys * w.Hq
    gbps = nbytes / (ms_kernel * 1e-3) / 1e9
    traffic, sclk = measured_profile(args.workload, "decode")
    out = {
        "metric": "paged decode HBM bandwidth (algorithmic bytes)", "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "block": w.extra["block"],
                   "cached_tokens": n_keys, "len_min": min(lens), "len_max": max(lens), "splits": splits,
                   "bytes_per_step": nbytes, "flops_per_step": fl, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbps / 8000.0, 4), "traffic": traffic, "kernel_ms": round(ms_kernel, 4),
                     "kernel_ms_median": round(per_launch[len(per_launch) // 2], 4),
                     "kernel_ms_min": round(per_launch[0], 4), "tflops": round(fl / (ms_kernel * 1e-3) / 1e12, 2)},
    }
    print(json.dumps(out), flush=True)


def bench_backward(w, args):
    """attn_bwd after one forward of the same inputs; FLOPs: 2.5x the forward's mask-adjusted
    count (the five products of the gradient: S, dP, dV, dK, dQ; the kernels recompute S and dP
    once more for dQ, which is not counted)."""
    x = I.inputs(w)
    g = torch.Generator("cpu").manual_seed(2000 + w.k)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).to("cuda")
    o, lse = _lib.fwd(q, k, v, scale=w.scale, mask=w.mask)
    ws = torch.empty(w.B * w.Hq * w.N, device="cuda", dtype=torch.float32)
    fl = 2.5 * flops.attention_flops(w.B, w.Hq, w.N, w.N, w.d, w.mask, w.window, None)

    def step():
        _lib.bwd(q, k, v, o, do, lse, scale=w.scale, mask=w.mask, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_kernel = evs[0].elapsed_time(evs[-1]) / args.steps
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    achieved = fl / (ms_kernel * 1e-3) / 1e12
    traffic, _ = measured_profile(args.workload, "bwd")
    out = {
        "metric": "attention bwd TFLOPS (2.5x the mask-adjusted forward FLOPs)",
        "value": round(fl / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "mask": mask_name(w.mask), "flops_per_step": fl, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                     "kernel_ms": round(ms_kernel, 4), "kernel_ms_median": round(per_launch[len(per_launch) // 2], 4),
                     "kernel_ms_min": round(per_launch[0], 4)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--calibrate-copy", action="store_true", help="only run a 1 GiB device copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by independent (batch, head) groups with no exchange)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    _lib.load()

    w = I.WORKLOADS[args.workload]
    if w.extra.get("decode"):
        bench_decode(w, args)
        return
    if w.extra.get("backward"):
        bench_backward(w, args)
        return
    x = I.inputs(w)
    dev = {k: (None if v is None else v.to("cuda").contiguous()) for k, v in x.items()}
    q, k, v = dev["q"], dev["k"], dev["v"]
    lse = torch.empty(w.B, w.Hq, w.N, device="cuda", dtype=torch.float32)
    fl = flops.attention_flops(w.B, w.Hq, w.N, w.N, w.d, w.mask, w.window, x["doc_ids"])
    extra = {}
    if w.dtype == "fp8":
        q8, k8, v8 = _lib.fp8_prepare(q, k, v, dev["signs"])
        o = torch.empty(w.B, w.Hq, w.N, w.d, dtype=torch.bfloat16, device="cuda")

        def step():
            _lib.fwd_fp8(q8, k8, v8, w.B, w.Hq, w.Hkv, w.N, w.d, scale=w.scale, out=o, lse=lse)

        def prep():
            _lib.fp8_prepare(q, k, v, dev["signs"])
    elif w.extra.get("varlen"):
        # packed sequences through attn_fwd_varlen: [H][total][d] views of the B = 1 tensors
        cu = I.cu_seqlens(x["doc_ids"][0]).to("cuda")
        ws = torch.empty(w.N, dtype=torch.int32, device="cuda")
        o = torch.empty_like(q)
        extra = {"sequences": int(cu.numel() - 1)}

        def step():
            _lib.fwd_varlen(q[0], k[0], v[0], cu, scale=w.scale, mask=w.mask & ~I.MASK_DOC, window=w.window,
                            softcap=w.softcap, alibi_slopes=dev["slopes"], out=o[0], lse=lse[0], workspace=ws)
    else:
        o = torch.empty_like(q)

        def step():
            _lib.fwd(q, k, v, scale=w.scale, mask=w.mask, window=w.window, doc_ids=dev["doc_ids"],
                     softcap=w.softcap, alibi_slopes=dev["slopes"], out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # events on the launch stream around every launch of the timed region
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_kernel = evs[0].elapsed_time(evs[-1]) / args.steps
    per_launch = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    value = fl / (ms_step * 1e-3) / 1e12
    achieved = fl / (ms_kernel * 1e-3) / 1e12
    dt = {"f32": "f32", "bf16": "bf16", "fp8": "fp8"}[w.dtype]
    peak = PEAK_TFLOPS[dt]
    if w.dtype == "fp8":
        # the prepare step (Hadamard + quantisation) is HBM-bound: timed on its own
        for _ in range(2):
            prep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            prep()
        e1.record()
        torch.cuda.synchronize()
        ms_prep = e0.elapsed_time(e1) / 10
        # read Q, K, V (bf16); write value + residual codes of Q and K, V's codes, the scales
        v_plane = w.B * w.Hkv * (-(-w.N // 128) * 128) * w.d   # V's unused residual plane
        prep_bytes = 2 * (q.numel() + k.numel() + v.numel()) + q8.numel() + k8.numel() + v8.numel() - v_plane
        # the same step with the rotary embedding of Q and K fused in front
        rc, rs = (t.to("cuda") for t in I.rope_tables(w.N, w.d))
        for _ in range(2):
            _lib.fp8_prepare(q, k, v, dev["signs"], rope_cos=rc, rope_sin=rs)
        e0.record()
        for _ in range(10):
            _lib.fp8_prepare(q, k, v, dev["signs"], rope_cos=rc, rope_sin=rs)
        e1.record()
        torch.cuda.synchronize()
        ms_rope = e0.elapsed_time(e1) / 10
        rope_bytes = prep_bytes + 2 * rc.numel() * 4
        extra = {"prepare_ms": round(ms_prep, 4), "prepare_GBps": round(prep_bytes / ms_prep / 1e6, 1),
                 "prepare_rope_ms": round(ms_rope, 4), "prepare_rope_GBps": round(rope_bytes / ms_rope / 1e6, 1),
                 "end_to_end_tflops": round(fl / ((ms_prep + ms_kernel) * 1e-3) / 1e12, 2)}
    traffic, sclk = measured_profile(args.workload, "varlen" if w.extra.get("varlen") else dt)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "mask": mask_name(w.mask), "window": w.window, "softcap": w.softcap,
                   "alibi": w.alibi, "flops_per_step": fl, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_ms": round(ms_kernel, 4),
                     "kernel_ms_median": round(per_launch[len(per_launch) // 2], 4),
                     "kernel_ms_min": round(per_launch[0], 4),
                     # the same peak scaled to the graphics clock the counter run of this
                     # kernel measured (busy cycles / kernel time), when it is on record
                     "sclk_mhz": sclk,
                     "peak_at_sclk": None if sclk is None else round(peak * sclk / PEAK_MHZ, 1),
                     "frac_at_sclk": None if sclk is None else round(achieved / (peak * sclk / PEAK_MHZ), 4)},
    }
    if extra and w.dtype == "fp8":
        out["fp8_prepare"] = extra
    elif extra:
        out["config"].update(extra)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], results = run_cpu_baseline(w, x, args.cpu_seconds)
        if w.extra.get("varlen"):
            results = {}   # the packed layout is checked by the varlen tests, not here
        out["parity"] = parity_of_timed_output(w, o, lse, results)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

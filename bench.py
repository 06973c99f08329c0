#!/usr/bin/env python3
"""Benchmark of GQA over a KV cache on one MI355X.

Timed step: one gqa_decode call on the 70B-class layer (B=32, Hq=64, Hkv=8,
d=128, every sequence at L=4096, bf16 cache, fp32 arithmetic), with q, the
caches and the output resident in device memory.  The cache is rotated over
several independent copies so consecutive steps never find it in the 256 MiB
Infinity Cache or the L2.  Prints one JSON line.

Also measured and reported in the same line: the causal prefill (B=2,
P=4096, Hq=32, Hkv=8, d=128) against the bf16 matrix-core peak, the
head-sharing sweep (B=16, Hq=64, d=128, L=2048, Hkv in 64/16/8/4/1), and the
CPU oracle on the decode workload as a baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "GQA decode: achieved HBM TB/s + µs/step, Hq=64 Hkv=8 d=128 B=32 L=4096"


DECODE_SOURCES = ("gqa_kv_cache_amd/csrc/common.hpp", "gqa_kv_cache_amd/csrc/decode.hpp",
                  "gqa_kv_cache_amd/csrc/gqa_api.hip")
PREFILL_SOURCES = ("gqa_kv_cache_amd/csrc/common.hpp", "gqa_kv_cache_amd/csrc/prefill.hpp",
                   "gqa_kv_cache_amd/csrc/gqa_api.hip")
EXT_SOURCES = ("gqa_kv_cache_amd/csrc/common.hpp", "gqa_kv_cache_amd/csrc/decode.hpp",
               "gqa_kv_cache_amd/csrc/decode_ex.hpp", "gqa_kv_cache_amd/csrc/gqa_api.hip")
DECODE_PMC = "profiles/decode_bf16_B32_Hq64_Hkv8_d128_L4096.pmc.txt"
EXT_FP8_PMC = {"e4m3": "profiles/decode_ex_e4m3_B32_Hq64_Hkv8_d128_L4096.pmc.txt",
               "e5m2": "profiles/decode_ex_e5m2_B32_Hq64_Hkv8_d128_L4096.pmc.txt"}
PREFILL_PMC = "profiles/prefill_bf16_B2_P4096_Hq32_Hkv8_d128_causal.pmc.txt"


def source_digest(paths) -> str:
    """sha256 over the kernel sources a profile was taken on."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pmc_traffic(summary_rel, sources):
    """HBM bytes per launch from a committed FETCH_SIZE/WRITE_SIZE summary.

    The summary records the digest of the kernel sources it was measured on;
    if those sources have changed since, the figure no longer applies and
    None is returned.
    """
    path = os.path.join(ROOT, summary_rel)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(sources):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, torch):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def time_calls(fn, n_steps, n_warmup, torch, rotate=1):
    """Run fn(i) warm-up + timed; returns (wall ms/step, event ms/step, per-call event ms list)."""
    for i in range(n_warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(n_steps):
        fn(i % rotate)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / n_steps
    ev_ms = start.elapsed_time(end) / n_steps
    # per-call durations, bracketed one by one on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i % rotate)
        b.record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) for a, b in evs]
    return wall_ms, ev_ms, per_call


def median(xs):
    s = sorted(xs)
    return s[len(s) // 2]


def pct(xs, p):
    s = sorted(xs)
    return s[min(len(s) - 1, int(p / 100.0 * len(s)))]


def bench_decode_case(case, steps, warmup, copies, torch, gqa):
    q = to_dev(case.q, torch)
    ks = [to_dev(case.k, torch)]
    vs = [to_dev(case.v, torch)]
    for _ in range(copies - 1):
        ks.append(ks[0].clone())
        vs.append(vs[0].clone())
    sl = torch.from_numpy(case.seqlens).cuda()
    out = torch.empty_like(q)
    B, Hq, d = case.q.shape
    _, Lmax, Hkv, _ = case.k.shape
    dt = gqa.BF16 if case.dtype == "bf16" else gqa.F32
    need = gqa.decode_workspace_size(B, Hq, Hkv, d, Lmax, dt, 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    splits = gqa.decode_num_splits(B, Hq, Hkv, d, Lmax, dt, 0)

    def fn(i):
        gqa.decode(q, ks[i], vs[i], sl, case.scale, out=out, workspace=ws)

    wall_ms, ev_ms, per_call = time_calls(fn, steps, warmup, torch, rotate=copies)
    nbytes = gqa.decode_bytes(case.seqlens, Hq, Hkv, d, dt)
    flops = gqa.decode_flops(case.seqlens, Hq, d)
    res = dict(bytes=nbytes, flops=flops, splits=splits, wall_ms=wall_ms, event_ms=ev_ms,
               call_ms_median=median(per_call), call_ms_mean=sum(per_call) / len(per_call),
               call_ms_p10=pct(per_call, 10), call_ms_p90=pct(per_call, 90))
    del ks, vs
    return res, out


def bench_decode_ex(case, steps, warmup, torch, gqa, min_total_bytes=1.0e9):
    """Time gqa_decode_ex (no append) over rotated cache copies; returns a result dict."""
    def dev(a):
        if a.dtype.name == "uint8":
            return torch.from_numpy(a).cuda()
        return to_dev(a, torch)

    cache_bytes = case.k.nbytes + case.v.nbytes
    copies = max(2, min(8, math.ceil(min_total_bytes / cache_bytes)))
    q = to_dev(case.q, torch)
    ks = [dev(case.k)]
    vs = [dev(case.v)]
    for _ in range(copies - 1):
        ks.append(ks[0].clone())
        vs.append(vs[0].clone())
    sl = torch.from_numpy(case.seqlens).cuda()
    kw = {}
    if case.kv_format:
        kw["k_scale"] = torch.from_numpy(case.k_scale).cuda()
        kw["v_scale"] = torch.from_numpy(case.v_scale).cuda()
        kw["kv_format"] = case.kv_format
    if case.block_table is not None:
        kw["block_table"] = torch.from_numpy(case.block_table).cuda()
        kw["block_size"] = case.block_size
    out = torch.empty_like(q)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")

    def fn(i):
        gqa.decode_ex(q, ks[i], vs[i], sl, scale=case.scale, window=case.window, out=out,
                      workspace=ws, **kw)

    wall_ms, ev_ms, per_call = time_calls(fn, steps, warmup, torch, rotate=copies)
    B, T, Hq, d = case.q.shape
    Hkv = case.k.shape[2]
    elt = 1 if case.kv_format else 2
    # rows some token of the sequence can see, read once per KV head; q and out
    first = [max(0, int(n) - T - case.window + 1) if case.window > 0 else 0 for n in case.seqlens]
    rows = sum(int(n) - f for n, f in zip(case.seqlens, first))
    nbytes = rows * 2 * Hkv * d * elt + 2 * B * T * Hq * d * 2
    us = ev_ms * 1e3
    del ks, vs
    return {"workload": case.name, "T": T, "kv_dtype": case.kv_format or "bf16",
            "paged_block_size": case.block_size or None, "window": case.window or None,
            "bytes": nbytes, "us_per_step": us, "us_per_call_median": median(per_call) * 1e3,
            "achieved_TBps": nbytes / (us * 1e-6) / 1e12,
            "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "new_tokens_per_s": B * T / (us * 1e-6), "cache_copies_rotated": copies}


def cpu_baseline(case, gpu_out, torch, min_seconds=10.0, max_passes=200):
    """Time the fp64 oracle on the decode workload on the host cores."""
    import numpy as np
    from oracle import counts, reference as orc

    passes, total = 0, 0.0
    ref = None
    while passes < max_passes and (passes == 0 or total < min_seconds):
        t0 = time.perf_counter()
        ref = orc.decode(case.q, case.k, case.v, case.seqlens, case.scale)
        total += time.perf_counter() - t0
        passes += 1
    B, Hq, d = case.q.shape
    Hkv = case.k.shape[2]
    nbytes = counts.decode_bytes(case.seqlens, Hq, Hkv, d, 2) * passes
    got = (gpu_out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
           << np.uint32(16)).view(np.float32).astype(np.float64)
    err = np.abs(got - ref)
    ok = bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))
    return {
        "value": nbytes / total / 1e12, "unit": "TB/s", "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": "whole decode workload (all 32 sequences x 64 query heads x 4096 rows), "
                  "%d pass(es), fp64 C oracle with OpenMP, %.2f s" % (passes, total),
        "us_per_step": total / passes * 1e6,
        "cpu": platform.processor() or platform.machine(),
        "gpu_vs_oracle_max_abs_err": float(err.max()), "gpu_vs_oracle_within_tol": ok,
    }


def bench_prefill(steps, warmup, torch, gqa):
    import gqa_inputs as gi
    c = gi.prefill_causal()
    q, k, v = to_dev(c.q, torch), to_dev(c.k, torch), to_dev(c.v, torch)
    out = torch.empty_like(q)

    def fn(i):
        gqa.prefill(q, k, v, causal=True, scale=c.scale, out=out)

    wall_ms, ev_ms, per_call = time_calls(fn, steps, warmup, torch)
    B, P, Hq, d = c.q.shape
    Hkv = c.k.shape[2]
    flops = gqa.prefill_flops(B, P, Hq, d, True)
    mean_ms = sum(per_call) / len(per_call)
    tflops = flops / (ev_ms * 1e-3) / 1e12
    return {
        "workload": c.name, "flops": flops, "bytes": gqa.prefill_bytes(B, P, Hq, Hkv, d, gqa.BF16),
        "us_per_call_median": median(per_call) * 1e3, "us_per_call_mean": mean_ms * 1e3,
        "us_per_step_stream": ev_ms * 1e3,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                     "traffic": pmc_traffic(PREFILL_PMC, PREFILL_SOURCES),
                     "kernel": "prefill_bf16"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=3, help="rotating copies of the KV cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--ragged", action="store_true", help="also time the ragged batch (8 GiB cache)")
    ap.add_argument("--no-extended", action="store_true",
                    help="skip the extended decode (FP8, several tokens, paged, window)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_inputs as gi
    import gqa_kv_cache_amd as gqa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gqa.load()
    log("generating the decode workload")
    case = gi.decode_70b(invalid="zero")
    log("timing decode: %d warm-up + %d steps, %d cache copies" % (args.warmup, args.steps, args.copies))
    res, out = bench_decode_case(case, args.steps, args.warmup, args.copies, torch, gqa)
    torch.cuda.synchronize()
    ms = res["event_ms"]  # average duration per step over the timed region (stream events)
    value = res["bytes"] / (ms * 1e-3) / 1e12
    achieved = res["bytes"] / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "B": 32, "Hq": 64, "Hkv": 8, "d": 128, "L": 4096,
                   "cache_layout": "[B,L,Hkv,d]", "accumulate": "fp32", "splits": res["splits"],
                   "cache_copies_rotated": args.copies, "parallelism": "single GPU"},
        "decode": {"bytes_per_step": res["bytes"], "flops_per_step": res["flops"],
                   "us_per_call_median": res["call_ms_median"] * 1e3,
                   "us_per_call_p10": res["call_ms_p10"] * 1e3,
                   "us_per_call_p90": res["call_ms_p90"] * 1e3,
                   "us_per_step_wall": res["wall_ms"] * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": pmc_traffic(DECODE_PMC, DECODE_SOURCES),
                     "kernel": "decode_split_bf16" if res["splits"] == 1
                               else "decode_split_bf16 + decode_merge",
                     "launches_per_step": 1 if res["splits"] == 1 else 2},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the decode workload")
        line["cpu_baseline"] = cpu_baseline(case, out, torch)
    del out
    if not args.no_prefill:
        log("timing prefill")
        line["prefill"] = bench_prefill(max(10, args.steps // 4), max(3, args.warmup // 4), torch, gqa)
    if not args.no_sweep:
        sweep = []
        for hkv in gi.SWEEP_HKV:
            log("timing sweep Hkv=%d" % hkv)
            c = gi.sweep_decode(hkv)
            kv_bytes = c.k.nbytes * 2
            copies = max(2, min(8, math.ceil(1.0e9 / kv_bytes)))
            r, o = bench_decode_case(c, max(20, args.steps // 2), args.warmup, copies, torch, gqa)
            us = r["call_ms_mean"] * 1e3
            fl_alu_us = r["flops"] / 78.6e12 * 1e6
            sweep.append({"Hkv": hkv, "bytes": r["bytes"], "flops": r["flops"], "splits": r["splits"],
                          "us_per_call_mean": us, "us_per_call_median": r["call_ms_median"] * 1e3,
                          "achieved_TBps": r["bytes"] / (us * 1e-6) / 1e12,
                          "hbm_frac": r["bytes"] / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                          "time_at_hbm_peak_us": r["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6,
                          "fp32_vector_alu_time_us": fl_alu_us})
            del o
        line["sweep"] = sweep
    if not args.no_extended:
        ext = []
        L70 = dict(B=32, T=1, Hq=64, Hkv=8, d=128, Lmax=4096, seqlens=[4096] * 32, dtype="bf16",
                   invalid="zero")
        variants = [
            ("decode_ex_e4m3_B32_Hq64_Hkv8_d128_L4096", dict(kv="fp8")),
            ("decode_ex_e5m2_B32_Hq64_Hkv8_d128_L4096", dict(kv="e5m2")),
            ("decode_ex_bf16_T4_B32_Hq64_Hkv8_d128_L4096", dict(T=4)),
            ("decode_ex_bf16_paged64_B32_Hq64_Hkv8_d128_L4096", dict(paged=True, block_size=64)),
            ("decode_ex_bf16_paged16_B32_Hq64_Hkv8_d128_L4096", dict(paged=True, block_size=16)),
            ("decode_ex_bf16_window1024_B32_Hq64_Hkv8_d128_L4096", dict(window=1024)),
        ]
        for name, extra in variants:
            log("timing %s" % name)
            a = dict(L70)
            a.update(extra)
            c = gi.decode_ex_case(seed=60, name=name, **a)
            r = bench_decode_ex(c, max(20, args.steps // 2), args.warmup, torch, gqa)
            if c.kv_format:
                r["traffic"] = pmc_traffic(EXT_FP8_PMC[c.kv_format], EXT_SOURCES)
            ext.append(r)
            del c
        line["extended"] = ext
    if args.ragged:
        log("generating the ragged workload (8 GiB cache)")
        c = gi.ragged_decode(invalid="zero")
        r, o = bench_decode_case(c, max(10, args.steps // 4), max(3, args.warmup // 4), 1, torch, gqa)
        us = r["call_ms_mean"] * 1e3
        line["ragged"] = {"workload": c.name, "bytes": r["bytes"], "flops": r["flops"],
                          "splits": r["splits"], "us_per_call_mean": us,
                          "achieved_TBps": r["bytes"] / (us * 1e-6) / 1e12,
                          "hbm_frac": r["bytes"] / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                          "note": "one cache copy (8 GiB exceeds every cache level)"}
        del o
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of one MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: mla_append of one
new token per sequence, then mla_decode (absorb W_UK, attention over the
latent cache, merge + W_UV) for every sequence. The append and the absorb
stage go through mla_append_absorb (one launch: neither reads what the other
writes), then mla_decode_attend_combine. The default workload is the
DeepSeek-V2-Lite-shaped decode (B=64, H=16, L ~ U[1024, 4096], bf16 cache,
d_model 2048). Inputs are synthetic and seeded; several replicas of the
cache and weights are rotated so each step reads its cache from HBM, not
from the 256 MB Infinity Cache.

Prints one JSON line. `value` is the step's algorithmic bytes (cache rows,
weights, activations and outputs the method must move) per second, over a
timed region of whole steps with events only at its ends (the larger of the
wall clock and the GPU events); untimed warmup steps come first, enough for
the chip to reach its sustained clock. A second pass with an event between
every two steps gives the per-step p10/p50/p90. The attention
kernel's own duration (the roofline entry) is then measured as the same
number of attention launches back to back on the launch stream, rotating over
the replicas, between two HIP events. A second workload (the 128-head V2
shape by default) is measured the same way and reported under "secondary",
with its attention rate also against the bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-cache GB/s + TFLOP/s, % of MI355X roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA, MI355X
KERNEL_SOURCES = ["head_latent_attention_14_amd/csrc/decode_attn.hip",
                  "head_latent_attention_14_amd/csrc/decode_attn_stream.hip",
                  "head_latent_attention_14_amd/csrc/attn_tile.h",
                  "head_latent_attention_14_amd/csrc/common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter runs, if
    they were taken on the current kernel source for this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("kernel_source_sha") != kernel_source_hash():
        return None
    return r.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # timed steps: the wall clock around them carries a fixed cost (first
    # launch, final synchronisation; about 90 us), which 300 steps amortise
    ap.add_argument("--steps", type=int, default=300)
    # untimed warmup: the 128-head step needs a few hundred steps (tens of ms)
    # before the chip settles at its sustained clock (110.7 -> 94.7 us/step
    # measured between 10 and 500 warmup steps)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="v2lite_bf16")
    ap.add_argument("--secondary", default="v2_bf16",
                    help="a second workload measured the same way and reported under "
                         "'secondary' (empty: none)")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed 2x the MALL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the known-size "
                         "reference that scales hardware byte counters), then exit")
    return ap.parse_args()


def cpu_baseline(p, seconds: float):
    """Time the fp64 oracle on whole sequences of the same problem until about
    `seconds` of CPU work; report its rate in the metric's unit."""
    from oracle import mla as omla
    from oracle.problem import OracleView
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = None
    view = OracleView(p)
    B, H = p.q_nope.shape[:2]
    e_c = {"f32": 4, "bf16": 2, "fp8": 1}[p.wl.cache] + 0
    sf = 4 if p.wl.cache == "fp8" else 0
    e_a = {"f32": 4, "bf16": 2}[p.wl.act]
    t0 = time.perf_counter()
    done = 0           # sequences decoded (passes over the batch repeat it)
    tokens = 0
    while time.perf_counter() - t0 < seconds and done < 64 * B:
        b = done % B
        view.decode([(b, h) for h in range(H)])
        tokens += int(p.seq_len[b])
        done += 1
    el = time.perf_counter() - t0
    # the sample's share of the step's algorithmic bytes
    by = tokens * (576 * e_c + sf) + 2 * H * 128 * 512 * e_a * done / B + done * H * (192 + 128) * e_a
    cores = len(os.sched_getaffinity(0))
    return {"value": by / el / 1e9, "unit": "GB/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"fp64 unabsorbed oracle, {done} sequence decodes over the {B} sequences "
                      f"(all {H} heads, {tokens} cached tokens, {el:.1f} s, "
                      f"{cores} host cores visible)"}


def measure(mla, W, torch, name: str, steps: int, warmup: int, replicas: int = 0):
    """Time `steps` decode steps of workload `name` (append when the workload
    has it, then absorb -> attend -> combine). Returns the measurements."""
    wl = W.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    p = W.make_problem(wl)
    B, H = wl.B, wl.H
    ab = W.algorithmic_bytes(p)
    fl = W.algorithmic_flops(p)
    e_a = {"f32": 4, "bf16": 2}[wl.act]
    e_c = {"f32": 4, "bf16": 2, "fp8": 1}[wl.cache]
    append_bytes = 0
    if wl.append:
        # h, W_DKV, W_KR read; one row written per token
        append_bytes = B * wl.d_model * e_a + 576 * wl.d_model * e_a + B * 576 * e_c
    step_bytes = ab["total"] + append_bytes
    step_flops = fl["total"] + (2 * B * wl.d_model * 576 if wl.append else 0)

    # ---- replicas so that every step reads its inputs from HBM, not the 256 MB MALL ----
    per_rep = p.rows.numel() * p.rows.element_size() + ab["weights"]
    R = replicas or max(2, math.ceil(2 * 256e6 / per_rep) + 1)
    scale = 1.0 / math.sqrt(192.0)
    stream = torch.cuda.current_stream()
    reps = []
    for _ in range(R):
        rows = p.rows.to(dev)
        cache = mla.LatentCache(rows=rows, seq_start=torch.from_numpy(p.seq_start).to(dev),
                                seq_capacity=torch.from_numpy(p.seq_capacity).to(dev),
                                row_scale=p.row_scale.to(dev) if p.row_scale is not None else None)
        r = dict(cache=cache, seq_len=torch.from_numpy(p.seq_len).to(dev),
                 q_nope=p.q_nope.to(dev), q_pe=p.q_pe.to(dev), w_uk=p.w_uk.to(dev),
                 w_uv=p.w_uv.to(dev),
                 out=torch.empty(B, H, 128, dtype=p.q_nope.dtype, device=dev),
                 lse=torch.empty(B, H, dtype=torch.float32, device=dev))
        r["ws"] = mla.alloc_workspace(cache, H, p.q_nope.dtype)
        # arguments marshalled once per replica: a step is a few foreign calls
        r["dec"] = mla.PreparedDecode(r["cache"], r["seq_len"], r["q_nope"], r["q_pe"], r["w_uk"],
                                      r["w_uv"], scale, r["out"], r["lse"], r["ws"], stream)
        if wl.append:
            r.update(h=p.h.to(dev), w_dkv=p.w_dkv.to(dev), w_kr=p.w_kr.to(dev),
                     tok_seq=torch.from_numpy(p.tok_seq).to(dev),
                     tok_pos=torch.from_numpy(p.tok_pos).to(dev))
            # the append and the decode's absorb stage in one call (one launch
            # where it applies), then attend and combine in one more call
            r["app"] = mla.PreparedAppendAbsorb(r["cache"], r["h"], r["w_dkv"], r["w_kr"],
                                                r["tok_seq"], r["tok_pos"], wl.rope_base,
                                                r["seq_len"], r["q_nope"], r["q_pe"], r["w_uk"],
                                                r["w_uv"], scale, r["out"], r["lse"], r["ws"],
                                                stream)
        reps.append(r)

    def step(i):
        r = reps[i % R]
        if wl.append:
            r["app"]()
            r["dec"].attend_combine()
        else:
            r["dec"]()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: `steps` whole steps, events only at its two ends
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    gpu_ms = start.elapsed_time(end) / steps
    ms = max(wall_ms, gpu_ms)

    # the distribution over steps: another `steps` steps, an event between
    # every two (outside the timed region above)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        evs[i].record(stream)
        step(warmup + steps + i)
    evs[steps].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))

    def pct(q):
        return round(per[min(len(per) - 1, int(round(q * (len(per) - 1))))], 2)
    step_pct = {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)}

    # the attention kernel's own duration: `steps` launches back to back on the
    # launch stream, rotating over the replicas (each absorbed first, so every
    # launch reads its cache from HBM), between two events
    for r in reps:
        r["dec"].absorb()
    torch.cuda.synchronize()
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for i in range(steps):
        reps[i % R]["dec"].attend()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / steps
    del reps
    torch.cuda.empty_cache()
    return dict(wl=wl, p=p, T=p.T, B=B, H=H, R=R, ms=ms, wall_ms=wall_ms, gpu_ms=gpu_ms,
                step_pct=step_pct, step_bytes=step_bytes,
                step_flops=step_flops, attn_bytes=ab["cache"], attn_flops=fl["attention"],
                attn_ms=attn_ms)


def gpu_info(torch):
    """The device as the runtime reports it (name, compute units, clock)."""
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "compute_units": pr.multi_processor_count,
            "arch": getattr(pr, "gcnArchName", None)}
    clk = getattr(pr, "clock_rate", None)               # kHz where the build exposes it
    info["max_clock_mhz"] = round(clk / 1e3) if clk else None
    return info


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_reference:
        n = args.copy_reference << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes": n, "launches": 5}))
        return
    import head_latent_attention_14_amd as mla
    import workloads as W

    torch.cuda.set_device(0)
    m = measure(mla, W, torch, args.workload, args.steps, args.warmup, args.replicas)
    wl, ms = m["wl"], m["ms"]
    value = m["step_bytes"] / (ms * 1e-3) / 1e9
    attn_gbs = m["attn_bytes"] / (m["attn_ms"] * 1e-3) / 1e9
    traffic = recorded_traffic(args.workload)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-cache/bf16"}[wl.cache],
        "data": "synthetic (seeded normal draws; random-init weights of the DeepSeek-V2(-Lite) "
                "MLA shapes)",
        "config": {"workload": f"{wl.name}: MLA decode step, append {'1 token/seq + ' if wl.append else ''}"
                               f"decode, B={m['B']}, H={m['H']}, L~U[{wl.lo},{wl.hi}], {wl.cache} latent cache",
                   "B": m["B"], "H": m["H"], "T": m["T"], "d_c": 512, "d_r": 64,
                   "d_model": wl.d_model if wl.append else None, "replicas": m["R"]},
        "tflops": round(m["step_flops"] / (ms * 1e-3) / 1e12, 3),
        "step_us_percentiles": m["step_pct"],
        "step_us_host_gpu": [round(m["wall_ms"] * 1e3, 2), round(m["gpu_ms"] * 1e3, 2)],
        "gpu": gpu_info(torch),
        "attended_tokens_per_s": round(m["T"] / (ms * 1e-3), 1),
        "step_bytes": int(m["step_bytes"]),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "attention (mla_decode_attend)",
                     "kernel_avg_us": round(m["attn_ms"] * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(m["attn_bytes"])},
    }
    if args.secondary and args.secondary != args.workload:
        s = measure(mla, W, torch, args.secondary, args.steps, args.warmup)
        sw = s["wl"]
        s_attn = s["attn_bytes"] / (s["attn_ms"] * 1e-3) / 1e9
        out["secondary"] = {
            "workload": f"{sw.name}: MLA decode step, B={s['B']}, H={s['H']}, "
                        f"L~U[{sw.lo},{sw.hi}], {sw.cache} latent cache",
            "ms_per_step": round(s["ms"], 5),
            "step_us_percentiles": s["step_pct"],
            "step_us_host_gpu": [round(s["wall_ms"] * 1e3, 2), round(s["gpu_ms"] * 1e3, 2)],
            "value_GBps": round(s["step_bytes"] / (s["ms"] * 1e-3) / 1e9, 2),
            "tflops": round(s["step_flops"] / (s["ms"] * 1e-3) / 1e12, 3),
            "hbm_frac_step": round(s["step_bytes"] / (s["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "attention_kernel_us": round(s["attn_ms"] * 1e3, 3),
            "attention_GBps": round(s_attn, 2),
            "attention_hbm_frac": round(s_attn / HBM_PEAK_GBS, 4),
            "attention_tflops": round(s["attn_flops"] / (s["attn_ms"] * 1e-3) / 1e12, 2),
            "attention_mfma_frac": round(s["attn_flops"] / (s["attn_ms"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "attention_traffic": recorded_traffic(args.secondary),
        }
    if not args.no_cpu_baseline:
        p = W.make_problem(wl)
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

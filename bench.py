#!/usr/bin/env python3
"""Benchmark of MLA decode steps on one MI355X.

A step is one pass of the whole hot path over one batch: for every sequence,
absorb W_UK into the query, attend over the sequence's latent cache (split-K
partials), merge the partials and apply W_UV; workloads that append (the
DeepSeek-V2-Lite shape) first write one new latent row per sequence
(mla_append_absorb, then mla_decode_attend_combine). Inputs are synthetic
and seeded; several replicas of the cache and weights rotate so every step
reads its cache from HBM, not from the 256 MB Infinity Cache.

Prefill (causal multi-query attention, mla_prefill) is measured on its own
workloads after the decode ones and reported under "prefill": prompt tokens/s
and the matrix TFLOP/s of a whole call (up-projection of every cached row to
per-head K/V, plus attention over the (query, row) pairs a query may see)
against the bf16 MFMA peak, with a sampled parity check against the oracle.

The headline workload is the DeepSeek-V2-shaped decode (B=32, H=128,
L ~ U[2048, 8192], bf16 cache). The DeepSeek-V2-Lite step (B=64, H=16, with
append), the 128K-token decode (B=4, H=128) and the fp8- and fp6-cache
decodes (B=128, H=128) are measured the same way and reported under "workloads", each with
its own roofline block; they run first, so the headline is timed with the
chip at its sustained clock. For each workload: W untimed warmup steps, then
exactly K timed steps with events only at the ends of the timed region
(`ms_per_step` is the larger of the wall clock and the GPU events); a second
pass with an event between every two steps gives p10/p50/p90. The attention
kernel's own duration (the roofline entry) is K attention launches back to
back on the launch stream, rotating over the replicas, between two HIP events.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-cache GB/s + TFLOP/s, % of MI355X roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # dense, MI355X
HEADLINE = "v2_bf16"
OTHERS = ["v2lite_bf16", "long_bf16", "fp8_cache", "fp6_cache"]
PREFILLS = ["prefill_bf16", "prefill_chunk_fp8", "prefill_chunk_fp6"]
# every source that decides what the attention launch reads and writes: the
# kernels, the work split (api.cpp, gemm_tile.h) and the shared headers
KERNEL_SOURCES = sorted(glob.glob(os.path.join(ROOT, "head_latent_attention_14_amd", "csrc", "*")))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter runs, if
    they were taken on the current kernel sources for this workload."""
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, help="the headline workload")
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma-separated workloads measured first and reported under "
                         "'workloads' (empty: none)")
    ap.add_argument("--prefill", default=",".join(PREFILLS),
                    help="comma-separated prefill workloads reported under 'prefill' (empty: none)")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed 2x the MALL")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warm-up (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the known-size "
                         "reference that scales hardware byte counters), then exit")
    return ap.parse_args()


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')}", i.get("num_threads")
    except Exception:
        pass
    return None, None


def cpu_baseline(p, seconds: float):
    """Time the fp64 oracle on whole sequences of the same problem until about
    `seconds` of CPU work; report its rate in the metric's unit."""
    from oracle.problem import OracleView
    blas, blas_threads = blas_info()
    view = OracleView(p)
    B, H = p.q_nope.shape[:2]
    import workloads as W
    row = W.ROW_BYTES[p.wl.cache] + (4 if p.wl.cache == "fp8" else 0)   # row (+ fp8 scale)
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
    by = tokens * row + 2 * H * 128 * 512 * e_a * done / B + done * H * (192 + 128) * e_a
    # the unabsorbed oracle's own fp64 work: K and V expansions plus scores and values
    flops = tokens * H * (4 * 128 * 512 + 2 * (128 + 64) + 2 * 128)
    cores = len(os.sched_getaffinity(0))
    return {"value": by / el / 1e9, "unit": "GB/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"fp64 unabsorbed oracle, {done} sequence decodes over the {B} sequences "
                      f"(all {H} heads, {tokens} cached tokens, {el:.1f} s, "
                      f"{cores} host cores visible)",
            "blas": blas, "blas_threads": blas_threads,
            "attended_tokens_per_s": round(tokens / el, 1),
            "fp64_gflops": round(flops / el / 1e9, 2), "seconds": round(el, 2)}


def gpu_clock_mhz():
    """Current shader clock as the amdgpu kernel driver reports it (sysfs pp_dpm_sclk, else
    rocm-smi)."""
    for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            for line in open(f):
                if "*" in line:
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        for card in d.values():
            for k, v in card.items():
                if "sclk" in k.lower():
                    return float(str(v).strip("()Mhz").replace("Mhz", ""))
    except Exception:
        pass
    return None


def gpu_info(torch):
    """The device as the runtime reports it (name, compute units, clocks)."""
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "compute_units": pr.multi_processor_count,
            "arch": getattr(pr, "gcnArchName", None)}
    clk = getattr(pr, "clock_rate", None)               # kHz where the build exposes it
    info["max_clock_mhz"] = round(clk / 1e3) if clk else None
    return info


def parity_sample(p, o, lse, n_seq: int = 2):
    """rel-L2 and max-abs of the measured run's outputs against the oracle on
    every head of `n_seq` sequences (the first and the longest)."""
    from oracle.problem import OracleView
    B, H = p.q_nope.shape[:2]
    seqs = sorted({0, int(np.argmax(p.seq_len))})[:n_seq]
    pairs = [(b, h) for b in seqs for h in range(H)]
    ro, rl = OracleView(p).decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    gl = np.array([lse[b, h] for b, h in pairs])
    err = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
    bound = {"f32": 1e-5, "bf16": 2e-2, "fp8": 4e-2, "fp6": 4e-2}[p.wl.cache]
    return {"rel_l2": float(f"{err:.4g}"), "bound": bound, "ok": bool(err <= bound),
            "max_abs": float(f"{np.abs(got - ro).max():.4g}"),
            "lse_max_abs": float(f"{np.abs(gl - rl).max():.4g}"),
            "sample": f"all {H} heads of sequences {seqs}"}


def measure(mla, W, torch, name: str, steps: int, warmup: int, replicas: int = 0,
            parity: bool = False, settle_ms: float = 300.0):
    """Time `steps` decode steps of workload `name` (append when the workload
    has it, then absorb -> attend -> combine). Returns the measurements."""
    wl = W.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    p = W.make_problem(wl)
    B, H = wl.B, wl.H
    ab = W.algorithmic_bytes(p)
    fl = W.algorithmic_flops(p)
    e_a = {"f32": 4, "bf16": 2}[wl.act]
    append_bytes = 0
    if wl.append:
        # h, W_DKV, W_KR read; one row written per token
        append_bytes = B * wl.d_model * e_a + 576 * wl.d_model * e_a + B * W.ROW_BYTES[wl.cache]
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

    # the chip reaches its sustained clock only after tens of milliseconds of
    # load: steps run for `settle_ms` of wall time first (untimed, like the
    # warm-up), so a small --warmup does not time the clock ramp
    t_settle = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
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
    clock = gpu_clock_mhz()

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

    # append alone, plain RoPE and YaRN (the same kernel with another
    # frequency table; launch-bound at these sizes, so µs only)
    append_us = None
    if wl.append:
        r = reps[0]
        seq_t, pos_t = r["tok_seq"], r["tok_pos"]
        calls = {
            "rope": lambda: mla.mla_append(r["cache"], r["h"], r["w_dkv"], r["w_kr"], seq_t, pos_t,
                                           wl.rope_base, stream),
            "yarn": lambda: mla.mla_append_yarn(r["cache"], r["h"], r["w_dkv"], r["w_kr"], seq_t,
                                                pos_t, base=wl.rope_base, stream=stream),
        }
        append_us = {}
        for k, fn in calls.items():
            fn()
            torch.cuda.synchronize()
            b0 = torch.cuda.Event(enable_timing=True)
            b1 = torch.cuda.Event(enable_timing=True)
            b0.record(stream)
            for _ in range(20):
                fn()
            b1.record(stream)
            torch.cuda.synchronize()
            append_us[k] = round(b0.elapsed_time(b1) / 20 * 1e3, 2)

    par = None
    if parity:
        # the outputs of one full step of replica 0 against the oracle
        step(0)
        torch.cuda.synchronize()
        r = reps[0]
        par = parity_sample(p, r["out"].double().cpu().numpy(), r["lse"].double().cpu().numpy())
    del reps
    torch.cuda.empty_cache()
    return dict(wl=wl, p=p, T=p.T, B=B, H=H, R=R, ms=ms, wall_ms=wall_ms, gpu_ms=gpu_ms,
                step_pct=step_pct, step_bytes=step_bytes,
                step_flops=step_flops, attn_bytes=ab["cache"], attn_flops=fl["attention"],
                attn_ms=attn_ms, clock_mhz=clock, parity=par, append_us=append_us)


def measure_prefill(mla, W, torch, name: str, steps: int, warmup: int) -> dict:
    """One mla_prefill call per step over a seeded prefill problem (inputs in
    HBM); steps timed between two events, plus a sampled parity check."""
    wl = W.PREFILL_WORKLOADS[name]
    p = W.make_prefill_problem(wl)
    dev = torch.device("cuda")
    scale = p.row_scale.to(dev) if p.row_scale is not None else None
    cache = mla.LatentCache(rows=p.rows.to(dev), seq_start=torch.from_numpy(p.seq_start).to(dev),
                            seq_capacity=torch.from_numpy(p.seq_capacity).to(dev), row_scale=scale)
    seq_len = torch.from_numpy(p.seq_len).to(dev)
    q_start = torch.from_numpy(p.q_start).to(dev)
    q_nope, q_pe = p.q_nope.to(dev), p.q_pe.to(dev)
    w_uk, w_uv = p.w_uk.to(dev), p.w_uv.to(dev)
    n_q, H = p.q_nope.shape[:2]
    out = torch.empty(n_q, H, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(n_q, H, dtype=torch.float32, device=dev)
    ws = mla.alloc_prefill_workspace(cache, H, n_q, p.T)
    sm = 1.0 / math.sqrt(192.0)

    def call():
        mla.mla_prefill(cache, seq_len, q_start, p.T, q_nope, q_pe, w_uk, w_uv, sm, out, lse, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = max(e0.elapsed_time(e1) / steps, wall)
    fl = W.prefill_flops(p)
    # parity: every query of the last sequence, heads 0 and H-1
    from oracle.problem import PrefillOracleView
    b = len(p.seq_len) - 1
    q0, q1 = int(p.q_start[b]), int(p.q_start[b + 1])
    heads = [0, H - 1]
    ro, _ = PrefillOracleView(p).prefill(heads)
    got = out[q0:q1].double().cpu().numpy()[:, heads]
    ref = ro[q0:q1][:, heads]
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    tfl = fl["total"] / (ms * 1e-3) / 1e12
    return {
        "workload": (f"{name}: causal multi-query prefill, B={len(p.seq_len)}, H={H}, "
                     f"L~U[{wl.lo},{wl.hi}], "
                     + ("every position a query" if wl.chunk == 0 else f"last {wl.chunk} positions queries")
                     + f", {wl.cache} cache"),
        "ms_per_call": round(ms, 4),
        "prompt_tokens_per_s": round(n_q / (ms * 1e-3), 1),
        "n_q": n_q, "T": p.T,
        "tflops": round(tfl, 2),
        "mfma_dtype": "bf16",
        "mfma_frac": round(tfl / MFMA_PEAK_TFLOPS["bf16"], 4),
        "matrix_flops": {"kv_up_projection": fl["kv"], "attention": fl["attn"]},
        "parity": {"rel_l2": err, "bound": 2e-2 if wl.cache == "bf16" else 4e-2,
                   "sample": f"every query of sequence {b}, heads {heads}"},
    }


def describe(wl, m) -> str:
    return (f"{wl.name}: MLA decode step, {'append 1 token/seq + ' if wl.append else ''}"
            f"decode, B={m['B']}, H={m['H']}, L~U[{wl.lo},{wl.hi}], {wl.cache} latent cache")


def roofline(m, name: str) -> dict:
    """The attention kernel against the roofline that binds the workload: HBM
    when its matrix flop per algorithmic byte is below the MFMA ridge (peak
    flop/s over peak bytes/s), else the MFMA peak. The MFMA peak is that of
    the narrowest matrix arithmetic the cache format allows (bf16 for a bf16
    cache, fp8 for the fp8 and fp6 caches, fp32 for fp32), whatever
    instructions the kernel runs; both rates are reported either way, and the
    matrix rate also against the bf16 peak (the fp8 and fp6 caches are
    contracted on bf16 MFMA after widening)."""
    wl = m["wl"]
    gbs = m["attn_bytes"] / (m["attn_ms"] * 1e-3) / 1e9
    tf = m["attn_flops"] / (m["attn_ms"] * 1e-3) / 1e12
    mfma_dtype = {"f32": "f32", "bf16": "bf16"}.get(wl.cache, "fp8")
    mfma_peak = MFMA_PEAK_TFLOPS[mfma_dtype]
    t_hbm = m["attn_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = m["attn_flops"] / (mfma_peak * 1e12)
    if t_mfma > t_hbm:
        head = {"bound": "mfma", "achieved": round(tf, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tf / mfma_peak, 4)}
    else:
        head = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    used = "f32" if wl.cache == "f32" else "bf16"
    return {**head, "traffic": recorded_traffic(name),
            "kernel": "attention (mla_decode_attend)",
            "kernel_avg_us": round(m["attn_ms"] * 1e3, 3),
            "algorithmic_bytes_per_launch": int(m["attn_bytes"]),
            "algorithmic_flops_per_launch": int(m["attn_flops"]),
            "flop_per_byte": round(m["attn_flops"] / m["attn_bytes"], 1),
            "ridge_flop_per_byte": round(mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9), 1),
            "gbs": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tflops": round(tf, 2), "mfma_dtype": mfma_dtype,
            "mfma_frac": round(tf / mfma_peak, 4),
            "mfma_used": used, "mfma_used_frac": round(tf / MFMA_PEAK_TFLOPS[used], 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every run here uses a single GPU; the design notes say how the path would "
              "shard)", file=sys.stderr)
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
    others = [w for w in args.others.split(",") if w and w != args.workload]
    blocks = {}
    for name in others:
        s = measure(mla, W, torch, name, args.steps, args.warmup, settle_ms=args.settle_ms)
        blocks[name] = {
            "workload": describe(s["wl"], s),
            "ms_per_step": round(s["ms"], 5),
            "value": round(s["step_bytes"] / (s["ms"] * 1e-3) / 1e9, 2), "unit": "GB/s",
            "tflops": round(s["step_flops"] / (s["ms"] * 1e-3) / 1e12, 3),
            "step_us_percentiles": s["step_pct"],
            "step_us_host_gpu": [round(s["wall_ms"] * 1e3, 2), round(s["gpu_ms"] * 1e3, 2)],
            "T": s["T"], "step_bytes": int(s["step_bytes"]), "clock_mhz": s["clock_mhz"],
            "roofline": roofline(s, name),
        }
        if s["append_us"]:
            blocks[name]["append_us"] = s["append_us"]
        print(f"# measured {name}: {s['ms'] * 1e3:.2f} us/step, attention "
              f"{s['attn_ms'] * 1e3:.2f} us", file=sys.stderr, flush=True)

    prefill = {}
    for name in [w for w in args.prefill.split(",") if w]:
        prefill[name] = measure_prefill(mla, W, torch, name, args.steps, args.warmup)
        print(f"# measured {name}: {prefill[name]['ms_per_call'] * 1e3:.1f} us/call",
              file=sys.stderr, flush=True)

    m = measure(mla, W, torch, args.workload, args.steps, args.warmup, args.replicas,
                parity=not args.no_parity, settle_ms=args.settle_ms)
    wl, ms = m["wl"], m["ms"]
    value = m["step_bytes"] / (ms * 1e-3) / 1e9
    gi = gpu_info(torch)
    gi["clock_mhz_after_timed_steps"] = m["clock_mhz"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-cache/bf16", "fp6": "fp6-cache/bf16"}[wl.cache],
        "data": "synthetic (seeded normal draws; random-init weights of the DeepSeek-V2(-Lite) "
                "MLA shapes)",
        "config": {"workload": describe(wl, m),
                   "B": m["B"], "H": m["H"], "T": m["T"], "d_c": 512, "d_r": 64,
                   "d_model": wl.d_model if wl.append else None, "replicas": m["R"]},
        "tflops": round(m["step_flops"] / (ms * 1e-3) / 1e12, 3),
        "step_us_percentiles": m["step_pct"],
        "step_us_host_gpu": [round(m["wall_ms"] * 1e3, 2), round(m["gpu_ms"] * 1e3, 2)],
        "gpu": gi,
        "attended_tokens_per_s": round(m["T"] / (ms * 1e-3), 1),
        "step_bytes": int(m["step_bytes"]),
        "roofline": roofline(m, args.workload),
        "parity": m["parity"],
        "workloads": blocks,
        "prefill": prefill,
    }
    if not args.no_cpu_baseline:
        p = W.make_problem(wl)
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

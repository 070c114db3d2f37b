#!/usr/bin/env python3
"""Benchmark of the IsoQuant packed-KV decode step on one MI355X.

Headline workload (the metric's configuration, synthetic): decode attention
over packed 3-bit K/V at 32K context -- 64 sequences of 32,768 tokens, 32
query heads / 4 KV heads (GQA 8:1), head_dim 128, 3-bit IsoQuant-Full codes,
fp16 I/O.  One step = quantize and append one new K and one new V vector per
sequence and KV head (into the last row), then decode attention for every
query head over the packed caches.  100 steps are timed by default.

Prints one JSON line: value = packed-KV (+ q, o) bytes the steps' attention
reads and writes per second of step time (GB/s); the dominant kernel's
roofline (its algorithmic bytes per launch over its average launch time,
measured with HIP events on its stream, also as a fraction of the read rate
the GPU reaches for a plain stream, measured in the same run); the FP64
oracle timed on the host as a baseline; and, as labelled extras, the batched decode-with-append workload
(64 ragged sequences up to 32K, 16/8 heads, d=256, 3-bit Fast) with its own
roofline and oracle baseline, stage-1 quantize / dequantize rates over the
whole d x bits x variant x dtype sweep on 2^20 unit vectors (with the
oracle's stage-1 rate), single-call latencies (4,096-vector stage-1
round trip, one 8K and one 32K sequence), the RoPE sub-block case and the
deferred-prefill compression.

  --calibrate-copy  also runs one plain device-to-device copy of 256 MiB first
                    (the reference kernel for scaling the HBM byte counters).
  --no-stage1       skips the stage-1 sweep (shorter profiled runs).
  --summarize-counters FETCH_CSV WRITE_CSV
                    reads the counter_collection.csv of a rocprofv3 FETCH_SIZE
                    pass and of a WRITE_SIZE pass over a --calibrate-copy run,
                    scales both by what they read for the 256 MiB copy, and
                    writes the decode kernel's HBM bytes per launch to
                    profiles/decode_partial_hbm_traffic.json (tagged with a
                    hash of the kernel sources); no GPU needed.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPY_BYTES = 256 << 20

# The metric's configuration: packed 3-bit K/V at 32K context with the
# long-context head layout (32 query / 4 KV heads, d=128, Full), batched over
# 64 sequences so that one decode step streams 839 MB of packed K/V.
HEADLINE = dict(name="headline", batch=64, kv_len=32768, num_q_heads=32, num_kv_heads=4, head_dim=128, bits=3,
                variant="full", seed=40,
                label="decode with append at 32K context: 64 sequences x 32,768 tokens, 32 query / 4 KV heads, "
                      "head_dim 128, 3-bit IsoQuant-Full K and V, fp16 I/O; each step quantizes and appends one "
                      "K/V token per sequence (into the last row), then attends over all 32,768")
# The batched decode-with-append configuration: ragged contexts up to 32K.
BATCHED_APPEND = dict(name="batched_append_c5", batch=64, len_lo=1024, len_hi=32768, num_q_heads=16,
                      num_kv_heads=8, head_dim=256, bits=3, variant="fast", length_seed=45, seed=46,
                      label="batched decode with append: 64 sequences, context lengths uniform in [1024, 32768] "
                            "(+1 per step), 16 query heads / 8 KV heads, head_dim 256, 3-bit IsoQuant-Fast, fp16 "
                            "I/O; each step quantize+append one K/V token per sequence, then attend")
PARTIAL_KERNEL = "partial_kernel"

# Sources of the decode kernel; HBM counter readings recorded for it are
# reported only while these are unchanged.
KERNEL_SOURCES = ["compressed_space_attention_isoquant_amd/csrc/decode_kernels.h",
                  "compressed_space_attention_isoquant_amd/csrc/decode_256.hip",
                  "compressed_space_attention_isoquant_amd/csrc/decode_128.hip",
                  "compressed_space_attention_isoquant_amd/csrc/decode_args.h",
                  "compressed_space_attention_isoquant_amd/csrc/iq_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_hbm_traffic.json")


def row_bytes(d, bits):
    return d * bits // 8


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and blank space are left
    out, so that a comment edit keeps the recorded counter readings."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload_name)
    if not entry or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-stage1", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="the 32K headline and the batched-append workload only (the profiled command)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--stage1-only", action="store_true", help="the stage-1 sweep only (the profiled command)")
    ap.add_argument("--summarize-stage1", metavar="COUNTER_CSV",
                    help="VALU / HBM summary of the stage-1 kernels from a rocprofv3 --pmc run")
    ap.add_argument("--fresh-runs", type=int, default=2,
                    help="extra independent headline runs, each in a fresh process")
    ap.add_argument("--headline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.summarize_stage1:
        return summarize_stage1(args.summarize_stage1)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; runs on several GPUs are not "
                                   "part of it", "n_gpus": args.gpus}))
        return 2

    # independent runs of the headline in fresh processes, started before this
    # process touches the GPU
    fresh = []
    if not (args.headline_child or args.no_extras or args.decode_only or args.stage1_only):
        for _ in range(max(0, args.fresh_runs)):
            fresh.append(run_fresh_headline(args.steps, args.warmup))

    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        a = torch.empty((COPY_BYTES,), dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.stage1_only:
        print(json.dumps(run_stage1(torch, dev)))
        return 0
    head = run_decode_workload(torch, dev, HEADLINE, args.steps, args.warmup)
    if args.headline_child:
        print(json.dumps({"value": head["value"], "ms_per_step": head["ms_per_step"],
                          "partial_ms": head["partial_ms"]}))
        return 0
    extras = {}
    ceiling = run_stream_ceiling(torch, dev)
    if not args.no_extras:
        c5 = run_decode_workload(torch, dev, BATCHED_APPEND, max(10, args.steps // 2), args.warmup)
        extras["batched_append_c5"] = workload_record(BATCHED_APPEND, c5, "batched_append_c5")
        if not args.decode_only:
            extras["rope_32k"] = run_rope_32k(torch, dev)
            extras["c1_latency"] = run_c1_latency(torch, dev)
            extras["c3_latency"] = run_c3_latency(torch, dev)
            extras["c4_latency"] = run_c3_latency(torch, dev, T=32768, with_argmax=True)
            extras["prefill_compress"] = run_prefill_compress(torch, dev)
        if not args.no_stage1 and not args.decode_only:
            extras["stage1"] = run_stage1(torch, dev)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(HEADLINE, head["lengths"], args.cpu_seconds)
        if "batched_append_c5" in extras:
            extras["batched_append_c5"]["cpu_baseline"] = cpu_baseline(BATCHED_APPEND, c5["lengths"],
                                                                       args.cpu_seconds / 2)
        if "stage1" in extras:
            extras["stage1"]["cpu_baseline"] = cpu_baseline_stage1(args.cpu_seconds / 2)

    rec = workload_record(HEADLINE, head, "headline")
    rec["roofline"]["frac_of_measured_read_ceiling"] = round(rec["roofline"]["achieved"] / ceiling["gbs"], 4)
    if "batched_append_c5" in extras:
        r5 = extras["batched_append_c5"]["roofline"]
        r5["frac_of_measured_read_ceiling"] = round(r5["achieved"] / ceiling["gbs"], 4)
    result = {
        "metric": "packed-KV decode-attn GB/s (% HBM peak) at 32K ctx; quantize Mvec/s",
        "value": rec["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u3 codes, f16/f32 arithmetic",
        "data": "synthetic (seeded torch draws on the GPU: N(0,1) K/V with 4 x10 outlier channels per KV head, "
                "N(0,1) queries)",
        "config": rec["config"],
        "pct_hbm_peak": rec["pct_hbm_peak"],
        "steps_per_s": rec["steps_per_s"],
        "partial_kernel_ms": rec["partial_kernel_ms"],
        "partial_kernel_ms_spread": rec["partial_kernel_ms_spread"],
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        "stream_read_ceiling": ceiling,
    }
    if fresh:
        vals = [head["value"]] + [f["value"] for f in fresh]
        pms = [head["partial_ms"]] + [f["partial_ms"] for f in fresh]
        result["independent_runs"] = {
            "processes": len(vals), "values_gbs": [round(v, 2) for v in vals],
            "partial_kernel_ms": [round(v, 5) for v in pms],
            "mean_gbs": round(float(np.mean(vals)), 2), "std_gbs": round(float(np.std(vals)), 2),
            "cv": round(float(np.std(vals) / np.mean(vals)), 4)}
    result.update(extras)
    print(json.dumps(result))
    return 0


def run_stream_ceiling(torch, dev, nbytes=2 << 30, reps=10):
    """The read rate this GPU reaches for a plain stream: the library's
    probe (include/iq_probe.h) reads a 2 GiB buffer once per call with
    16-byte non-temporal loads over every compute unit; median of `reps` calls timed with
    HIP events on the stream it runs on."""
    from compressed_space_attention_isoquant_amd import binding as B

    buf = torch.zeros((nbytes,), dtype=torch.uint8, device=dev)
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        B.iq_probe_stream_read(buf, sink)
    times = []
    for _ in range(reps):
        e0, e1 = _events(torch)
        e0.record(stream)
        B.iq_probe_stream_read(buf, sink)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    ms = float(np.median(times))
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench] streaming-read ceiling {gbs:.1f} GB/s ({ms:.4f} ms per 2 GiB)", file=sys.stderr, flush=True)
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "ms": round(ms, 4), "kernel": "iq_probe_stream_read (16-byte non-temporal loads, grid-stride, 8 workgroups per CU)"}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def workload_record(w, r, traffic_name):
    """The JSON fields of one timed decode workload: its step rate, and the
    roofline of its dominant (split) kernel."""
    per = r["per_step_ms"]
    return {
        "value": round(r["value"], 2), "unit": "GB/s", "ms_per_step": round(r["ms_per_step"], 5),
        "steps": len(per),
        "config": {"workload": w["label"], "batch": w["batch"], "num_q_heads": w["num_q_heads"],
                   "num_kv_heads": w["num_kv_heads"], "head_dim": w["head_dim"], "bits": w["bits"],
                   "variant": w["variant"], "mean_kv_len": round(float(np.mean(r["lengths"])), 1),
                   "attention_bytes_per_step": int(r["attn_bytes_per_step"])},
        "pct_hbm_peak": round(100.0 * r["value"] / HBM_PEAK_GBS, 2),
        "steps_per_s": round(1e3 / r["ms_per_step"], 1),
        "partial_kernel_ms": round(r["partial_ms"], 5),
        # per-step spread of the split kernel; the first steps' times next to
        # the median show whether the slow steps are the early ones (clock and
        # cache warm-up) or spread over the run
        "partial_kernel_ms_spread": {"std": round(float(np.std(per)), 5), "min": round(float(np.min(per)), 5),
                                     "median": round(float(np.median(per)), 5),
                                     "max": round(float(np.max(per)), 5),
                                     "cv": round(float(np.std(per) / np.mean(per)), 4),
                                     "first_steps": [round(float(x), 5) for x in per[:5]],
                                     # the slowest steps with the host time their enqueue took
                                     "slowest_steps": [{"step": int(i), "ms": round(float(per[i]), 5),
                                                        "host_enqueue_ms": round(float(r["host_enqueue_ms"][i]), 4)}
                                                       for i in np.argsort(per)[::-1][:3]],
                                     "host_enqueue_ms_median": round(float(np.median(r["host_enqueue_ms"])), 4)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["achieved"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(traffic_name),
            "kernel": f"{PARTIAL_KERNEL}<{w['head_dim']},{w['bits']},{w['num_q_heads'] // w['num_kv_heads']}> "
                      "(split decode over packed K/V)",
            "algorithmic_bytes_per_launch": int(r["partial_bytes_per_launch"]),
        },
    }


def run_decode_workload(torch, dev, w, steps, warmup):
    """One decode workload, timed.  Set-up (not timed): every cache row of K
    and V holds a quantized synthetic token.  A step appends one new K and one
    new V token per sequence and KV head (one batched launch) and runs decode
    attention for every query head over the packed caches: the ragged
    workload's sequences grow by one token per step; the uniform workload
    appends into its last row, so each step attends over exactly kv_len
    tokens.  HIP events on the stream the split kernel is launched on bracket
    that (dominant) kernel in every timed step."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    batch, hq, hkv, d, bits = (w[k] for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim", "bits"))
    variant = {"full": B.IQ_FULL, "fast": B.IQ_FAST}[w["variant"]]
    n_total = warmup + steps
    if w.get("kv_len"):
        lens = np.full(batch, w["kv_len"], np.int64)
        grow = 0
        cap = int(w["kv_len"])
    else:
        lens = inputs.batch_lengths(w["length_seed"], batch, w["len_lo"], w["len_hi"]).astype(np.int64)
        grow = 1
        cap = (int(lens.max()) + n_total + 1) // 2 * 2       # decode needs an even capacity
    seed = w["seed"]
    quats = torch.from_numpy(inputs.quaternions(hkv, d)).to(dev)
    cfg = B.Config(d, bits, variant, hkv, quats, B.iq_codebook(bits, d))
    rng = np.random.default_rng(seed)
    ch_k = inputs.outlier_channels(rng, hkv, d)
    ch_v = inputs.outlier_channels(rng, hkv, d)

    kc = B.new_cache(batch, hkv, cap, d, bits, dev)
    vc = B.new_cache(batch, hkv, cap, d, bits, dev)
    sb, st = 8, 4096
    for cache, idx, ch in ((kc, 0, ch_k), (vc, 1, ch_v)):
        for b0 in range(0, batch, sb):
            nb = min(sb, batch - b0)
            sub = B.PackedCache(cache.codes[b0:b0 + nb], cache.norms[b0:b0 + nb])
            for t0 in range(0, cap, st):
                nt = min(st, cap - t0)
                x = inputs.device_kv(seed + 1 + idx, (b0 // sb) * 1000 + t0 // st, nb * nt, ch, d, dev)
                pos = torch.full((nb,), t0, dtype=torch.int32, device=dev)
                B.iq_quantize_append(cfg, x.view(nb, nt, hkv, d), pos, sub)
                del x
    torch.cuda.synchronize()
    P = 8   # distinct new-token / query draws cycled over the steps
    knew = [inputs.device_kv(seed + 3, s, batch, ch_k, d, dev).view(batch, 1, hkv, d) for s in range(P)]
    vnew = [inputs.device_kv(seed + 4, s, batch, ch_v, d, dev).view(batch, 1, hkv, d) for s in range(P)]
    qs = [inputs.device_normal(seed + 5, s, (batch, hq, d), dev, torch.float16) for s in range(P)]
    pos_dev = [torch.from_numpy((lens - 1 + grow * g).astype(np.int32)).to(dev) for g in range(n_total)]
    len_dev = [torch.from_numpy((lens + grow * g).astype(np.int32)).to(dev) for g in range(n_total)]
    max_len = [int(lens.max()) + grow * g for g in range(n_total)]
    out = torch.empty((batch, hq, d), dtype=torch.float16, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    ws = torch.empty((B.iq_decode_workspace_bytes(cfg, batch, hq, max(max_len)),), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()
    rb = row_bytes(d, bits)
    events = []

    # the step's K and V appends in one launch (same rotation, two caches)
    append_kv = [B.prepare_append_many([cfg, cfg], [knew[s], vnew[s]], [kc, vc]) for s in range(P)]

    # host time spent enqueuing each timed split phase: a step whose events
    # are far apart while its enqueue took long was held up by the host, not
    # by the GPU
    host_ms = []
    step_events = [_events(torch) for _ in range(steps)]

    def step(g, record):
        s = g % P
        append_kv[s](pos_dev[g])
        if record:
            e0, e1 = step_events[g - warmup]
            e0.record(stream)
            h0 = time.perf_counter()
        # the two phases of iq_decode_attention, so that the events bracket the
        # split (dominant) phase alone
        B.iq_decode_attention_partial(cfg, qs[s], kc, vc, len_dev[g], max_len[g], scale, ws, track_argmax=False)
        if record:
            host_ms.append((time.perf_counter() - h0) * 1e3)
            e1.record(stream)
            events.append((e0, e1))
        B.iq_decode_attention_merge(cfg, batch, hq, max_len[g], out, lse, None, ws)

    for g in range(warmup):
        step(g, False)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()                             # no collector pauses inside the timed steps
    try:
        t0 = time.perf_counter()
        for g in range(warmup, n_total):
            step(g, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    finally:
        gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / steps
    per_step = np.array([a.elapsed_time(b) for a, b in events])
    partial_ms = float(per_step.mean())
    kv = np.array([float((lens + grow * g).sum()) * hkv * 2 * (rb + 2) for g in range(warmup, n_total)])
    qo = batch * hq * d * 2
    attn_bytes = kv + 2 * qo                 # packed K/V with norms read, q read, o written
    partial_bytes = kv + qo                  # the split phase reads K/V and q; its partial states are O(pieces*d)
    value = attn_bytes.sum() / (t1 - t0) / 1e9
    achieved = partial_bytes.mean() / (partial_ms * 1e-3) / 1e9
    print(f"[bench] {w['name']}: step {ms_per_step:.4f} ms, split phase {partial_ms:.4f} ms, "
          f"{achieved:.1f} GB/s", file=sys.stderr, flush=True)
    del kc, vc, ws
    return dict(value=value, ms_per_step=ms_per_step, partial_ms=partial_ms, achieved=achieved,
                attn_bytes_per_step=attn_bytes.mean(), partial_bytes_per_launch=partial_bytes.mean(),
                lengths=lens, per_step_ms=per_step, host_enqueue_ms=np.array(host_ms))


def run_fresh_headline(steps, warmup):
    """The headline workload in a fresh Python process (its own GPU context,
    allocations and caches); returns its value, step and partial-kernel times."""
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--headline-child", "--steps", str(steps),
           "--warmup", str(warmup), "--no-cpu-baseline"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"fresh headline run failed ({r.returncode}):\n{r.stderr[-2000:]}")
    sys.stderr.write(r.stderr)
    sys.stderr.flush()
    return json.loads(r.stdout.strip().splitlines()[-1])


def run_rope_32k(torch, dev, reps=20):
    """Supplementary: the uniform 32K shape with a RoPE sub-block: keys of
    128 content coordinates (3-bit Full) plus 64 fp16 RoPE coordinates,
    values of 128; 64 sequences x 32,768 tokens, 32 query / 4 KV heads.
    Times the fused decode call (split + merge)."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    batch, T, hq, hkv, d, bits, r = 64, 32768, 32, 4, 128, 3, 64
    quats = torch.from_numpy(inputs.quaternions(hkv, d)).to(dev)
    cfg = B.Config(d, bits, B.IQ_FULL, hkv, quats, B.iq_codebook(bits, d))
    rng = np.random.default_rng(7)
    ch_k = inputs.outlier_channels(rng, hkv, d)
    ch_v = inputs.outlier_channels(rng, hkv, d)
    kc = B.new_cache(batch, hkv, T, d, bits, dev)
    vc = B.new_cache(batch, hkv, T, d, bits, dev)
    rope = torch.empty((batch, hkv, T, r), dtype=torch.int16, device=dev)
    sb = 8
    zero = torch.zeros((sb,), dtype=torch.int32, device=dev)
    for b0 in range(0, batch, sb):
        kx = torch.cat([inputs.device_kv(70, b0, sb * T, ch_k, d, dev),
                        inputs.device_normal(71, b0, (sb * T, hkv, r), dev, torch.float16)], dim=-1)
        B.iq_quantize_append_rope(cfg, kx.view(sb, T, hkv, d + r), r, zero,
                                  B.PackedCache(kc.codes[b0:b0 + sb], kc.norms[b0:b0 + sb]), rope[b0:b0 + sb])
        vx = inputs.device_kv(72, b0, sb * T, ch_v, d, dev)
        B.iq_quantize_append(cfg, vx.view(sb, T, hkv, d), zero, B.PackedCache(vc.codes[b0:b0 + sb], vc.norms[b0:b0 + sb]))
        del kx, vx
    q = inputs.device_normal(73, 0, (batch, hq, d + r), dev, torch.float16)
    kv_len = torch.full((batch,), T, dtype=torch.int32, device=dev)
    out = torch.empty((batch, hq, d), dtype=torch.float16, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    ws = torch.empty((B.iq_decode_workspace_bytes(cfg, batch, hq, T),), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d + r)
    stream = torch.cuda.current_stream()

    def call():
        B.iq_decode_attention_rope(cfg, q, kc, rope, vc, kv_len, T, scale, out, lse, None, ws)

    for _ in range(3):
        call()
    e0, e1 = _events(torch)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kv = batch * hkv * T * (2 * (row_bytes(d, bits) + 2) + 2 * r)
    qo = batch * hq * (d + r) * 2 + batch * hq * d * 2
    gbs = (kv + qo) / (ms * 1e-3) / 1e9
    print(f"[bench] RoPE 32K decode {ms:.4f} ms, {gbs:.1f} GB/s", file=sys.stderr, flush=True)
    del kc, vc, rope
    return {"workload": "64 sequences x 32768 tokens, 32 query / 4 KV heads, keys of 128 content coordinates "
                        "(3-bit IsoQuant-Full) + 64 fp16 RoPE coordinates, values of 128; fused decode call",
            "ms": round(ms, 5), "value": round(gbs, 2), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_call": int(kv + qo)}


def run_c3_latency(torch, dev, reps=20, T=8192, with_argmax=False):
    """Supplementary: one sequence of T tokens (8,192; 32,768 for the
    needle-search shape, which also writes the per-head argmax), 32 query /
    4 KV heads, d=128, 3-bit Full (3.3 / 13.1 MB of packed K/V: both fit the
    256 MB last-level cache).  Latency of one decode call (order, partial,
    merge), warm (back to back) and cold (512 MiB written between calls,
    events around the call only)."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    hq, hkv, d, bits = 32, 4, 128, 3
    quats = torch.from_numpy(inputs.quaternions(hkv, d)).to(dev)
    cfg = B.Config(d, bits, B.IQ_FULL, hkv, quats, B.iq_codebook(bits, d))
    rng = np.random.default_rng(3)
    kc = B.new_cache(1, hkv, T, d, bits, dev)
    vc = B.new_cache(1, hkv, T, d, bits, dev)
    zero = torch.zeros((1,), dtype=torch.int32, device=dev)
    for cache, idx in ((kc, 0), (vc, 1)):
        ch = inputs.outlier_channels(rng, hkv, d)
        B.iq_quantize_append(cfg, inputs.device_kv(70 + idx, 0, T, ch, d, dev).view(1, T, hkv, d), zero, cache)
    q = inputs.device_normal(72, 0, (1, hq, d), dev, torch.float16)
    kv_len = torch.full((1,), T, dtype=torch.int32, device=dev)
    out = torch.empty((1, hq, d), dtype=torch.float32, device=dev)
    arg = torch.empty((1, hq), dtype=torch.int32, device=dev) if with_argmax else None
    lse = torch.empty((1, hq), dtype=torch.float32, device=dev) if with_argmax else None
    ws = torch.empty((B.iq_decode_workspace_bytes(cfg, 1, hq, T),), dtype=torch.uint8, device=dev)
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def timed(cold):
        ts = []
        for _ in range(reps):
            if cold:
                flush.fill_(1)
            e0, e1 = _events(torch)
            e0.record(stream)
            B.iq_decode_attention(cfg, q, kc, vc, kv_len, T, 1.0 / math.sqrt(d), out, lse, arg, ws)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3

    timed(False)
    warm, cold = timed(False), timed(True)
    del flush
    print(f"[bench] {T // 1024}K single-sequence decode latency warm {warm:.1f} us, cold {cold:.1f} us",
          file=sys.stderr, flush=True)
    return {"workload": f"one sequence of {T} tokens, 32 query / 4 KV heads, d=128, 3-bit Full, fp16 q, "
                        f"fp32 out{', lse and argmax' if with_argmax else ''}; median of {reps} calls",
            "warm_us": round(warm, 1), "cold_us": round(cold, 1),
            "packed_kv_bytes": int(T * hkv * 2 * (row_bytes(d, bits) + 2))}


def run_prefill_compress(torch, dev, reps=5):
    """Supplementary: bulk compression of a finished prefill (deferred
    prefill, [RQ] Appendix C): 28 layers x (K, V) of [1][2048][8][128] fp16,
    3-bit Full, each layer with its own rotation; one iq_quantize_append_many
    call for all 56 tensors, and for comparison one iq_quantize_append call
    per tensor (n_new = 2048)."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    layers, T, hkv, d, bits = 28, 2048, 8, 128, 3
    cb = B.iq_codebook(bits, d)
    cfgs = []
    for layer in range(layers):
        quats = torch.from_numpy(inputs.quaternions(hkv, d, seed=layer)).to(dev)
        cfgs += [B.Config(d, bits, B.IQ_FULL, hkv, quats, cb)] * 2
    rng = np.random.default_rng(6)
    xs, caches = [], []
    for layer in range(layers):
        for idx in range(2):
            ch = inputs.outlier_channels(rng, hkv, d)
            xs.append(inputs.device_kv(60 + idx, layer, T, ch, d, dev).view(1, T, hkv, d))
            caches.append(B.new_cache(1, hkv, T, d, bits, dev))
    zero = torch.zeros((1,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    append_all = B.prepare_append_many(cfgs, xs, caches)
    ms = timed(lambda: append_all(zero))
    per_call_ms = timed(lambda: [B.iq_quantize_append(c, x, zero, o) for c, x, o in zip(cfgs, xs, caches)])
    nvec = layers * 2 * T * hkv
    moved = nvec * (d * 2 + row_bytes(d, bits) + 2)
    print(f"[bench] prefill compression {ms:.3f} ms for {layers} layers x K,V of {T}x{hkv}x{d} fp16 "
          f"({per_call_ms:.3f} ms with one call per tensor)", file=sys.stderr, flush=True)
    return {"workload": f"deferred-prefill compression: {layers} layers x (K, V) [1][{T}][{hkv}][{d}] fp16, "
                        f"{bits}-bit Full, one iq_quantize_append_many call for the {2 * layers} tensors",
            "ms": round(ms, 4), "input_mib": round(nvec * d * 2 / 2 ** 20, 1),
            "mvec_s": round(nvec / (ms * 1e-3) / 1e6, 1), "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
            "per_call_ms": round(per_call_ms, 4)}


def run_stage1(torch, dev):
    """Quantize / dequantize rates on 2^20 unit vectors for every setting of
    the stage-1 sweep (d x bits x variant x I/O dtype)."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    n = 1 << 20
    stream = torch.cuda.current_stream()
    rates = {}
    for d in (128, 256, 512):
        params = {v: torch.from_numpy(inputs.rotation_params(1, d, v)).to(dev)
                  for v in (B.IQ_FULL, B.IQ_FAST, B.IQ_PLANAR)}
        for bits in (2, 3, 4):
            for variant, vname in ((B.IQ_FULL, "full"), (B.IQ_FAST, "fast"), (B.IQ_PLANAR, "planar")):
                cfg = B.Config(d, bits, variant, 1, params[variant], B.iq_codebook(bits, d))
                c1 = B.new_cache(1, 1, n, d, bits, dev)
                sp = torch.zeros((1,), dtype=torch.int32, device=dev)
                for dt, dname in ((torch.float16, "fp16"), (torch.float32, "fp32")):
                    x = inputs.device_unit_vectors(2, n, d, dev, dt).view(1, n, 1, d)
                    o = torch.empty_like(x)
                    B.iq_quantize_append(cfg, x, sp, c1)
                    B.iq_dequantize(cfg, c1, sp, n, o)
                    reps = 10
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                    ev[0].record(stream)
                    for _ in range(reps):
                        B.iq_quantize_append(cfg, x, sp, c1)
                    ev[1].record(stream)
                    for _ in range(reps):
                        B.iq_dequantize(cfg, c1, sp, n, o)
                    ev[2].record(stream)
                    torch.cuda.synchronize()
                    qms = ev[0].elapsed_time(ev[1]) / reps
                    dms = ev[1].elapsed_time(ev[2]) / reps
                    io = n * (d * x.element_size() + row_bytes(d, bits) + 2)
                    qg, dg = io / (qms * 1e-3) / 1e9, io / (dms * 1e-3) / 1e9
                    rates[f"d{d}_b{bits}_{vname}_{dname}"] = {
                        "quantize_mvec_s": round(n / (qms * 1e-3) / 1e6, 1),
                        "dequantize_mvec_s": round(n / (dms * 1e-3) / 1e6, 1),
                        "quantize_gbs": round(qg, 1), "dequantize_gbs": round(dg, 1),
                        "quantize_hbm_frac": round(qg / HBM_PEAK_GBS, 4),
                        "dequantize_hbm_frac": round(dg / HBM_PEAK_GBS, 4)}
                    del x, o
                del c1
    for vname in ("full", "fast", "planar"):
        r = rates[f"d128_b3_{vname}_fp16"]
        print(f"[bench] stage-1 d=128 b=3 {vname} fp16: quantize {r['quantize_mvec_s']} Mvec/s, "
              f"dequantize {r['dequantize_mvec_s']} Mvec/s", file=sys.stderr, flush=True)
    h = rates["d128_b3_full_fp16"]
    return {"workload": "2^20 unit vectors per setting, d in {128,256,512} x bits in {2,3,4} x "
                        "{Full,Fast,Planar} x {fp16,fp32} I/O; HBM fractions are the algorithmic bytes "
                        "(d x input bytes + d x b / 8 + 2 per vector, the reverse for dequantize) over the "
                        "kernel time, against 8 TB/s",
            "quantize_mvec_s_d128_b3_full_fp16": h["quantize_mvec_s"], "rates": rates}


def run_c1_latency(torch, dev, reps=20):
    """The stage-1 parity configuration as a latency: 4,096 unit vectors,
    d=128, fp32, 3-bit Full; one quantize (append) call and one dequantize
    call, each timed alone with HIP events (median of reps, warm)."""
    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    n, d, bits = 4096, 128, 3
    cfg = B.Config(d, bits, B.IQ_FULL, 1, torch.from_numpy(inputs.quaternions(1, d)).to(dev),
                   B.iq_codebook(bits, d))
    x = torch.from_numpy(inputs.unit_vectors(n, d, np.float32, seed=1)).to(dev).view(1, n, 1, d)
    o = torch.empty_like(x)
    cache = B.new_cache(1, 1, n, d, bits, dev)
    sp = torch.zeros((1,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = _events(torch)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3

    q_us = timed(lambda: B.iq_quantize_append(cfg, x, sp, cache))
    d_us = timed(lambda: B.iq_dequantize(cfg, cache, sp, n, o))
    print(f"[bench] C1 4096 x 128 fp32: quantize {q_us:.1f} us, dequantize {d_us:.1f} us",
          file=sys.stderr, flush=True)
    return {"workload": "4,096 unit vectors, d=128, fp32 I/O, 3-bit Full (one head); single calls, median of "
                        f"{reps}, warm", "quantize_us": round(q_us, 2), "dequantize_us": round(d_us, 2),
            "quantize_mvec_s": round(n / q_us, 1)}


# Kernels whose HBM traffic is recorded, by the workload they run in.
TRAFFIC_KERNELS = {"headline": "partial_kernel<128, 3, 8, false, 0>",
                   "batched_append_c5": "partial_kernel<256, 3, 2, false, 0>"}


def summarize_counters(fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  Each is scaled by
    (true bytes / reading) of the 256 MiB device copy, whose kernel reads and
    writes exactly 256 MiB."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return by

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    # the runtime's buffer-copy blit kernel carries the 256 MiB device copy;
    # its largest dispatch is that copy (every other blit here is tiny)
    copy_names = [k for k in fetch if "copybuffer" in k.lower() and k in write]
    if not copy_names:
        raise SystemExit("no buffer-copy kernel in the counter files (run the passes with --calibrate-copy)")
    copy_name = max(copy_names, key=lambda k: max(write[k]))
    true_kib = COPY_BYTES / 1024
    f_read = true_kib / max(fetch[copy_name])
    f_write = true_kib / max(write[copy_name])
    out = {"commands": [
               "export TMPDIR=/tmp",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof_out/pmc_fetch -o f -- python3 bench.py "
               "--steps 3 --warmup 1 --no-cpu-baseline --decode-only --calibrate-copy",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof_out/pmc_write -o w -- python3 bench.py "
               "--steps 3 --warmup 1 --no-cpu-baseline --decode-only --calibrate-copy",
               "python3 bench.py --summarize-counters prof_out/pmc_fetch/f_counter_collection.csv "
               "prof_out/pmc_write/w_counter_collection.csv"],
           "kernel_source_hash": kernel_source_hash(),
           "copy_calibration": {"kernel": copy_name[:120], "bytes": COPY_BYTES,
                                "fetch_kib": max(fetch[copy_name]), "write_kib": max(write[copy_name]),
                                "read_factor": round(f_read, 4), "write_factor": round(f_write, 4)},
           "workloads": {}}
    for wname, kname in TRAFFIC_KERNELS.items():
        hits = [k for k in fetch if kname in k]
        if not hits:
            continue
        fk = float(np.mean(fetch[hits[0]]))
        wk = float(np.mean(write.get(hits[0], [0.0])))
        out["workloads"][wname] = {"kernel": kname, "dispatches": len(fetch[hits[0]]),
                                   "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                                   "hbm_bytes_per_launch": int(round((fk * f_read + wk * f_write) * 1024))}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


# read + write rate of a plain device-to-device copy measured on the GPU
# (torch copy_ of 4 GiB): the practical HBM ceiling for kernels that both
# read and write
COPY_CEILING_GBS = 4880.0
STAGE1_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "stage1_valu_and_hbm.md")


def summarize_stage1(counter_csv):
    """Per stage-1 kernel (d, bits, variant, I/O type): from one rocprofv3
    --pmc pass with SQ_INSTS_VALU and GRBM_GUI_ACTIVE, the VALU instructions
    per vector and the VALU issue utilisation (wave64 instructions x 4 cycles
    over the SIMD cycles of the dispatch: 1024 SIMDs, GRBM_GUI_ACTIVE being
    counted per XCD, 8 XCDs), next to the HBM rate of the algorithmic bytes
    over the dispatch's duration.  The larger fraction names the binding
    roofline."""
    import csv
    import re

    n = 1 << 20
    disp = {}
    for r in csv.DictReader(open(counter_csv)):
        # mangled (the _Float16 instantiations) or demangled (float) names
        m = (re.search(r"(quantize|dequantize)_kernelILi(\d+)ELi(\d)ELi(\d)E(DF16_|f)E", r["Kernel_Name"]) or
             re.search(r"(quantize|dequantize)_kernel<(\d+), (\d), (\d), (_Float16|float)>", r["Kernel_Name"]))
        if not m:
            continue
        io = "fp16" if m.group(5) in ("DF16_", "_Float16") else "fp32"
        e = disp.setdefault(r["Dispatch_Id"], {"key": (m.group(1), int(m.group(2)), int(m.group(3)),
                                                        int(m.group(4)), io),
                                                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for e in disp.values():
        if "SQ_INSTS_VALU" in e and "GRBM_GUI_ACTIVE" in e:
            agg.setdefault(e["key"], []).append(e)
    vname = {0: "Full", 1: "Fast", 2: "Planar"}
    lines = ["# Stage-1 kernels: VALU and HBM fractions", "",
             "Commands (from the repository root, on one MI355X):", "", "```", "export TMPDIR=/tmp",
             "rocprofv3 --pmc SQ_INSTS_VALU SQ_WAVES GRBM_GUI_ACTIVE --output-format csv -d prof_out/pmc_s1 "
             "-o s -- python3 bench.py --stage1-only",
             "python3 bench.py --summarize-stage1 prof_out/pmc_s1/s_counter_collection.csv", "```", "",
             f"2^20 vectors per dispatch; medians over the dispatches of each kernel.  VALU: wave64 VALU "
             f"instructions per vector x 64 lanes (lane-ops per vector), and the issue ratio = "
             f"SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x the dispatch's cycles, GRBM_GUI_ACTIVE / 8 being "
             f"the cycles of one XCD); it exceeds 1 where part of the instructions take fewer than four "
             f"cycles, and near or above 1 the VALU issues without pause.  HBM: (d x input bytes + "
             f"d x b / 8 + 2) bytes per vector for quantize, the reverse for dequantize, over the dispatch's "
             f"duration (counter collection serialises dispatches, so the durations are those of a lone "
             f"kernel), as a fraction of 8 TB/s.  Bound: HBM where the rate reaches 90% of what a plain "
             f"device-to-device copy moves on this GPU (read + write, {COPY_CEILING_GBS / 1e3:.2f} TB/s), "
             f"VALU where the issue ratio reaches 0.9, else neither (issue stalls).", "",
             "| kernel | d | b | variant | I/O | us | G vec/s | VALU lane-ops / vec | VALU issue ratio | HBM GB/s | HBM frac | bound |",
             "|---|---:|---:|---|---|---:|---:|---:|---:|---:|---:|---|"]
    for key in sorted(agg, key=lambda k: (k[0] != "quantize", k[1], k[2], k[3], k[4])):
        kind, d, b, v, io = key
        es = agg[key]
        ns = float(np.median([e["ns"] for e in es]))
        valu = float(np.median([e["SQ_INSTS_VALU"] for e in es]))
        util = float(np.median([e["SQ_INSTS_VALU"] * 4 / (128.0 * e["GRBM_GUI_ACTIVE"]) for e in es]))
        nbytes = n * (d * (2 if io == "fp16" else 4) + row_bytes(d, b) + 2)
        gbs = nbytes / ns
        frac = gbs / HBM_PEAK_GBS
        hbm_bound, valu_bound = gbs >= 0.9 * COPY_CEILING_GBS, util >= 0.9
        bound = ("HBM + VALU" if valu_bound else "HBM") if hbm_bound else ("VALU" if valu_bound else "neither")
        lines.append(f"| {kind} | {d} | {b} | {vname[v]} | {io} | {ns / 1e3:.1f} | {n / ns:.2f} | "
                     f"{valu * 64 / n:.0f} | {util:.2f} | {gbs:.0f} | {frac:.2f} | {bound} |")
    text = "\n".join(lines) + "\n"
    os.makedirs(os.path.dirname(STAGE1_FILE), exist_ok=True)
    with open(STAGE1_FILE, "w") as f:
        f.write(text)
    print(text)
    return 0


def _oracle_worker(w, T, seconds):
    """One process: the oracle's dequantize-then-attend on one (sequence,
    KV head) pair of T rows of workload w with its G query heads, repeated
    for about ``seconds``.  Returns (repetitions, elapsed seconds)."""
    import oracle as O
    from compressed_space_attention_isoquant_amd import inputs

    d, bits = w["head_dim"], w["bits"]
    variant = {"full": O.FULL, "fast": O.FAST}[w["variant"]]
    group = w["num_q_heads"] // w["num_kv_heads"]
    rng = np.random.default_rng(44)
    ch = inputs.outlier_channels(rng, 1, d)[0]
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    k[:, ch] *= inputs.OUTLIER_SCALE
    v[:, ch] *= inputs.OUTLIER_SCALE
    k, v = k.astype(np.float16), v.astype(np.float16)
    q = rng.standard_normal((group, d)).astype(np.float16)
    quats = inputs.quaternions(1, d)
    cb = O.codebook(bits, d)
    rk = O.quantize(k, quats[0], cb, variant)
    rv = O.quantize(v, quats[0], cb, variant)
    kr, kn = O.pack(rk["codes"], bits)[None], rk["norm16"][None]
    vr, vn = O.pack(rv["codes"], bits)[None], rv["norm16"][None]
    reps, t0 = 0, time.perf_counter()
    while True:
        O.attend(q, kr, kn, vr, vn, quats, cb, bits, variant, 1.0 / math.sqrt(d))
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return reps, time.perf_counter() - t0


# The box grants one GPU 16 host cores, whatever the host has: the baseline's
# process pool is held to that share.
CPU_SHARE = 16


def _host_workers(max_workers=CPU_SHARE):
    return max(1, min(max_workers, len(os.sched_getaffinity(0))))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def _pool_map(fn, argsets):
    """Run fn over argsets in one spawned process per entry, BLAS held to one
    thread per process."""
    import concurrent.futures as cf
    import multiprocessing as mp

    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        with cf.ProcessPoolExecutor(max_workers=len(argsets), mp_context=mp.get_context("spawn")) as ex:
            return list(ex.map(fn, *zip(*argsets)))
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val


def cpu_baseline(w, lengths, seconds):
    """The FP64 oracle's dequantize-then-attend on a bounded sample of
    workload w: each of W worker processes (one per host core of the box's
    share) runs one (sequence, KV head) pair at the median context length
    with its query heads for about ``seconds``.  Aggregate packed-KV GB/s
    over the workers."""
    d, bits = w["head_dim"], w["bits"]
    T = int(np.median(lengths))
    group = w["num_q_heads"] // w["num_kv_heads"]
    workers = _host_workers()
    res = _pool_map(_oracle_worker, [(w, T, seconds)] * workers)
    nbytes = T * 2 * (row_bytes(d, bits) + 2)
    rate = sum(r * nbytes / dt for r, dt in res)
    per = float(np.mean([dt / r for r, dt in res]))
    return {"value": round(rate / 1e9, 5), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "one_core_value": round(nbytes / per / 1e9, 5), "cpu_model": _cpu_model(),
            "host_cores_visible": len(os.sched_getaffinity(0)),
            "sample": f"{workers} processes (one BLAS thread each), each repeating one (sequence, KV head) "
                      f"pair of this workload at context length {T}: {T} packed K/V rows, "
                      f"{group} query heads, d={d}, {bits}-bit {w['variant']}; {sum(r for r, _ in res)} "
                      f"repetitions in all, {per:.3f} s each (NumPy FP64)"}


def _oracle_stage1_worker(d, bits, n, seconds):
    """One process: the oracle's quantize (normalise, WHT, SO(4), Lloyd-Max,
    pack) of chunks of n unit vectors, d, bits, Full, fp16 input, repeated
    for about ``seconds``.  Returns (vectors, elapsed seconds)."""
    import oracle as O
    from compressed_space_attention_isoquant_amd import inputs

    x = inputs.unit_vectors(n, d, np.float16, seed=2)
    quats = inputs.quaternions(1, d)
    cb = O.codebook(bits, d)
    done, t0 = 0, time.perf_counter()
    while True:
        r = O.quantize(x, quats[0], cb, O.FULL)
        O.pack(r["codes"], bits)
        done += n
        if time.perf_counter() - t0 >= seconds:
            break
    return done, time.perf_counter() - t0


def cpu_baseline_stage1(seconds, d=128, bits=3, n=8192):
    """The oracle's stage-1 quantize rate (vectors/s) over the machine's host-core
    share, each worker quantizing chunks of n vectors of the sweep's d=128,
    3-bit, Full, fp16 setting for about ``seconds``."""
    workers = _host_workers()
    res = _pool_map(_oracle_stage1_worker, [(d, bits, n, seconds)] * workers)
    rate = sum(v / dt for v, dt in res)
    return {"value": round(rate / 1e6, 4), "unit": "Mvec/s", "cores": workers, "kind": "oracle",
            "one_core_value": round(float(np.mean([v / dt for v, dt in res])) / 1e6, 4),
            "sample": f"{workers} processes, each quantizing chunks of {n} unit vectors (d={d}, {bits}-bit Full, "
                      f"fp16 in) for about {seconds:.0f} s; {sum(v for v, _ in res)} vectors in all (NumPy FP64)"}


if __name__ == "__main__":
    sys.exit(main())

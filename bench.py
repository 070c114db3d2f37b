#!/usr/bin/env python3
"""Benchmark of the IsoQuant packed-KV decode step on one MI355X.

Workload (fp16 I/O, synthetic): 64 independent sequences at 32,768 tokens of
context, 32 query heads / 4 KV heads (GQA 8:1), head_dim 128, 3-bit
IsoQuant-Full codes for K and V (838.9 MB of packed KV).  One step = quantize
and append one new K and one new V vector per sequence and KV head (into the
last row, so every step attends over exactly 32,768 rows), then decode
attention for the 32 query heads of every sequence over the packed caches.

Prints one JSON line: value = packed-KV bytes the step's attention reads per
second of step time (GB/s), plus the dominant kernel's roofline, the stage-1
quantize/dequantize rates on 2^20 vectors (d=128, 3-bit, Full, fp16), and the
FP64 oracle timed on the host as a baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

WORKLOAD = dict(batch=64, kv_len=32768, num_q_heads=32, num_kv_heads=4, head_dim=128, bits=3,
                variant="full")


def packed_row_bytes(d, bits):
    return d * bits // 8


def kv_bytes(w):
    """Every packed K and V row and its fp16 norm, read once."""
    rows = w["batch"] * w["num_kv_heads"] * w["kv_len"]
    return rows * 2 * (packed_row_bytes(w["head_dim"], w["bits"]) + 2)


def attention_bytes(w):
    """Algorithmic HBM bytes of one decode attention: the packed K/V with
    norms, q read (fp16) and o written (fp16)."""
    return kv_bytes(w) + 2 * w["batch"] * w["num_q_heads"] * w["head_dim"] * 2


def partial_bytes(w):
    """Algorithmic HBM bytes of the split (partial) kernel: packed K/V with
    norms and q (fp16).  Its partial states are O(splits x d) per head and not
    counted."""
    return kv_bytes(w) + w["batch"] * w["num_q_heads"] * w["head_dim"] * 2


def append_bytes(w):
    """Two quantize-appends per step: fp16 vectors in, packed rows + norms out."""
    n = w["batch"] * w["num_kv_heads"]
    return 2 * n * (w["head_dim"] * 2 + packed_row_bytes(w["head_dim"], w["bits"]) + 2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        return 2

    import torch

    from compressed_space_attention_isoquant_amd import binding as B
    from compressed_space_attention_isoquant_amd import inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = dict(WORKLOAD)
    batch, T, hq, hkv, d, bits = (w[k] for k in ("batch", "kv_len", "num_q_heads", "num_kv_heads",
                                                 "head_dim", "bits"))
    variant = B.IQ_FULL
    quats = torch.from_numpy(inputs.quaternions(hkv, d)).to(dev)
    cfg = B.Config(d, bits, variant, hkv, quats, B.iq_codebook(bits, d))
    rng = np.random.default_rng(4)
    ch_k = inputs.outlier_channels(rng, hkv, d)
    ch_v = inputs.outlier_channels(rng, hkv, d)

    # ---- set-up: prefill caches with T-1 tokens per sequence (not timed) ----
    kc = B.new_cache(batch, hkv, T, d, bits, dev)
    vc = B.new_cache(batch, hkv, T, d, bits, dev)
    zero = torch.zeros((batch,), dtype=torch.int32, device=dev)
    for cache, idx, ch in ((kc, 0, ch_k), (vc, 1, ch_v)):
        x = inputs.device_kv(40, idx, batch * (T - 1), ch, d, dev).view(batch, T - 1, hkv, d)
        B.iq_quantize_append(cfg, x, zero, cache)
        del x
    torch.cuda.synchronize()
    P = 8   # distinct new-token / query draws cycled over the steps
    knew = [inputs.device_kv(41, s, batch, ch_k, d, dev).view(batch, 1, hkv, d) for s in range(P)]
    vnew = [inputs.device_kv(42, s, batch, ch_v, d, dev).view(batch, 1, hkv, d) for s in range(P)]
    qs = [inputs.device_normal(43, s, (batch, hq, d), dev, torch.float16) for s in range(P)]
    last = torch.full((batch,), T - 1, dtype=torch.int32, device=dev)
    kv_len = torch.full((batch,), T, dtype=torch.int32, device=dev)
    out = torch.empty((batch, hq, d), dtype=torch.float16, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    arg = torch.empty((batch, hq), dtype=torch.int32, device=dev)
    ws = torch.empty((B.iq_decode_workspace_bytes(cfg, batch, hq, T),), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    events = []

    def step(s, record):
        B.iq_quantize_append(cfg, knew[s % P], last, kc)
        B.iq_quantize_append(cfg, vnew[s % P], last, vc)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        # the two phases of iq_decode_attention, so that the events bracket the
        # partial (dominant) kernel alone
        B.iq_decode_attention_partial(cfg, qs[s % P], kc, vc, kv_len, T, scale, ws, track_argmax=False)
        if record:
            e1.record(stream)
            events.append((e0, e1))
        B.iq_decode_attention_merge(cfg, batch, hq, T, out, lse, None, ws)

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    print(f"[bench] decode step {ms_per_step:.4f} ms, partial kernel {attn_ms:.4f} ms", file=sys.stderr, flush=True)

    abytes = attention_bytes(w)
    step_bytes = abytes + append_bytes(w)
    value = abytes / (ms_per_step * 1e-3) / 1e9
    achieved = partial_bytes(w) / (attn_ms * 1e-3) / 1e9

    # ---- stage-1 rates: 2^20 vectors, d=128, 3-bit, Full, fp16 I/O ----------
    n = 1 << 20
    cfg1 = B.Config(d, bits, variant, 1, quats[:1].contiguous(), B.iq_codebook(bits, d))
    x1 = inputs.device_unit_vectors(2, n, d, dev, torch.float16).view(1, n, 1, d)
    c1 = B.new_cache(1, 1, n, d, bits, dev)
    o1 = torch.empty_like(x1)
    sp1 = torch.zeros((1,), dtype=torch.int32, device=dev)
    for _ in range(3):
        B.iq_quantize_append(cfg1, x1, sp1, c1)
        B.iq_dequantize(cfg1, c1, sp1, n, o1)
    reps = 20
    eq = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    eq[0].record(stream)
    for _ in range(reps):
        B.iq_quantize_append(cfg1, x1, sp1, c1)
    eq[1].record(stream)
    for _ in range(reps):
        B.iq_dequantize(cfg1, c1, sp1, n, o1)
    eq[2].record(stream)
    torch.cuda.synchronize()
    q_ms = eq[0].elapsed_time(eq[1]) / reps
    dq_ms = eq[1].elapsed_time(eq[2]) / reps
    row = packed_row_bytes(d, bits)
    stage1 = {
        "quantize_mvec_s": n / (q_ms * 1e-3) / 1e6,
        "quantize_gbs": n * (2 * d + row + 2) / (q_ms * 1e-3) / 1e9,
        "dequantize_mvec_s": n / (dq_ms * 1e-3) / 1e6,
        "dequantize_gbs": n * (2 * d + row + 2) / (dq_ms * 1e-3) / 1e9,
        "workload": "2^20 unit vectors, d=128, 3-bit, IsoQuant-Full, fp16 in/out",
    }
    print(f"[bench] stage-1 quantize {q_ms:.4f} ms, dequantize {dq_ms:.4f} ms", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, ch_k, ch_v, args.cpu_seconds)

    result = {
        "metric": "packed-KV decode-attn GB/s (% HBM peak) at 32K ctx; quantize Mvec/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded torch/NumPy draws: N(0,1) K/V with 4 x10 outlier channels per head)",
        "config": {
            "workload": "decode step: append 1 K + 1 V token per sequence, then attention over packed "
                        "3-bit K/V; 64 seqs x 32768 ctx, Hq=32, H_kv=4, d=128, IsoQuant-Full, fp16 I/O",
            "batch": batch, "kv_len": T, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
            "bits": bits, "variant": "full", "packed_kv_bytes_per_step": abytes,
            "step_bytes": step_bytes,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "partial_kernel_ms": round(attn_ms, 5),
        "stage1": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in stage1.items()},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "partial_kernel<128,3,8> (split-K decode over packed K/V)",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result))
    return 0


def cpu_baseline(w, ch_k, ch_v, seconds):
    """The FP64 oracle's dequantize-then-attend on a bounded sample of the same
    workload: one (sequence, KV head) pair at the full context with its 8 query
    heads, repeated for about ``seconds`` of host time."""
    import oracle as O
    from compressed_space_attention_isoquant_amd import inputs

    d, bits, T = w["head_dim"], w["bits"], w["kv_len"]
    group = w["num_q_heads"] // w["num_kv_heads"]
    rng = np.random.default_rng(44)
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    k[:, ch_k[0]] *= inputs.OUTLIER_SCALE
    v[:, ch_v[0]] *= inputs.OUTLIER_SCALE
    k, v = k.astype(np.float16), v.astype(np.float16)
    q = rng.standard_normal((group, d)).astype(np.float16)
    quats = inputs.quaternions(w["num_kv_heads"], d)[:1]
    cb = O.codebook(bits, d)
    rk = O.quantize(k, quats[0], cb, O.FULL)
    rv = O.quantize(v, quats[0], cb, O.FULL)
    kr, kn = O.pack(rk["codes"], bits)[None], rk["norm16"][None]
    vr, vn = O.pack(rv["codes"], bits)[None], rv["norm16"][None]
    reps, t0 = 0, time.perf_counter()
    while True:
        O.attend(q, kr, kn, vr, vn, quats, cb, bits, O.FULL, 1.0 / math.sqrt(d))
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = T * 2 * (packed_row_bytes(d, bits) + 2)
    return {"value": round(nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one (sequence, KV head) pair: {T} packed K/V rows, {group} query heads, "
                      f"{reps} repetitions, {dt:.3f} s each (single-threaded NumPy FP64)"}


if __name__ == "__main__":
    sys.exit(main())

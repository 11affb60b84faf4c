#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

One step = one paged_attn_forward over one batch of the workload (plan,
block-table gather, fp8 dequantisation when present, scores, mask, online
softmax, P.V, split merge: the whole path).  Successive steps rotate over
copies of the batch placed at disjoint physical pages, about 1 GiB in total,
so every step reads its KV from HBM rather than from the 256 MB
Infinity Cache or the L2s.

Prints one JSON line: KV GB/s for decode/verify workloads (TFLOP/s for the
chunked prefill), the roofline of the kernel time measured with HIP events
on the launch stream, and the fp64 CPU oracle timed on a bounded sample of
the same workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--all]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV GB/s (% of HBM peak) decode/verify; TFLOP/s (% MFMA peak) chunked prefill"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
ROTATE_BYTES = 1 << 30         # KV bytes the timed steps rotate over (4x the Infinity Cache)
MAX_COPIES = 64

WORKLOADS = {
    "tiny_decode": "tiny decode: 1 seq, q_len 1, 4/1 heads, D 64, 257 tokens, fp16 KV",
    "decode": "single-token decode: 1 seq, q_len 1, 32/8 heads, D 128, 4,097 tokens, bf16 KV, 16-token pages",
    "verify": "speculative verify: 1 seq, q_len 8 causal, 32/8 heads, D 128, 61,448 tokens, fp16 KV, 1% K x4",
    "verify_window": "speculative verify, 2048-token window, out-of-window pages NaN (61,448 tokens, fp16 KV)",
    "prefill": "chunked prefill: 2,048-token chunk on 65,536 cached, 24/4 heads, D 128, bf16 KV",
    "mixed_fp8": "mixed batch: 4 seqs, 200,001/131,076/32,776/4,097 tokens, q_len 1/4/8/1, 32/8 heads, fp8 e4m3 KV",
}
DTYPE_NAME = {"f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3 (kv) / fp32 accumulate"}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "paged_attention_long_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("kernel_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def measure(workload: str, steps: int, warmup: int):
    import numpy as np
    import torch

    import paged_attention_long_amd as pal
    from synth import named
    from synth.gen import replicate
    from synth.torch_upload import upload_batch, upload_pool

    t0 = time.time()
    base = named(workload)[0]
    kv_bytes = base.kv_bytes()
    flops = base.flops()
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / kv_bytes)))
    batches = replicate(base, copies, seed=1)
    pools = upload_pool(batches)
    devs = [upload_batch(b) for b in batches]
    log(f"[bench] {workload}: inputs ready in {time.time() - t0:.1f}s ({copies} rotating copies, "
        f"{kv_bytes / 1e6:.2f} MB KV per step)")

    cfg = pal.make_config(base.num_q_heads, base.num_kv_heads, base.head_dim, base.q_dtype, base.kv_dtype,
                          base.num_seqs, int(base.q_lens.max()), base.num_tokens)
    h = pal.paged_attn_create(cfg)
    out = torch.empty((base.num_tokens, base.num_q_heads, base.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((base.num_tokens, base.num_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        d = devs[i % copies]
        pal.paged_attn_forward(h, d["q"], pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                               base.window, base.scale, d["kv_scale"], out, lse, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        ev0[i].record(stream)
        step(warmup + i)
        ev1[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kt = np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)]) * 1e-3     # seconds per forward
    pal.paged_attn_destroy(h)
    assert torch.isfinite(out).all().item(), "non-finite output"

    k_mean = float(kt.mean())
    if workload == "prefill":
        unit = "TFLOP/s"
        value = flops * steps / wall / 1e12
        achieved = flops / k_mean / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                "frac": achieved / BF16_MFMA_PEAK_TFS}
    else:
        unit = "GB/s"
        value = kv_bytes * steps / wall / 1e9
        achieved = kv_bytes / k_mean / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = load_traffic(workload)
    res = {
        "value": value, "unit": unit, "ms_per_step": wall / steps * 1e3, "roofline": roof,
        "kernel_us": {"mean": k_mean * 1e6, "median": float(np.median(kt)) * 1e6, "min": float(kt.min()) * 1e6,
                      "max": float(kt.max()) * 1e6},
        "kv_bytes_per_step": kv_bytes, "flops_per_step": flops, "rotating_copies": copies,
        "dtype": DTYPE_NAME[base.kv_dtype],
    }
    log(f"[bench] {workload}: {value:.1f} {unit} (wall), kernel mean {k_mean * 1e6:.2f} us -> "
        f"{achieved:.1f} {roof['unit']} = {roof['frac'] * 100:.1f}% of peak")
    return res, base


def cpu_baseline(workload: str, base, budget_s: float = 12.0):
    """The fp64 oracle on this host: full attention of the workload's batch
    (decode-sized workloads) or a bounded slice of its rows, repeated until
    the time budget is spent."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    kv_bytes = base.kv_bytes()
    t0 = time.perf_counter()
    reps = 0
    if workload in ("tiny_decode", "decode", "verify_window"):
        while True:
            oracle.attention(base)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        sample = f"full {workload} batch (all {base.num_tokens * base.num_q_heads} rows), {reps} repetitions"
        return {"value": kv_bytes * reps / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": el}
    # Larger workloads: rows of one KV head at a time, scaled by the head count.
    Hk, G = base.num_kv_heads, base.group
    rows = []
    cu = np.concatenate([[0], np.cumsum(base.q_lens)])
    for b in range(base.num_seqs):
        for t in range(int(cu[b]), int(cu[b + 1])):
            rows.append((t, 0))
    done_heads = 0
    while True:
        g = done_heads % Hk
        hh = g * G + (done_heads // Hk) % G
        oracle.attention_rows(base, [(t, hh) for t, _ in rows])
        done_heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    frac = done_heads / base.num_q_heads
    sample = f"all tokens of {done_heads} query head(s) of {base.num_q_heads}; scaled by heads"
    if workload == "prefill":
        return {"value": base.flops() * frac / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": sample, "seconds": el}
    return {"value": kv_bytes * frac / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": el}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="also measure every other workload (per_config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    res, base = measure(args.workload, args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "name": args.workload,
                   "kv_bytes_per_step": res["kv_bytes_per_step"], "flops_per_step": res["flops_per_step"],
                   "rotating_copies": res["rotating_copies"], "parallelism": "single GPU"},
        "roofline": res["roofline"], "kernel_us": res["kernel_us"],
    }
    if args.all:
        per = {}
        for w in ("decode", "verify", "verify_window", "prefill", "mixed_fp8"):
            if w == args.workload:
                continue
            try:
                r, _ = measure(w, max(20, args.steps // 4), max(5, args.warmup // 2))
                per[w] = {"value": r["value"], "unit": r["unit"], "roofline": r["roofline"],
                          "kernel_us": r["kernel_us"]}
            except Exception as e:  # report, do not hide
                per[w] = {"error": repr(e)}
        line["per_config"] = per
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, base)
    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()

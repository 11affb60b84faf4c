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
    "append_fp8": "cache append: 64 seqs x 256 new rows, 8 KV heads, D 128, bf16 rows quantised into fp8 e4m3 pages",
}
# inputs as stored; every product is accumulated, and every softmax step computed, in fp32
DTYPE_NAME = {"f16": "f16 in / f32 accumulate", "bf16": "bf16 in / f32 accumulate",
              "fp8_e4m3": "fp8_e4m3 kv, bf16 q / f32 accumulate"}


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


def measure(workload: str, steps: int, warmup: int, use_graph: bool = True):
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

    pos = base.q_lens[base.q_lens > 0]
    cfg = pal.make_config(base.num_q_heads, base.num_kv_heads, base.head_dim, base.q_dtype, base.kv_dtype,
                          base.num_seqs, int(base.q_lens.max()), base.num_tokens, min_q_len=int(pos.min()))
    h = pal.paged_attn_create(cfg)
    out = torch.empty((base.num_tokens, base.num_q_heads, base.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((base.num_tokens, base.num_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        d = devs[i % copies]
        pal.paged_attn_forward(h, d["q"], pools["k"], pools["v"], d["block_table"], d["seq_lens"], d["q_lens"],
                               base.window, base.scale, d["kv_scale"], out, lse,
                               stream=torch.cuda.current_stream())

    def timed(fn):
        """Wall clock and HIP-event time of fn(), synchronised on both sides."""
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - w0, e0.elapsed_time(e1) * 1e-3

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Eager: one launch per step from Python.
    eager_wall, eager_ev = timed(lambda: [step(warmup + i) for i in range(steps)])
    graph_wall = graph_ev = None
    if use_graph:
        # The same K steps captured once into a HIP graph and replayed: no
        # host launch cost between the forwards.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        graph_wall, graph_ev = timed(g.replay)
    pal.paged_attn_destroy(h)
    assert torch.isfinite(out).all().item(), "non-finite output"

    wall = graph_wall if use_graph else eager_wall
    k_mean = (graph_ev if use_graph else eager_ev) / steps
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
    # A forward is the attention launch(es) plus the split-merge launch; the
    # events bracket whole forwards, so achieved and traffic are per forward.
    roof["scope"] = "one forward: attention kernel(s) + split-merge kernel, HIP events over the timed region / steps"
    work = flops if workload == "prefill" else kv_bytes
    res = {
        "value": value, "unit": unit, "ms_per_step": wall / steps * 1e3, "roofline": roof,
        "forward_us": {"graph_events": graph_ev / steps * 1e6 if use_graph else None,
                       "eager_events": eager_ev / steps * 1e6, "eager_wall": eager_wall / steps * 1e6},
        "eager_value": work * steps / eager_wall / (1e12 if workload == "prefill" else 1e9),
        "timing": "graph replay of the timed steps" if use_graph else "eager launches",
        "forwards_run": warmup + steps + (2 * steps if use_graph else 0),
        "kv_bytes_per_step": kv_bytes, "flops_per_step": flops, "rotating_copies": copies,
        "dtype": DTYPE_NAME[base.kv_dtype],
    }
    log(f"[bench] {workload}: {value:.1f} {unit} ({res['timing']}, wall), {k_mean * 1e6:.2f} us per forward "
        f"(events) -> {achieved:.1f} {roof['unit']} = {roof['frac'] * 100:.1f}% of peak; eager "
        f"{res['eager_value']:.1f} {unit}")
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


COPY_KERNEL_TAG = "neg_kernel"     # torch.neg: reads N bytes, writes N bytes
OUR_KERNEL_TAGS = ("decode_valu_kernel", "tile_attn_kernel", "merge_kernel", "merge_slots_kernel")


def calibrate_copy(mib: int) -> None:
    """Runs a plain elementwise kernel of known traffic (torch.neg over mib
    MiB of fp32, three times) so a counter pass over the same process can
    scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {COPY_KERNEL_TAG} over {mib} MiB read + {mib} MiB written, x3")
    del src, dst


def _csv_rows(path_glob: str):
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(path_glob, recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name: str) -> str:
    if COPY_KERNEL_TAG in name:
        return COPY_KERNEL_TAG
    for tag in OUR_KERNEL_TAGS:
        if tag in name:
            i = name.find(tag)
            j = name.find("(", i)
            return name[i:j if j > 0 else None]
    return name[:60]


def reduce_profiles(prof_dir: str, workload: str, calib_mib: int, commands: list) -> dict:
    """Turns one workload's rocprofv3 runs (kernel trace + stats, a FETCH_SIZE
    pass, a WRITE_SIZE pass) into profiles/<kernel>_<workload>.md and its
    entry in profiles/traffic.json."""
    import collections

    stats = [r for r in _csv_rows(os.path.join(prof_dir, "kt", "**", "*kernel_stats.csv"))]
    per = {}
    for cname, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        vals = collections.defaultdict(list)
        for r in _csv_rows(os.path.join(prof_dir, sub, "**", "*counter_collection.csv")):
            if r["Counter_Name"] == cname:
                vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        per[cname] = vals
    calib_bytes = calib_mib << 20
    fetch_copy = per["FETCH_SIZE"][COPY_KERNEL_TAG]
    write_copy = per["WRITE_SIZE"][COPY_KERNEL_TAG]
    if not fetch_copy or not write_copy:
        raise RuntimeError("no calibration kernel in the counter passes")
    # KiB per dispatch -> bytes: scale so the copy reads / writes exactly its size
    f_scale = calib_bytes / (sum(fetch_copy) / len(fetch_copy) * 1024)
    w_scale = calib_bytes / (sum(write_copy) / len(write_copy) * 1024)
    ours = sorted(k for k in per["FETCH_SIZE"] if any(t in k for t in OUR_KERNEL_TAGS))
    kern = {}
    for k in ours:
        fv, wv = per["FETCH_SIZE"][k], per["WRITE_SIZE"].get(k, [])
        kern[k] = {"dispatches": len(fv), "fetch_kib": sum(fv) / len(fv),
                   "write_kib": (sum(wv) / len(wv)) if wv else float("nan")}
    # dispatches per forward: dispatches in the counter pass / forwards that (eager) run made
    with open(os.path.join(prof_dir, "fetch", "bench.json")) as f:
        fetch_run = json.loads(f.read().strip().splitlines()[-1])
    with open(os.path.join(prof_dir, "kt", "bench.json")) as f:
        n_fwd = json.loads(f.read().strip().splitlines()[-1])
    from synth import named

    base = named(workload)[0]
    alg = base.flops() if workload == "prefill" else base.kv_bytes()
    hbm = 0.0
    for k, v in kern.items():
        v["per_forward"] = v["dispatches"] / max(1, fetch_run["forwards_run"])
        v["hbm_bytes"] = v["fetch_kib"] * 1024 * f_scale + v["write_kib"] * 1024 * w_scale
        hbm += v["hbm_bytes"] * v["per_forward"]
    lines = [f"# {', '.join(kern) or 'kernels'}: {workload}", "",
             f"Workload: {WORKLOADS[workload]}.", "", "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if any(t in r["Name"] for t in OUR_KERNEL_TAGS):
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", f"The traced bench.py run: {n_fwd['timing']}, forward time from HIP events "
              f"{json.dumps(n_fwd['forward_us'])} us, roofline {json.dumps(n_fwd['roofline'])}.", "",
              "## HBM traffic (FETCH_SIZE, WRITE_SIZE passes)", "",
              f"Calibration: {COPY_KERNEL_TAG} over {calib_mib} MiB reads and writes {calib_bytes} B each; "
              f"counters read {sum(fetch_copy) / len(fetch_copy):.0f} KiB fetched and "
              f"{sum(write_copy) / len(write_copy):.0f} KiB written per dispatch, so bytes = "
              f"FETCH_SIZE x 1024 x {f_scale:.4f} and WRITE_SIZE x 1024 x {w_scale:.4f}.", "",
              "| kernel | dispatches | per forward | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per dispatch |",
              "|---|---|---|---|---|---|"]
    for k, v in kern.items():
        lines.append(f"| {k} | {v['dispatches']} | {v['per_forward']:.2f} | {v['fetch_kib']:.0f} | "
                     f"{v['write_kib']:.0f} | {v['hbm_bytes']:.4g} |")
    unit = "flop" if workload == "prefill" else "B of KV"
    lines += ["", f"HBM bytes per forward: {hbm:.4g}; algorithmic {alg:.4g} {unit} per forward"
              + ("" if workload == "prefill" else f" (ratio {hbm / alg:.3f})") + ".", ""]
    name = "_".join(sorted({k.split("<")[0] for k in kern})) or "kernels"
    out_md = os.path.join(ROOT, "profiles", f"{name}_{workload}.md")
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(tj) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = {"kernel_hash": kernel_source_hash(), "hbm_bytes_per_launch": hbm,
                      "fetch_scale": f_scale, "write_scale": w_scale, "summary": os.path.basename(out_md)}
    with open(tj, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    log(f"[bench] wrote {out_md} and the {workload} entry of {tj}")
    return data[workload]


APPEND_SHAPE = dict(num_seqs=64, rows=256, hkv=8, head_dim=128)


def _append_inputs(seed: int = 7):
    """Seeded append workload: each sequence's last `rows` positions get new
    rows; its block table maps those pages to distinct pool pages."""
    import numpy as np

    sh = APPEND_SHAPE
    rng = np.random.default_rng(seed)
    seq_lens = rng.integers(sh["rows"], 60000, sh["num_seqs"]).astype(np.int32)
    q_lens = np.full(sh["num_seqs"], sh["rows"], dtype=np.int32)
    width = int((seq_lens.max() + 15) // 16)
    per = sh["rows"] // 16 + 1
    pages = sh["num_seqs"] * per
    perm = rng.permutation(pages).astype(np.int32)
    bt = np.zeros((sh["num_seqs"], width), dtype=np.int32)
    for b, sl in enumerate(seq_lens.tolist()):
        first = (sl - sh["rows"]) // 16
        last = (sl - 1) // 16
        bt[b, first:last + 1] = perm[b * per:b * per + (last - first + 1)]
    T = int(q_lens.sum())
    x = rng.standard_normal((2, T, sh["hkv"], sh["head_dim"])).astype(np.float32)
    scale = rng.uniform(0.01, 0.05, (2, sh["hkv"])).astype(np.float32)
    return seq_lens, q_lens, bt, pages, x, scale


def measure_append(steps: int, warmup: int, use_graph: bool = True):
    import numpy as np
    import torch

    import paged_attention_long_amd as pal

    sh = APPEND_SHAPE
    seq_lens, q_lens, bt, pages, x, scale = _append_inputs()
    T = int(q_lens.sum())
    dev = torch.device("cuda")
    kn = torch.from_numpy(x[0]).to(dev).to(torch.bfloat16).contiguous()
    vn = torch.from_numpy(x[1]).to(dev).to(torch.bfloat16).contiguous()
    kc = torch.zeros((pages, sh["hkv"], 16, sh["head_dim"]), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    d_bt, d_sl, d_ql = (torch.from_numpy(a).to(dev) for a in (bt, seq_lens, q_lens))
    d_sc = torch.from_numpy(scale.reshape(-1)).to(dev)
    cfg = pal.make_config(sh["hkv"] * 4, sh["hkv"], sh["head_dim"], "bf16", "fp8_e4m3", sh["num_seqs"], sh["rows"], T)
    h = pal.paged_attn_create(cfg)
    stream = torch.cuda.current_stream()

    def step(st=None):
        pal.paged_attn_append(h, kn, vn, kc, vc, d_bt, d_sl, d_ql, d_sc, stream=st or stream)

    try:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(); [step() for _ in range(steps)]; e1.record(); torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / steps
        us = eager_us
        timing = "eager launches"
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(steps):
                    step(torch.cuda.current_stream())
            g.replay(); torch.cuda.synchronize()
            e0.record(); g.replay(); e1.record(); torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            timing = "graph replay of the timed steps"
    finally:
        pal.paged_attn_destroy(h)
    nbytes = 2 * T * sh["hkv"] * sh["head_dim"] * (2 + 1)     # read the 16-bit rows, write the fp8 codes
    gbs = nbytes / us / 1e3
    print(f"[bench] append_fp8: {gbs:.1f} GB/s ({timing}), {us:.2f} us per call = {100 * gbs / HBM_PEAK_GBS:.1f}% of peak",
          file=sys.stderr, flush=True)
    res = {
        "value": gbs, "unit": "GB/s", "ms_per_step": us / 1e3, "dtype": "bf16 in / fp8 e4m3 out",
        "kv_bytes_per_step": nbytes, "flops_per_step": 0, "rotating_copies": 1,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "scope": "one append call (new K and V rows read, fp8 codes written)"},
        "timing": timing, "forward_us": {"events": us, "eager_events": eager_us},
        "eager_value": nbytes / eager_us / 1e3, "forwards_run": warmup + steps * (2 if use_graph else 1) + 1,
    }
    return res, (seq_lens, q_lens, bt, pages, x, scale)


def cpu_baseline_append(base):
    """The oracle's append on the host cores, on the first sequences' rows."""
    import numpy as np

    import oracle

    seq_lens, q_lens, bt, pages, x, scale = base
    sh = APPEND_SHAPE
    bits = np.stack([x[w].astype(np.float32) for w in range(2)])
    import torch
    b16 = torch.from_numpy(bits).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pool = np.zeros((pages, sh["hkv"], 16, sh["head_dim"]), dtype=np.uint8)
    n_seq = 2
    rows = n_seq * sh["rows"]
    t0 = time.time()
    reps = 0
    while True:
        oracle.append_kv(b16[0, :rows], b16[1, :rows], "bf16", pool, pool, "fp8_e4m3", bt[:n_seq], seq_lens[:n_seq],
                         q_lens[:n_seq], scale, 16)
        reps += 1
        if time.time() - t0 > 10:
            break
    sec = time.time() - t0
    nbytes = reps * 2 * rows * sh["hkv"] * sh["head_dim"] * 3
    return {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows of {n_seq} sequences, {reps} repetitions", "seconds": sec}


def profile_commands(workload: str, calib_mib: int = 512) -> list:
    """The rocprofv3 runs behind profiles/<kernel>_<workload>.md, from the
    repository root $REPO (counters in passes of their own, as the profiler
    collects them)."""
    out = f"$REPO/gpurun_out/prof/{workload}"
    run = f"python3 $REPO/bench.py --workload {workload} --no-cpu-baseline"
    return [
        "cd /tmp && export TMPDIR=/tmp",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/kt -o run -- "
        f"{run} --steps 50 --warmup 5 --json-out {out}/kt/bench.json",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- "
        f"{run} --steps 5 --warmup 1 --eager --calibrate-copy {calib_mib} --json-out {out}/fetch/bench.json",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- "
        f"{run} --steps 5 --warmup 1 --eager --calibrate-copy {calib_mib} --json-out {out}/write/bench.json",
        f"python3 bench.py --workload {workload} --reduce-profiles gpurun_out/prof/{workload}   # on any host",
    ]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="also measure every other workload (per_config)")
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no graph replay)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a copy kernel of known size (for counter scaling)")
    ap.add_argument("--profile-commands", action="store_true", help="print the rocprofv3 commands and exit")
    ap.add_argument("--reduce-profiles", default=None, metavar="DIR",
                    help="summarise the rocprofv3 runs in DIR into profiles/ (no GPU needed)")
    ap.add_argument("--json-out", default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.profile_commands:
        print("\n".join(profile_commands(args.workload)))
        return
    if args.reduce_profiles:
        reduce_profiles(args.reduce_profiles, args.workload, 512, profile_commands(args.workload))
        return

    import torch

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
    if args.workload == "append_fp8":
        res, base = measure_append(args.steps, args.warmup, use_graph=not args.eager)
    else:
        res, base = measure(args.workload, args.steps, args.warmup, use_graph=not args.eager)
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "name": args.workload,
                   "kv_bytes_per_step": res["kv_bytes_per_step"], "flops_per_step": res["flops_per_step"],
                   "rotating_copies": res["rotating_copies"], "parallelism": "single GPU"},
        "roofline": res["roofline"], "timing": res["timing"], "forward_us": res["forward_us"],
        "eager_value": res["eager_value"], "forwards_run": res["forwards_run"],
    }
    if args.all:
        per = {}
        for w in ("decode", "verify", "verify_window", "prefill", "mixed_fp8"):
            if w == args.workload:
                continue
            try:
                r, _ = measure(w, max(20, args.steps // 4), max(5, args.warmup // 2), use_graph=not args.eager)
                per[w] = {"value": r["value"], "unit": r["unit"], "roofline": r["roofline"],
                          "forward_us": r["forward_us"], "eager_value": r["eager_value"]}
            except Exception as e:  # report, do not hide
                per[w] = {"error": repr(e)}
        line["per_config"] = per
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline_append(base) if args.workload == "append_fp8"
                                else cpu_baseline(args.workload, base))
    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()

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
    "prefill_d256": "chunked prefill at head_dim 256: 2,048-token chunk on 65,536 cached, 16/2 heads, bf16 KV",
    "mixed_fp8": "mixed batch: 4 seqs, 200,001/131,076/32,776/4,097 tokens, q_len 1/4/8/1, 32/8 heads, fp8 e4m3 KV",
    "mixed_int8": "mixed batch as mixed_fp8 on an int8 KV cache with a fp32 scale per cached row",
    "prefill_int8": "chunked prefill on an int8 KV cache (fp32 row scales): 2,048-token chunk on 65,536 cached, 24/4 heads, D 128",
    "append_fp8": "cache append: 64 seqs x 256 new rows, 8 KV heads, D 128, bf16 rows quantised into fp8 e4m3 pages",
}
# inputs as stored; every product is accumulated, and every softmax step computed, in fp32
DTYPE_NAME = {"f16": "f16 in / f32 accumulate", "bf16": "bf16 in / f32 accumulate",
              "fp8_e4m3": "fp8_e4m3 kv, bf16 q / f32 accumulate",
              "int8": "int8 kv (fp32 row scales), bf16 q / f32 accumulate"}


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


PATHS = {"auto": 0, "valu": 1, "mfma": 2}
# Workloads measured on the VALU path as well as on the automatic (MFMA tile) one.
ALT_PATH_WORKLOADS = ("verify", "mixed_fp8")
# workloads measured in TFLOP/s against the bf16 MFMA peak (the rest: KV bytes against HBM)
FLOP_WORKLOADS = ("prefill", "prefill_d256", "prefill_int8")
# Timed regions per measurement: the median is reported, and the spread
# (max - min) / median across them ("run it three times, watch the drift").
REPEATS = 3
WARM_REPLAYS = 3   # untimed replays of the captured graph before the timed ones (clocks settle) ...
WARM_SECONDS = 0.2  # ... for at least this long (a cold GPU ramps its clock over tens of milliseconds)


class Prepared:
    """One workload's inputs on the device: rotating copies of the batch at
    disjoint physical pages in one pool."""

    def __init__(self, workload: str):
        import torch

        from synth import named
        from synth.gen import replicate
        from synth.torch_upload import upload_batch, upload_pool

        t0 = time.time()
        self.workload = workload
        self.base = named(workload)[0]
        self.kv_bytes = self.base.kv_bytes()
        self.flops = self.base.flops()
        self.copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / self.kv_bytes)))
        batches = replicate(self.base, self.copies, seed=1)
        self.pools = upload_pool(batches)
        self.devs = [upload_batch(b) for b in batches]
        b = self.base
        self.out = torch.empty((b.num_tokens, b.num_q_heads, b.head_dim), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((b.num_tokens, b.num_q_heads), dtype=torch.float32, device="cuda")
        log(f"[bench] {workload}: inputs ready in {time.time() - t0:.1f}s ({self.copies} rotating copies, "
            f"{self.kv_bytes / 1e6:.2f} MB KV per step)")

    def handle(self, path: str = "auto"):
        import paged_attention_long_amd as pal

        b = self.base
        pos = b.q_lens[b.q_lens > 0]
        cfg = pal.make_config(b.num_q_heads, b.num_kv_heads, b.head_dim, b.q_dtype, b.kv_dtype, b.num_seqs,
                              int(b.q_lens.max()), b.num_tokens, min_q_len=int(pos.min()))
        h = pal.paged_attn_create(cfg)
        if path != "auto":
            pal.paged_attn_set_tuning(h, path=PATHS[path])
        return h

    def step(self, h, i: int):
        import torch

        import paged_attention_long_amd as pal

        d = self.devs[i % self.copies]
        ksc = self.pools["row_scale"] if "row_scale" in self.pools else d["kv_scale"]
        pal.paged_attn_forward(h, d["q"], self.pools["k"], self.pools["v"], d["block_table"], d["seq_lens"],
                               d["q_lens"], self.base.window, self.base.scale, ksc, self.out, self.lse,
                               stream=torch.cuda.current_stream())

    def free(self):
        import torch

        self.pools = self.devs = self.out = self.lse = None
        torch.cuda.empty_cache()


def _timed(fn):
    """Wall clock and HIP-event time of fn(), synchronised on both sides; the
    events are recorded on the stream the forwards are launched on."""
    import torch

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - w0, e0.elapsed_time(e1) * 1e-3


def time_path(prep: Prepared, path: str, steps: int, warmup: int, repeats: int = REPEATS, graph: bool = True):
    """Warm-up forwards, one eager timed region, then `repeats` timed replays
    of a HIP graph holding `steps` forwards (no host launch cost between
    them); with graph=False, `repeats` eager timed regions instead.  Returns
    per-forward times in microseconds."""
    import torch

    import paged_attention_long_amd as pal

    h = prep.handle(path)
    try:
        for i in range(warmup):
            prep.step(h, i)
        torch.cuda.synchronize()
        eager_wall, eager_ev = _timed(lambda: [prep.step(h, warmup + i) for i in range(steps)])
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    prep.step(h, i)
            warm = 0
            t_warm = time.perf_counter()
            while warm < WARM_REPLAYS or time.perf_counter() - t_warm < WARM_SECONDS:
                g.replay()
                torch.cuda.synchronize()
                warm += 1
            runs = [_timed(g.replay) for _ in range(repeats)]
            del g
        else:
            runs = [(eager_wall, eager_ev)] + [
                _timed(lambda: [prep.step(h, i) for i in range(steps)]) for _ in range(repeats - 1)]
    finally:
        pal.paged_attn_destroy(h)
    assert torch.isfinite(prep.out).all().item(), f"{prep.workload}/{path}: non-finite output"
    walls = sorted(w / steps * 1e6 for w, _ in runs)
    evs = [e / steps * 1e6 for _, e in runs]
    ev_sorted = sorted(evs)
    med_ev = ev_sorted[len(ev_sorted) // 2]
    return {
        "path": path,
        "graph_event_us": med_ev,
        "graph_event_runs_us": evs,
        "graph_wall_us": walls[len(walls) // 2],
        "spread": (ev_sorted[-1] - ev_sorted[0]) / med_ev,
        "eager_event_us": eager_ev / steps * 1e6,
        "eager_wall_us": eager_wall / steps * 1e6,
        "timing": "graph replay of the timed steps" if graph else "eager launches",
        "forwards_run": warmup + steps + steps * (warm + repeats) if graph else warmup + steps * repeats,
    }


def rates(prep: Prepared, t: dict) -> dict:
    """Throughput and roofline of one timing (prefill in TFLOP/s against the
    bf16 MFMA peak, the others in KV GB/s against HBM)."""
    if prep.workload in FLOP_WORKLOADS:
        work, unit, peak, bound, scale = prep.flops, "TFLOP/s", BF16_MFMA_PEAK_TFS, "mfma", 1e-6
    else:
        work, unit, peak, bound, scale = prep.kv_bytes, "GB/s", HBM_PEAK_GBS, "hbm", 1e-3
    value = work / t["graph_wall_us"] * scale
    achieved = work / t["graph_event_us"] * scale
    return {
        "value": value, "unit": unit,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                     "traffic": load_traffic(prep.workload),
                     "scope": "one forward (every kernel it launches), HIP events on the launch stream over "
                              f"the timed region ({t['timing']}) / steps, median of the repeats"},
        "eager_value": work / t["eager_wall_us"] * scale,
    }


def measure(workload: str, steps: int, warmup: int, paths=("auto",), repeats: int = REPEATS, graph: bool = True):
    prep = Prepared(workload)
    try:
        res = {}
        for path in paths:
            t = time_path(prep, path, steps, warmup, repeats, graph)
            r = rates(prep, t)
            r["timing"] = t
            res[path] = r
            log(f"[bench] {workload}/{path}: {r['value']:.1f} {r['unit']} ({t['timing']}, wall); "
                f"{t['graph_event_us']:.2f} us per forward (events, median of {repeats}, spread "
                f"{100 * t['spread']:.2f}%) -> {r['roofline']['frac'] * 100:.1f}% of peak")
        return res, prep.base
    finally:
        prep.free()


def cpu_baseline(workload: str, base, budget_s: float = 10.0):
    """The fp64 oracle, unmodified, on this host: full attention of the
    workload's batch (decode-sized workloads) or all rows of some query heads
    (larger ones, scaled by the head count), repeated until the budget is
    spent.  cores: the CPUs this process may run on; blas_threads: the
    threads numpy's BLAS uses."""
    import numpy as np

    import oracle

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    kv_bytes = base.kv_bytes()
    t0 = time.perf_counter()
    reps = 0
    common = {"cores": cores, "blas_threads": blas, "kind": "oracle"}
    if workload in ("tiny_decode", "decode", "verify_window"):
        while True:
            oracle.attention(base)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        sample = f"full {workload} batch (all {base.num_tokens * base.num_q_heads} rows), {reps} repetitions"
        return {"value": kv_bytes * reps / el / 1e9, "unit": "GB/s", **common, "sample": sample, "seconds": el}
    # Larger workloads: all tokens of one query head at a time, scaled by the head count.
    Hk, G = base.num_kv_heads, base.group
    cu = np.concatenate([[0], np.cumsum(base.q_lens)])
    toks = [t for b in range(base.num_seqs) for t in range(int(cu[b]), int(cu[b + 1]))]
    done_heads = 0
    while True:
        g = done_heads % Hk
        hh = g * G + (done_heads // Hk) % G
        oracle.attention_rows(base, [(t, hh) for t in toks])
        done_heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    frac = done_heads / base.num_q_heads
    sample = f"all tokens of {done_heads} query head(s) of {base.num_q_heads}; scaled by heads"
    if workload in FLOP_WORKLOADS:
        return {"value": base.flops() * frac / el / 1e12, "unit": "TFLOP/s", **common, "sample": sample,
                "seconds": el}
    return {"value": kv_bytes * frac / el / 1e9, "unit": "GB/s", **common, "sample": sample, "seconds": el}


# ------------------------------------------------------------------ kernel trace of the replayed forwards
MARKER_TAG = "bitwise_not"     # a torch kernel launched between workloads in the traced child run


def _marker():
    import torch

    x = torch.zeros(64, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    x.bitwise_not_()
    torch.cuda.synchronize()


def trace_child(workloads, steps: int, warmup: int, replays: int) -> None:
    """Runs inside rocprofv3 --kernel-trace: per workload, warm-up forwards,
    untimed replays of a graph of `steps` forwards for at least WARM_SECONDS
    (as in the timed runs, so the clock has settled), then a marker kernel,
    `replays` replays of the graph, and a marker again, so the replayed
    dispatches can be told apart."""
    import torch

    import paged_attention_long_amd as pal

    for w in workloads:
        prep = Prepared(w)
        h = prep.handle("auto")
        try:
            for i in range(warmup):
                prep.step(h, i)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    prep.step(h, i)
            torch.cuda.synchronize()
            t_warm = time.perf_counter()
            while time.perf_counter() - t_warm < WARM_SECONDS:
                g.replay()
                torch.cuda.synchronize()
            _marker()
            for _ in range(replays):
                g.replay()
            torch.cuda.synchronize()
            _marker()
            del g
        finally:
            pal.paged_attn_destroy(h)
            prep.free()
        log(f"[bench] traced {w}: {replays} x {steps} replayed forwards")


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def parse_kernel_trace(csv_path: str, workloads, forwards: int) -> dict:
    """Per workload, the replayed dispatches between its two markers: per
    kernel the dispatches per forward and the median duration; the kernel
    time of one forward and its dominant kernel."""
    import csv

    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows)
    marks = [i for i, e in enumerate(ev) if MARKER_TAG in e[2]]
    if len(marks) != 2 * len(workloads):
        raise RuntimeError(f"expected {2 * len(workloads)} marker dispatches, found {len(marks)}")
    out = {}
    for k, w in enumerate(workloads):
        # the library's kernels only (the markers' own fill kernels fall in between)
        seg = [e for e in ev[marks[2 * k] + 1:marks[2 * k + 1]] if any(t in e[2] for t in OUR_KERNEL_TAGS)]
        per = {}
        for s0, s1, name in seg:
            per.setdefault(_short(name), []).append((s1 - s0) * 1e-3)
        kern = {n: {"per_forward": len(d) / forwards, "median_us": _median(d), "min_us": min(d), "max_us": max(d)}
                for n, d in per.items()}
        total = sum(v["median_us"] * v["per_forward"] for v in kern.values())
        dom = max(kern, key=lambda n: kern[n]["median_us"] * kern[n]["per_forward"]) if kern else None
        out[w] = {"kernels": kern, "kernel_us_per_forward": total, "dominant": dom}
    return out


def kernel_trace(workloads, steps: int = 10, warmup: int = 3, replays: int = 5, timeout_s: int = 300):
    """Runs this file under rocprofv3 --kernel-trace in a child process (the
    profiler runs the program itself, after --) and returns the parsed
    replayed-dispatch durations, or {"error": ...}."""
    import glob
    import shutil
    import subprocess
    import tempfile

    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(prof):
        return {"error": "rocprofv3 not found"}
    tmp = tempfile.mkdtemp(prefix="pa_ktrace_", dir="/tmp")
    cmd = [prof, "--kernel-trace", "--output-format", "csv", "-d", tmp, "-o", "run", "--",
           sys.executable, os.path.abspath(__file__), "--trace-child", ",".join(workloads), "--steps", str(steps),
           "--warmup", str(warmup), "--replays", str(replays)]
    env = dict(os.environ, TMPDIR="/tmp")
    t0 = time.time()
    try:
        r = subprocess.run(cmd, cwd="/tmp", env=env, timeout=timeout_s, stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        rc = r.returncode
        tail = r.stdout[-2000:]
    except subprocess.TimeoutExpired:
        return {"error": f"rocprofv3 child timed out after {timeout_s}s"}
    files = glob.glob(os.path.join(tmp, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return {"error": f"no kernel trace (rocprofv3 rc {rc})", "tail": tail}
    try:
        res = parse_kernel_trace(files[0], workloads, steps * replays)
    except Exception as e:  # report, do not hide
        return {"error": repr(e), "rc": rc}
    shutil.rmtree(tmp, ignore_errors=True)
    log(f"[bench] kernel trace of {len(workloads)} workloads in {time.time() - t0:.1f}s (rocprofv3 rc {rc})")
    return {"command": "rocprofv3 --kernel-trace --output-format csv -- python3 bench.py --trace-child "
                       f"{','.join(workloads)} --steps {steps} --warmup {warmup} --replays {replays}",
            "profiler_rc": rc, "replayed_forwards": steps * replays, "workloads": res}


def kernel_roofline(prep_like: dict, tr: dict) -> dict:
    """Roofline of the dominant kernel from its replayed-dispatch median, and
    the kernel-only time of the whole forward."""
    dom = tr["dominant"]
    k = tr["kernels"][dom]
    work, unit, peak, scale = prep_like["work"], prep_like["unit"], prep_like["peak"], prep_like["scale"]
    return {"kernel": dom, "median_us": k["median_us"], "per_forward": k["per_forward"],
            "achieved": work / (k["median_us"] * k["per_forward"]) * scale, "unit": unit, "peak": peak,
            "frac": work / (k["median_us"] * k["per_forward"]) * scale / peak,
            "forward_kernels_us": tr["kernel_us_per_forward"],
            "forward_kernels_frac": work / tr["kernel_us_per_forward"] * scale / peak}


COPY_KERNEL_TAG = "neg_kernel"     # torch.neg: reads N bytes, writes N bytes
OUR_KERNEL_TAGS = ("decode_valu_kernel", "tile_attn_kernel", "tile256_kernel", "merge_kernel", "merge_row_kernel",
                   "merge_slots_kernel",
                   "append_kernel", "zero_words_kernel")


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
    if workload == "append_fp8":
        sh = APPEND_SHAPE   # 16-bit rows read, fp8 codes written, K and V
        alg = 2 * sh["num_seqs"] * sh["rows"] * sh["hkv"] * sh["head_dim"] * 3
    else:
        from synth import named

        base = named(workload)[0]
        alg = base.flops() if workload in FLOP_WORKLOADS else base.kv_bytes()
    hbm = 0.0
    for k, v in kern.items():
        v["per_forward"] = v["dispatches"] / max(1, fetch_run["forwards_run"])
        v["hbm_bytes"] = v["fetch_kib"] * 1024 * f_scale + v["write_kib"] * 1024 * w_scale
        hbm += v["hbm_bytes"] * v["per_forward"]
    lines = [f"# {', '.join(kern) or 'kernels'}: {workload}", "",
             f"Workload: {WORKLOADS[workload]}.", "", "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    # The timed graph replays are the last steps x repeats dispatches of each
    # kernel in the traced run (warm-up and eager dispatches come first).
    trace_rows = _csv_rows(os.path.join(prof_dir, "kt", "**", "*kernel_trace.csv"))
    replayed = n_fwd.get("steps", 0) * n_fwd.get("repeats", REPEATS)
    by_kernel = collections.defaultdict(list)
    for r in sorted(trace_rows, key=lambda r: int(r["Start_Timestamp"])):
        if any(t in r["Kernel_Name"] for t in OUR_KERNEL_TAGS):
            by_kernel[_short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "All dispatches of the run (warm-up, eager and replayed forwards):", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if any(t in r["Name"] for t in OUR_KERNEL_TAGS):
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    if replayed and by_kernel:
        lines += ["", f"The timed graph replays only (the last {replayed} dispatches of each kernel):", "",
                  "| kernel | dispatches | median us | average us | min us | max us |", "|---|---|---|---|---|---|"]
        for k, d in sorted(by_kernel.items()):
            d = d[-replayed:]
            lines.append(f"| {k} | {len(d)} | {_median(d):.2f} | {sum(d) / len(d):.2f} | {min(d):.2f} | "
                         f"{max(d):.2f} |")
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
    unit = "flop" if workload in FLOP_WORKLOADS else "B of KV"
    lines += ["", f"HBM bytes per forward: {hbm:.4g}; algorithmic {alg:.4g} {unit} per forward"
              + ("" if workload in FLOP_WORKLOADS else f" (ratio {hbm / alg:.3f})") + ".", ""]
    trace_avg = {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
    lines += _mfma_summary(prof_dir, trace_avg)
    lines += _valu_summary(prof_dir, trace_avg)
    lines += _issue_summary(prof_dir)
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


def measure_append(steps: int, warmup: int, use_graph: bool = True, repeats: int = REPEATS):
    """Times the cache append over rotating copies: each copy has its own new
    rows and its own page range, about 1 GiB in all, so every call reads its
    rows from HBM and writes pages no recent call touched."""
    import numpy as np
    import torch

    import paged_attention_long_amd as pal

    sh = APPEND_SHAPE
    seq_lens, q_lens, bt, pages, x, scale = _append_inputs()
    T = int(q_lens.sum())
    nbytes = 2 * T * sh["hkv"] * sh["head_dim"] * (2 + 1)     # read the 16-bit rows, write the fp8 codes
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / nbytes)))
    dev = torch.device("cuda")
    kn0 = torch.from_numpy(x[0]).to(dev).to(torch.bfloat16).contiguous()
    vn0 = torch.from_numpy(x[1]).to(dev).to(torch.bfloat16).contiguous()
    kns = [kn0] + [kn0.clone() for _ in range(copies - 1)]
    vns = [vn0] + [vn0.clone() for _ in range(copies - 1)]
    kc = torch.zeros((pages * copies, sh["hkv"], 16, sh["head_dim"]), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    d_bts = [torch.from_numpy(bt + np.int32(c * pages)).to(dev) for c in range(copies)]
    d_sl, d_ql = (torch.from_numpy(a).to(dev) for a in (seq_lens, q_lens))
    d_sc = torch.from_numpy(scale.reshape(-1)).to(dev)
    cfg = pal.make_config(sh["hkv"] * 4, sh["hkv"], sh["head_dim"], "bf16", "fp8_e4m3", sh["num_seqs"], sh["rows"], T)
    h = pal.paged_attn_create(cfg)

    def step(i):
        c = i % copies
        pal.paged_attn_append(h, kns[c], vns[c], kc, vc, d_bts[c], d_sl, d_ql, d_sc,
                              stream=torch.cuda.current_stream())

    try:
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        eager_wall, eager_ev = _timed(lambda: [step(warmup + i) for i in range(steps)])
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    step(i)
            warm = 0
            t_warm = time.perf_counter()
            while warm < WARM_REPLAYS or time.perf_counter() - t_warm < WARM_SECONDS:
                g.replay()
                torch.cuda.synchronize()
                warm += 1
            runs = [_timed(g.replay) for _ in range(repeats)]
            timing = "graph replay of the timed steps"
        else:
            runs = [(eager_wall, eager_ev)] + [_timed(lambda: [step(i) for i in range(steps)])
                                              for _ in range(repeats - 1)]
            timing = "eager launches"
    finally:
        pal.paged_attn_destroy(h)
    evs = sorted(e / steps * 1e6 for _, e in runs)
    walls = sorted(w / steps * 1e6 for w, _ in runs)
    us, wall_us = evs[len(evs) // 2], walls[len(walls) // 2]
    gbs = nbytes / us / 1e3
    log(f"[bench] append_fp8: {nbytes / wall_us / 1e3:.1f} GB/s ({timing}, wall), {us:.2f} us per call "
        f"(events) = {100 * gbs / HBM_PEAK_GBS:.1f}% of peak, {copies} rotating copies")
    res = {
        "value": nbytes / wall_us / 1e3, "unit": "GB/s", "ms_per_step": wall_us / 1e3,
        "dtype": "bf16 in / fp8 e4m3 out", "kv_bytes_per_step": nbytes, "flops_per_step": 0,
        "rotating_copies": copies,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic("append_fp8"),
                     "scope": "one append call (new K and V rows read, fp8 codes written), HIP events"},
        "timing": {"timing": timing, "graph_event_us": us, "graph_event_runs_us": [e / steps * 1e6 for _, e in runs],
                   "spread": (evs[-1] - evs[0]) / us, "eager_event_us": eager_ev / steps * 1e6,
                   "eager_wall_us": eager_wall / steps * 1e6},
        "eager_value": nbytes / (eager_wall / steps * 1e6) / 1e3,
        "forwards_run": warmup + steps + (steps * (warm + repeats) if use_graph else steps * (repeats - 1)),
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
    # elementwise numpy code: one thread does the work whatever the affinity
    return {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": 1, "affinity_cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{rows} rows of {n_seq} sequences, {reps} repetitions", "seconds": sec}


# Counter passes of the MFMA-bound workloads (one rocprofv3 run each).
MFMA_PASSES = (("mfma_util", "MfmaUtil"), ("mfma_raw", "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"),
               ("mfma_mops", "SQ_INSTS_VALU_MFMA_MOPS_BF16"))


VALU_PASS = "SQ_INSTS_VALU SQ_WAVES"

# Issue and wait counters of the MFMA-bound workloads (wave-cycles, in units
# of four cycles as the profiler counts them): where the waves' time goes.
ISSUE_PASSES = (("issue", "SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
                          "SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_MISC"),
                ("lds", "SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT "
                        "SQ_LDS_ADDR_CONFLICT"))


def _issue_summary(prof_dir: str) -> list:
    """Markdown lines for the issue/wait and LDS passes (empty if they were not run)."""
    import collections

    vals = {sub: collections.defaultdict(lambda: collections.defaultdict(list)) for sub, _ in ISSUE_PASSES}
    for sub, _ in ISSUE_PASSES:
        for r in _csv_rows(os.path.join(prof_dir, sub, "**", "*counter_collection.csv")):
            k = _short(r["Kernel_Name"])
            if any(t in k for t in OUR_KERNEL_TAGS):
                vals[sub][k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not any(vals.values()):
        return []
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    lines = ["## Issue and waits (SQ_WAVE_CYCLES, SQ_ACTIVE_INST_*, SQ_WAIT_*; LDS)", "",
             "Per dispatch, averaged over the dispatches of the eager counter runs.  Each share is of the "
             "waves' resident time (SQ_WAVE_CYCLES of the same pass), with the profiler's meanings: issuing "
             "(SQ_ACTIVE_INST_ANY), waiting on a counter or event (SQ_WAIT_ANY), an instruction waiting to "
             "issue (SQ_WAIT_INST_ANY), VALU issue (SQ_ACTIVE_INST_VALU), LDS instructions waiting to issue "
             "(SQ_WAIT_INST_LDS); the shares overlap.  VALU issue slots beyond one per VALU instruction "
             "(SQ_ACTIVE_INST_VALU - SQ_INSTS_VALU) against SQ_INSTS_VALU_TRANS_F32 give the issue slots of "
             "a transcendental.", "",
             "| kernel | wave-cycles (x4) | issuing % | waiting % | instr. waiting % | VALU issue % | "
             "VALU instr. | exp/log instr. | extra VALU slots | LDS instr. | LDS wait % | bank conflicts | "
             "addr. conflicts |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(set(vals["issue"]) | set(vals["lds"])):
        c, d = vals["issue"][k], vals["lds"][k]
        wc, wl = mean(c.get("SQ_WAVE_CYCLES", [])), mean(d.get("SQ_WAVE_CYCLES", []))
        pc = lambda n: 100.0 * mean(c.get(n, [])) / wc
        extra = mean(c.get("SQ_ACTIVE_INST_VALU", [])) - mean(c.get("SQ_INSTS_VALU", []))
        lines.append(f"| {k} | {wc:.4g} | {pc('SQ_ACTIVE_INST_ANY'):.1f} | {pc('SQ_WAIT_ANY'):.1f} | "
                     f"{pc('SQ_WAIT_INST_ANY'):.1f} | {pc('SQ_ACTIVE_INST_VALU'):.1f} | "
                     f"{mean(c.get('SQ_INSTS_VALU', [])):.4g} | {mean(c.get('SQ_INSTS_VALU_TRANS_F32', [])):.4g} | "
                     f"{extra:.4g} | {mean(d.get('SQ_INSTS_LDS', [])):.4g} | "
                     f"{100.0 * mean(d.get('SQ_WAIT_INST_LDS', [])) / wl:.1f} | "
                     f"{mean(d.get('SQ_LDS_BANK_CONFLICT', [])):.4g} | {mean(d.get('SQ_LDS_ADDR_CONFLICT', [])):.4g} |")
    return lines + [""]


def _valu_summary(prof_dir: str, trace_avg_us: dict) -> list:
    """Markdown lines for the VALU instruction pass (empty if it was not run)."""
    import collections

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv_rows(os.path.join(prof_dir, "valu", "**", "*counter_collection.csv")):
        k = _short(r["Kernel_Name"])
        if any(t in k for t in OUR_KERNEL_TAGS):
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not vals:
        return []
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    lines = ["## Vector ALU (SQ_INSTS_VALU, SQ_WAVES)", "",
             "Per dispatch.  A CU issues at most one 64-lane VALU instruction per cycle (four SIMDs, four "
             "cycles each), so the chip's VALU floor is instructions / (256 CUs x the clock); at 2.4 GHz:", "",
             "| kernel | VALU instructions | waves | per wave | VALU floor us at 2.4 GHz | kernel us (trace avg) |",
             "|---|---|---|---|---|---|"]
    for k, c in sorted(vals.items()):
        ins, waves = mean(c.get("SQ_INSTS_VALU", [])), mean(c.get("SQ_WAVES", []))
        lines.append(f"| {k} | {ins:.4g} | {waves:.4g} | {ins / waves:.0f} | {ins / (256 * 2.4e3):.1f} | "
                     f"{trace_avg_us.get(k, float('nan')):.1f} |")
    return lines + [""]


def _mfma_summary(prof_dir: str, trace_avg_us: dict) -> list:
    """Markdown lines for the MFMA counter passes (empty if they were not run)."""
    import collections

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for sub, _ in MFMA_PASSES:
        for r in _csv_rows(os.path.join(prof_dir, sub, "**", "*counter_collection.csv")):
            k = _short(r["Kernel_Name"])
            if any(t in k for t in OUR_KERNEL_TAGS):
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not vals:
        return []
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    lines = ["## Matrix cores (MfmaUtil; SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE; SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
             "Per dispatch, averaged over the dispatches of the eager counter runs.  MfmaUtil is the profiler's "
             "derived counter: MFMA-busy SIMD cycles / (GPU-active cycles x 1,024 SIMDs).  The raw "
             "GRBM_GUI_ACTIVE as the profiler reports it sums the 8 XCDs, so the clock is GRBM_GUI_ACTIVE / "
             "kernel time / 8 (given for the matrix kernels only: over a kernel of a few microseconds the "
             "counter window, dispatch to completion, is longer than the traced kernel time).  Executed "
             "flop = MFMA ops x 512.", "",
             "| kernel | MfmaUtil % | MFMA busy cycles | GPU-active cycles | kernel us (trace avg) | "
             "cycles / us | clock GHz (/ 8 XCDs) | executed TFLOP | executed TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, c in sorted(vals.items()):
        us = trace_avg_us.get(k, float("nan"))
        gui = mean(c.get("GRBM_GUI_ACTIVE", []))
        fl = mean(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])) * 512
        clk = f"{gui / us:.1f} | {gui / us / 8e3:.2f}" if fl > 0 else "n/a | n/a"
        lines.append(f"| {k} | {mean(c.get('MfmaUtil', [])):.1f} | {mean(c.get('SQ_VALU_MFMA_BUSY_CYCLES', [])):.4g} | "
                     f"{gui:.4g} | {us:.1f} | {clk} | {fl / 1e12:.4f} | {fl / us / 1e6:.1f} |")
    return lines + [""]


def profile_commands(workload: str, calib_mib: int = 512) -> list:
    """The rocprofv3 runs behind profiles/<kernel>_<workload>.md, from the
    repository root $REPO (counters in passes of their own, as the profiler
    collects them)."""
    out = f"$REPO/gpurun_out/prof/{workload}"
    run = (f"python3 $REPO/bench.py --workload {workload} --no-cpu-baseline --no-per-config --no-kernel-trace "
           f"--path auto")
    return [
        "cd /tmp && export TMPDIR=/tmp",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/kt -o run -- "
        f"{run} --steps 50 --warmup 5 --json-out {out}/kt/bench.json",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- "
        f"{run} --steps 5 --warmup 1 --repeats 1 --eager --calibrate-copy {calib_mib} --json-out {out}/fetch/bench.json",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- "
        f"{run} --steps 5 --warmup 1 --repeats 1 --eager --calibrate-copy {calib_mib} --json-out {out}/write/bench.json",
    ] + ([
        # matrix-core utilisation of the prefill kernels: the profiler's MfmaUtil
        # (MFMA-busy SIMD cycles over GPU-active cycles x SIMDs), the raw busy
        # and GPU-active cycles, and the bf16 MFMA operations (512 flop each);
        # then the waves' issue and wait cycles and the LDS counters
        f"rocprofv3 --pmc {ctrs} --output-format csv -d {out}/{sub} -o run -- "
        f"{run} --steps 5 --warmup 1 --repeats 1 --eager --json-out {out}/{sub}/bench.json"
        for sub, ctrs in MFMA_PASSES + ISSUE_PASSES] if workload in FLOP_WORKLOADS else []) + ([
        # the append's vector-ALU instruction count (its limiter)
        f"rocprofv3 --pmc {VALU_PASS} --output-format csv -d {out}/valu -o run -- "
        f"{run} --steps 5 --warmup 1 --repeats 1 --eager --json-out {out}/valu/bench.json"
    ] if workload == "append_fp8" else []) + [
        f"python3 bench.py --workload {workload} --reduce-profiles gpurun_out/prof/{workload}   # on any host",
    ]


# Per-configuration entries of the default run: steps sized so each timed
# region lasts a few milliseconds.
PER_CONFIG = {"tiny_decode": 300, "decode": 200, "verify": 60, "verify_window": 200, "prefill": 20,
              "mixed_int8": 20, "prefill_d256": 20, "prefill_int8": 10}
CPU_BUDGET_HEADLINE_S = 10.0
CPU_BUDGET_PER_CONFIG_S = 3.0


def _entry(workload: str, res: dict, base, trace: dict, cpu: dict = None) -> dict:
    auto = res["auto"]
    t = auto["timing"]
    e = {"value": auto["value"], "unit": auto["unit"], "path": "auto", "roofline": auto["roofline"],
         "forward_us": {"graph_event_median": t["graph_event_us"], "graph_event_runs": t["graph_event_runs_us"],
                        "spread": t["spread"], "graph_wall_median": t["graph_wall_us"],
                        "eager_events": t["eager_event_us"], "eager_wall": t["eager_wall_us"]},
         "eager_value": auto["eager_value"], "kv_bytes_per_step": base.kv_bytes(), "flops_per_step": base.flops()}
    tr = (trace or {}).get("workloads", {}).get(workload)
    if tr:
        work = base.flops() if workload in FLOP_WORKLOADS else base.kv_bytes()
        unit = e["unit"]
        peak = BF16_MFMA_PEAK_TFS if workload in FLOP_WORKLOADS else HBM_PEAK_GBS
        e["roofline"] = dict(e["roofline"], kernel=kernel_roofline(
            {"work": work, "unit": unit, "peak": peak, "scale": 1e-6 if workload in FLOP_WORKLOADS else 1e-3}, tr),
            kernels=tr["kernels"])
    for path, r in res.items():
        if path != "auto":
            e.setdefault("alt_paths", {})[path] = {
                "value": r["value"], "unit": r["unit"], "frac": r["roofline"]["frac"],
                "forward_us": {"graph_event_median": r["timing"]["graph_event_us"], "spread": r["timing"]["spread"]}}
    if cpu is not None:
        e["cpu_baseline"] = cpu
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=REPEATS, help="timed regions per measurement (median, spread)")
    ap.add_argument("--workload", default="mixed_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-per-config", action="store_true",
                    help="headline workload only (the default run also measures every other config)")
    ap.add_argument("--no-kernel-trace", action="store_true", help="skip the rocprofv3 kernel-trace child run")
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no graph replay)")
    ap.add_argument("--path", default=None, choices=sorted(PATHS),
                    help="time this path only (default: auto, plus valu for verify and mixed_fp8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a copy kernel of known size (for counter scaling)")
    ap.add_argument("--profile-commands", action="store_true", help="print the rocprofv3 commands and exit")
    ap.add_argument("--reduce-profiles", default=None, metavar="DIR",
                    help="summarise the rocprofv3 runs in DIR into profiles/ (no GPU needed)")
    ap.add_argument("--trace-child", default=None, metavar="WORKLOADS", help=argparse.SUPPRESS)
    ap.add_argument("--replays", type=int, default=5, help=argparse.SUPPRESS)
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
    if args.trace_child:
        trace_child(args.trace_child.split(","), args.steps, args.warmup, args.replays)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
    w = args.workload
    if w == "append_fp8":
        head, base = measure_append(args.steps, args.warmup, use_graph=not args.eager, repeats=args.repeats)
        t = head["timing"]
        line = {
            "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
            "config": {"workload": WORKLOADS[w], "name": w, "kv_bytes_per_step": head["kv_bytes_per_step"],
                       "rotating_copies": head["rotating_copies"], "parallelism": "single GPU"},
            "roofline": head["roofline"], "timing": t["timing"], "forward_us": t,
            "eager_value": head["eager_value"], "forwards_run": head["forwards_run"],
        }
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_append(base)
        _emit(line, args.json_out)
        return

    per_config = (w == "mixed_fp8") and not args.no_per_config and not args.eager
    if args.path:
        paths = (args.path,)
    else:
        paths = ("auto", "valu") if (w in ALT_PATH_WORKLOADS and not args.eager) else ("auto",)
    res, base = measure(w, args.steps, args.warmup, paths, args.repeats, graph=not args.eager)
    if "auto" not in res:
        res = {"auto": res[paths[0]]}
    auto = res["auto"]
    t = auto["timing"]
    kinds = {"f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3", "int8": "int8"}
    line = {
        "metric": METRIC, "value": auto["value"], "unit": auto["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t["graph_wall_us"] / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[kinds[base.kv_dtype]], "data": "synthetic",
        "config": {"workload": WORKLOADS[w], "name": w, "kv_bytes_per_step": base.kv_bytes(),
                   "flops_per_step": base.flops(), "parallelism": "single GPU", "path": paths[0]},
        "roofline": auto["roofline"], "timing": t["timing"],
        "forward_us": {"graph_event_median": t["graph_event_us"], "graph_event_runs": t["graph_event_runs_us"],
                       "spread": t["spread"], "graph_wall_median": t["graph_wall_us"],
                       "eager_events": t["eager_event_us"], "eager_wall": t["eager_wall_us"]},
        "eager_value": auto["eager_value"], "forwards_run": t["forwards_run"], "repeats": args.repeats,
    }
    line["config"]["rotating_copies"] = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / base.kv_bytes())))
    cpu_budget = CPU_BUDGET_HEADLINE_S
    per, bases = {}, {}
    if per_config:
        for pw, steps in PER_CONFIG.items():
            try:
                r, b = measure(pw, steps, max(5, args.warmup),
                               ("auto", "valu") if pw in ALT_PATH_WORKLOADS else ("auto",), args.repeats)
                per[pw], bases[pw] = r, b
            except Exception as e:  # report, do not hide
                per[pw] = {"error": repr(e)}
    trace = None
    if not args.no_kernel_trace and not args.eager:
        # The first workload a profiled process traces runs its kernels
        # slower than later ones, warm-up replays notwithstanding (the mixed
        # batch's tile kernel: 134.7-137.7 us median when traced first, 126.6 us
        # after the 257-token decode, as in its own profile run), so the
        # 257-token decode, a few milliseconds of work, always leads.
        traced = [w] + [pw for pw in per if "error" not in per[pw]]
        trace = kernel_trace(["tiny_decode"] + [x for x in traced if x != "tiny_decode"])
        line["kernel_trace"] = {k: v for k, v in trace.items() if k != "workloads"}
        if "error" in trace:
            log(f"[bench] kernel trace failed: {trace['error']}")
    head = _entry(w, res, base, trace)
    line["roofline"] = head["roofline"]
    if "alt_paths" in head:
        line["alt_paths"] = head["alt_paths"]
    if per_config:
        line["per_config"] = {}
        for pw, r in per.items():
            if "error" in r:
                line["per_config"][pw] = r
                continue
            cpu = None if args.no_cpu_baseline else cpu_baseline(pw, bases[pw], CPU_BUDGET_PER_CONFIG_S)
            line["per_config"][pw] = dict(_entry(pw, r, bases[pw], trace, cpu), config=WORKLOADS[pw],
                                          steps=PER_CONFIG[pw])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, base, cpu_budget)
    _emit(line, args.json_out)


def _emit(line: dict, json_out) -> None:
    text = json.dumps(line)
    print(text, flush=True)
    if json_out:
        os.makedirs(os.path.dirname(os.path.abspath(json_out)), exist_ok=True)
        with open(json_out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()

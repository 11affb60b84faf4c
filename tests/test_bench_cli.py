"""Host-side checks of bench.py's contract (no GPU): one GPU only, the
profiler passes it prints, and the HBM-traffic figure it reports only while
the committed counters match the kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("workload", sorted(bench.WORKLOADS))
def test_profile_commands_keep_counters_and_traces_apart(workload):
    cmds = bench.profile_commands(workload)
    prof = [c for c in cmds if c.startswith("rocprofv3")]
    mfma = workload in bench.FLOP_WORKLOADS
    valu = workload == "append_fp8"
    n_mfma = len(bench.MFMA_PASSES) + len(bench.ISSUE_PASSES)
    assert len(prof) == 3 + (n_mfma if mfma else 0) + (1 if valu else 0)
    trace, fetch, write = prof[:3]
    assert "--kernel-trace" in trace and "--stats" in trace and "--pmc" not in trace
    passes = [(fetch, "FETCH_SIZE"), (write, "WRITE_SIZE")]
    if mfma:
        passes += [(c, ctrs) for c, (_, ctrs) in zip(prof[3:], bench.MFMA_PASSES + bench.ISSUE_PASSES)]
    if valu:
        passes += [(prof[3], bench.VALU_PASS)]
    for c, counter in passes:
        assert f"--pmc {counter} " in c
        for banned in ("--sys-trace", "--runtime-trace", "--kernel-trace", " -s ", " -r "):
            assert banned not in c
    # at most 8 SQ and 2 GRBM counters in one pass
    for _, ctrs in bench.MFMA_PASSES + bench.ISSUE_PASSES + (("valu", bench.VALU_PASS),):
        names = ctrs.split()
        assert sum(n.startswith("SQ_") for n in names) <= 8 and sum(n.startswith("GRBM_") for n in names) <= 2
    # the program itself follows "--" (no launcher in between)
    for c in prof:
        assert " -- python3 " in c
        assert f"--workload {workload}" in c


def test_traffic_is_dropped_when_kernel_sources_change(monkeypatch):
    real = bench.kernel_source_hash()
    data = bench.load_traffic("decode")
    if data is None:
        pytest.skip("no counter summary for the current kernel sources")
    assert data > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16 if real != "0" * 16 else "1" * 16)
    assert bench.load_traffic("decode") is None


def test_kernel_source_hash_covers_every_source_file(tmp_path, monkeypatch):
    """The hash changes with the text of any file of the library's sources."""
    src = os.path.join(ROOT, "paged_attention_long_amd", "csrc")
    csrc = tmp_path / "paged_attention_long_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in sorted(os.listdir(src)):
        with open(os.path.join(src, name), "rb") as f:
            (csrc / name).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash()
    for name in sorted(os.listdir(csrc)):
        p = csrc / name
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench.kernel_source_hash() != h0, name
        p.write_bytes(orig)
    assert bench.kernel_source_hash() == h0


def test_kernel_trace_parser_takes_dispatches_between_markers(tmp_path):
    """Replayed dispatches are those between each workload's two marker
    kernels; per kernel the median duration and dispatches per forward."""
    rows = [("warm tile_attn_kernel<128, 3, 2, 1>(pa::DecodeArgs)", 0, 500)]
    t = 1000
    names = ["tile_attn_kernel<128, 3, 2, 1>(pa::DecodeArgs)", "merge_row_kernel<128>(pa::MergeArgs)"]
    for w, durs in (("mixed_fp8", (100, 10)), ("decode", (12, 5))):
        rows.append(("void at::native::bitwise_not_kernel(x)", t, t + 1)); t += 10
        for k in range(4):
            for n, d in zip(names, durs):
                rows.append((n, t, t + d * 1000 + k)); t += d * 1000 + 50
        rows.append(("void at::native::bitwise_not_kernel(x)", t, t + 1)); t += 10
    p = tmp_path / "run_kernel_trace.csv"
    with open(p, "w") as f:
        f.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, a, b in rows:
            f.write(f'KERNEL_DISPATCH,"{n}",{a},{b}\n')
    res = bench.parse_kernel_trace(str(p), ["mixed_fp8", "decode"], forwards=4)
    m = res["mixed_fp8"]
    assert m["dominant"] == "tile_attn_kernel<128, 3, 2, 1>"
    assert m["kernels"]["tile_attn_kernel<128, 3, 2, 1>"]["per_forward"] == 1.0
    assert abs(m["kernels"]["tile_attn_kernel<128, 3, 2, 1>"]["median_us"] - 100.0015) < 1e-6
    assert abs(m["kernel_us_per_forward"] - (100.0015 + 10.0015)) < 1e-6
    assert res["decode"]["kernels"]["merge_row_kernel<128>"]["median_us"] < 6


def test_every_launched_kernel_is_recognised():
    """Each kernel the library launches has a tag the trace and counter
    reductions know (an unrecognised one would drop out of the tables)."""
    import re
    names = set()
    for f in os.listdir(os.path.join(ROOT, "paged_attention_long_amd", "csrc")):
        if f.endswith(".hip"):
            src = open(os.path.join(ROOT, "paged_attention_long_amd", "csrc", f)).read()
            names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+_kernel)\s*\(", src))
    names.discard("debug_gather_kernel")   # test-only, never traced
    assert len(names) >= 8, sorted(names)
    for n in names:
        assert any(tag == n for tag in bench.OUR_KERNEL_TAGS), n


def test_default_run_is_the_mixed_batch():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="mixed_fp8"' in src
    assert {"tiny_decode", "decode", "verify", "verify_window", "prefill"} <= set(bench.PER_CONFIG)

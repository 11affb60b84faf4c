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
    assert len(prof) == 3
    trace, fetch, write = prof
    assert "--kernel-trace" in trace and "--stats" in trace and "--pmc" not in trace
    for c, counter in ((fetch, "FETCH_SIZE"), (write, "WRITE_SIZE")):
        assert f"--pmc {counter}" in c
        for banned in ("--sys-trace", "--runtime-trace", "--kernel-trace", " -s ", " -r "):
            assert banned not in c
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

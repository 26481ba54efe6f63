"""Host-side logic of bench.py (no GPU): the one-GPU contract and the counter file's keying."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                       # no JSON line


def test_counters_apply_only_to_the_source_they_were_taken_on(tmp_path, monkeypatch):
    f = tmp_path / "counters.txt"
    f.write_text("# comment: 1\nkernel_source_sha256_16: abcdef0123456789\nhbm_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.counters_traffic("abcdef0123456789") == 12345.0
    assert bench.counters_traffic("0000000000000000") is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.txt"))
    assert bench.counters_traffic("abcdef0123456789") is None


def test_committed_counters_parse_and_exceed_the_algorithmic_bytes():
    """The committed summary names a source hash and a per-launch byte count; the bytes measured
    (reads + writes) cannot be below the launch's algorithmic bytes (65,536 rows x 360 B plus
    2.36 MB of queries)."""
    kv = {}
    for line in open(bench.COUNTERS_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert len(kv["kernel_source_sha256_16"]) == 16
    assert float(kv["hbm_bytes_per_launch"]) >= 65536 * 360 + 32 * 64 * 576 * 2
    assert len(bench.kernel_source_hash()) == 16


def test_timed_steps_are_whole_graphs_whatever_the_step_count():
    """Every timed replay is one multi-step graph: full passes over the rotations, then one graph
    of the remaining steps over the first rotations; the warmup's remainder covers the last
    rotations, so the timed steps do not start on inputs the warmup just read."""
    assert bench._graph_plan(48, 20, False) == [(20, 0)]
    assert bench._graph_plan(48, 960, False) == [(48, 0)] * 20
    assert bench._graph_plan(48, 100, False) == [(48, 0), (48, 0), (4, 0)]
    assert bench._graph_plan(48, 5, True) == [(5, 43)]
    assert bench._graph_plan(48, 96, True) == [(48, 0)] * 2
    assert bench._graph_plan(48, 0, True) == []
    for n in (1, 20, 47, 48, 49, 960, 1000):
        assert sum(k for k, _ in bench._graph_plan(48, n, False)) == n

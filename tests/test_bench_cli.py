"""bench.py's command line without a GPU: the one-GPU rule, argument checks,
and the pure helpers the JSON line is built from."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    e = dict(os.environ, **(env or {}))
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True,
                          text=True, timeout=300, env=e)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2


def test_bad_step_counts_are_refused():
    assert _run("--steps", "0").returncode == 2
    assert _run("--warmup", "-1").returncode == 2


def test_algorithmic_bytes_of_the_large_model():
    sys.path.insert(0, ROOT)
    import bench
    b = bench.algorithmic_bytes(1, 75600, 5120, 2, 256)
    act = 75600 * 5120 * 2
    assert b["fwd"] == 2 * act + 2 * 5120 * 2 + 8 * 75600
    assert b["bwd_fused"] == 3 * act + 5120 * 2 + 8 * 75600 + 2 * 256 * 5120 * 4
    assert b["bwd_finish"] == 2 * 256 * 5120 * 4 + 2 * 5120 * 4
    s = bench.segment_bytes(1000, 3072, 2, 4, 8 * 3072 * 10)
    assert s["fwd"] == 2 * 1000 * 3072 * 2 + 2 * 4 * 3072 * 2 + 8 * 1000


def test_committed_counters_match_the_sources():
    """The committed HBM-traffic records are keyed to the kernel sources;
    bench.py reports them only while the hash matches."""
    sys.path.insert(0, ROOT)
    import bench
    for k in ("fwd", "bwd_fused", "bwd_finish"):
        path = os.path.join(ROOT, "profiles", f"{k}_large_model_pmc.json")
        rec = json.load(open(path))
        assert rec["kernel"] == k and rec["workload"] == "large_model"
        got = bench.load_traffic(k, "large_model", rec["source_hash"])
        assert got == rec["hbm_bytes_per_launch"]
        assert bench.load_traffic(k, "large_model", "0" * 16) is None

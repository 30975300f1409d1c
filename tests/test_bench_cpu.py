"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic byte counts the
roofline entry divides by, and the traffic table's validity rule."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS, ConvShape  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "error" in line


def _touched_brute(s):
    """x elements some forward window reads, counted one by one."""
    seen = set()
    for p in range(s.P):
        for q in range(s.Q):
            for r in range(s.R):
                for t in range(s.S):
                    h, w = p * s.stride[0] - s.pad[0] + r, q * s.stride[1] - s.pad[1] + t
                    if 0 <= h < s.H and 0 <= w < s.W:
                        seen.add((h, w))
    return len(seen) * s.N * s.C


@pytest.mark.parametrize("s", [ConvShape(2, 3, 8, 8, 4, 1, 1, (0, 0), (2, 2), 4, 4),
                               ConvShape(1, 2, 9, 7, 3, 3, 3, (0, 1), (3, 2), 3, 4),
                               ConvShape(1, 1, 10, 10, 1, 2, 2, (0, 0), (4, 4), 3, 3)])
def test_algorithmic_bytes(s):
    """fwd: x elements read once (only those a window touches) + W + y fp32; the backward passes
    read their whole inputs and write their output once."""
    es = 2
    nchw, nkpq, kcrs = s.N * s.C * s.H * s.W, s.N * s.K * s.P * s.Q, s.K * s.C * s.R * s.S
    assert bench.alg_bytes(s, "fwd", es) == _touched_brute(s) * es + kcrs * es + nkpq * 4
    assert bench.alg_bytes(s, "bwd_data", es) == nkpq * es + kcrs * es + nchw * 4
    assert bench.alg_bytes(s, "bwd_filter", es) == _touched_brute(s) * es + nkpq * es + kcrs * 4


def test_traffic_table_matches_the_sources():
    """Every committed traffic entry was taken on the current kernel sources (else the bench would
    report traffic null), and covers every pass of every measured configuration."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    h = bench.source_hash()
    for key, e in t["entries"].items():
        assert e["source_hash"] == h, key
        assert e["bytes_per_launch"] > 0 and e["kernels"], key
    for name, dt in bench.EXTRA_CONFIGS + [("deep3x3", "bf16")]:
        if name == "tiny":
            continue
        for p in WORKLOADS[name].passes:
            assert f"{name}/{dt}/{p}" in t["entries"], (name, dt, p)
            assert bench.stored_traffic(name, dt, p) == t["entries"][f"{name}/{dt}/{p}"]["bytes_per_launch"]
    assert bench.stored_traffic("deep3x3", "f64", "fwd") is None

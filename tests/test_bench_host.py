"""Host logic of bench.py (no GPU): percentiles, the code hash that keys the
recorded byte counters, the records themselves, and the one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_pct_matches_numpy_percentiles():
    xs = [3.0, 1.0, 2.0, 10.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0]
    p = bench.pct(xs)
    assert p["p50"] == np.median(xs)
    assert p["p10"] == np.percentile(xs, 10) and p["p90"] == np.percentile(xs, 90)
    assert bench.pct([]) is None


def test_code_hash_ignores_comments_and_whitespace_only():
    a = 'int f(int x) {  // doubles\n  return 2 * x; /* block\n comment */ }\nconst char* s = "a // b";\n'
    b = 'int f(int x) {\n\n  return 2 * x;   }\nconst char* s = "a // b";  // trailing\n'
    c = 'int f(int x) {\n  return 3 * x; }\nconst char* s = "a // b";\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert '"a // b"' in bench._code_only(a)  # a comment marker inside a string literal is code


def test_recorded_traffic_only_for_known_kernel_and_workload():
    for k in bench.KERNEL_SOURCES:
        assert len(bench.source_sha(k)) == 16
        assert bench.recorded_traffic(k, "no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

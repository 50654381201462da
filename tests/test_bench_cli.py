"""bench.py's argument checks, which run before any GPU work: more than one
GPU is refused with a message, and so are the fp8 score outside the skewed fp8
workload's plain decode and several rows per request outside the V2-Lite
decode."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr


def test_fp8_score_only_for_the_skewed_fp8_decode():
    for args in (["--fp8-score"], ["--fp8-score", "--workload", "v2_lite"],
                 ["--fp8-score", "--workload", "skewed_fp8", "--append"]):
        r = run(*args)
        assert r.returncode == 2, args
        assert "--fp8-score applies to the skewed_fp8" in r.stderr


def test_rows_per_request_only_for_the_v2_lite_decode():
    for args in (["--rows-per-request", "4"], ["--rows-per-request", "0", "--workload", "v2_lite"],
                 ["--rows-per-request", "2", "--workload", "v2_lite", "--append"]):
        r = run(*args)
        assert r.returncode == 2, args
        assert "--rows-per-request applies to the v2_lite" in r.stderr

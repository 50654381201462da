"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner (every params variant: plain, graph-safe, never split, fp32
output, the fp8 score, shared rows, tree-verify suffix tokens; several
compute-unit counts), the host index checks and the C oracle are compiled with g++/gcc and
-fsanitize=address,undefined into one host program (tests/sanitize/
host_driver.cpp), which plans the page layouts of every workload plus empty
and degenerate batches. Any sanitizer report aborts the program and fails the
test. No GPU and no HIP runtime are involved."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_mla_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def write_case(path, batch, suffix=0):
    B = batch.batch
    has_qo = int(not np.array_equal(batch.qo_indptr, np.arange(B + 1)))
    head = np.array([B, batch.page_size, batch.num_heads, has_qo, batch.cache.shape[0], suffix], np.int32)
    parts = [head]
    if has_qo:
        parts.append(batch.qo_indptr.astype(np.int32))
    parts += [batch.kv_indptr.astype(np.int32), batch.kv_last_page_len.astype(np.int32),
              batch.kv_indices[:int(batch.kv_indptr[-1])].astype(np.int32)]
    with open(path, "wb") as f:
        for p in parts:
            f.write(np.ascontiguousarray(p).tobytes())


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("gcc/g++ not available")
    d = tmp_path_factory.mktemp("san")
    oracle_o = d / "oracle.o"
    subprocess.check_call(["gcc", "-std=c11", "-c", *SAN, "-o", str(oracle_o),
                           os.path.join(ROOT, "oracle", "mla_oracle.c")])
    exe = d / "host_driver"
    subprocess.check_call(["g++", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
                           "-o", str(exe), os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                           os.path.join(CSRC, "mla_plan.cpp"), os.path.join(CSRC, "mla_validate.cpp"),
                           str(oracle_o), "-lm"])
    return exe, d


def test_planner_validation_and_oracle_are_clean(driver):
    exe, d = driver
    cases = []

    def add(name, batch, suffix=0):
        p = d / f"{name}.bin"
        write_case(p, batch, suffix)
        cases.append(str(p))

    add("tiny", workloads.tiny(layout_only=True))
    add("v2_lite", workloads.v2_lite(layout_only=True))
    add("v3", workloads.v3(layout_only=True))
    add("skewed_fp8", workloads.skewed_fp8(layout_only=True))
    tv = workloads.tree_verify(batch=4, prefix_len=300, pool_slots=4096)
    add("tree_prefix_rows", tv.prefix)  # 64 query rows per request (qo_indptr)
    add("tree_single_pass", tv.prefix, suffix=tv.max_tree_depth)
    # degenerate batches: no requests, requests without tokens, one token
    add("empty", workloads.random_decode_batch(1, [], num_heads=16, page_size=1, pool_pages=4))
    add("zero_lengths", workloads.random_decode_batch(2, [0, 0, 0], num_heads=128, page_size=64))
    add("one_token", workloads.random_decode_batch(3, [1], num_heads=128, page_size=64))
    add("odd_pages", workloads.random_decode_batch(4, [0, 1, 47, 48, 49, 1000], num_heads=16, page_size=48))
    # several query rows per request (shared-rows units of up to 4 rows at 16 heads, 2 at 32)
    add("rows16", workloads.random_decode_batch(7, [0, 40, 3000, 9000, 1], num_heads=16, page_size=16,
                                                rows_per_request=[3, 4, 9, 1, 2]))
    add("rows32", workloads.random_decode_batch(8, [5000, 2, 700], num_heads=32, page_size=1,
                                                rows_per_request=[5, 2, 0]))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe), *cases], capture_output=True, text=True, env=env, timeout=600)
    print(res.stdout[-3000:])
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    assert res.stdout.strip().endswith("ok")
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

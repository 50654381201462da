"""A wait in the 128-head decode kernel that depends on the compiler's output.

After an item's page-index loads, the kernel issues the 36 loads of the bf16
query and waits until at most 36 vector memory operations are outstanding.
Loads retire in issue order, so that wait covers the page indices only if at
least 36 loads were issued after the last index load. The loads are ordinary
C++ loads, so their count and placement are the compiler's choice. This test
compiles the kernel source for gfx950 to assembly (host only, no GPU) and
checks the invariant at every tagged wait of every instantiation. (Kernels whose
tiles each lie in one page read a scalar page number per tile instead and have
no such wait.)"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# A vector memory load that counts in vmcnt and retires in order with the
# index loads (scratch stores do not retire in order with loads and are not
# counted).
_VLOAD = re.compile(r"^\s*(global_load_|buffer_load_|scratch_load_|flat_load_)")
_IDX = re.compile(r"^\s*global_load_lds_dword\s")
_TAG = re.compile(r"s_waitcnt vmcnt\((\d+)\)\s*; mla-query-wait")


@pytest.fixture(scope="module")
def h128_asm(tmp_path_factory):
    from paged_mla_decode_amd import build as B
    out = tmp_path_factory.mktemp("isa") / "h128.s"
    flags = [f for f in B.COMMON if f != "-fPIC"]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(B.CSRC, "mla_decode_h128.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().splitlines()


def test_query_wait_leaves_only_query_loads_in_flight(h128_asm):
    lines = h128_asm
    kernels, tagged = 0, 0
    with_idx = set()
    current = None
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w*decode_h128_kernel\w*):", line)
        if m:
            current = m.group(1)
            kernels += 1
            continue
        if current and _IDX.match(line):
            with_idx.add(current)
        t = _TAG.search(line)
        if not t:
            continue
        tagged += 1
        need = int(t.group(1))
        loads = 0
        j = i - 1
        while j >= 0 and not _IDX.match(lines[j]):
            if _VLOAD.match(lines[j]):
                loads += 1
            if re.match(r"^_Z\w*:", lines[j]):
                break
            j -= 1
        assert j >= 0 and _IDX.match(lines[j]), f"{current}: no page-index load before the query wait"
        assert loads >= need, (f"{current}: only {loads} vector loads between the last page-index "
                               f"load and 'vmcnt({need})' (line {i + 1})")
    assert kernels >= 8
    # Every instantiation that stages page indices through LDS has the tagged
    # wait, but the fp8-score one; those with page-uniform tiles (a scalar load
    # of one page number per tile) load no page indices and have none.
    assert len(with_idx) >= 8 and kernels > len(with_idx)
    assert tagged >= len(with_idx) - 1, (tagged, len(with_idx), kernels)

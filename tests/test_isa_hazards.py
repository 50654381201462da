"""Wait states the 128-head decode kernel leaves out on purpose.

Its MFMAs are inline assembly, so the compiler inserts none of the wait states
the hardware needs between a VALU instruction that writes a register and an
MFMA that reads it. The MFMAs whose operands come straight from memory (the
bf16 tile and probabilities from LDS, the query from global memory) are issued
without the two wait states the others carry (mla_device.h, kWait). That is
right only as long as the compiler never places a VALU write of one of their
source registers (A, B or C) just before them, which is its choice: this test
compiles the kernel for gfx950 (host only, no GPU) and checks, for every MFMA
not preceded by its wait states, the four instructions before it."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WINDOW = 4  # issued instructions (an s_nop N counts N + 1) checked before each MFMA


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


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


def test_mfmas_without_wait_states_read_no_fresh_valu_result(h128_asm):
    ins, kernel = [], None
    unguarded = 0
    for line in h128_asm:
        m = re.match(r"^(_Z\w*decode_h128_kernel\w*):", line)
        if m:
            kernel, ins = m.group(1), []
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        ins.append(t)
        op = t.split()[0]
        if not op.startswith("v_mfma"):
            continue
        prev = ins[-2].split() if len(ins) >= 2 else [""]
        if prev[0] == "s_nop" and int(prev[1], 0) >= 1:
            continue  # the MFMA carries its two wait states
        unguarded += 1
        toks = [x.strip(",") for x in t.split()[1:]]
        srcs = set().union(*(_regs(x) for x in toks[1:4]))
        dist = 0
        for p in reversed(ins[:-1]):
            pop = p.split()[0]
            dist += int(p.split()[1], 0) + 1 if pop == "s_nop" else 1
            if dist > WINDOW:
                break
            if pop.startswith("v_") and not pop.startswith("v_mfma"):
                dst = _regs(p.split()[1].strip(","))
                assert not (dst & srcs), f"{kernel}: '{p}' writes a source of '{t}' {dist} instructions before it"
    assert unguarded > 0  # the bf16 instantiations use the MFMAs without wait states

"""The direct-to-LDS load statements write SCC, and the compiler must know it.

Each 16-byte direct global->LDS load is an inline-assembly statement that sets
M0 with s_add_u32, which also writes SCC (its carry). Unless the statement
declares SCC clobbered, the compiler may set SCC with a comparison, place such
statements after it and branch on SCC behind them, so that the branch reads the
carry instead of the comparison. This test compiles the decode kernels for
gfx950 (host only, no GPU) and checks every branch on SCC: within its basic
block, the last instruction before it that writes SCC must not be one of those
statements."""
import os
import re
import subprocess

import pytest

# SALU instructions that write SCC (a superset is harmless: it only ends the
# backward walk early at an instruction that does set the flag).
_SCC_WRITE = re.compile(
    r"^s_(cmp|cmpk|bitcmp|add_|addc_|sub_|subb_|addk_|and_|or_|xor_|andn2_|orn2_|nand_|nor_|xnor_|"
    r"lshl|lshr|ashr|bfe_|min_|max_|abs_|absdiff_|not_|bcnt|lshl\d_add)")


def _compile(tmp_path_factory, src):
    from paged_mla_decode_amd import build as B
    out = tmp_path_factory.mktemp("isa") / (os.path.splitext(src)[0] + ".s")
    flags = [f for f in B.COMMON if f != "-fPIC"]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-o", str(out), os.path.join(B.CSRC, src)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text().splitlines()


@pytest.mark.parametrize("src", ["mla_decode_h128.hip", "mla_kernels.hip"])
def test_no_branch_reads_the_carry_of_a_dma_statement(tmp_path_factory, src):
    lines = [l.strip() for l in _compile(tmp_path_factory, src)]
    kernel, branches, dmas = None, 0, 0
    for i, t in enumerate(lines):
        m = re.match(r"^(_Z\w+):", t)
        if m:
            kernel = m.group(1)
            continue
        if t.startswith("s_add_u32 m0"):
            dmas += 1
        if not t.startswith("s_cbranch_scc"):
            continue
        branches += 1
        for p in reversed(lines[:i]):
            if p.endswith(":") or p.startswith("_Z"):
                break  # block start: SCC comes from elsewhere
            assert not p.startswith("s_add_u32 m0"), f"{kernel}: '{t}' reads SCC written by '{p}'"
            if _SCC_WRITE.match(p):
                break
    assert dmas > 0 and branches > 0

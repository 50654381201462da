"""The decode kernel's LDS tile layout and address decompositions, checked on
the host for every lane and instance (tests/layout_check.cpp)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_tile_layout_decompositions(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-Wall",
                           "-I", os.path.join(ROOT, "paged_mla_decode_amd", "csrc"),
                           os.path.join(HERE, "layout_check.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "layout ok" in out.stdout

"""Without the built library the package refuses to run: the binding raises
ImportError naming the missing file, and no call reaches a fallback. (A copy
of the package's Python sources without libmla_decode.so, in a subprocess.)"""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_package_without_the_library_raises(tmp_path):
    pkg = tmp_path / "paged_mla_decode_amd"
    pkg.mkdir()
    for name in os.listdir(os.path.join(ROOT, "paged_mla_decode_amd")):
        if name.endswith(".py"):
            shutil.copy(os.path.join(ROOT, "paged_mla_decode_amd", name), pkg / name)
    assert not (pkg / "libmla_decode.so").exists()
    code = ("import paged_mla_decode_amd as m\n"
            "try:\n"
            "    m.mla_status_string(0)\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e)\n"
            "    raise SystemExit(3)\n"
            "raise SystemExit(0)\n")
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=str(tmp_path),
                       timeout=300)
    assert r.returncode == 3, (r.stdout, r.stderr)
    assert "no fallback" in r.stdout and "libmla_decode.so" in r.stdout


def test_the_package_never_reaches_the_oracle():
    """The product path (the package's Python and native sources) imports,
    links or names nothing under oracle/: only tests/, smoke() and bench.py's
    cpu_baseline leg use the oracle."""
    import re
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b)|mla_oracle|oracle_mla", re.M)
    root = os.path.join(ROOT, "paged_mla_decode_amd")
    for dirpath, _, files in os.walk(root):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not pat.search(text), os.path.join(dirpath, f)

"""The product path has no CPU fallback: a copy of the package without its
built library must refuse to load (the binding raises on import), and nothing
in the package imports the oracle."""

import os
import re
import shutil
import subprocess
import sys

from conftest import ROOT

PKG = "combine_router_softmax_expert_amd"


def test_binding_raises_without_the_library(tmp_path):
    dst = tmp_path / PKG
    shutil.copytree(os.path.join(ROOT, PKG), dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    import combine_router_softmax_expert_amd.binding\n"
            "except RuntimeError as e:\n"
            "    print('refused:', e); sys.exit(0)\n"
            "sys.exit(3)\n") % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout


def test_package_never_imports_the_oracle():
    pattern = re.compile(r"^\s*(from\s+oracle\b|import\s+oracle\b|from\s+\.+oracle\b)", re.M)
    for dirpath, _, files in os.walk(os.path.join(ROOT, PKG)):
        for f in files:
            if f.endswith(".py"):
                assert not pattern.search(open(os.path.join(dirpath, f)).read()), f
    assert pattern.search("from oracle import oracle as orc\n")   # the check itself works

"""The product path stands alone: importing the package without its built
library fails loudly (no CPU fallback), and nothing in the package or its
native sources reaches into the oracle (test infrastructure only)."""

import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "vocab_embedding_softmax_amd")


def test_import_without_library_fails(tmp_path):
    dst = tmp_path / "vocab_embedding_softmax_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import vocab_embedding_softmax_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libvce.so is missing" in r.stderr, r.stderr[-2000:]


def test_package_and_sources_never_use_the_oracle():
    pat = re.compile(r"^\s*(import|from)\s+oracle\b|\boracle\.", re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not pat.search(src), os.path.join(dirpath, f)
    hdr = open(os.path.join(ROOT, "include", "vce.h"), encoding="utf-8").read()
    assert "oracle" not in hdr

"""Host-side logic of bench.py (no GPU): the one-GPU refusal and the guard
that keeps the committed traffic counters tied to the kernel sources they
were read on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == 2


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    for name in bench.GEMM_SOURCES:
        with open(os.path.join(bench.CSRC, name)) as f:
            (tmp_path / name).write_text(f.read())
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_hash()
    p = tmp_path / bench.GEMM_SOURCES[0]
    p.write_text(p.read_text() + "\n// a comment line\n\n")
    assert bench.kernel_source_hash() == h0
    p.write_text(p.read_text() + "static int vce_extra_symbol;\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_counters_follow_the_sources(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        text = f.read()
    recorded = [l.split()[1] for l in text.splitlines() if l.startswith("source_hash ")]
    assert len(recorded) == 1
    # a summary read on the current sources gives every kernel's bytes
    current = tmp_path / "current.txt"
    current.write_text("\n".join(("source_hash " + bench.kernel_source_hash()
                                   if l.startswith("source_hash ") else l)
                                  for l in text.splitlines()) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(current))
    for tag in ("fwd", "grad", "dh", "dw"):
        assert bench.measured_traffic(tag) > 0
    # a summary taken on other sources is not used
    stale = tmp_path / "traffic.txt"
    stale.write_text("\n".join(("source_hash 0123456789abcdef" if l.startswith("source_hash ")
                                else l) for l in text.splitlines()) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("grad") is None

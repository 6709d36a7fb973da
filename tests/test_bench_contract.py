"""bench.py's command-line contract and its host-side bookkeeping (CPU only).

* More than one GPU is refused with a message and a non-zero status, before
  any GPU work.
* The recorded HBM traffic of a workload is reported only while the kernel
  sources hash to the value it was measured on; comment edits keep the hash.
"""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_follows_the_source_hash(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        table = json.load(f)
    name, entry = next(iter(table.items()))
    monkeypatch.setattr(bench, "source_hash", lambda: entry["source_hash"])
    assert bench.measured_traffic(name) == entry["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("no_such_workload") is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "fp8_block_scaled_nt_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.h").write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    (csrc / "k.h").write_text("/* header */\nint f(int x) {\n\n  return x + 1;  // two\n}\n")
    assert bench.source_hash() == h0
    (csrc / "k.h").write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash() != h0

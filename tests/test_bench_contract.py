"""Host-side checks of bench.py: the one-GPU contract and the bookkeeping
that ties committed counter records to the kernel sources they measured."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {\n  // add one\n  return x + 1;  /* done */\n}\n"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_tokens(a) == bench._code_tokens(b)
    assert bench._code_tokens(a) != bench._code_tokens(c)


def test_traffic_records_are_complete():
    for name in ("decode_1m_counters", "prefill_8m_counters", "route_1m_counters"):
        path = os.path.join(ROOT, "profiles", name + ".json")
        with open(path) as f:
            rec = json.load(f)
        for key in ("kernel", "sources", "sources_sha256", "fetch_size_kib_per_dispatch",
                    "write_size_kib_per_dispatch", "hbm_bytes_per_launch",
                    "algorithmic_bytes_per_launch", "copy_calibration", "commands"):
            assert key in rec, (name, key)
        for src in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, src)), src
        # the measured bytes are close to the kernel's algorithmic bytes
        assert 0.9 < rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.2


def test_traffic_lookup_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    rec = {"sources": [str(src)], "sources_sha256": bench._sources_sha256([str(src)]),
           "hbm_bytes_per_launch": 1234.0}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "rec.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("rec") == 1234.0
    src.write_text("// a comment only\n__global__ void k() {}\n")
    assert bench.measured_traffic("rec") == 1234.0
    src.write_text("__global__ void k() { int x = 1; }\n")
    assert bench.measured_traffic("rec") is None
    assert bench.measured_traffic("missing") is None

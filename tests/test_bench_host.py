"""Host logic of bench.py that runs without a GPU: the one-GPU contract and
the digest that ties the recorded HBM traffic to the kernel sources it was
measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout


def test_traffic_follows_the_recorded_counters():
    t = bench.TRAFFIC_MEASURED
    if bench._sources_digest() != t["digest"]:
        # kernel sources changed since the counters were taken: no figure
        assert bench._traffic_bytes() is None
        return
    want = round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))
    assert bench._traffic_bytes() == want
    # the counters cover the launch's algorithmic bytes and little more
    algorithmic = 36_971_152
    assert 1.0 <= want / algorithmic < 1.1


def test_traffic_is_null_once_a_source_changes(monkeypatch):
    monkeypatch.setitem(bench.TRAFFIC_MEASURED, "digest", "0" * 64)
    assert bench._traffic_bytes() is None


def test_cpu_model_is_text_or_none():
    m = bench._cpu_model()
    assert m is None or (isinstance(m, str) and m)

"""Host-side pieces of bench.py: the traffic figure read from the committed
counter summary is used only while the decode sources match the hash it
records, and the GPU-count contract."""
import subprocess
import sys
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_read_traffic_follows_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# header: ignored\nhbm_bytes_per_launch: 76425988   (fetch + write)\n"
                 f"decode_source_sha256: {bench.decode_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic() == 76425988.0
    monkeypatch.setattr(bench, "decode_source_hash", lambda: "0" * 64)
    assert bench.read_traffic() is None


def test_read_traffic_missing_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)

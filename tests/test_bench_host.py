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


def test_cpu_baseline_times_the_oracle_on_all_and_one_thread():
    """The CPU leg runs the oracle's append + attention on the headline
    step's inputs, on the affinity's threads and then on one thread, and
    returns the oracle's own output for the parity check."""
    import numpy as np
    import oracle
    from transformer_kv_cache_amd import synth
    w = synth.make_workload("cpu_leg", seed=1, dtype="f32", L=2, B=1, Hq=2, Hkv=2, D=64, Tmax=40,
                            hist=[20], step_lens=(1,))
    r = bench.cpu_baseline(w, 0.2)
    assert r["steps"] >= 1 and r["us_per_step"] > 0 and r["one_thread_us_per_step"] > 0
    assert r["threads"] >= 1
    q, k, v = w.steps[0]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.append(kc, vc, k, v, w.hist)
    assert np.array_equal(r["out"], oracle.attention(q, kc, vc, w.hist, w.scale))
    m = bench.cpu_model()
    assert m is None or isinstance(m, str)

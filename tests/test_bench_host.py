"""Host-side checks of bench.py's measurement plumbing (no GPU): the committed HBM counter
readings are only reported while the sources of the measured launch are unchanged, and
--gpus above 1 is refused with a message."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_profiled_launch_names_existing_sources():
    csrc = os.path.join(ROOT, "block_sparse_gqa_paged_amd", "csrc")
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), (kernel, f)
        assert len(bench.kernel_source_hash(kernel)) == 16


def test_committed_decode_traffic_is_reported_only_for_its_sources():
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    k = rec["kernels"]["attn_decode"]
    # the counters read the cache once: within 2% of the algorithmic K+V bytes
    assert 1.0 <= k["bytes_per_launch"] / 1204576256 < 1.02
    fresh = k["source_hash"] == bench.kernel_source_hash("attn_decode")
    assert bench.traffic_from_profiles("attn_decode") == (k["bytes_per_launch"] if fresh else None)


def test_stale_readings_are_not_reported(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    rec["kernels"]["attn_decode"]["source_hash"] = "0" * 16
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "f" * 16)
    assert bench.traffic_from_profiles("attn_decode") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]

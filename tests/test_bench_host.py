"""Host-side pieces of bench.py: the one-GPU guard and the HBM traffic record
(counter figures are reported only while the kernel sources still hash to
the value the counters were taken with)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_record_parses_and_scales(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    for f in bench.TRAFFIC_SOURCES:
        (src / f).write_bytes(f.encode())
    import hashlib
    h = hashlib.sha256(b"".join(f.encode() for f in bench.TRAFFIC_SOURCES)).hexdigest()
    prof = tmp_path / "p.md"
    rec = {"sources_sha256": h, "fetch_kib": 100.0, "write_kib": 50.0, "fetch_factor": 2.0, "write_factor": 1.0}
    prof.write_text("# x\n\ntraffic-record: " + json.dumps(rec) + "\n")
    pkg = tmp_path / "megatron_tensor_transformer_col_amd"
    pkg.mkdir()
    os.symlink(src, pkg / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.col_gemm_traffic() == 1024.0 * (200.0 + 50.0)
    (src / bench.TRAFFIC_SOURCES[0]).write_bytes(b"changed kernel")
    assert bench.col_gemm_traffic() is None          # stale counters are not reported
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.col_gemm_traffic() is None


def test_committed_traffic_record_is_well_formed():
    line = next(l for l in open(bench.TRAFFIC_PROFILE) if l.startswith("traffic-record:"))
    rec = json.loads(line.split(":", 1)[1])
    assert set(rec) >= {"sources_sha256", "fetch_kib", "write_kib", "fetch_factor", "write_factor"}
    assert rec["fetch_kib"] > 0 and rec["write_kib"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

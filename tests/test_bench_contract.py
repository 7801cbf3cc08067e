"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, and the committed HBM-traffic figure is used only while the
kernel sources still hash to the value stamped beside it."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def _stamped(tmp_path, sha, enc=123, dec=456):
    p = tmp_path / "traffic.md"
    p.write_text(f"    kernel_source_sha256: {sha}\n    encode_hbm_bytes_per_launch: {enc}\n"
                 f"    decode_hbm_bytes_per_launch: {dec}\n")
    return str(p)


def test_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _stamped(tmp_path, bench.kernel_source_hash()))
    assert bench.measured_traffic("encode") == 123
    assert bench.measured_traffic("decode") == 456
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _stamped(tmp_path, "0" * 64))
    assert bench.measured_traffic("encode") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("decode") is None


def test_source_hash_covers_the_kernel_files():
    names = sorted(os.path.basename(f) for f in bench.KERNEL_SOURCES)
    assert names == ["kvc_arch.h", "kvc_internal.h", "kvc_kernels.hip"]
    assert all(os.path.exists(f) for f in bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 64

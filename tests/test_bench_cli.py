"""Host-side behaviour of bench.py that needs no GPU: the refusal of more
than one GPU, and the rule that the recorded HBM traffic and VALU activity
are reported only for the kernel source they were measured on."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hpp"
    src.write_text("// kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"w": {"kernel_sha256_16": bench.kernel_hash(),
                                     "bytes_per_launch": 1234}}))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    assert bench.recorded_traffic("w") == 1234
    assert bench.recorded_traffic("other") is None
    src.write_text("// kernel source, changed\n")
    assert bench.recorded_traffic("w") is None


def test_valu_fraction_from_the_record(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hpp"
    src.write_text("// kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    rec = tmp_path / "traffic.json"
    cycles = bench.N_SIMDS * bench.CLOCK_HZ * 1e-3 * 0.5      # half of a 1 ms launch
    rec.write_text(json.dumps({"w": {"kernel_sha256_16": bench.kernel_hash(),
                                     "valu_active_simd_cycles": cycles}}))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    assert bench.valu_roofline("w", 1.0)["frac"] == pytest.approx(0.5)
    assert bench.valu_roofline("w", 2.0)["frac"] == pytest.approx(0.25)
    src.write_text("// kernel source, changed\n")
    assert bench.valu_roofline("w", 1.0) is None



def test_cpu_baseline_context():
    """The CPU model and the oracle's one-thread times reported beside the
    CPU baseline (host only)."""
    assert bench.cpu_model() and bench.cpu_model() != ""
    res = bench.one_thread_times()
    assert res["tiny_s"] > 0 and res["gpt2s_s"] > 0
    assert "4 of 96 heads" in res["gpt2s_sample"]


def test_issue_model_from_the_record(tmp_path, monkeypatch):
    """Recorded instruction counts times the measured issue costs, summed
    (MFMA and VALU issue one after the other), over 1024 SIMDs."""
    src = tmp_path / "kernel.hpp"
    src.write_text("// kernel source\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    rec = tmp_path / "traffic.json"
    n = 1024 * 1000
    rec.write_text(json.dumps({"w": {"kernel_sha256_16": bench.kernel_hash(),
                                     "valu_active_simd_cycles": 1.0, "valu_insts": 3 * n,
                                     "valu_trans_insts": n, "mfma_insts": n}}))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    want_us = (2 * bench.ISSUE_NS["valu"] + bench.ISSUE_NS["trans"] + bench.ISSUE_NS["mfma"])
    got = bench.valu_roofline("w", want_us * 2e-3)
    assert got["issue_model_us"] == pytest.approx(want_us, abs=0.05)
    assert got["issue_frac"] == pytest.approx(0.5, abs=1e-3)


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))

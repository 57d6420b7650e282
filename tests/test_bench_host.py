"""Host-side logic of bench.py (CPU only: nothing here touches a GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_records_are_keyed_to_their_kernel_sources():
    # a record whose sha1 is that of the named sources yields its value; any
    # other sha1 (the sources changed since the counters were taken) yields None
    import hashlib
    srcs = ("mx_pack.hip", "mx_device.h", "mx_kernels.h")
    h = hashlib.sha1()
    for f in srcs:
        with open(os.path.join(ROOT, "microscaling_block_scaled_mx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    assert bench.measured_traffic({"bytes_per_launch": 5.0, "sources": srcs, "sources_sha1": h.hexdigest()}) == 5.0
    assert bench.measured_traffic({"instructions_per_launch": 7.0, "sources": srcs,
                                   "sources_sha1": h.hexdigest()}) == 7.0
    assert bench.measured_traffic({"bytes_per_launch": 5.0, "sources": srcs, "sources_sha1": "0" * 40}) is None
    for rec in (bench.GEMM_TRAFFIC, bench.PACK_TRAFFIC, bench.PACK_VALU):
        assert len(rec["sources_sha1"]) == 40 and rec["sources"]


def test_alu_roofline_arithmetic(monkeypatch):
    # 1228.8 G wavefront-instructions/s = 256 CUs x 4 SIMDs x 2.4 GHz x 2
    # instructions per 4 cycles: the fp32 vector 157.3 TFLOP/s over the 128
    # flops of one wave64 FMA
    assert bench.VALU_PEAK_GIPS == pytest.approx(1228.8)
    assert bench.VALU_PEAK_GIPS == pytest.approx(157.3e12 / 128 / 1e9, rel=1e-3)
    monkeypatch.setattr(bench, "measured_traffic", lambda rec: 1.2288e7)
    r = bench.alu_roofline(20.0)  # 1.2288e7 instructions in 20 us = 614.4 G/s
    assert r["bound"] == "alu" and r["achieved"] == pytest.approx(614.4)
    assert r["frac"] == pytest.approx(0.5)
    monkeypatch.setattr(bench, "measured_traffic", lambda rec: None)
    assert bench.alu_roofline(20.0) is None


def test_pack_algorithmic_bytes_per_element():
    # bf16 in (2 B) plus, per packed axis, the codes (bits / 8 B) and one E8M0
    # byte per 32 elements
    assert bench.PACK_OUT[4] == pytest.approx(0.5 + 1 / 32)
    assert bench.PACK_OUT[6] == pytest.approx(0.75 + 1 / 32)
    assert bench.PACK_OUT[8] == pytest.approx(1.0 + 1 / 32)
    # the dual pack of the MXFP6 linear step: X [4096,3072], W [3072,3072], dY [4096,3072]
    M, N, K = 4096, 3072, 3072
    assert (M * K + N * K + M * N) * (2 + 2 * bench.PACK_OUT[6]) == 123273216

"""Host-side logic of bench.py (no GPU): the roofline arithmetic of every reported
entry, the weight rotation that keeps timed launches out of the caches, the counter
summaries' hash gate, and the refusal of more than one GPU."""
import math
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (stdlib-only at import time)


def test_roofline_entry_hbm_bound():
    # one token through a 4096 x 4096 layer: 4 MB of packed weights, 33.5 M operations
    N = K = 4096
    nbytes = N * K // 4 + 4 * N + 2 * K + 4 * N
    ops = 2.0 * N * K
    us = 3.0
    e = bench.roofline_entry(us, ops, nbytes)
    assert e["bound"] == "hbm"
    assert e["frac_hbm_peak"] == pytest.approx(nbytes / us / 1e3 / bench.HBM_PEAK_GBS, abs=1e-4)
    ai = ops / nbytes
    assert e["ops_per_byte"] == pytest.approx(ai, abs=0.01)
    # attainable = AI x 8 TB/s (in TOPS) while below the matrix-core peak
    assert e["attainable_TOPS"] == pytest.approx(ai * bench.HBM_PEAK_GBS / 1e3, abs=0.1)
    # fraction of the attainable time = ideal time / measured time
    assert e["frac_of_attainable"] == pytest.approx(
        nbytes / (bench.HBM_PEAK_GBS * 1e3) / us, abs=1e-4)
    assert "frac_mfma_peak" not in e


def test_roofline_entry_mfma_bound():
    M, N, K = 2048, 14336, 4096
    nbytes = N * K // 4 + 4 * N + M * K + 4 * M + 2 * M * N
    ops = 2.0 * M * N * K
    us = 120.0
    e = bench.roofline_entry(us, ops, nbytes)
    assert e["bound"] == "mfma"
    assert e["attainable_TOPS"] == bench.INT8_MFMA_PEAK_TOPS
    assert e["frac_mfma_peak"] == pytest.approx(ops / us / 1e6 / bench.INT8_MFMA_PEAK_TOPS,
                                                abs=1e-4)
    assert e["frac_of_attainable"] == pytest.approx(e["frac_mfma_peak"], abs=1e-4)
    assert "frac_hbm_peak" not in e


def test_roofline_bound_switches_at_the_ridge_point():
    # ridge: ops / bytes = 5.0e15 / 8.0e12 = 625 operations per byte
    ridge = bench.INT8_MFMA_PEAK_TOPS * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert ridge == pytest.approx(625.0)
    assert bench.roofline_entry(1.0, 600.0 * 1e6, 1e6)["bound"] == "hbm"
    assert bench.roofline_entry(1.0, 650.0 * 1e6, 1e6)["bound"] == "mfma"


@pytest.mark.parametrize("nbytes", [1 << 20, 17367040, 117440512, 1 << 30, 3 << 30])
def test_rotation_exceeds_the_rotation_bytes(nbytes):
    t = torch.zeros(4, dtype=torch.uint8)
    copies = bench.rotation([t], nbytes)
    R = len(copies)
    assert R == max(2, math.ceil(bench.ROTATE_BYTES / nbytes))
    assert R * nbytes >= bench.ROTATE_BYTES
    assert copies[0][0] is t                       # entry 0: the tensors themselves
    assert all(c[0] is not t and torch.equal(c[0], t) for c in copies[1:])
    assert len({id(c[0]) for c in copies}) == R    # every copy its own storage


def test_load_summary_applies_only_to_its_kernel_source(tmp_path):
    p = tmp_path / "summary.txt"
    p.write_text("# comment = ignored\nkernel_source_sha256 = abc\nhbm_bytes_per_launch = 42\n")
    vals = bench.load_summary(str(p), "abc")
    assert vals == {"kernel_source_sha256": "abc", "hbm_bytes_per_launch": "42"}
    assert bench.load_summary(str(p), "def") is None
    assert bench.load_summary(str(tmp_path / "missing.txt"), "abc") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

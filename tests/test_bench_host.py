"""Host-side parts of bench.py: the one-GPU contract and the algorithmic
byte counts its roofline entries divide by (no GPU needed)."""
import os
import subprocess
import sys

import bench
from long_context_sparse_csa2_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_bytes_c2():
    # indexer K of every scanned entry (68 B: 64 B E2M1 codes + 4 E8M0 scale
    # bytes), the Full scan over 4 x 2^20 entries and 4 Reindex scans of the
    # 2048 x 8 pool; per attention call and query 512 main rows of 288 B,
    # 128 SWA rows of 516 B, the bf16 query and the fp32 output (64 x 512)
    wl = synth.WORKLOADS["c2"]
    q = 4
    want = q * 2**20 * 68 + 4 * q * 16384 * 68 + 5 * q * (512 * 288 + 128 * 516 + 64 * 512 * 2 + 64 * 512 * 4)
    assert bench.step_bytes(wl) == want == 311_240_704
    assert bench.step_bytes(synth.WORKLOADS["c3"]) is None        # prefill: rows come from cache


def test_scan_traffic_is_current_or_null():
    t = bench.scan_traffic("c2")
    if t is not None:                  # counters taken on the current scan source
        # at least the algorithmic bytes, and no large re-read
        assert 285_212_672 <= t <= 1.2 * (285_212_672 + 16_777_216)

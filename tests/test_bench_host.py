"""Host-side parts of bench.py, on a machine without a GPU: the one-GPU refusal, the algorithmic
byte count of the layer workload (every input and output once, the state never in HBM), and that
the committed HBM-traffic summary was taken on the current scan sources (otherwise the bench line
reports its traffic as null)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LAYER_BYTES = 675_106_816   # 8 x 2048 x 5120, N 16, bf16: x, delta, z in, y out, B, C, A, D, h_last


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_layer_algorithmic_bytes():
    B, L, D, N = 8, 2048, 5120, 16
    tok = B * L * D * 2
    by_hand = 4 * tok + 2 * B * L * N * 2 + D * N * 4 + D * 4 + B * D * N * 4
    assert by_hand == LAYER_BYTES
    assert bench.scan_bytes(B, L, D, N, 2) == LAYER_BYTES


def test_traffic_summary_matches_sources():
    t = bench.read_traffic()
    assert t is not None, "profiles/ traffic summary was taken on other scan sources"
    assert LAYER_BYTES <= t < 1.2 * LAYER_BYTES

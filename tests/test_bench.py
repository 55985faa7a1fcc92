"""bench.py's host-side contract (CPU): the single-GPU refusal and the byte counts its
bandwidth figures divide by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_expert_bytes_closed_form():
    # codes: 3 projections x H x I x 0.5 B; scale + bias: 3 x H x (I/64) x 2 x 2 B
    assert bench.expert_bytes(2048, 512) == 1_769_472
    assert bench.expert_bytes(512, 128) == 3 * 512 * 128 // 2 + 3 * 512 * 2 * 4


def test_decode_algorithmic_bytes():
    # 9 experts + router rows (bf16 [256][2048]) + x (bf16) + y (fp32) + ids and weights
    H, I, E, k = 2048, 512, 256, 8
    assert 9 * bench.expert_bytes(H, I) + E * H * 2 + H * 2 + H * 4 + k * 8 == 16_986_176


def test_traffic_is_tied_to_the_measured_source():
    t = bench.ffn_traffic_bytes()
    # either the counters belong to this gemm.hip (a byte count) or they are withheld
    assert t is None or (isinstance(t, int) and t > 0)

"""The benchmark's host side, on the CPU: the multi-GPU refusal and the algorithmic-work formulas its
roofline figures divide by (hand-computed values for one small shape)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from inputs import MoEShape  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr and "one GPU" in r.stderr


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_algorithmic_work_formulas(fmt):
    # H 256, I 128, 4 local experts, top-2; 10 routed pairs from 6 tokens
    sh = MoEShape("alg", 1, 6, 256, 128, 8, 4, 2, 64, weight_format=fmt)
    a = bench.algorithmic(sh, R=10, N=6)
    assert a["gemm1_flop"] == 2 * 10 * 256 * (2 * 128)          # 2 flop per MAC, N = 2I outputs
    assert a["gemm2_flop"] == 2 * 10 * 128 * 256
    assert a["route_bytes"] == 6 * 2 * 8 + 10 * 4
    assert a["fill_bytes"] == 10 * (2 * 256 + 2 * 2 * 4 + 16)    # row in+out, 2 scales in+out, meta + entry
    assert a["combine_bytes"] == 10 * 2 * 256 + 6 * (2 * 256 + 2 * 12)
    weights = 4 * (2 * 128 * 256 + 256 * 128)                     # W1 and W2 elements of 4 experts
    if fmt == "fp8":                                                # one byte each, fp32 per 128 x 128 block
        assert a["weight_bytes"] == weights + 4 * (2 * 1 * 2 + 2 * 1) * 4
    else:                                                           # half a byte each, one byte per 32
        assert a["weight_bytes"] == weights // 2 + weights // 32
    with_shared = bench.algorithmic(sh.replace(num_shared_experts=1), R=10, N=6, shared_rows=3)
    assert with_shared["gemm1_flop"] == 2 * 13 * 256 * 256

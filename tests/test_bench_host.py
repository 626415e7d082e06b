"""CPU checks of bench.py's contract: the algorithmic byte counts behind its
roofline fractions, written out here from the tensor shapes of the batch-16,
64-node, 32-head, d = 128 workload, the one-GPU guard, and that the
committed traffic summary belongs to the fused kernel's current code."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

B, N, H, D = 16, 64, 32, 128
STATE = B * H * D * D * 4            # fp32 S0, 32 MiB


def test_verify_bytes_are_the_tensors_touched_once():
    qkv = 3 * B * N * H * D * 2      # bf16 q, k, v: 8 MiB each
    gates = 2 * B * N * H * 4        # fp32 alpha, beta
    parent = B * N * 4
    out = B * N * H * D * 4          # fp32 out, 16 MiB
    assert bench.verify_bytes(B, N, H, D, D) == qkv + gates + parent + STATE + out == 75763712
    # fp32 q/k/v (the all-fp32 leg) doubles the q/k/v bytes only
    assert bench.verify_bytes(B, N, H, D, D, elem=4) == 2 * qkv + gates + parent + STATE + out


def test_commit_and_fused_bytes():
    m = 139                           # path nodes summed over the batch
    per_node = H * (2 * D * 2 + 2 * 4)   # k, v rows (bf16) and alpha, beta of every head
    commit = 2 * STATE + m * per_node + m * 4 + B * 4
    assert bench.commit_bytes(B, H, D, D, [m]) == commit
    # the fused step reads the state once for both halves
    assert bench.fused_bytes(B, N, H, D, D, [m]) == bench.verify_bytes(B, N, H, D, D) + commit - STATE


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_committed_traffic_matches_the_current_fused_kernel():
    """the committed rocprofv3 traffic summary was taken on the fused
    kernel's current code (bench.py reports no traffic otherwise), and its
    ratio to the algorithmic bytes stays near 1"""
    t = bench.read_traffic(bench.HEADLINE_STEP)
    assert t is not None, "profiles/ traffic summary is stale: re-take it"
    assert 1.0 <= t / bench.fused_bytes(B, N, H, D, D, [139]) < 1.1

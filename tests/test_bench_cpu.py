"""Host-side contract of bench.py (no GPU needed)."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_flops_count_kept_pairs_through_three_projections():
    sys.path.insert(0, ROOT)
    import bench

    class W:
        num_experts, hidden, intermediate = 4, 256, 384
        ids = np.array([[0, 3], [5, 1], [-1, 2]])  # 5 and -1 are dropped

    f = bench.prefill_step_flops(W)
    kept = 4
    assert f["gemm_gateup"] == 2.0 * kept * 256 * 2 * 384
    assert f["gemm_down"] == 2.0 * kept * 384 * 256
    assert f["gemm_experts"] == f["gemm_gateup"] + f["gemm_down"]


def test_kernel_source_hash_covers_the_expert_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench

    h = bench.kernel_source_sha()
    assert len(h) == 64 and h == bench.kernel_source_sha()
    csrc = os.path.join(ROOT, "trellis_quantized_moe_amd", "csrc")
    with open(os.path.join(csrc, "gemm_wide.hip")) as f:
        src = f.read()
    # every local header the expert kernel includes is hashed
    for line in src.splitlines():
        if line.startswith('#include "'):
            name = line.split('"')[1]
            assert name in bench.KERNEL_SOURCES, name

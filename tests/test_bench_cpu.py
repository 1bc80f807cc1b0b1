"""The benchmark's contract on the host: it refuses more than one GPU, and
its byte counts are the algorithmic ones (each matrix once per unique expert,
in the NVFP4 layout) that its GB/s figures divide by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from speculative_block_verify_amd import api, inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_nvfp4_matrix_bytes():
    # codes (half a byte per value) + one E4M3 scale per 16 values + the fp32 tensor scale
    assert bench.nvfp4_bytes(512, 2048) == 512 * 2048 // 2 + 512 * 2048 // 16 + 4 == 589828


@pytest.mark.parametrize("U,K", [(1, 1), (16, 2), (93, 16)])
def test_gateup_bytes_decompose_the_step_bytes(U, K):
    shape = inputs.LAGUNA
    H, I, Is, k = shape.hidden, shape.inter, shape.shared_inter, shape.top_k
    cfg = api.make_cfg(shape, K)
    step = api.moe_verify_weight_bytes(cfg, U, K)  # router + routed + shared + activations
    gu = bench.gateup_bytes(shape, U, K)
    # the router + gate/up launch: the bf16 router, gate + up of each unique
    # expert and the shared one, x in, h out
    assert gu == 2 * shape.n_experts * H + U * 2 * bench.nvfp4_bytes(I, H) + 2 * bench.nvfp4_bytes(Is, H) \
        + K * H * 2 + (K * k * I + K * Is) * 4
    # the step: those matrices, the down matrices, the bf16 router, x in and y out once each
    down = (U + 1) * bench.nvfp4_bytes(H, I)
    assert step == U * 2 * bench.nvfp4_bytes(I, H) + 2 * bench.nvfp4_bytes(Is, H) + down + 2 * shape.n_experts * H \
        + 2 * 2 * K * H


def test_near_tie_rows_counts_the_kth_gap():
    import numpy as np
    l = np.zeros((2, 3, 16), np.float32)
    l[..., :] = np.arange(16, dtype=np.float32)[::-1]     # well separated
    l[0, 1, 8] = l[0, 1, 7] - 1e-6                          # rank 8 nearly ties rank 7 (k = 8)
    assert bench.near_tie_rows(l, 8) == 1
    assert bench.near_tie_rows(l, 4) == 0


def test_host_info_names_cores_and_model():
    info = bench.host_info()
    assert info["host_cores"] >= 1 and isinstance(info["cpu_model"], str)
    assert bench.DTYPE.startswith("nvfp4 weights")


def test_kernel_source_hash_covers_the_launch_glue():
    assert any(p.endswith("moe_abi.hip") for p in bench.KERNEL_SOURCES)

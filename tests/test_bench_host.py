"""The benchmark's work figures on the host: algorithmic FLOPs and bytes per call of each
workload, against values worked out by hand from the workload shapes (matmul FLOPs only:
2TdN + sum over targets of 2Tdr + 2T r N_t for the forward; the backward adds 2TNd and, per
target, V = G B, the LoRA term of dh, the U recompute, dB and dA; bytes are x, gamma, W, bias,
A_t, B_t, positions and out, each once).  No GPU is needed."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from layer_rmsnorm_qkv_amd import workloads as wl  # noqa: E402

# name: (forward FLOP, backward FLOP, forward bytes)
EXPECTED = {
    # T 8, d 64, N 128, r 4 on q (64 cols) and v (32 cols), float32
    "tiny": (145408.0, 167936.0, 42784),
    # T 8192, d 4096, N 6144, r 8 on q (4096) and v (1024), bf16
    "llama3": (414061690880.0, 416880263168.0, 218357760),
    # T 16384, d 4096, N 12288, r 64 on q, k, v (4096 each), bf16
    "llama2": (1700807049216.0, 1778116460544.0, 640753664),
    # T 64, same shape as llama2 plus bias
    "decode": (6643777536.0, 6945767424.0, 105939200),
    # T 16384, llama3 shape
    "train": (828123381760.0, 833760526336.0, 386162688),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_algorithmic_work(name):
    f, b, by = bench.algorithmic_work(wl.get(name))
    ef, eb, eby = EXPECTED[name]
    assert f == pytest.approx(ef, rel=1e-12)
    assert b == pytest.approx(eb, rel=1e-12)
    assert by == eby


def test_dominant_kernel_work():
    # tiled forward: every matmul FLOP of the forward
    assert bench.dominant_kernel_work(wl.get("llama3"), "tiled", False) == (414061690880.0, "flop")
    # tiled backward main product: 2 T d (N + sum of ranks) = 2 * 16384 * 4096 * (6144 + 16)
    assert bench.dominant_kernel_work(wl.get("train"), "tiled", True) == (2.0 * 16384 * 4096 * 6160, "flop")
    # decode streaming kernel: x, gamma, W, bias, the targets' A and B (rank 64 on q, k and v:
    # 64 x d and N x 64 elements), every output, positions
    T, d, N = 64, 4096, 12288
    expected = 2 * (T * d + d + N * d + N + 3 * 64 * d + N * 64 + T * N) + 4 * T
    assert bench.dominant_kernel_work(wl.get("decode"), "decode", False) == (expected, "bytes")


def test_multi_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr

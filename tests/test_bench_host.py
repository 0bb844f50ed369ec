"""Host-side logic of bench.py (no GPU): the kernel each workload's call routes to, the
roofline's algorithmic byte and flop counts summed by hand, and the command-line refusals."""
import sys

import pytest

import bench
from workloads import WORKLOADS


@pytest.mark.parametrize("cid,kernel", [(1, "k_gemm"), (2, "k_gemm_int4"), (3, "k_gemm_mx"), (4, "k_gemm_mx"),
                                        (5, "k_gemm_decode_mx")])
def test_gemm_kernel_routing(cid, kernel):
    """Workload 1 (K = 64) is below the INT4 kernel's six stages of 256 codes, so the library
    runs the general kernel there."""
    wl = WORKLOADS[cid]
    assert bench.gemm_kernel(wl, wl.B)[0] == kernel


def test_algorithmic_bytes_int4_default():
    wl = WORKLOADS[2]  # B 256, M = N = 4096, rank 32, INT4, bf16
    parts = {
        "activation codes": 256 * 4096 // 2,
        "residual codes": 4096 * 4096 // 2,
        "s_x and s_R": 4 + 4,
        "down [B, r]": 256 * 32 * 2,
        "L2^T [N, r]": 4096 * 32 * 2,
        "Y": 256 * 4096 * 2,
    }
    w = bench.algorithmic(wl, wl.B)
    assert w["gemm_bytes"] == sum(parts.values()) == 11288584
    assert w["flops"] == 2.0 * 256 * 4096 * 4096


def test_algorithmic_bytes_mx_decode():
    wl = WORKLOADS[5]  # B 16, M = N = 8192, rank 128, MXFP4, bf16
    parts = {
        "activation codes": 16 * 8192 // 2,
        "activation E8M0": 16 * 8192 // 32,
        "residual codes": 8192 * 8192 // 2,
        "residual E8M0": 8192 * 8192 // 32,
        "down [B, r]": 16 * 128 * 2,
        "L2^T [N, r]": 8192 * 128 * 2,
        "Y": 16 * 8192 * 2,
    }
    assert bench.algorithmic(wl, wl.B)["gemm_bytes"] == sum(parts.values()) == 38084608


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"], ["--steps", "0"], ["--warmup", "-1"]])
def test_refusals_exit_before_touching_a_gpu(argv, monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    assert bench.main() == 2
    err = capsys.readouterr().err
    assert ("one GPU only" in err) if argv[0] == "--gpus" else ("--steps" in err)

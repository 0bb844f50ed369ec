"""Host-side logic of bench.py (no GPU): the kernel each workload's call routes to, the
roofline's algorithmic byte and flop counts summed by hand, and the command-line refusals."""
import sys

import pytest

import bench
from workloads import WORKLOADS


@pytest.mark.parametrize("cid,kernel", [(1, "k_gemm_int4"), (2, "k_gemm_int4"), (3, "k_gemm_mx"), (4, "k_gemm_mx"),
                                        (5, "k_gemm_decode_mx")])
def test_gemm_kernel_routing(cid, kernel):
    """Workload 1 (K = 64: one stage of 256 codes, fewer than the six the INT kernel keeps in
    flight) takes the INT kernel's short-K path."""
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


def test_call_bytes_mlp_up():
    """The whole call's algorithmic bytes at the MXFP4 MLP up-projection workload (B 4096,
    M 3072, N 12288, rank 32, bf16): what the method must move, intermediates excluded."""
    wl = WORKLOADS[4]
    parts = {
        "x": 4096 * 3072 * 2,
        "scale": 3072 * 4,
        "Y": 4096 * 12288 * 2,
        "residual codes": 3072 * 12288 // 2,
        "residual E8M0": 3072 * 12288 // 32,
        "L1 + L2": (3072 + 12288) * 32 * 2,
    }
    assert bench.algorithmic(wl, wl.B)["call_bytes"] == sum(parts.values()) == 146878464


@pytest.mark.parametrize("steps", [1, 5, 16, 20, 31, 800, 5000])
def test_gemm_sampling_keeps_16_launches(steps):
    """The sampled GEMM timing records every launch of a short run and at least 16 launches of
    any run."""
    every = bench.sampling_stride(steps)
    sampled = len(range(0, steps, every))
    assert sampled >= min(16, steps)


def test_roofline_fractions():
    """Both fractions of the GEMM kernel and of the whole call, from hand-computed times."""
    wl = WORKLOADS[4]
    w = bench.algorithmic(wl, wl.B)
    r = bench.roofline(wl, wl.B, w, gemm_ms=0.1, call_ms=0.125)
    assert r["bound"] == "mfma" and r["kernel"] == "k_gemm_mx"
    assert r["frac"] == pytest.approx(w["flops"] / 1e-4 / 1e12 / 10100.0)
    assert r["frac_hbm"] == pytest.approx(w["gemm_bytes"] / 1e-4 / 1e9 / 8000.0)
    assert r["call"]["frac_mfma"] == pytest.approx(w["flops"] / 1.25e-4 / 1e12 / 10100.0)
    assert r["call"]["frac_hbm"] == pytest.approx(w["call_bytes"] / 1.25e-4 / 1e9 / 8000.0)
    d = WORKLOADS[5]
    assert bench.roofline(d, d.B, bench.algorithmic(d, d.B), 0.01, 0.015)["bound"] == "hbm"


def test_default_workload_is_the_largest(monkeypatch):
    """With no --workload the bench runs the MXFP4 MLP up-projection (4096 x 3072 x 12288), the
    largest configuration that fits one GPU."""
    seen = {}
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    monkeypatch.setattr(bench, "run", lambda args: seen.setdefault("w", args.workload))
    assert bench.main() == 0 and seen["w"] == 4
    flops = {c: WORKLOADS[c].B * WORKLOADS[c].M * WORKLOADS[c].N for c in WORKLOADS}
    assert max(flops, key=flops.get) == 4


def test_measured_ceiling(tmp_path):
    """The GEMM's rate against the committed measured ceiling of its own kind: the FP4 loop for
    MXFP4 shapes, the INT8 loop for INT ones, the read stream for HBM-bound shapes; none
    without a ceilings file."""
    import json

    c = {"fp4_mfma": {"tflops": 8000.0}, "int8_mfma": {"tflops": 4000.0}, "hbm_read": {"gbs": 5000.0}}
    path = tmp_path / "ceilings.json"
    path.write_text(json.dumps(c))
    for cid, probe, peak in ((4, "fp4_mfma", 8000.0), (2, "int8_mfma", 4000.0), (5, "hbm_read", 5000.0)):
        wl = WORKLOADS[cid]
        r = bench.roofline(wl, wl.B, bench.algorithmic(wl, wl.B), 0.05, 0.06)
        m = bench.measured_ceiling(wl, r, str(path))
        assert m["probe"] == probe and m["peak"] == peak
        assert m["frac"] == pytest.approx(r["achieved"] / peak)
    assert bench.measured_ceiling(WORKLOADS[4], r, str(tmp_path / "absent.json")) is None


@pytest.mark.parametrize("B,kernel", [(256, "k_gemm_int4"), (512, "k_gemm_int4"), (1024, "k_gemm_int_big"), (4096, "k_gemm_int_big")])
def test_int_routing_by_batch(B, kernel):
    """INT4 at 4096 x 4096: 64 x 64 tiles up to three rounds of the chip, the large tiles from four."""
    assert bench.gemm_kernel(WORKLOADS[2], B)[0] == kernel

"""bench.py's accounting and command-line contract, on the CPU: the algorithmic
work it prices each stage at (the roofline numerators) against closed forms of
the Qwen3-30B-A3B-shaped layer, and the one-GPU exit."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from scale_only_quantization_amd import fqlib as F  # noqa: E402
from scale_only_quantization_amd.layer import LayerDims  # noqa: E402

E, H, I, T, K = 128, 2048, 768, 16384, 8
R = T * K
DIMS = LayerDims(E, H, I, T, K)


def test_gemm_flops_closed_form():
    fwd, bwd = bench.stage_work(DIMS, F.preset("nvfp4"))
    work = {**fwd, **bwd}
    fc1 = 2.0 * R * (2 * I) * H          # [R, H] x [H, 2I]
    fc2 = 2.0 * R * H * I                # [R, I] x [I, H]
    assert work["fc1"] == ("mfma", fc1) and work["fc1_dgrad"] == ("mfma", fc1) and work["fc1_wgrad"] == ("mfma", fc1)
    assert work["fc2"] == ("mfma", fc2) and work["fc2_dgrad"] == ("mfma", fc2) and work["fc2_wgrad"] == ("mfma", fc2)
    total = sum(v for kind, v in work.values() if kind == "mfma")
    assert total == pytest.approx(3.711e12, rel=1e-3)      # 3 (fc1 + fc2) = 226.5 MFLOP per token


def test_hbm_bytes_closed_form():
    fwd, bwd = bench.stage_work(DIMS, F.preset("nvfp4"))
    bf = 2
    w1, w2 = E * 2 * I * H, E * H * I                     # elements
    # weight fake-quant: read W, write W^, read one fp32 scale per 16-block
    assert fwd["w1_fq"] == ("hbm", 2 * bf * w1 + 4 * w1 // 16)
    assert fwd["w2_fq"] == ("hbm", 2 * bf * w2 + 4 * w2 // 16)
    # permute: each token row read once, each routed row written once
    assert fwd["permute_a1"] == ("hbm", bf * T * H + bf * R * H)
    # SwiGLU: read [R, 2I], write [R, I]
    assert fwd["swiglu_a2"] == ("hbm", bf * R * 2 * I + bf * R * I)
    # combine: read routed rows and their weights, write token rows
    assert fwd["combine"] == ("hbm", bf * R * H + bf * T * H + 4 * R)
    # A1 backward: read X and dX, gather dX^, write nothing else of that size
    assert bwd["unpermute_a1"] == ("hbm", 2 * bf * T * H + bf * R * H)
    # nvfp4 weight-scale gradients are formed in the weight-gradient GEMM
    assert bwd["w1_scale_grad"] == ("hbm", 0) and bwd["w2_scale_grad"] == ("hbm", 0)


def test_dy_permute_without_topk_weight_gradient():
    q = F.preset("w8a8")
    _, full = bench.stage_work(DIMS, q, full_bwd=True)
    _, part = bench.stage_work(DIMS, q, full_bwd=False)
    assert full["permute_dy"][1] - part["permute_dy"][1] == 2 * R * H    # no read of Y_r
    assert bench.WORKLOADS["qwen3_w8a8"][3] is False
    assert all(bench.WORKLOADS[w][3] for w in ("qwen3", "qwen3_w4afp8", "qwen3_fp8"))


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_scale_bytes_follow_the_descriptors():
    # INT4 group-128 weights: one fp32 scale per 128 elements; INT8 per row: one per row
    bf = 2
    w1, w2 = E * 2 * I * H, E * H * I
    fwd, bwd = bench.stage_work(DIMS, F.preset("w4a16"))
    assert fwd["w1_fq"] == ("hbm", 2 * bf * w1 + 4 * w1 // 128)
    assert fwd["w2_fq"] == ("hbm", 2 * bf * w2 + 4 * w2 // 128)
    # per-32-column partials of the GEMM epilogue, read once, and the scales written
    assert bwd["w1_scale_grad"] == ("hbm", 4 * w1 // 32 + 4 * w1 // 128)
    fwd, bwd = bench.stage_work(DIMS, F.preset("w8a8"))
    assert fwd["w1_fq"] == ("hbm", 2 * bf * w1 + 4 * E * 2 * I)
    assert bwd["w2_scale_grad"] == ("hbm", 4 * w2 // 32 + 4 * E * H)


def test_measured_path_takes_nothing_from_the_checker():
    # the timed layer is configured by the library's own presets: oracle/ and
    # tests/ appear in bench.py only inside the CPU-baseline leg
    src = open(os.path.join(ROOT, "bench.py")).read().splitlines()
    start = next(i for i, l in enumerate(src) if l.startswith("def cpu_baseline("))
    end = next(i for i in range(start + 1, len(src)) if src[i].startswith("def "))
    for i, line in enumerate(src):
        if ("oracle" in line or "tests" in line) and not start <= i < end:
            raise AssertionError(f"bench.py:{i + 1} outside cpu_baseline: {line.strip()}")

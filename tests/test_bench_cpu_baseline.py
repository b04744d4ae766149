"""CPU: bench.py's oracle baseline leg on every path, with small host inputs
(the GPU legs of the benchmark are not run here)."""

import dataclasses

import pytest
import torch

import bench
from reduce_add_rmsnorm_amd.inputs import WORKLOADS, make_inputs

BUDGET = 0.2


def _check(cb, unit):
    assert cb["kind"] == "oracle" and cb["unit"] == unit and cb["cores"] == 1
    assert cb["value"] > 0 and cb["seconds"] > 0 and cb["sample"]
    par = cb["parallel"]
    assert par["unit"] == unit and par["value"] > 0 and 1 <= par["cores"] <= 2
    assert cb["host"]["logical_cpus"] >= 1


def test_fused_leg_counts_shard_rows():
    w = WORKLOADS["C2"]
    x = make_inputs(w, rank=w.rank, device=torch.device("cpu"))
    cb = bench.cpu_baseline("fused", w, x, BUDGET, 2)
    _check(cb, "GB/s")
    assert cb["tokens_per_s"] > 0 and f"of {w.shard_rows} rows" in cb["sample"]
    # GB/s and tokens/s describe the same timed rows
    per_row = w.algorithmic_bytes() / w.shard_rows
    assert cb["value"] == pytest.approx(cb["tokens_per_s"] * per_row / 1e9, rel=2e-3)


@pytest.mark.parametrize("path", ["gather", "fc2", "dsacp"])
def test_layout_legs(path):
    w = dataclasses.replace(WORKLOADS["C5"], num_tokens=256, num_tokens_pad=256)  # tp 4, S 64
    tp, S, H = w.tp, w.shard_rows, w.hidden
    g = torch.Generator().manual_seed(1)
    if path == "gather":
        shards = [torch.randint(0, 256, (S, H), generator=g, dtype=torch.uint8) for _ in range(tp)]
        scales = [torch.rand(S, generator=g) for _ in range(tp)]
        x, nbytes = (shards, scales, None, None), 2 * w.num_tokens * (H + 4)
    elif path == "fc2":
        srcs = [torch.randn(w.num_tokens_pad, H // tp, generator=g).to(torch.bfloat16) for _ in range(tp)]
        x, nbytes = (srcs, None), 2 * w.num_tokens_pad * (H // tp) * 2
    else:
        attn = [torch.randn(S, H, generator=g).to(torch.bfloat16) for _ in range(tp)]
        x, nbytes = (attn, None), 2 * tp * S * (H // tp) * 2
    cb = bench.cpu_baseline(path, w, x, BUDGET, 2, nbytes=nbytes)
    _check(cb, "GB/s")


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_leg_counts_flops(fp8):
    w = WORKLOADS["C2"]
    M, K, N = 64, 64, 256
    g = torch.Generator().manual_seed(2)
    if fp8:
        x = (torch.randint(0, 120, (M, K), generator=g, dtype=torch.uint8), torch.rand(M, generator=g),
             torch.randint(0, 120, (N, K), generator=g, dtype=torch.uint8), torch.rand(N, generator=g), None)
    else:
        x = (torch.randn(M, K, generator=g).to(torch.bfloat16), torch.randn(N, K, generator=g).to(torch.bfloat16),
             None)
    cb = bench.cpu_baseline("gemm", w, x, BUDGET, 2, nbytes=2 * M * K * N, fp8_gemm=fp8)
    _check(cb, "TFLOP/s")
    assert f"of {M} token rows" in cb["sample"]


# ---- command line: refusals that come before any device is touched

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120,
                          env={**os.environ, **(env or {})})


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU only" in r.stderr


@pytest.mark.parametrize("args", [["--quant", "fp8"], ["--path", "gemm", "--quant", "mxfp8"],
                                  ["--path", "gather", "--quant", "mxfp4"]])
def test_inconsistent_options_are_refused(args):
    r = _bench(*args)
    assert r.returncode == 2 and "error" in r.stderr and r.stdout == ""


# ---- roofline.traffic: counter bytes only while the kernel source is the one they were taken on

def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    rec = {"C5": {"kernel": "sprms_kernel", "kernel_sha256_16": bench.kernel_hash("fused"),
                  "hbm_bytes_per_launch": 123456789},
           "C4": {"kernel": "sprms_kernel", "kernel_sha256_16": "0" * 16, "hbm_bytes_per_launch": 1},
           "C5-gemm-None": {"kernel": "matmul_scatter_kernel", "kernel_sha256_16": bench.kernel_hash("gemm"),
                            "hbm_bytes_per_launch": 42}}
    f = tmp_path / "pmc_traffic.md"
    f.write_text("# counters\n\n<!-- traffic " + __import__("json").dumps(rec) + " -->\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("C5") == 123456789
    assert bench.measured_traffic("C4") is None                 # taken on another source
    assert bench.measured_traffic("C3") is None                 # never measured
    assert bench.measured_traffic("C5-gemm-None", "gemm") == 42
    assert bench.measured_traffic("C5-gemm-None", "fused") is None  # hash of the wrong kernel
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("C5") is None


"""The library used from plain C on the GPU: tests/c_gpu_client.c (gcc,
include/sprms.h and HIP's C runtime API, no Python or C++) enqueues the fused
call on its own stream for three workload forms and checks each against the
oracle's sp_oracle_reduce_add_rmsnorm given the same arguments."""

import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_client_matches_the_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import __graft_entry__ as ge

    exe = ge.C_GPU_CLIENT
    if not os.path.exists(exe):
        ge.build_c_gpu_client()
    print("plain-C client: 3 cases (bf16 + bias, dynamic e4m3 in place, static e4m3 f32)", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "all cases ok" in r.stdout

"""The product path has no fallback: without the built HIP library every
entry point of the binding raises, and the product package never imports
the oracle (which only the tests, the smoke check and the benchmark's CPU
baseline may use)."""

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "reduce_add_rmsnorm_amd")

PROBE = r"""
import sys
sys.path.insert(0, {root!r})
import torch
import reduce_add_rmsnorm_amd as sp
sp.LIB_PATH = "/nonexistent/libsprms.so"
sp._lib = None
calls = {{
    "load": lambda: sp.load(),
    "sp_reduce_add_rmsnorm": lambda: sp.sp_reduce_add_rmsnorm(
        torch.zeros((2, 4, 8)), torch.zeros((4, 8)), torch.zeros(8), None, 1e-6, 0, None,
        torch.zeros((4, 8), dtype=torch.bfloat16), None, tp_rank=0, num_tokens=8),
    "prepare": lambda: sp.prepare(
        torch.zeros((2, 4, 8)), torch.zeros((4, 8)), torch.zeros(8), None, 1e-6, 0, None,
        torch.zeros((4, 8), dtype=torch.bfloat16), None, tp_rank=0, num_tokens=8),
    "sp_all_gather_unpad": lambda: sp.sp_all_gather_unpad([torch.zeros((4, 8))] * 2, None,
                                                          torch.zeros((8, 8)), None, num_tokens=8),
    "sp_fc2_regroup": lambda: sp.sp_fc2_regroup([torch.zeros((4, 8))] * 2, [torch.zeros((2, 16))] * 2, otp=1),
    "sp_dsacp_heads_to_tokens": lambda: sp.sp_dsacp_heads_to_tokens([torch.zeros((4, 16))] * 2,
                                                                    [torch.zeros((8, 8))] * 2),
    "sp_matmul_scatter": lambda: sp.sp_matmul_scatter(torch.zeros((8, 8), dtype=torch.bfloat16),
                                                      torch.zeros((8, 8), dtype=torch.bfloat16),
                                                      [torch.zeros((2, 4, 8))] * 2, rank=0),
    "sp_shard_geometry": lambda: sp.sp_shard_geometry(8, 8, 2, 0),
    "sp_error_string": lambda: sp.sp_error_string(0),
}}
for name, f in calls.items():
    try:
        f()
    except ImportError as e:
        assert "not built" in str(e), (name, e)
        continue
    raise SystemExit(f"{{name}} did not raise without the library")
print("all raise")
"""


def test_every_entry_point_raises_without_the_library():
    r = subprocess.run([sys.executable, "-c", PROBE.format(root=ROOT)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all raise" in r.stdout


def test_product_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), f"{f} imports the oracle"

"""The C ABI boundary on the CPU: the library loads, exports every entry point
include/sprms.h declares, and its host-side checks behave as documented.
No kernel is launched (no GPU here): only sp_validate, sp_shard_geometry and
the error-string functions are called, with fake device addresses."""

import json
import os
import re
import subprocess

import pytest

import reduce_add_rmsnorm_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sprms.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(sp_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = sp.load()
    names = declared_functions()
    assert set(names) == set(sp.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", sp.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in nm.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_error_strings():
    for code in (sp.SP_OK, sp.SP_ERR_NULL, sp.SP_ERR_SHAPE, sp.SP_ERR_DTYPE, sp.SP_ERR_ALIGN,
                 sp.SP_ERR_UNSUPPORTED, sp.SP_ERR_HIP):
        assert sp.sp_error_string(code) and sp.sp_error_string(code) != "unknown status"
    assert sp.sp_error_string(12345) == "unknown status"


def test_shard_geometry_matches_worked_example():
    with open(os.path.join(ROOT, "tests", "golden", "shard_geometry.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert sp.sp_shard_geometry(c["num_tokens"], c["num_tokens_pad"], c["tp"], c["rank"]) == (
            c["shard_rows"], c["local_start"], c["valid_rows"])
    assert sp.sp_shard_geometry(1000, 1024, 8, 7) == (128, 896, 104)
    assert sp.sp_shard_geometry(1000, 1024, 8, 0) == (128, 0, 128)


@pytest.mark.parametrize("args", [(10, 12, 5, 0), (13, 12, 4, 0), (10, 12, 4, 4), (10, 12, 4, -1),
                                  (-1, 12, 4, 0)])
def test_shard_geometry_rejects(args):
    with pytest.raises(sp.SprmsError) as e:
        sp.sp_shard_geometry(*args)
    assert e.value.status == sp.SP_ERR_SHAPE


# ------------------------------------------------------------ sp_validate

BASE = 1 << 40  # fake, well-separated, 16-byte aligned device addresses
GB = 1 << 32


def problem(**kw):
    d = dict(tp=8, tp_rank=7, shard_rows=128, hidden=4096, num_tokens=1000,
             partial_dtype=sp.SP_BF16, act_dtype=sp.SP_BF16, out_dtype=sp.SP_BF16,
             residual_rows=128, deepstack_rows=0, residual_out=None)
    d.update(kw)
    return sp.sp_problem(**d)


def ptrs(**kw):
    d = dict(partials=BASE, residual=BASE + GB, weight=BASE + 2 * GB, bias=None, eps=1e-6,
             quant_mode=sp.SP_QUANT_NONE, deepstack=None, out=BASE + 3 * GB, out_scale=None)
    d.update(kw)
    return d


def validate(p, **kw):
    a = ptrs(**kw)
    status = sp.sp_validate(p, a["partials"], a["residual"], a["weight"], a["bias"], a["eps"],
                            a["quant_mode"], a["deepstack"], a["out"], a["out_scale"])
    return status, sp.sp_last_error()


def test_valid_problems_pass():
    assert validate(problem())[0] == sp.SP_OK
    assert validate(problem(residual_out=BASE + 4 * GB))[0] == sp.SP_OK
    assert validate(problem(residual_rows=8 * 128))[0] == sp.SP_OK
    assert validate(problem(out_dtype=sp.SP_FP8_E4M3), quant_mode=sp.SP_QUANT_DYNAMIC_TOKEN,
                    out_scale=BASE + 5 * GB)[0] == sp.SP_OK
    assert validate(problem(deepstack_rows=1024), deepstack=BASE + 6 * GB)[0] == sp.SP_OK
    assert validate(problem(tp=1, tp_rank=0, num_tokens=128))[0] == sp.SP_OK
    assert validate(problem(shard_rows=0, num_tokens=0, residual_rows=0), partials=None, residual=None,
                    weight=None, out=None)[0] == sp.SP_OK  # empty shard


@pytest.mark.parametrize("case,expect", [
    (dict(p=dict(tp=0)), sp.SP_ERR_SHAPE),
    (dict(p=dict(tp=65, tp_rank=0)), sp.SP_ERR_SHAPE),
    (dict(p=dict(tp_rank=8)), sp.SP_ERR_SHAPE),
    (dict(p=dict(tp_rank=-1)), sp.SP_ERR_SHAPE),
    (dict(p=dict(num_tokens=1025)), sp.SP_ERR_SHAPE),
    (dict(p=dict(num_tokens=-1)), sp.SP_ERR_SHAPE),
    (dict(p=dict(hidden=4100)), sp.SP_ERR_SHAPE),
    (dict(p=dict(hidden=32776)), sp.SP_ERR_SHAPE),
    (dict(p=dict(hidden=0)), sp.SP_ERR_SHAPE),
    (dict(p=dict(shard_rows=-1)), sp.SP_ERR_SHAPE),
    (dict(p=dict(residual_rows=129)), sp.SP_ERR_SHAPE),
    (dict(p=dict(deepstack_rows=128)), sp.SP_ERR_SHAPE),                  # rows without pointer
    (dict(p=dict(deepstack_rows=100), a=dict(deepstack=BASE + 6 * GB)), sp.SP_ERR_SHAPE),
    (dict(p=dict(partial_dtype=sp.SP_FP8_E4M3)), sp.SP_ERR_DTYPE),
    (dict(p=dict(act_dtype=7)), sp.SP_ERR_DTYPE),
    (dict(p=dict(out_dtype=sp.SP_FP8_E4M3)), sp.SP_ERR_DTYPE),            # fp8 without quant
    (dict(a=dict(quant_mode=sp.SP_QUANT_STATIC_TENSOR, out_scale=BASE + 5 * GB)), sp.SP_ERR_DTYPE),
    (dict(a=dict(quant_mode=3)), sp.SP_ERR_UNSUPPORTED),                  # dynamic per-tensor
    (dict(a=dict(quant_mode=-1)), sp.SP_ERR_UNSUPPORTED),
    (dict(a=dict(partials=None)), sp.SP_ERR_NULL),
    (dict(a=dict(out=None)), sp.SP_ERR_NULL),
    (dict(p=dict(out_dtype=sp.SP_FP8_E4M3), a=dict(quant_mode=sp.SP_QUANT_DYNAMIC_TOKEN)),
     sp.SP_ERR_NULL),                                                      # no out_scale
    (dict(a=dict(partials=BASE + 8)), sp.SP_ERR_ALIGN),
    (dict(a=dict(out=BASE + 3 * GB + 4)), sp.SP_ERR_ALIGN),
    (dict(p=dict(residual_out=BASE + 4 * GB + 2)), sp.SP_ERR_ALIGN),
    (dict(a=dict(eps=-1.0)), sp.SP_ERR_SHAPE),
    (dict(a=dict(eps=float("nan"))), sp.SP_ERR_SHAPE),
    (dict(a=dict(out=BASE + 4096)), sp.SP_ERR_SHAPE),                     # out overlaps partials
    (dict(p=dict(residual_out=BASE + 2 * GB)), sp.SP_ERR_SHAPE),          # residual_out on weight
    (dict(p=dict(residual_out=BASE + 3 * GB)), sp.SP_ERR_SHAPE),          # residual_out on out
])
def test_invalid_problems_are_rejected(case, expect):
    status, msg = validate(problem(**case.get("p", {})), **case.get("a", {}))
    assert status == expect, msg
    assert msg and msg != "no error"


def test_null_descriptor():
    lib = sp.load()
    assert lib.sp_validate(None, None, None, None, None, 0.0, 0, None, None, None) == sp.SP_ERR_NULL


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((2, 4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sp.sp_reduce_add_rmsnorm(x, x[0], x[0, 0], None, 1e-6, 0, None, x[0], None, tp_rank=0,
                                 num_tokens=8)

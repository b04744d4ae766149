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
    (dict(p=dict(partial_stride=128 * 4096 - 8)), sp.SP_ERR_SHAPE),       # partials would overlap
    (dict(p=dict(partial_stride=128 * 4096 + 4)), sp.SP_ERR_ALIGN),       # 8-byte plane step
    (dict(p=dict(flags=2)), sp.SP_ERR_UNSUPPORTED),
])
def test_invalid_problems_are_rejected(case, expect):
    status, msg = validate(problem(**case.get("p", {})), **case.get("a", {}))
    assert status == expect, msg
    assert msg and msg != "no error"


RES_ROW = 4096 * 2   # bytes of one bf16 residual row of problem()
FP8_STATIC = dict(quant_mode=sp.SP_QUANT_STATIC_TENSOR)


@pytest.mark.parametrize("case,expect", [
    # residual rows updated in place (residual_out NULL) inside the partials
    (dict(a=dict(residual=BASE + 4096)), sp.SP_ERR_SHAPE),
    # ... also when residual_out names those rows explicitly
    (dict(p=dict(residual_out=BASE + 4096), a=dict(residual=BASE + 4096)), sp.SP_ERR_SHAPE),
    # the in-place rows cover the weight, the bias or the deepstack
    (dict(a=dict(residual=BASE + 2 * GB - 64 * RES_ROW)), sp.SP_ERR_SHAPE),
    (dict(a=dict(bias=BASE + GB + 5 * RES_ROW)), sp.SP_ERR_SHAPE),
    (dict(p=dict(deepstack_rows=128), a=dict(deepstack=BASE + GB + 64 * RES_ROW)), sp.SP_ERR_SHAPE),
    # a replicated residual: only block tp_rank is written, block 0 may hold the weight
    (dict(p=dict(residual_rows=1024), a=dict(weight=BASE + GB + 64)), sp.SP_OK),
    (dict(p=dict(residual_rows=1024), a=dict(weight=BASE + GB + 7 * 128 * RES_ROW + 64)),
     sp.SP_ERR_SHAPE),
    # the static scale is read by every workgroup: not on out, nor on the residual written
    (dict(p=dict(out_dtype=sp.SP_FP8_E4M3), a=dict(out_scale=BASE + 3 * GB + 64, **FP8_STATIC)),
     sp.SP_ERR_SHAPE),
    (dict(p=dict(out_dtype=sp.SP_FP8_E4M3), a=dict(out_scale=BASE + GB + 64, **FP8_STATIC)),
     sp.SP_ERR_SHAPE),
    (dict(p=dict(out_dtype=sp.SP_FP8_E4M3), a=dict(out_scale=BASE + 5 * GB, **FP8_STATIC)), sp.SP_OK),
    # (tp-1)*partial_stride + S*H elements must be a span of at most 2^47 bytes
    (dict(p=dict(partial_stride=2 ** 63 - 64)), sp.SP_ERR_SHAPE),       # wrapped to 0 before
    (dict(p=dict(partial_stride=2 ** 62)), sp.SP_ERR_SHAPE),
    (dict(p=dict(partial_stride=2 ** 43)), sp.SP_ERR_SHAPE),            # 7 * 2^44 bytes
    (dict(p=dict(partial_stride=2 ** 42), a=dict(out=BASE - 2 ** 30, residual=BASE - 2 ** 31,
                                                weight=BASE - 2 ** 32)), sp.SP_OK),
])
def test_written_bytes_may_not_be_read_or_span_too_far(case, expect):
    status, msg = validate(problem(**case.get("p", {})), **case.get("a", {}))
    assert status == expect, msg


def test_out_alignment_is_the_store_width():
    """out needs the width of one lane's 8-element store: 16 bytes for bf16
    and f32, 8 for e4m3, 4 for packed e2m1 (MX scale bytes need none)."""
    fp8 = dict(quant_mode=sp.SP_QUANT_DYNAMIC_TOKEN, out_scale=BASE + 5 * GB)
    mx = dict(quant_mode=sp.SP_QUANT_MX_BLOCK, out_scale=BASE + 5 * GB + 1)
    cases = [(sp.SP_BF16, {}, 8, sp.SP_ERR_ALIGN), (sp.SP_F32, {}, 8, sp.SP_ERR_ALIGN),
             (sp.SP_FP8_E4M3, fp8, 8, sp.SP_OK), (sp.SP_FP8_E4M3, fp8, 4, sp.SP_ERR_ALIGN),
             (sp.SP_FP8_E4M3, mx, 8, sp.SP_OK), (sp.SP_FP4_E2M1, mx, 4, sp.SP_OK),
             (sp.SP_FP4_E2M1, mx, 2, sp.SP_ERR_ALIGN), (sp.SP_BF16, {}, 16, sp.SP_OK)]
    for dt, q, off, want in cases:
        status, msg = validate(problem(out_dtype=dt), out=BASE + 3 * GB + off, **q)
        assert status == want, (dt, off, msg)


def test_one_partial_takes_any_stride_without_overflow():
    # with tp = 1 the stride addresses nothing, so the span check cannot bound
    # it; the alignment test must still hold without forming stride * 2 (the
    # products below overflow int64)
    one = dict(tp=1, tp_rank=0, num_tokens=128)
    assert validate(problem(partial_stride=2 ** 62, **one))[0] == sp.SP_OK
    assert validate(problem(partial_stride=2 ** 63 - 8, **one))[0] == sp.SP_OK
    assert validate(problem(partial_stride=2 ** 63 - 1, **one))[0] == sp.SP_ERR_ALIGN
    assert validate(problem(partial_stride=2 ** 62 + 4, partial_dtype=sp.SP_F32, **one))[0] == sp.SP_OK
    assert validate(problem(partial_stride=2 ** 62 + 2, partial_dtype=sp.SP_F32, **one))[0] == sp.SP_ERR_ALIGN


def test_strided_and_valid_rows_only_problems_pass():
    assert validate(problem(partial_stride=1024 * 4096))[0] == sp.SP_OK
    assert validate(problem(flags=sp.SP_FLAG_VALID_ROWS_ONLY))[0] == sp.SP_OK
    # with valid rows only, out may end right where the 104 valid rows end
    status, msg = validate(problem(flags=sp.SP_FLAG_VALID_ROWS_ONLY), out=BASE - 104 * 4096 * 2)
    assert status == sp.SP_OK, msg
    assert validate(problem(), out=BASE - 104 * 4096 * 2)[0] == sp.SP_ERR_SHAPE


def _gather(tp=2, S=4, H=16, T=8, dtype=sp.SP_BF16, shards=None, scales=None, out=BASE + 8 * GB,
            out_scale=None, sb=0):
    import ctypes as C
    lib = sp.load()
    g = sp.sp_gather_problem(tp=tp, dtype=dtype, shard_rows=S, hidden=H, num_tokens=T, scale_row_bytes=sb)
    shards = shards if shards is not None else [BASE + q * GB for q in range(tp)]
    src = (C.c_void_p * len(shards))(*shards)
    ssrc = None if scales is None else (C.c_void_p * len(scales))(*scales)
    return lib.sp_all_gather_unpad(C.byref(g), src, ssrc, out, out_scale, None), sp.sp_last_error()


@pytest.mark.parametrize("case,expect", [
    (dict(tp=0), sp.SP_ERR_SHAPE),
    (dict(tp=65, shards=[BASE] * 65), sp.SP_ERR_SHAPE),
    (dict(T=9), sp.SP_ERR_SHAPE),
    (dict(H=12), sp.SP_ERR_SHAPE),
    (dict(dtype=9), sp.SP_ERR_DTYPE),
    (dict(shards=[BASE, 0]), sp.SP_ERR_NULL),
    (dict(shards=[BASE, BASE + GB + 8]), sp.SP_ERR_ALIGN),
    (dict(out=BASE + 8 * GB + 4), sp.SP_ERR_ALIGN),
    (dict(out=BASE + 64), sp.SP_ERR_SHAPE),                        # out overlaps shard 0
    (dict(scales=[BASE + 4 * GB, BASE + 5 * GB]), sp.SP_ERR_NULL),  # no out_scale
    (dict(out_scale=BASE + 6 * GB), sp.SP_ERR_NULL),                # no shard scales
    # with scales (4 bytes a row): nothing written may overlap what is read, or each other
    # (only rejections here: an accepted call would launch on these fake addresses)
    (dict(sb=4, scales=[BASE + 4 * GB, BASE + 5 * GB], out_scale=BASE + GB + 16), sp.SP_ERR_SHAPE),
    (dict(sb=4, scales=[BASE + 4 * GB, BASE + 8 * GB + 64], out_scale=BASE + 6 * GB), sp.SP_ERR_SHAPE),
    (dict(sb=4, scales=[BASE + 4 * GB, BASE + 5 * GB], out_scale=BASE + 8 * GB + 240), sp.SP_ERR_SHAPE),
    (dict(sb=4, scales=[BASE + 4 * GB, BASE + 5 * GB], out_scale=BASE + 5 * GB + 12), sp.SP_ERR_SHAPE),
])
def test_gather_rejects_invalid_problems(case, expect):
    status, msg = _gather(**case)
    assert status == expect, msg


def test_gather_empty_is_a_no_op():
    assert _gather(T=0)[0] == sp.SP_OK
    assert _gather(S=0, T=0)[0] == sp.SP_OK


def _fc2(G=4, otp=2, dtype=sp.SP_BF16, N=8, Cc=8, rank=-1, src=None, dst=None):
    import ctypes as C
    lib = sp.load()
    f = sp.sp_fc2_problem(global_tp=G, otp=otp, dtype=dtype, rank=rank, tokens=N, cols=Cc)
    src = src if src is not None else [BASE + q * GB for q in range(G)]
    dst = dst if dst is not None else [BASE + (G + q) * GB for q in range(G)]
    s = (C.c_void_p * len(src))(*src)
    d = (C.c_void_p * len(dst))(*dst)
    return lib.sp_fc2_regroup(C.byref(f), s, d, None), sp.sp_last_error()


@pytest.mark.parametrize("case,expect", [
    (dict(G=1, otp=1, src=[BASE], dst=[BASE + GB]), sp.SP_ERR_SHAPE),
    (dict(G=65, otp=5, src=[BASE] * 65, dst=[BASE + GB] * 65), sp.SP_ERR_SHAPE),
    (dict(otp=4), sp.SP_ERR_SHAPE),                       # otp == G
    (dict(otp=3), sp.SP_ERR_SHAPE),                       # does not divide G
    (dict(otp=0), sp.SP_ERR_SHAPE),
    (dict(rank=4), sp.SP_ERR_SHAPE),
    (dict(rank=-2), sp.SP_ERR_SHAPE),
    (dict(rank=1, dst=[BASE + 4 * GB, 0, BASE + 6 * GB, BASE + 7 * GB]), sp.SP_ERR_NULL),
    # only dst[rank] is checked: NULL and overlapping unwritten entries are ignored, so the
    # call gets as far as the misaligned source
    (dict(rank=1, dst=[0, BASE + 5 * GB, BASE + 5 * GB, 0],
          src=[BASE, BASE + GB + 4, BASE + 2 * GB, BASE + 3 * GB]), sp.SP_ERR_ALIGN),
    (dict(dtype=sp.SP_FP4_E2M1), sp.SP_ERR_DTYPE),
    (dict(dtype=7), sp.SP_ERR_DTYPE),
    (dict(N=10), sp.SP_ERR_SHAPE),                        # not a multiple of G
    (dict(N=-4), sp.SP_ERR_SHAPE),
    (dict(N=1 << 31), sp.SP_ERR_SHAPE),
    (dict(Cc=3), sp.SP_ERR_SHAPE),                        # 6-byte rows
    (dict(Cc=0), sp.SP_ERR_SHAPE),
    (dict(G=64, otp=32, N=(1 << 31) - 64, Cc=1024, src=[BASE + q * GB for q in range(64)],
          dst=[BASE + (64 + q) * GB for q in range(64)]), sp.SP_ERR_SHAPE),  # grid too large
    (dict(G=2, otp=1, N=1 << 27, Cc=64, src=[BASE, BASE + 64 * GB],
          dst=[BASE + 128 * GB, BASE + 192 * GB]), sp.SP_ERR_SHAPE),  # grid fits, work-items do not
    (dict(src=[BASE, BASE + GB, 0, BASE + 3 * GB]), sp.SP_ERR_NULL),
    (dict(dst=[BASE + 4 * GB, BASE + 5 * GB, BASE + 6 * GB, 0]), sp.SP_ERR_NULL),
    (dict(src=[BASE, BASE + GB + 4, BASE + 2 * GB, BASE + 3 * GB]), sp.SP_ERR_ALIGN),  # 16-B rows
    (dict(dst=[BASE + 4 * GB, BASE + 5 * GB, BASE + 2 * GB + 16, BASE + 7 * GB]), sp.SP_ERR_SHAPE),
    (dict(dst=[BASE + 4 * GB, BASE + 5 * GB, BASE + 4 * GB + 16, BASE + 7 * GB]), sp.SP_ERR_SHAPE),
])
def test_fc2_regroup_rejects_invalid_problems(case, expect):
    status, msg = _fc2(**case)
    assert status == expect, msg
    if case.get("N") == 1 << 27:
        assert "dispatch" in msg
    if case.get("rank") == 1 and case.get("src"):
        assert "src[1]" in msg


def test_fc2_rank_mode_checks_only_its_own_destination():
    # dst[1] sits on top of dst[0], which rank 0's call does not write: the
    # call passes the pointer checks and stops at the dispatch limit
    status, msg = _fc2(G=2, otp=1, rank=0, N=1 << 27, Cc=64, src=[BASE, BASE + 64 * GB],
                       dst=[BASE + 128 * GB, BASE + 128 * GB + 16])
    assert status == sp.SP_ERR_SHAPE and "dispatch" in msg, msg


def _dsacp(tp=4, dtype=sp.SP_BF16, rank=-1, reserved=0, S=8, D=8, attn=None, out=None):
    import ctypes as C
    lib = sp.load()
    f = sp.sp_dsacp_problem(tp=tp, dtype=dtype, rank=rank, reserved=reserved, shard_rows=S,
                            head_cols=D)
    attn = attn if attn is not None else [BASE + q * GB for q in range(max(tp, 1))]
    out = out if out is not None else [BASE + (64 + q) * GB for q in range(max(tp, 1))]
    a = (C.c_void_p * len(attn))(*attn)
    o = (C.c_void_p * len(out))(*out)
    return lib.sp_dsacp_heads_to_tokens(C.byref(f), a, o, None), sp.sp_last_error()


@pytest.mark.parametrize("case,expect", [
    (dict(tp=0), sp.SP_ERR_SHAPE),
    (dict(tp=65, attn=[BASE] * 65, out=[BASE + GB] * 65), sp.SP_ERR_SHAPE),
    (dict(rank=4), sp.SP_ERR_SHAPE),
    (dict(rank=-2), sp.SP_ERR_SHAPE),
    (dict(reserved=3), sp.SP_ERR_UNSUPPORTED),
    (dict(dtype=sp.SP_FP4_E2M1), sp.SP_ERR_DTYPE),
    (dict(dtype=9), sp.SP_ERR_DTYPE),
    (dict(S=-1), sp.SP_ERR_SHAPE),
    (dict(S=1 << 29), sp.SP_ERR_SHAPE),                  # tp*S = 2^31
    (dict(D=0), sp.SP_ERR_SHAPE),
    (dict(D=1), sp.SP_ERR_SHAPE),                        # 2-byte pieces
    (dict(attn=[BASE, 0, BASE + 2 * GB, BASE + 3 * GB]), sp.SP_ERR_NULL),
    (dict(out=[BASE + 64 * GB, BASE + 65 * GB, 0, BASE + 67 * GB]), sp.SP_ERR_NULL),
    (dict(attn=[BASE, BASE + GB, BASE + 2 * GB + 8, BASE + 3 * GB]), sp.SP_ERR_ALIGN),
    (dict(D=2, out=[BASE + 64 * GB, BASE + 65 * GB + 2, BASE + 66 * GB, BASE + 67 * GB]),
     sp.SP_ERR_ALIGN),                                   # 4-byte pieces, 2-byte offset
    (dict(out=[BASE + 64 * GB, BASE + GB + 64, BASE + 66 * GB, BASE + 67 * GB]), sp.SP_ERR_SHAPE),
    (dict(out=[BASE + 64 * GB, BASE + 65 * GB, BASE + 64 * GB + 32, BASE + 67 * GB]),
     sp.SP_ERR_SHAPE),
    (dict(rank=2, out=[0, 0, BASE + 66 * GB, 0], S=1 << 24, D=8), sp.SP_ERR_SHAPE),  # dispatch
])
def test_dsacp_rejects_invalid_problems(case, expect):
    status, msg = _dsacp(**case)
    assert status == expect, msg
    if case.get("rank") == 2:
        assert "dispatch" in msg


def test_dsacp_empty_is_a_no_op():
    assert _dsacp(S=0)[0] == sp.SP_OK
    assert _dsacp(S=0, tp=1, attn=[BASE + 2], out=[BASE + GB + 2])[0] == sp.SP_OK


def test_fc2_regroup_empty_is_a_no_op():
    assert _fc2(N=0)[0] == sp.SP_OK
    # 4-byte rows need only 4-byte alignment; N == 0 never touches the pointers
    assert _fc2(N=0, Cc=2, src=[BASE + 4, BASE + GB, BASE + 2 * GB, BASE + 3 * GB])[0] == sp.SP_OK


def _mm(tp=4, rank=1, S=64, K=896, N=1024, in_dtype=sp.SP_BF16, out_dtype=sp.SP_F32, x=BASE,
        w=BASE + GB, dst=None, xs_rows=0, ws_rows=0, scaled=False, xs=BASE + 60 * GB,
        ws=BASE + 61 * GB):
    import ctypes as C
    lib = sp.load()
    p = sp.sp_matmul_problem(tp=tp, rank=rank, shard_rows=S, k=K, n=N, in_dtype=in_dtype,
                             out_dtype=out_dtype, x_scale_rows=xs_rows, w_scale_rows=ws_rows)
    dst = dst if dst is not None else [BASE + (2 + r) * GB for r in range(max(tp, 1))]
    d = (C.c_void_p * len(dst))(*dst)
    if scaled:
        rc = lib.sp_scaled_matmul_scatter(C.byref(p), x, xs, w, ws, d, None)
    else:
        rc = lib.sp_matmul_scatter(C.byref(p), x, w, d, None)
    return rc, sp.sp_last_error()


FP8 = dict(scaled=True, in_dtype=sp.SP_FP8_E4M3, xs_rows=1, ws_rows=1)


@pytest.mark.parametrize("case,expect", [
    (dict(FP8, in_dtype=sp.SP_BF16), sp.SP_ERR_DTYPE),
    (dict(FP8, K=24), sp.SP_ERR_SHAPE),                  # e4m3 chunks are 16 elements
    (dict(FP8, K=8), sp.SP_ERR_SHAPE),
    (dict(FP8, xs_rows=3), sp.SP_ERR_SHAPE),             # neither 1 nor M = 256
    (dict(FP8, xs_rows=0), sp.SP_ERR_SHAPE),
    (dict(FP8, ws_rows=1023), sp.SP_ERR_SHAPE),          # neither 1 nor N = 1024
    (dict(FP8, xs=0), sp.SP_ERR_NULL),
    (dict(FP8, ws=0), sp.SP_ERR_NULL),
    (dict(FP8, xs=BASE + 60 * GB + 2), sp.SP_ERR_ALIGN),
    # slot 1 of dst[2] starts at BASE + 4 GB + 64*1024*4: a per-token scale there overlaps it
    (dict(FP8, xs_rows=256, xs=BASE + 4 * GB + 64 * 1024 * 4), sp.SP_ERR_SHAPE),
    (dict(xs_rows=1), sp.SP_ERR_SHAPE),                   # the bf16 entry takes no scales
    (dict(in_dtype=sp.SP_FP8_E4M3), sp.SP_ERR_DTYPE),     # e4m3 goes through the scaled entry
])
def test_scaled_matmul_scatter_rejects_invalid_problems(case, expect):
    status, msg = _mm(**case)
    assert status == expect, msg


def test_scaled_matmul_scatter_empty_is_a_no_op():
    assert _mm(S=0, x=0, w=0, **FP8)[0] == sp.SP_OK


@pytest.mark.parametrize("case,expect", [
    (dict(tp=0), sp.SP_ERR_SHAPE),
    (dict(tp=65, dst=[BASE + (2 + r) * GB for r in range(65)]), sp.SP_ERR_SHAPE),
    (dict(rank=4), sp.SP_ERR_SHAPE),
    (dict(rank=-1), sp.SP_ERR_SHAPE),
    (dict(in_dtype=sp.SP_F32), sp.SP_ERR_DTYPE),
    (dict(out_dtype=sp.SP_FP8_E4M3), sp.SP_ERR_DTYPE),
    (dict(S=-1), sp.SP_ERR_SHAPE),
    (dict(S=1 << 29), sp.SP_ERR_SHAPE),                   # tp*S = 2^31
    (dict(K=4), sp.SP_ERR_SHAPE),
    (dict(K=900), sp.SP_ERR_SHAPE),
    (dict(K=(1 << 20) + 8), sp.SP_ERR_SHAPE),
    (dict(N=1028), sp.SP_ERR_SHAPE),
    (dict(x=0), sp.SP_ERR_NULL),
    (dict(w=0), sp.SP_ERR_NULL),
    (dict(dst=[BASE + 2 * GB, 0, BASE + 4 * GB, BASE + 5 * GB]), sp.SP_ERR_NULL),
    (dict(x=BASE + 8), sp.SP_ERR_ALIGN),
    (dict(dst=[BASE + 2 * GB, BASE + 3 * GB + 4, BASE + 4 * GB, BASE + 5 * GB]), sp.SP_ERR_ALIGN),
    # slot 1 of dst[0] (bytes [64*1024*4, 2*64*1024*4)) on top of x
    (dict(dst=[BASE - 64 * 1024 * 4, BASE + 3 * GB, BASE + 4 * GB, BASE + 5 * GB]), sp.SP_ERR_SHAPE),
    # slots of two destinations overlap
    (dict(dst=[BASE + 2 * GB, BASE + 2 * GB + 1024, BASE + 4 * GB, BASE + 5 * GB]), sp.SP_ERR_SHAPE),
])
def test_matmul_scatter_rejects_invalid_problems(case, expect):
    status, msg = _mm(**case)
    assert status == expect, msg


def test_matmul_scatter_empty_is_a_no_op():
    assert _mm(S=0, x=0, w=0)[0] == sp.SP_OK


def test_null_descriptor():
    lib = sp.load()
    assert lib.sp_validate(None, None, None, None, None, 0.0, 0, None, None, None) == sp.SP_ERR_NULL


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((2, 4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sp.sp_reduce_add_rmsnorm(x, x[0], x[0, 0], None, 1e-6, 0, None, x[0], None, tp_rank=0,
                                 num_tokens=8)
    with pytest.raises(ValueError):
        sp.sp_all_gather_unpad([x[0], x[1]], None, torch.zeros((8, 8), dtype=torch.bfloat16),
                               None, num_tokens=8)
    with pytest.raises(ValueError):
        sp.sp_fc2_regroup([x[0], x[1]], [x[0].clone(), x[1].clone()], otp=1)
    with pytest.raises(ValueError):
        sp.sp_dsacp_heads_to_tokens([x[0], x[1]], [x[0].clone(), x[1].clone()])
    with pytest.raises(ValueError):
        sp.sp_matmul_scatter(x[0], x[1], [x.clone()], rank=0)


def test_plain_c_client_compiles_links_and_runs(tmp_path):
    """A C program that includes only include/sprms.h builds with gcc, links
    against libsprms.so and gets the documented answers from the host-only
    entry points."""
    sp.load()
    exe = tmp_path / "c_abi_check"
    lib_dir = os.path.dirname(sp.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe), "-L", lib_dir,
                    "-lsprms", f"-Wl,-rpath,{lib_dir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "c abi ok" in out.stdout


def test_last_error_is_per_thread():
    """Calls on several threads at once: each thread reads back the detail of
    its own last failure (the library keeps no other state across calls)."""
    import threading

    cases = {
        "tp": (problem(tp=0), {}),
        "hidden": (problem(hidden=4100), {}),
        "quant": (problem(), dict(quant_mode=3)),
        "align": (problem(), dict(partials=BASE + 8)),
    }
    expect = {"tp": "tp=0", "hidden": "hidden=4100", "quant": "quant_mode=3", "align": "aligned"}
    errors = []
    barrier = threading.Barrier(len(cases))

    def worker(name):
        p, kw = cases[name]
        barrier.wait()
        for _ in range(200):
            status, msg = validate(p, **kw)
            if status == sp.SP_OK or expect[name] not in msg:
                errors.append((name, status, msg))
                return

    threads = [threading.Thread(target=worker, args=(n,)) for n in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


# sizes so large that multiplying them first would wrap int64 past the range
# checks: each must be rejected, never accepted as a small or empty problem
TP64 = dict(tp=64, dst=[BASE + (2 + r) * GB for r in range(64)])


@pytest.mark.parametrize("case", [
    dict(TP64, S=1 << 58),            # 64 * 2^58 = 2^64 wraps to 0
    dict(TP64, S=(1 << 57) + 1),      # wraps negative
    dict(S=(1 << 62) + 3),            # tp = 4: wraps to 12
])
def test_matmul_scatter_rejects_shard_rows_that_would_wrap(case):
    status, msg = _mm(**case)
    assert status == sp.SP_ERR_SHAPE, msg


@pytest.mark.parametrize("case", [
    dict(tp=64, S=1 << 58, attn=[BASE + q * GB for q in range(64)], out=[BASE + (64 + q) * GB for q in range(64)]),
    dict(S=(1 << 62) + 2),
    dict(D=1 << 62),                  # head_cols * 2 bytes * tp wraps
    dict(D=(1 << 61) + 2),
])
def test_dsacp_rejects_sizes_that_would_wrap(case):
    status, msg = _dsacp(**case)
    assert status == sp.SP_ERR_SHAPE, msg


@pytest.mark.parametrize("Cc", [1 << 62, (1 << 61) + 2, (1 << 60) + 2])
def test_fc2_rejects_cols_that_would_wrap(Cc):
    status, msg = _fc2(Cc=Cc)
    assert status == sp.SP_ERR_SHAPE, msg

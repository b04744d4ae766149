"""ctypes wrapper around the plain C oracle (``sprms_oracle.c``).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Inputs are numpy
arrays: float32 arrays for f32 tensors and uint16 arrays holding raw
bfloat16 bit patterns for bf16 tensors.  The wrapper only marshals arrays;
every step of the computation is in the C file.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

ORC_F32, ORC_BF16, ORC_E4M3, ORC_E2M1 = 0, 1, 2, 3
QUANT_NONE, QUANT_STATIC_TENSOR, QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK = 0, 1, 2, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sprms_oracle.c")
# SPRMS_ORACLE_LIB lets the mutation tests load a deliberately broken copy.
_LIB = os.environ.get("SPRMS_ORACLE_LIB") or os.path.join(_HERE, "liboracle_sprms.so")

# -ffp-contract=off keeps every double operation as written (no fused
# multiply-add), so the oracle's arithmetic is exactly what its source says.
GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
           "-Wextra", "-fPIC", "-shared", "-o", _LIB, _SRC, "-lm"]


class OracleError(RuntimeError):
    pass


class _Problem(C.Structure):
    _fields_ = [
        ("tp", C.c_int32),
        ("tp_rank", C.c_int32),
        ("shard_rows", C.c_int64),
        ("hidden", C.c_int64),
        ("num_tokens", C.c_int64),
        ("partial_dtype", C.c_int32),
        ("act_dtype", C.c_int32),
        ("out_dtype", C.c_int32),
        ("residual_rows", C.c_int64),
        ("deepstack_rows", C.c_int64),
        ("partial_scale", C.c_double),
    ]


class AbiProblem(C.Structure):
    """The descriptor of sp_oracle_reduce_add_rmsnorm: the library
    descriptor's field layout, defined here on its own."""
    _fields_ = [
        ("tp", C.c_int32),
        ("tp_rank", C.c_int32),
        ("shard_rows", C.c_int64),
        ("hidden", C.c_int64),
        ("num_tokens", C.c_int64),
        ("partial_dtype", C.c_int32),
        ("act_dtype", C.c_int32),
        ("out_dtype", C.c_int32),
        ("residual_rows", C.c_int64),
        ("deepstack_rows", C.c_int64),
        ("residual_out", C.c_void_p),
        ("partial_stride", C.c_int64),
        ("flags", C.c_int32),
        ("partial_scale", C.c_float),
    ]


def build() -> str:
    """Compile the oracle with gcc (always; used by the repository build step)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = C.CDLL(_LIB)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    lib.orc_shard_geometry.argtypes = [i64, i64, i32, i32, C.POINTER(i64), C.POINTER(i64),
                                       C.POINTER(i64)]
    lib.orc_shard_geometry.restype = C.c_int
    lib.orc_reduce_add_rmsnorm.argtypes = [
        C.POINTER(_Problem), vp, vp, vp, vp, C.c_float, i32, vp, C.c_float, i64, vp, vp, vp,
        vp, vp, vp]
    lib.orc_reduce_add_rmsnorm.restype = C.c_int
    lib.sp_oracle_reduce_add_rmsnorm.argtypes = [C.POINTER(AbiProblem), vp, vp, vp, vp, C.c_float,
                                                 C.c_int, vp, vp, vp, vp]
    lib.sp_oracle_reduce_add_rmsnorm.restype = C.c_int
    lib.orc_bf16_from_double.argtypes = [C.c_double]
    lib.orc_bf16_from_double.restype = C.c_uint16
    lib.orc_bf16_to_double.argtypes = [C.c_uint16]
    lib.orc_bf16_to_double.restype = C.c_double
    lib.orc_e4m3_from_double.argtypes = [C.c_double]
    lib.orc_e4m3_from_double.restype = C.c_uint8
    lib.orc_e4m3_to_double.argtypes = [C.c_uint8]
    lib.orc_e4m3_to_double.restype = C.c_double
    lib.orc_all_gather_unpad.argtypes = [i32, i64, i64, i64, C.POINTER(vp), i64, C.POINTER(vp),
                                         vp, vp]
    lib.orc_all_gather_unpad.restype = C.c_int
    lib.orc_fc2_batch_ids.argtypes = [i32, i32, vp]
    lib.orc_fc2_batch_ids.restype = C.c_int
    lib.orc_fc2_regroup.argtypes = [i32, i32, i64, i64, i32, C.POINTER(vp), C.POINTER(vp)]
    lib.orc_fc2_regroup.restype = C.c_int
    lib.orc_dsacp_heads_to_tokens.argtypes = [i32, i64, i64, C.POINTER(vp), C.POINTER(vp)]
    lib.orc_dsacp_heads_to_tokens.restype = C.c_int
    lib.orc_matmul_scatter.argtypes = [i32, i32, i64, i64, i64, i32, vp, vp, i64, vp,
                                       C.POINTER(vp)]
    lib.orc_matmul_scatter.restype = C.c_int
    lib.orc_scaled_matmul_scatter.argtypes = [i32, i32, i64, i64, i64, i32, vp, vp, i64, vp, vp, i64,
                                              i64, vp, C.POINTER(vp)]
    lib.orc_scaled_matmul_scatter.restype = C.c_int
    lib.orc_e2m1_from_double.argtypes = [C.c_double]
    lib.orc_e2m1_from_double.restype = C.c_uint8
    lib.orc_e2m1_to_double.argtypes = [C.c_uint8]
    lib.orc_e2m1_to_double.restype = C.c_double
    lib.orc_e2m1_from_double_n.argtypes = [vp, i64, vp]
    lib.orc_e2m1_from_double_n.restype = None
    lib.orc_bf16_from_double_n.argtypes = [vp, i64, vp]
    lib.orc_bf16_from_double_n.restype = None
    lib.orc_e4m3_from_double_n.argtypes = [vp, i64, vp]
    lib.orc_e4m3_from_double_n.restype = None
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ORC_F32
    if a.dtype == np.uint16:
        return ORC_BF16
    raise OracleError(f"unsupported array dtype {a.dtype} (float32 or uint16 bf16 bits)")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def shard_geometry(num_tokens: int, num_tokens_pad: int, tp: int, rank: int):
    """(shard_rows, local_start, valid_rows) for rank's contiguous shard."""
    lib = _load()
    s, st, v = C.c_int64(), C.c_int64(), C.c_int64()
    rc = lib.orc_shard_geometry(num_tokens, num_tokens_pad, tp, rank, C.byref(s), C.byref(st),
                                C.byref(v))
    if rc != 0:
        raise OracleError(f"orc_shard_geometry failed: {rc}")
    return s.value, st.value, v.value


def reduce_add_rmsnorm(partials, residual, weight, bias, eps, quant_mode, deepstack=None, *,
                       tp_rank, num_tokens, out_dtype=ORC_BF16, static_scale=1.0, rows=None,
                       want_debug=True, partial_scale=1.0):
    """Run the oracle on host arrays.

    partials [tp, S, H]; residual [S or tp*S, H]; weight/bias [H];
    deepstack None or [S or tp*S, H].  ``rows`` selects shard rows (default
    all).  Returns a dict with residual_out, out (uint16 bf16 bits, float32 or
    uint8 e4m3 codes), out_scale (dynamic mode), z and y (float64, if
    ``want_debug``), all compact over the selected rows.
    """
    lib = _load()
    partials = np.ascontiguousarray(partials)
    residual = np.ascontiguousarray(residual)
    weight = np.ascontiguousarray(weight)
    bias = None if bias is None else np.ascontiguousarray(bias)
    deepstack = None if deepstack is None else np.ascontiguousarray(deepstack)
    tp, S, H = partials.shape
    act = _dtype_code(residual)
    for name, a in (("weight", weight), ("bias", bias), ("deepstack", deepstack)):
        if a is not None and _dtype_code(a) != act:
            raise OracleError(f"{name} dtype differs from the residual dtype")
    if quant_mode != QUANT_NONE and not (quant_mode == QUANT_MX_BLOCK and out_dtype == ORC_E2M1):
        out_dtype = ORC_E4M3
    prob = _Problem(tp=tp, tp_rank=tp_rank, shard_rows=S, hidden=H, num_tokens=num_tokens,
                    partial_dtype=_dtype_code(partials), act_dtype=act, out_dtype=out_dtype,
                    residual_rows=residual.shape[0],
                    deepstack_rows=0 if deepstack is None else deepstack.shape[0],
                    partial_scale=float(partial_scale))
    if rows is None:
        n = S
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.shape[0]
    res_out = np.zeros((n, H), dtype=residual.dtype)
    out_np = {ORC_F32: np.float32, ORC_BF16: np.uint16, ORC_E4M3: np.uint8, ORC_E2M1: np.uint8}
    out = np.zeros((n, H // 2 if out_dtype == ORC_E2M1 else H), dtype=out_np[out_dtype])
    if quant_mode == QUANT_MX_BLOCK:
        scale = np.zeros((n, H // 32), dtype=np.uint8)
    else:
        scale = np.zeros((n,), dtype=np.float32)
    z = np.zeros((n, H), dtype=np.float64) if want_debug else None
    y = np.zeros((n, H), dtype=np.float64) if want_debug else None
    rc = lib.orc_reduce_add_rmsnorm(C.byref(prob), _ptr(partials), _ptr(residual), _ptr(weight),
                                    _ptr(bias), float(eps), quant_mode, _ptr(deepstack),
                                    float(static_scale), n, _ptr(rows_arr), _ptr(res_out),
                                    _ptr(out), _ptr(scale), _ptr(z), _ptr(y))
    if rc != 0:
        raise OracleError(f"orc_reduce_add_rmsnorm failed: {rc}")
    result = {"residual_out": res_out, "out": out, "z": z, "y": y}
    if quant_mode in (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK):
        result["out_scale"] = scale
    return result


def sp_oracle_reduce_add_rmsnorm(problem: AbiProblem, partials, residual, weight, bias, eps,
                                 quant_mode, deepstack, out, out_scale) -> int:
    """The fused call with the library entry point's arguments, on host
    arrays (written in place: out, out_scale, problem.residual_out or the
    residual).  Returns the C status code."""
    lib = _load()
    return lib.sp_oracle_reduce_add_rmsnorm(C.byref(problem), _ptr(partials), _ptr(residual),
                                            _ptr(weight), _ptr(bias), float(eps), int(quant_mode),
                                            _ptr(deepstack), _ptr(out), _ptr(out_scale), None)


def bf16_from_double(x: float) -> int:
    return int(_load().orc_bf16_from_double(float(x)))


def bf16_to_double(bits: int) -> float:
    return float(_load().orc_bf16_to_double(int(bits)))


def e4m3_from_double(x: float) -> int:
    return int(_load().orc_e4m3_from_double(float(x)))


def e4m3_to_double(code: int) -> float:
    return float(_load().orc_e4m3_to_double(int(code)))


def bf16_from_double_array(x) -> np.ndarray:
    """Element-wise orc_bf16_from_double over a float64 array (uint16 bits)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_bf16_from_double_n(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_from_double_array(x) -> np.ndarray:
    """Element-wise orc_e4m3_from_double over a float64 array (uint8 codes)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_from_double_n(_ptr(x), x.size, _ptr(out))
    return out


def all_gather_unpad(shards, scales=None, *, num_tokens):
    """Gather tp host shard outputs [S, ...] (rows of any byte width) into
    [T, ...]; per-row scales [S, ...] likewise.  Returns (out, out_scale or None)."""
    lib = _load()
    shards = [np.ascontiguousarray(a) for a in shards]
    tp = len(shards)
    S = shards[0].shape[0]
    # row widths from the shapes, so that empty shards (S = 0) keep them
    row_bytes = int(np.prod(shards[0].shape[1:], dtype=np.int64)) * shards[0].dtype.itemsize
    out = np.zeros((num_tokens,) + shards[0].shape[1:], dtype=shards[0].dtype)
    src = (C.c_void_p * tp)(*[a.ctypes.data for a in shards])
    ssrc, out_scale, srow = None, None, 0
    if scales is not None:
        scales = [np.ascontiguousarray(a) for a in scales]
        ssrc = (C.c_void_p * tp)(*[a.ctypes.data for a in scales])
        srow = int(np.prod(scales[0].shape[1:], dtype=np.int64)) * scales[0].dtype.itemsize
        out_scale = np.zeros((num_tokens,) + scales[0].shape[1:], dtype=scales[0].dtype)
    rc = lib.orc_all_gather_unpad(tp, S, row_bytes, num_tokens, src, srow, ssrc, _ptr(out),
                                  _ptr(out_scale))
    if rc != 0:
        raise OracleError(f"orc_all_gather_unpad failed: {rc}")
    return out, out_scale


def e2m1_from_double(x: float) -> int:
    return int(_load().orc_e2m1_from_double(float(x)))


def e2m1_to_double(code: int) -> float:
    return float(_load().orc_e2m1_to_double(int(code)))


def e2m1_from_double_array(x) -> np.ndarray:
    """Element-wise orc_e2m1_from_double over a float64 array (one code per uint8)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e2m1_from_double_n(_ptr(x), x.size, _ptr(out))
    return out


def fc2_batch_ids(G: int, otp: int):
    """Reorganised batch ids: for each destination position j of an ODP group,
    the token segments it receives."""
    odp = G // otp
    ids = np.zeros((odp, otp), dtype=np.int32)
    rc = _load().orc_fc2_batch_ids(G, otp, _ptr(ids))
    if rc != 0:
        raise OracleError(f"orc_fc2_batch_ids failed: {rc}")
    return ids.tolist()


def fc2_regroup(srcs, otp: int):
    """Regroup G host arrays [N, C] (rank q's features of all tokens) into G
    arrays [N/odp, odp*C]."""
    lib = _load()
    srcs = [np.ascontiguousarray(a) for a in srcs]
    G = len(srcs)
    N, Cc = srcs[0].shape
    odp = G // otp
    dsts = [np.zeros((N // odp, odp * Cc), dtype=srcs[0].dtype) for _ in range(G)]
    sp_ = (C.c_void_p * G)(*[a.ctypes.data for a in srcs])
    dp_ = (C.c_void_p * G)(*[a.ctypes.data for a in dsts])
    rc = lib.orc_fc2_regroup(G, otp, N, Cc, srcs[0].dtype.itemsize, sp_, dp_)
    if rc != 0:
        raise OracleError(f"orc_fc2_regroup failed: {rc}")
    return dsts


def dsacp_heads_to_tokens(attn):
    """DSA-CP o_proj input exchange: tp host arrays [S, tp*D] (rank p's local
    tokens, every rank's heads) -> tp arrays [tp*S, D] (every token, rank q's
    heads)."""
    lib = _load()
    attn = [np.ascontiguousarray(a) for a in attn]
    tp = len(attn)
    S, W = attn[0].shape
    if W % tp:
        raise OracleError("row width is not a multiple of tp")
    D = W // tp
    outs = [np.zeros((tp * S, D), dtype=attn[0].dtype) for _ in range(tp)]
    ap = (C.c_void_p * tp)(*[a.ctypes.data for a in attn])
    op = (C.c_void_p * tp)(*[a.ctypes.data for a in outs])
    rc = lib.orc_dsacp_heads_to_tokens(tp, S, D * attn[0].dtype.itemsize, ap, op)
    if rc != 0:
        raise OracleError(f"orc_dsacp_heads_to_tokens failed: {rc}")
    return outs


def matmul_scatter(x, w, *, tp, rank, out_dtype=ORC_F32, rows=None, dst=None):
    """Rank `rank`'s row-parallel GEMM P = x w^T (x [tp*S, K], w [N, K], bf16
    bits as uint16) written into the tp receive buffers [tp][S][N] (slot
    `rank` of each).  ``dst`` may be given to collect several ranks' slots;
    ``rows`` selects the token rows computed."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    M, K = x.shape
    N = w.shape[0]
    if M % tp or w.shape[1] != K:
        raise OracleError("x must be [tp*S, K] and w [N, K]")
    S = M // tp
    dt = np.float32 if out_dtype == ORC_F32 else np.uint16
    if dst is None:
        dst = [np.zeros((tp, S, N), dtype=dt) for _ in range(tp)]
    dp = (C.c_void_p * tp)(*[d.ctypes.data for d in dst])
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib.orc_matmul_scatter(tp, rank, S, K, N, out_dtype, _ptr(x), _ptr(w),
                                0 if r is None else len(r), None if r is None else _ptr(r), dp)
    if rc != 0:
        raise OracleError(f"orc_matmul_scatter failed: {rc}")
    return dst


def scaled_matmul_scatter(x, x_scale, w, w_scale, *, tp, rank, out_dtype=ORC_F32, rows=None,
                          dst=None):
    """FP8 producer: x [tp*S, K] and w [N, K] e4m3 codes (uint8), x_scale
    [1] or [tp*S] and w_scale [1] or [N] float32; P = (x w^T) x_scale w_scale
    written into slot `rank` of the tp receive buffers [tp][S][N]."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xs = np.ascontiguousarray(x_scale, dtype=np.float32).reshape(-1)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32).reshape(-1)
    M, K = x.shape
    N = w.shape[0]
    if M % tp or w.shape[1] != K:
        raise OracleError("x must be [tp*S, K] and w [N, K]")
    S = M // tp
    dt = np.float32 if out_dtype == ORC_F32 else np.uint16
    if dst is None:
        dst = [np.zeros((tp, S, N), dtype=dt) for _ in range(tp)]
    dp = (C.c_void_p * tp)(*[d.ctypes.data for d in dst])
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib.orc_scaled_matmul_scatter(tp, rank, S, K, N, out_dtype, _ptr(x), _ptr(xs), xs.size,
                                       _ptr(w), _ptr(ws), ws.size, 0 if r is None else len(r),
                                       None if r is None else _ptr(r), dp)
    if rc != 0:
        raise OracleError(f"orc_scaled_matmul_scatter failed: {rc}")
    return dst

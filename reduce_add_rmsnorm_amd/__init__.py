"""Python binding of libsprms: fused sequence-parallel reduce + add + RMSNorm (+FP8)
for one rank's token shard on MI355X (gfx950).

The functions here have the names of the C entry points in include/sprms.h
and only marshal arguments: torch tensors are passed as device pointers, the
stream is torch's current HIP stream.  Every step of the computation runs in
the HIP kernels of libsprms.so; there is no other implementation behind these
names, and they raise if the library is not built.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

from .inputs import QUANT_DYNAMIC_TOKEN, QUANT_NONE, QUANT_STATIC_TENSOR  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsprms.so")

# sp_dtype
SP_F32, SP_BF16, SP_FP8_E4M3, SP_FP4_E2M1 = 0, 1, 2, 3
# sp_quant (3 is reserved for dynamic per-tensor scaling and always rejected)
SP_QUANT_NONE, SP_QUANT_STATIC_TENSOR, SP_QUANT_DYNAMIC_TOKEN, SP_QUANT_MX_BLOCK = 0, 1, 2, 4
# sp_status
SP_OK, SP_ERR_NULL, SP_ERR_SHAPE, SP_ERR_DTYPE, SP_ERR_ALIGN, SP_ERR_UNSUPPORTED, SP_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)

EXPORTED = ("sp_reduce_add_rmsnorm", "sp_validate", "sp_all_gather_unpad", "sp_fc2_regroup",
            "sp_dsacp_heads_to_tokens", "sp_matmul_scatter", "sp_scaled_matmul_scatter",
            "sp_shard_geometry",
            "sp_error_string", "sp_last_error")
SP_FLAG_VALID_ROWS_ONLY = 1


class SprmsError(RuntimeError):
    """A libsprms call returned a non-zero sp_status; `status` holds it and the
    message the library's detail (sp_last_error) for that call."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class sp_problem(C.Structure):
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


class sp_gather_problem(C.Structure):
    _fields_ = [
        ("tp", C.c_int32),
        ("dtype", C.c_int32),
        ("shard_rows", C.c_int64),
        ("hidden", C.c_int64),
        ("num_tokens", C.c_int64),
        ("scale_row_bytes", C.c_int64),
    ]


class sp_fc2_problem(C.Structure):
    _fields_ = [
        ("global_tp", C.c_int32),
        ("otp", C.c_int32),
        ("dtype", C.c_int32),
        ("rank", C.c_int32),
        ("tokens", C.c_int64),
        ("cols", C.c_int64),
    ]


class sp_dsacp_problem(C.Structure):
    _fields_ = [
        ("tp", C.c_int32),
        ("dtype", C.c_int32),
        ("rank", C.c_int32),
        ("reserved", C.c_int32),
        ("shard_rows", C.c_int64),
        ("head_cols", C.c_int64),
    ]


class sp_matmul_problem(C.Structure):
    _fields_ = [
        ("tp", C.c_int32),
        ("rank", C.c_int32),
        ("shard_rows", C.c_int64),
        ("k", C.c_int64),
        ("n", C.c_int64),
        ("in_dtype", C.c_int32),
        ("out_dtype", C.c_int32),
        ("x_scale_rows", C.c_int64),
        ("w_scale_rows", C.c_int64),
    ]


_lib = None


def load(build_if_missing: bool = False):
    """Load libsprms.so (the built HIP library); raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise ImportError(f"{LIB_PATH} is not built: run `python -m reduce_add_rmsnorm_amd.build`")
        from .build import build_library
        build_library()
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.sp_reduce_add_rmsnorm.argtypes = [C.POINTER(sp_problem), vp, vp, vp, vp, C.c_float, C.c_int,
                                          vp, vp, vp, vp]
    lib.sp_reduce_add_rmsnorm.restype = C.c_int
    lib.sp_validate.argtypes = [C.POINTER(sp_problem), vp, vp, vp, vp, C.c_float, C.c_int, vp, vp,
                                vp]
    lib.sp_validate.restype = C.c_int
    lib.sp_all_gather_unpad.argtypes = [C.POINTER(sp_gather_problem), C.POINTER(vp),
                                        C.POINTER(vp), vp, vp, vp]
    lib.sp_all_gather_unpad.restype = C.c_int
    lib.sp_fc2_regroup.argtypes = [C.POINTER(sp_fc2_problem), C.POINTER(vp), C.POINTER(vp), vp]
    lib.sp_fc2_regroup.restype = C.c_int
    lib.sp_dsacp_heads_to_tokens.argtypes = [C.POINTER(sp_dsacp_problem), C.POINTER(vp),
                                             C.POINTER(vp), vp]
    lib.sp_dsacp_heads_to_tokens.restype = C.c_int
    lib.sp_matmul_scatter.argtypes = [C.POINTER(sp_matmul_problem), vp, vp, C.POINTER(vp), vp]
    lib.sp_matmul_scatter.restype = C.c_int
    lib.sp_scaled_matmul_scatter.argtypes = [C.POINTER(sp_matmul_problem), vp, vp, vp, vp,
                                             C.POINTER(vp), vp]
    lib.sp_scaled_matmul_scatter.restype = C.c_int
    lib.sp_shard_geometry.argtypes = [i64, i64, i32, i32, C.POINTER(i64), C.POINTER(i64),
                                      C.POINTER(i64)]
    lib.sp_shard_geometry.restype = C.c_int
    lib.sp_error_string.argtypes = [C.c_int]
    lib.sp_error_string.restype = C.c_char_p
    lib.sp_last_error.argtypes = []
    lib.sp_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def _sp_dtype(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return SP_F32
    if dt == torch.bfloat16:
        return SP_BF16
    if dt in (torch.uint8, torch.float8_e4m3fn):
        return SP_FP8_E4M3
    if dt == torch.float4_e2m1fn_x2:
        return SP_FP4_E2M1
    raise TypeError(f"unsupported tensor dtype {dt}")


def _addr(x) -> Optional[int]:
    """Device address of a tensor (must be contiguous), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensors passed to libsprms must be contiguous")
    return x.data_ptr()


def _same_device(*tensors):
    """Every tensor given (None entries and lists of tensors allowed) is on the
    same GPU; returns that device.  A host tensor would hand the kernels a
    host address."""
    flat = []
    for t in tensors:
        if isinstance(t, (list, tuple)):
            flat.extend(x for x in t if x is not None)
        elif t is not None:
            flat.append(t)
    flat = [t for t in flat if not isinstance(t, int)]
    if not flat:
        raise ValueError("no tensor arguments")
    dev = flat[0].device
    for t in flat:
        if not t.is_cuda:
            raise ValueError("libsprms takes device tensors only (got a host tensor)")
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")
    return dev


def _stream_handle(device, stream):
    """hipStream_t of `stream` (a torch stream or a raw int handle); torch's
    current stream on `device` when None."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int):
    if status != SP_OK:
        raise SprmsError(status, sp_last_error())


def _partials_stride(partials) -> int:
    """Element stride between partials; rows within a partial must be packed."""
    tp, S, H = partials.shape
    if partials.stride(2) != 1 or (S > 1 and partials.stride(1) != H):
        raise ValueError("partials rows must be contiguous [S][H] blocks")
    return partials.stride(0) if tp > 1 else S * H


def make_problem(partials, residual, out, *, tp_rank: int, num_tokens: int, deepstack=None,
                 residual_out=None, valid_rows_only: bool = False,
                 out_dtype: Optional[int] = None, partial_scale: float = 1.0) -> sp_problem:
    """sp_problem from tensor shapes, strides and dtypes.  ``partials`` may be a
    [tp, S, H] view of a larger buffer (e.g. rows [r*S, (r+1)*S) of a
    [tp, T_pad, H] tensor) as long as each partial's rows are packed.
    ``out_dtype`` overrides the type inferred from ``out`` (e.g. SP_FP4_E2M1
    for a uint8 [S, H/2] buffer of packed codes)."""
    tp, S, H = partials.shape
    stride = _partials_stride(partials)
    return sp_problem(tp=tp, tp_rank=tp_rank, shard_rows=S, hidden=H, num_tokens=num_tokens,
                      partial_dtype=_sp_dtype(partials.dtype), act_dtype=_sp_dtype(residual.dtype),
                      out_dtype=_sp_dtype(out.dtype) if out_dtype is None else out_dtype,
                      residual_rows=residual.shape[0],
                      deepstack_rows=0 if deepstack is None else deepstack.shape[0],
                      residual_out=_addr(residual_out),
                      partial_stride=0 if stride == S * H else stride,
                      flags=SP_FLAG_VALID_ROWS_ONLY if valid_rows_only else 0,
                      partial_scale=partial_scale)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_fused_sizes(partials, residual, weight, bias, quant_mode, deepstack, out, out_scale, *,
                       tp_rank, num_tokens, residual_out, valid_rows_only, out_dtype):
    """Tensor sizes against what the kernels will touch.  The C ABI sees only
    pointers, so this is the one place a buffer that is too small for the
    descriptor built from `partials` is caught; int addresses are taken as
    given."""
    if partials.dim() != 3:
        raise ValueError("partials must be [tp, S, H]")
    tp, S, H = partials.shape
    rows = max(0, min(S, num_tokens - tp_rank * S)) if valid_rows_only else S
    act = residual.dtype if isinstance(residual, torch.Tensor) else None

    def rows_h(t, name, min_rows, rows_exact=None):
        if not isinstance(t, torch.Tensor):
            return
        if t.dim() != 2 or t.shape[1] != H:
            raise ValueError(f"{name} must be [rows, H={H}], got {tuple(t.shape)}")
        if rows_exact is not None and t.shape[0] not in rows_exact:
            raise ValueError(f"{name} must have {' or '.join(map(str, rows_exact))} rows, got {t.shape[0]}")
        if t.shape[0] < min_rows:
            raise ValueError(f"{name} has {t.shape[0]} rows, the call writes {min_rows}")
        if act is not None and t.dtype != act:
            raise ValueError(f"{name} must have the residual's dtype {act}, got {t.dtype}")

    rows_h(residual, "residual", 0, (S, tp * S))
    if deepstack is not None:
        rows_h(deepstack, "deepstack", 0, (S, tp * S))
    if residual_out is not None:
        rows_h(residual_out, "residual_out", rows)
    for t, name in ((weight, "weight"), (bias, "bias")):
        if isinstance(t, torch.Tensor):
            if t.numel() != H:
                raise ValueError(f"{name} must hold H={H} elements, got {t.numel()}")
            if act is not None and t.dtype != act:
                raise ValueError(f"{name} must have the residual's dtype {act}, got {t.dtype}")
    if isinstance(out, torch.Tensor):
        od = _sp_dtype(out.dtype) if out_dtype is None else out_dtype
        row_bytes = {SP_F32: 4 * H, SP_BF16: 2 * H, SP_FP8_E4M3: H, SP_FP4_E2M1: H // 2}.get(od)
        if row_bytes is not None:
            if out.dim() != 2 or out.shape[1] * out.element_size() != row_bytes:
                raise ValueError(f"out rows must be {row_bytes} bytes (H={H}), got shape {tuple(out.shape)} "
                                 f"of {out.dtype}")
            if out.shape[0] < rows:
                raise ValueError(f"out has {out.shape[0]} rows, the call writes {rows}")
    if isinstance(out_scale, torch.Tensor):
        if quant_mode in (SP_QUANT_STATIC_TENSOR, SP_QUANT_DYNAMIC_TOKEN):
            need = 1 if quant_mode == SP_QUANT_STATIC_TENSOR else rows
            if out_scale.dtype != torch.float32 or out_scale.numel() < need:
                raise ValueError(f"out_scale must be float32 with at least {need} elements, got "
                                 f"{out_scale.numel()} of {out_scale.dtype}")
        elif quant_mode == SP_QUANT_MX_BLOCK and _nbytes(out_scale) < rows * (H // 32):
            raise ValueError(f"out_scale must hold {rows} x {H // 32} E8M0 bytes, got {_nbytes(out_scale)}")


def _partials_addr(partials) -> int:
    _partials_stride(partials)
    return partials.data_ptr()


def sp_reduce_add_rmsnorm(partials, residual, weight, bias, eps, quant_mode, deepstack, out,
                          out_scale, *, tp_rank: int, num_tokens: int, residual_out=None,
                          valid_rows_only: bool = False, out_dtype: Optional[int] = None,
                          partial_scale: float = 1.0, stream=None) -> None:
    """Enqueue the fused shard path (see include/sprms.h for the contract).

    partials [tp, S, H] f32/bf16; residual [S or tp*S, H]; weight, bias [H];
    deepstack None or [S or tp*S, H]; out [S, H] bf16/f32, or uint8 /
    float8_e4m3fn for the e4m3 modes, or [S, H/2] uint8 / float4_e2m1fn_x2 for
    block-scaled e2m1 (pass out_dtype=SP_FP4_E2M1 with uint8); out_scale None,
    [1] f32 (static), [S] f32 (dynamic) or [S, H/32] uint8 E8M0 (block);
    residual_out [S, H] or None (in place).  With
    ``valid_rows_only`` the padding rows of the outputs are left untouched
    (out may then be a row block of an unpadded gathered tensor).
    ``partial_scale`` multiplies every partial before the sum.  Runs on
    ``stream`` (a torch stream or raw hipStream_t int; default: torch's
    current stream on partials' device).
    """
    lib = load()
    _check_fused_sizes(partials, residual, weight, bias, quant_mode, deepstack, out, out_scale,
                       tp_rank=tp_rank, num_tokens=num_tokens, residual_out=residual_out,
                       valid_rows_only=valid_rows_only, out_dtype=out_dtype)
    _same_device(partials, residual, weight, bias, deepstack, out, out_scale, residual_out)
    prob = make_problem(partials, residual, out, tp_rank=tp_rank, num_tokens=num_tokens,
                        deepstack=deepstack, residual_out=residual_out,
                        valid_rows_only=valid_rows_only, out_dtype=out_dtype,
                        partial_scale=partial_scale)
    with torch.cuda.device(partials.device):
        _check(lib.sp_reduce_add_rmsnorm(C.byref(prob), _partials_addr(partials), _addr(residual),
                                         _addr(weight), _addr(bias), float(eps), int(quant_mode),
                                         _addr(deepstack), _addr(out), _addr(out_scale),
                                         _stream_handle(partials.device, stream)))


def prepare(partials, residual, weight, bias, eps, quant_mode, deepstack, out, out_scale, *,
            tp_rank: int, num_tokens: int, residual_out=None, valid_rows_only: bool = False,
            out_dtype: Optional[int] = None, partial_scale: float = 1.0, stream=None):
    """Marshal the arguments of sp_reduce_add_rmsnorm once and return a
    no-argument callable that enqueues the call again (for timing loops).
    The tensors must stay alive and in place while the callable is used."""
    lib = load()
    _check_fused_sizes(partials, residual, weight, bias, quant_mode, deepstack, out, out_scale,
                       tp_rank=tp_rank, num_tokens=num_tokens, residual_out=residual_out,
                       valid_rows_only=valid_rows_only, out_dtype=out_dtype)
    _same_device(partials, residual, weight, bias, deepstack, out, out_scale, residual_out)
    prob = make_problem(partials, residual, out, tp_rank=tp_rank, num_tokens=num_tokens,
                        deepstack=deepstack, residual_out=residual_out,
                        valid_rows_only=valid_rows_only, out_dtype=out_dtype,
                        partial_scale=partial_scale)
    args = (C.byref(prob), _partials_addr(partials), _addr(residual), _addr(weight), _addr(bias),
            float(eps), int(quant_mode), _addr(deepstack), _addr(out), _addr(out_scale),
            _stream_handle(partials.device, stream))
    fn = lib.sp_reduce_add_rmsnorm

    def launch():
        _check(fn(*args))

    launch.problem = prob  # keep the descriptor alive with the callable
    return launch


def sp_all_gather_unpad(shards, shard_scales, out, out_scale, *, num_tokens: int,
                        dtype: Optional[int] = None, stream=None) -> None:
    """Gather tp shard outputs ([S, H] each, same dtype) into the unpadded
    out [T, H], and their scales ([S] f32 or [S, H/32] E8M0 bytes each) into
    out_scale; see include/sprms.h.  Rows are copied as bytes: packed e2m1
    shards may be given as uint8 [S, H/2] with dtype=SP_FP4_E2M1."""
    lib = load()
    tp = len(shards)
    S, W = shards[0].shape
    for t in shards:
        if t.shape != (S, W) or t.dtype != shards[0].dtype:
            raise ValueError("all shards must share shape and dtype")
    if out.dim() != 2 or out.shape[1] * out.element_size() != W * shards[0].element_size():
        raise ValueError(f"out rows must be as wide as the shards' ({W} x {shards[0].dtype})")
    rows = num_tokens if 0 <= num_tokens <= tp * S else 0   # other counts: the library's error
    if out.shape[0] < rows:
        raise ValueError(f"out has {out.shape[0]} rows, the call writes {rows}")
    srow = 0
    if shard_scales is not None:
        if len(shard_scales) != tp:
            raise ValueError("one scale tensor per shard")
        sb = _nbytes(shard_scales[0])
        if any(_nbytes(t) != sb for t in shard_scales) or (S and sb % S):
            raise ValueError("every shard's scales must be [S, row] of one size")
        srow = sb // max(S, 1)
        if isinstance(out_scale, torch.Tensor) and _nbytes(out_scale) < rows * srow:
            raise ValueError(f"out_scale must hold {rows} x {srow} bytes")
    _same_device(shards, shard_scales, out, out_scale)
    dt = _sp_dtype(shards[0].dtype) if dtype is None else dtype
    H = 2 * W if dt == SP_FP4_E2M1 else W
    g = sp_gather_problem(tp=tp, dtype=dt, shard_rows=S, hidden=H, num_tokens=num_tokens,
                          scale_row_bytes=srow)
    src = (C.c_void_p * tp)(*[_addr(t) for t in shards])
    ssrc = None
    if shard_scales is not None:
        ssrc = (C.c_void_p * tp)(*[_addr(t) for t in shard_scales])
    with torch.cuda.device(shards[0].device):
        _check(lib.sp_all_gather_unpad(C.byref(g), src, ssrc, _addr(out), _addr(out_scale),
                                       _stream_handle(shards[0].device, stream)))


def sp_fc2_regroup(srcs, dsts, *, otp: int, rank: int = -1, stream=None) -> None:
    """FlashComm2 o_proj input regrouping of G ranks: srcs[q] [N, C] ->
    dsts[r] [N/odp, odp*C], odp = G/otp; with rank >= 0 only dsts[rank] is
    written (the others may be None).  See include/sprms.h."""
    lib = load()
    G = len(srcs)
    N, Cc = srcs[0].shape
    for t in srcs:
        if t.shape != (N, Cc) or t.dtype != srcs[0].dtype:
            raise ValueError("all sources must share shape and dtype")
    if len(dsts) != G:
        raise ValueError("one destination per rank")
    for r, d in enumerate(dsts):  # [N/odp, odp*C]: the same elements as a source
        if d is not None and (d.dtype != srcs[0].dtype or d.numel() != N * Cc):
            raise ValueError(f"dsts[{r}] must hold {N * Cc} elements of {srcs[0].dtype}")
    _same_device(srcs, dsts)
    f = sp_fc2_problem(global_tp=G, otp=otp, dtype=_sp_dtype(srcs[0].dtype), rank=rank,
                       tokens=N, cols=Cc)
    src = (C.c_void_p * G)(*[_addr(t) for t in srcs])
    dst = (C.c_void_p * G)(*[_addr(t) for t in dsts])
    with torch.cuda.device(srcs[0].device):
        _check(lib.sp_fc2_regroup(C.byref(f), src, dst, _stream_handle(srcs[0].device, stream)))


def sp_dsacp_heads_to_tokens(attn, outs, *, rank: int = -1, stream=None) -> None:
    """DSA-CP o_proj input exchange of tp ranks: attn[p] [S, tp*D] (local
    tokens, every rank's heads) -> outs[q] [tp*S, D] (every token, rank q's
    heads); with rank >= 0 only outs[rank] is written (the others may be
    None).  See include/sprms.h."""
    lib = load()
    tp = len(attn)
    S, W = attn[0].shape
    for t in attn:
        if t.shape != (S, W) or t.dtype != attn[0].dtype:
            raise ValueError("all inputs must share shape and dtype")
    if W % tp or len(outs) != tp:
        raise ValueError("row width must be tp*D and there must be one output per rank")
    for q, o in enumerate(outs):  # [tp*S, D]
        if o is not None and (o.dtype != attn[0].dtype or o.shape != (tp * S, W // tp)):
            raise ValueError(f"outs[{q}] must be [{tp * S}, {W // tp}] of {attn[0].dtype}")
    _same_device(attn, outs)
    f = sp_dsacp_problem(tp=tp, dtype=_sp_dtype(attn[0].dtype), rank=rank, reserved=0,
                         shard_rows=S, head_cols=W // tp)
    src = (C.c_void_p * tp)(*[_addr(t) for t in attn])
    dst = (C.c_void_p * tp)(*[_addr(t) for t in outs])
    with torch.cuda.device(attn[0].device):
        _check(lib.sp_dsacp_heads_to_tokens(C.byref(f), src, dst,
                                            _stream_handle(attn[0].device, stream)))


def sp_matmul_scatter(x, w, dsts, *, rank: int, stream=None) -> None:
    """Rank `rank`'s row-parallel GEMM x w^T (x [tp*S, K] bf16, w [N, K] bf16)
    written into slot `rank` of each destination's receive buffer dsts[r]
    [tp, S, N] (bf16 or f32).  See include/sprms.h."""
    lib = load()
    tp = len(dsts)
    M, K = x.shape
    N = w.shape[0]
    if M % tp or w.shape[1] != K:
        raise ValueError("x must be [tp*S, K] and w [N, K]")
    S = M // tp
    for d in dsts:
        if d.shape != (tp, S, N) or d.dtype != dsts[0].dtype:
            raise ValueError("every receive buffer must be [tp, S, N] of one dtype")
    _same_device(x, w, dsts)
    p = sp_matmul_problem(tp=tp, rank=rank, shard_rows=S, k=K, n=N, in_dtype=_sp_dtype(x.dtype),
                          out_dtype=_sp_dtype(dsts[0].dtype))
    if _sp_dtype(w.dtype) != p.in_dtype:
        raise ValueError("x and w must share a dtype")
    dst = (C.c_void_p * tp)(*[_addr(d) for d in dsts])
    with torch.cuda.device(x.device):
        _check(lib.sp_matmul_scatter(C.byref(p), _addr(x), _addr(w), dst,
                                     _stream_handle(x.device, stream)))


def sp_scaled_matmul_scatter(x, x_scale, w, w_scale, dsts, *, rank: int, stream=None) -> None:
    """FP8 producer: x [tp*S, K] and w [N, K] e4m3 codes (uint8 or
    float8_e4m3fn), x_scale [1] or [tp*S] and w_scale [1] or [N] float32;
    (x w^T) x_scale w_scale written into slot `rank` of each dsts[r]
    [tp, S, N] (bf16 or f32).  See include/sprms.h."""
    lib = load()
    tp = len(dsts)
    M, K = x.shape
    N = w.shape[0]
    if M % tp or w.shape[1] != K:
        raise ValueError("x must be [tp*S, K] and w [N, K]")
    S = M // tp
    for d in dsts:
        if d.shape != (tp, S, N) or d.dtype != dsts[0].dtype:
            raise ValueError("every receive buffer must be [tp, S, N] of one dtype")
    if x_scale.dtype != torch.float32 or w_scale.dtype != torch.float32:
        raise ValueError("scales must be float32")
    _same_device(x, x_scale, w, w_scale, dsts)
    p = sp_matmul_problem(tp=tp, rank=rank, shard_rows=S, k=K, n=N, in_dtype=_sp_dtype(x.dtype),
                          out_dtype=_sp_dtype(dsts[0].dtype), x_scale_rows=x_scale.numel(),
                          w_scale_rows=w_scale.numel())
    if _sp_dtype(w.dtype) != p.in_dtype:
        raise ValueError("x and w must share a dtype")
    dst = (C.c_void_p * tp)(*[_addr(d) for d in dsts])
    with torch.cuda.device(x.device):
        _check(lib.sp_scaled_matmul_scatter(C.byref(p), _addr(x), _addr(x_scale), _addr(w),
                                            _addr(w_scale), dst, _stream_handle(x.device, stream)))


def sp_validate(problem: sp_problem, partials, residual, weight, bias, eps, quant_mode, deepstack,
                out, out_scale) -> int:
    """Host-side checks only (no HIP call).  Pointer arguments may be tensors,
    int addresses or None.  Returns the sp_status code."""
    lib = load()
    return lib.sp_validate(C.byref(problem), _addr(partials), _addr(residual), _addr(weight),
                           _addr(bias), float(eps), int(quant_mode), _addr(deepstack), _addr(out),
                           _addr(out_scale))


def sp_shard_geometry(num_tokens: int, num_tokens_pad: int, tp: int, rank: int):
    """(shard_rows, local_start, valid_rows) of rank's contiguous shard."""
    lib = load()
    s, st, v = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib.sp_shard_geometry(num_tokens, num_tokens_pad, tp, rank, C.byref(s), C.byref(st),
                                 C.byref(v)))
    return s.value, st.value, v.value


def sp_error_string(status: int) -> str:
    """The library's fixed name of an sp_status code."""
    return load().sp_error_string(int(status)).decode()


def sp_last_error() -> str:
    """Detail of the last failed call on this host thread ("no error" if none has failed)."""
    return load().sp_last_error().decode()

"""The oracle's entry point with the library boundary's argument list
(sp_oracle_reduce_add_rmsnorm), on the CPU: its descriptor has the library
descriptor's layout, and for every workload form it returns exactly what the
pinned oracle function orc_reduce_add_rmsnorm returns, with the boundary's
own conventions on top (in-place residual, valid-rows-only writes, strided
partials, the static scale read from out_scale, nothing written on error)."""

import ctypes as C
import dataclasses

import numpy as np
import pytest

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import to_host
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK, QUANT_NONE,
                                           QUANT_STATIC_TENSOR, WORKLOADS, make_inputs)

CODE = {np.dtype(np.float32): oracle.ORC_F32, np.dtype(np.uint16): oracle.ORC_BF16}


def test_descriptor_layout_matches_the_library():
    assert C.sizeof(oracle.AbiProblem) == C.sizeof(sp.sp_problem)
    names = [f[0] for f in oracle.AbiProblem._fields_]
    assert names == [f[0] for f in sp.sp_problem._fields_]
    for n in names:
        a, b = getattr(oracle.AbiProblem, n), getattr(sp.sp_problem, n)
        assert (a.offset, a.size) == (b.offset, b.size), n


def _small(name, S=12, pad=5):
    w = WORKLOADS[name]
    return dataclasses.replace(w, num_tokens=w.tp * S - pad, num_tokens_pad=w.tp * S,
                               hidden=min(w.hidden, 256))


def _host_inputs(w, rank):
    x = make_inputs(w, rank=rank, pad_fill=float("nan"))
    return {k: to_host(t) for k, t in x.items()}


def _problem(h, w, rank, out_dtype, **over):
    tp, S, H = h["partials"].shape
    p = oracle.AbiProblem(tp=tp, tp_rank=rank, shard_rows=S, hidden=H, num_tokens=w.num_tokens,
                          partial_dtype=CODE[h["partials"].dtype], act_dtype=CODE[h["residual"].dtype],
                          out_dtype=out_dtype, residual_rows=h["residual"].shape[0],
                          deepstack_rows=0 if h["deepstack"] is None else h["deepstack"].shape[0],
                          residual_out=None, partial_stride=0, flags=0, partial_scale=0.0)
    for k, v in over.items():
        setattr(p, k, v)
    return p


def _outputs(h, out_dtype, quant):
    tp, S, H = h["partials"].shape
    res = np.full((S, H), 0xA5A5 if h["residual"].dtype == np.uint16 else np.nan, h["residual"].dtype)
    out = np.full((S, H // 2 if out_dtype == oracle.ORC_E2M1 else H),
                  {oracle.ORC_F32: np.nan, oracle.ORC_BF16: 0xA5A5}.get(out_dtype, 0xA5),
                  {oracle.ORC_F32: np.float32, oracle.ORC_BF16: np.uint16}.get(out_dtype, np.uint8))
    sc = None
    if quant == QUANT_DYNAMIC_TOKEN:
        sc = np.full((S,), np.nan, np.float32)
    elif quant == QUANT_MX_BLOCK:
        sc = np.full((S, H // 32), 0xA5, np.uint8)
    elif quant == QUANT_STATIC_TENSOR:
        sc = np.array([0.02], np.float32)
    return res, out, sc


@pytest.mark.parametrize("name,rank", [("C1", 1), ("C2", 7), ("C3", 15), ("C4", 7), ("C5", 3), ("C5", 0)])
def test_equals_the_pinned_oracle_function(name, rank):
    w = _small(name)
    h = _host_inputs(w, rank)
    od = {QUANT_NONE: oracle.ORC_BF16}.get(w.quant_mode, oracle.ORC_E4M3)
    res, out, sc = _outputs(h, od, w.quant_mode)
    p = _problem(h, w, rank, od)
    p.residual_out = res.ctypes.data
    rc = oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], h["bias"],
                                             w.eps, w.quant_mode, h["deepstack"], out, sc)
    assert rc == 0
    ref = oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], h["bias"], w.eps,
                                    w.quant_mode, h["deepstack"], tp_rank=rank, num_tokens=w.num_tokens,
                                    out_dtype=od, static_scale=0.02, want_debug=False)
    np.testing.assert_array_equal(res.view(np.uint8), ref["residual_out"].view(np.uint8))
    np.testing.assert_array_equal(out.view(np.uint8), ref["out"].view(np.uint8))
    if w.quant_mode == QUANT_DYNAMIC_TOKEN:
        np.testing.assert_array_equal(sc, ref["out_scale"])


def test_block_scaled_e2m1():
    w = dataclasses.replace(_small("C5"), quant_mode=QUANT_MX_BLOCK)
    h = _host_inputs(w, 3)
    res, out, sc = _outputs(h, oracle.ORC_E2M1, QUANT_MX_BLOCK)
    p = _problem(h, w, 3, oracle.ORC_E2M1)
    p.residual_out = res.ctypes.data
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_MX_BLOCK, h["deepstack"], out, sc) == 0
    ref = oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], None, w.eps, QUANT_MX_BLOCK,
                                    h["deepstack"], tp_rank=3, num_tokens=w.num_tokens,
                                    out_dtype=oracle.ORC_E2M1, want_debug=False)
    np.testing.assert_array_equal(out, ref["out"])
    np.testing.assert_array_equal(sc, ref["out_scale"])


def test_in_place_replicated_residual():
    # C1 holds a replicated fp32 residual: rank 1 updates block 1 only
    w = _small("C1", S=16, pad=3)
    h = _host_inputs(w, 1)
    before = h["residual"].copy()
    res_sep, out_sep, _ = _outputs(h, oracle.ORC_BF16, QUANT_NONE)
    p = _problem(h, w, 1, oracle.ORC_BF16)
    p.residual_out = res_sep.ctypes.data
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], h["bias"], w.eps,
                                               QUANT_NONE, None, out_sep, None) == 0
    np.testing.assert_array_equal(h["residual"].view(np.uint8), before.view(np.uint8))   # read only
    _, out_inp, _ = _outputs(h, oracle.ORC_BF16, QUANT_NONE)
    p.residual_out = None
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], h["bias"], w.eps,
                                               QUANT_NONE, None, out_inp, None) == 0
    S = w.shard_rows
    np.testing.assert_array_equal(h["residual"][S:2 * S].view(np.uint8), res_sep.view(np.uint8))
    np.testing.assert_array_equal(h["residual"][:S].view(np.uint8), before[:S].view(np.uint8))
    np.testing.assert_array_equal(out_inp, out_sep)


def test_valid_rows_only_leaves_padding_rows_untouched():
    w = _small("C5", pad=5)
    h = _host_inputs(w, 3)
    S, v = w.shard_rows, w.shard_rows - 5
    res, out, sc = _outputs(h, oracle.ORC_E4M3, QUANT_DYNAMIC_TOKEN)
    full_res, full_out, full_sc = _outputs(h, oracle.ORC_E4M3, QUANT_DYNAMIC_TOKEN)
    p = _problem(h, w, 3, oracle.ORC_E4M3, flags=1)
    p.residual_out = res.ctypes.data
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_DYNAMIC_TOKEN, h["deepstack"], out, sc) == 0
    q = _problem(h, w, 3, oracle.ORC_E4M3)
    q.residual_out = full_res.ctypes.data
    assert oracle.sp_oracle_reduce_add_rmsnorm(q, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_DYNAMIC_TOKEN, h["deepstack"], full_out, full_sc) == 0
    np.testing.assert_array_equal(out[:v], full_out[:v])
    np.testing.assert_array_equal(res[:v], full_res[:v])
    np.testing.assert_array_equal(sc[:v], full_sc[:v])
    assert (out[v:] == 0xA5).all() and (res[v:] == 0xA5A5).all() and np.isnan(sc[v:]).all()
    assert not full_out[v:].any() and not full_res[v:].any() and not full_sc[v:].any()


def test_strided_partials_equal_packed():
    # rank r's rows of tp full [T_pad, H] partial tensors held in one buffer
    w = _small("C2", S=10, pad=7)
    r = 5
    tp, S, H = w.tp, w.shard_rows, w.hidden
    rng = np.random.default_rng(1)
    big = rng.standard_normal((tp, tp * S, H)).astype(np.float32)
    h = _host_inputs(w, r)
    h["partials"] = np.ascontiguousarray(big[:, r * S:(r + 1) * S]).view(np.float32)
    packed_res, packed_out, _ = _outputs(h, oracle.ORC_BF16, QUANT_NONE)
    p = _problem(h, w, r, oracle.ORC_BF16)      # f32 partials with a bf16 residual
    p.residual_out = packed_res.ctypes.data
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_NONE, None, packed_out, None) == 0
    str_res, str_out, _ = _outputs(h, oracle.ORC_BF16, QUANT_NONE)
    p.partial_stride = tp * S * H
    p.residual_out = str_res.ctypes.data
    view = big.reshape(-1)[r * S * H:]       # pointer at partial 0, row r*S
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, view, h["residual"], h["weight"], None, w.eps,
                                               QUANT_NONE, None, str_out, None) == 0
    np.testing.assert_array_equal(str_out, packed_out)
    np.testing.assert_array_equal(str_res, packed_res)
    p.partial_stride = S * H - 1
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, view, h["residual"], h["weight"], None, w.eps,
                                               QUANT_NONE, None, str_out, None) == oracle_err("SHAPE")


def oracle_err(name):
    return {"NULL": -1, "SHAPE": -2, "DTYPE": -3, "UNSUPPORTED": -5}[name]


def test_static_scale_is_read_from_out_scale():
    w = _small("C4")
    h = _host_inputs(w, 7)
    outs = []
    for s in (0.02, 0.05):
        res, out, _ = _outputs(h, oracle.ORC_E4M3, QUANT_STATIC_TENSOR)
        p = _problem(h, w, 7, oracle.ORC_E4M3)
        p.residual_out = res.ctypes.data
        sc = np.array([s], np.float32)
        assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                                   QUANT_STATIC_TENSOR, None, out, sc) == 0
        ref = oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], None, w.eps,
                                        QUANT_STATIC_TENSOR, None, tp_rank=7, num_tokens=w.num_tokens,
                                        out_dtype=oracle.ORC_E4M3, static_scale=s, want_debug=False)
        np.testing.assert_array_equal(out, ref["out"])
        outs.append(out)
    assert not np.array_equal(outs[0], outs[1])


def test_errors_write_nothing():
    w = _small("C5")
    h = _host_inputs(w, 3)
    res, out, sc = _outputs(h, oracle.ORC_E4M3, QUANT_DYNAMIC_TOKEN)
    p = _problem(h, w, 3, oracle.ORC_E4M3)
    p.residual_out = res.ctypes.data
    args = (h["partials"], h["residual"], h["weight"], None, w.eps)
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, *args, 3, h["deepstack"], out, sc) == oracle_err("UNSUPPORTED")
    p.flags = 2
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, *args, QUANT_DYNAMIC_TOKEN, h["deepstack"], out, sc) \
        == oracle_err("UNSUPPORTED")
    p.flags = 0
    p.tp_rank = w.tp
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, *args, QUANT_DYNAMIC_TOKEN, h["deepstack"], out, sc) \
        == oracle_err("SHAPE")
    p.tp_rank = 3
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, *args, QUANT_DYNAMIC_TOKEN, h["deepstack"], out, None) \
        == oracle_err("NULL")
    assert (out == 0xA5).all() and (res == 0xA5A5).all() and np.isnan(sc).all()


def test_in_place_residual_may_not_share_bytes_with_what_the_call_reads():
    # [PR18671] §5.2 raises on a layout mismatch rather than corrupting shared
    # storage; here the residual rows updated in place (residual_out NULL, or
    # the block in use) must not overlap the partials, gain, bias or deepstack.
    w = _small("C5")
    h = _host_inputs(w, 3)
    tp, S, H = h["partials"].shape
    _, out, sc = _outputs(h, oracle.ORC_E4M3, QUANT_DYNAMIC_TOKEN)
    buf = h["partials"].copy()
    inside = buf[1]  # partial 1's rows, used as this shard's residual
    before = buf.copy()
    for res_out in (None, inside.ctypes.data):
        p = _problem(h, w, 3, oracle.ORC_E4M3, residual_rows=S, residual_out=res_out)
        rc = oracle.sp_oracle_reduce_add_rmsnorm(p, buf, inside, h["weight"], None, w.eps,
                                                 QUANT_DYNAMIC_TOKEN, h["deepstack"], out, sc)
        assert rc == oracle_err("SHAPE")
    np.testing.assert_array_equal(buf, before)
    # the gain, the bias or the deepstack inside the residual block
    res = h["residual"][-S:].copy()
    for k in ("weight", "bias", "deepstack"):
        args = {"weight": h["weight"], "bias": None, "deepstack": h["deepstack"]}
        args[k] = res[2] if k != "deepstack" else res
        p = _problem(h, w, 3, oracle.ORC_E4M3, residual_rows=S,
                     deepstack_rows=0 if args["deepstack"] is None else args["deepstack"].shape[0])
        rc = oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], res, args["weight"], args["bias"],
                                                 w.eps, QUANT_DYNAMIC_TOKEN, args["deepstack"], out, sc)
        assert rc == oracle_err("SHAPE"), k
    # the same residual, on its own, updated in place is fine
    p = _problem(h, w, 3, oracle.ORC_E4M3)
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"].copy(), h["weight"],
                                               None, w.eps, QUANT_DYNAMIC_TOKEN, h["deepstack"],
                                               out, sc) == 0


def test_static_scale_may_not_share_bytes_with_an_output():
    w = _small("C4")
    h = _host_inputs(w, 7)
    res, out, _ = _outputs(h, oracle.ORC_E4M3, QUANT_STATIC_TENSOR)
    p = _problem(h, w, 7, oracle.ORC_E4M3)
    p.residual_out = res.ctypes.data
    sc = out.reshape(-1)[:4].view(np.float32)
    sc[0] = 0.02
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_STATIC_TENSOR, None, out, sc) == oracle_err("SHAPE")


@pytest.mark.parametrize("stride", [2 ** 62, 2 ** 63 - 64, 2 ** 46])
def test_partial_stride_that_overflows_or_spans_too_far_is_rejected(stride):
    # (tp - 1) * stride + S*H elements must be a byte span of at most 2^47;
    # nothing is read when it is not
    w = _small("C4")
    h = _host_inputs(w, 7)
    res, out, _ = _outputs(h, oracle.ORC_E4M3, QUANT_STATIC_TENSOR)
    p = _problem(h, w, 7, oracle.ORC_E4M3, partial_stride=stride)
    p.residual_out = res.ctypes.data
    sc = np.array([0.02], np.float32)
    assert oracle.sp_oracle_reduce_add_rmsnorm(p, h["partials"], h["residual"], h["weight"], None, w.eps,
                                               QUANT_STATIC_TENSOR, None, out, sc) == oracle_err("SHAPE")
    assert (out == 0xA5).all()

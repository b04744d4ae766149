"""NaN in a valid row, HIP path against the oracle on MI355X.

The pages say nothing about NaN; the reading both sides follow: IEEE
arithmetic throughout, and every NaN reaches the output in its format's own
NaN encoding (the rule is stated in include/sprms.h).  A NaN input element
makes that residual element and, through the row's sum of squares, every
output of its row NaN; a NaN gain or bias element makes its column (its
block, with block scaling; every row, with a per-token scale) NaN.

Checks: the NaN row's (column's, block's) e4m3 / e2m1 codes, E8M0 bytes and
per-token scale bytes are byte-equal to the oracle's; bf16 / f32 outputs are
NaN exactly where the oracle's are; everything the NaN does not feed is
bit-identical to a clean GPU run on the same inputs without it, and that
clean run is itself checked against the oracle (tests/parity.py).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import bf16_bits_to_f64, to_host
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK, QUANT_NONE,
                                           QUANT_STATIC_TENSOR, WORKLOADS, make_inputs)

pytestmark = pytest.mark.gpu

TP, S, H, RANK = 4, 16, 1024, 3
T = TP * S - 5           # rank 3: 11 valid rows, 5 padding rows
NAN_ROW, NAN_COL = 4, 37  # column 37 lies in block 1 (elements 32..63)
STATIC_SCALE = 0.01

# mode: (quant, out dtype of the call, oracle out dtype, bias)
MODES = {
    "bf16": (QUANT_NONE, torch.bfloat16, oracle.ORC_BF16, False),
    "f32": (QUANT_NONE, torch.float32, oracle.ORC_F32, False),
    "static": (QUANT_STATIC_TENSOR, torch.uint8, oracle.ORC_E4M3, False),
    "per_token": (QUANT_DYNAMIC_TOKEN, torch.uint8, oracle.ORC_E4M3, False),
    "per_token_bias": (QUANT_DYNAMIC_TOKEN, torch.uint8, oracle.ORC_E4M3, True),
    "mxfp8": (QUANT_MX_BLOCK, torch.uint8, oracle.ORC_E4M3, False),
    "mxfp4": (QUANT_MX_BLOCK, torch.uint8, oracle.ORC_E2M1, False),
}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _workload(mode):
    quant, out_t, _, bias = MODES[mode]
    return dataclasses.replace(WORKLOADS["C5"], tp=TP, num_tokens=T, num_tokens_pad=TP * S, hidden=H,
                               quant_mode=quant, out_dtype=out_t, bias=bias, deepstack=True,
                               fp4=mode == "mxfp4")


def _gpu(x, mode, dev):
    """One call through the C ABI on the given inputs; host copies of the outputs."""
    quant, out_t, _, _ = MODES[mode]
    fp4 = mode == "mxfp4"
    res_out = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((S, H // 2 if fp4 else H), dtype=out_t, device=dev)
    scale = None
    if quant == QUANT_STATIC_TENSOR:
        scale = torch.tensor([STATIC_SCALE], dtype=torch.float32, device=dev)
    elif quant == QUANT_DYNAMIC_TOKEN:
        scale = torch.empty((S,), dtype=torch.float32, device=dev)
    elif quant == QUANT_MX_BLOCK:
        scale = torch.empty((S, H // 32), dtype=torch.uint8, device=dev)
    sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], x["bias"], 1e-6, quant,
                             x["deepstack"], out, scale, tp_rank=RANK, num_tokens=T,
                             residual_out=res_out, out_dtype=sp.SP_FP4_E2M1 if fp4 else None)
    torch.cuda.synchronize()
    got = {"residual_out": to_host(res_out), "out": to_host(out)}
    if quant in (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK):
        got["out_scale"] = scale.cpu().numpy()
    return got


def _oracle(x, mode):
    quant, _, od, _ = MODES[mode]
    h = {k: to_host(t) for k, t in x.items()}
    return oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], h["bias"], 1e-6, quant,
                                     h["deepstack"], tp_rank=RANK, num_tokens=T, out_dtype=od,
                                     static_scale=STATIC_SCALE)


def _nan_mask(a, od):
    if od == oracle.ORC_BF16:
        return np.isnan(bf16_bits_to_f64(a))
    return np.isnan(a) if od == oracle.ORC_F32 else None


def _same_bytes(a, b):
    np.testing.assert_array_equal(np.ascontiguousarray(a).view(np.uint8),
                                  np.ascontiguousarray(b).view(np.uint8))


def _clean_checked(mode, dev):
    """Seeded inputs without NaN, checked against the oracle on every row."""
    w = _workload(mode)
    x = make_inputs(w, rank=RANK, device=dev, pad_fill=float("nan"))
    run_case(w, RANK, dev=dev, inputs={k: (None if v is None else v.clone()) for k, v in x.items()},
             static_scale=STATIC_SCALE, fp4=mode == "mxfp4")
    return x, _gpu(x, mode, dev)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("where", ["partial", "residual", "deepstack"])
def test_nan_input_element_reaches_every_output_of_its_row(dev, mode, where):
    say(f"NaN in {where} row {NAN_ROW} col {NAN_COL}, mode {mode}: tp={TP} S={S} H={H} rank {RANK}")
    quant, _, od, _ = MODES[mode]
    x, clean = _clean_checked(mode, dev)
    if where == "partial":
        x["partials"][2, NAN_ROW, NAN_COL] = float("nan")
    elif where == "residual":
        x["residual"][NAN_ROW, NAN_COL] = float("nan")
    else:
        x["deepstack"][RANK * S + NAN_ROW, NAN_COL] = float("nan")
    got, ref = _gpu(x, mode, dev), _oracle(x, mode)

    # the updated residual: NaN at that element only, the rest as in the clean run
    nan_res = np.isnan(bf16_bits_to_f64(got["residual_out"]))
    assert nan_res[NAN_ROW, NAN_COL] and nan_res.sum() == 1
    np.testing.assert_array_equal(nan_res, np.isnan(bf16_bits_to_f64(ref["residual_out"])))
    keep = ~nan_res
    np.testing.assert_array_equal(got["residual_out"][keep], clean["residual_out"][keep])

    # the NaN row: every output in its format's NaN encoding, as the oracle's
    if quant == QUANT_NONE:
        assert _nan_mask(got["out"][NAN_ROW], od).all()
        np.testing.assert_array_equal(_nan_mask(got["out"], od), _nan_mask(ref["out"], od))
    else:
        _same_bytes(got["out"][NAN_ROW], ref["out"][NAN_ROW])
    if "out_scale" in got:
        _same_bytes(got["out_scale"][NAN_ROW], ref["out_scale"][NAN_ROW])
    if quant == QUANT_DYNAMIC_TOKEN:
        assert got["out_scale"][NAN_ROW:NAN_ROW + 1].view(np.uint32)[0] == 0x7FC00000

    # every other row (padding rows included) is untouched by the NaN
    others = np.arange(S) != NAN_ROW
    for k in got:
        _same_bytes(got[k][others], clean[k][others])


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("which", ["weight", "bias"])
def test_nan_gain_or_bias_element_reaches_its_column(dev, mode, which):
    say(f"NaN {which} element {NAN_COL}, mode {mode}: tp={TP} S={S} H={H} rank {RANK}")
    quant, _, od, with_bias = MODES[mode]
    if which == "bias" and not with_bias:
        mode_w = dataclasses.replace(_workload(mode), bias=True)
    else:
        mode_w = _workload(mode)
    x = make_inputs(mode_w, rank=RANK, device=dev, pad_fill=float("nan"))
    run_case(mode_w, RANK, dev=dev, inputs={k: (None if v is None else v.clone()) for k, v in x.items()},
             static_scale=STATIC_SCALE, fp4=mode == "mxfp4")
    clean = _gpu(x, mode, dev)
    x[which][NAN_COL] = float("nan")
    got, ref = _gpu(x, mode, dev), _oracle(x, mode)
    v = T - RANK * S

    # the gain and bias do not enter the residual or rstd
    _same_bytes(got["residual_out"], clean["residual_out"])
    cols = np.arange(H) != NAN_COL
    if quant == QUANT_NONE:
        assert _nan_mask(got["out"][:v, NAN_COL], od).all()
        np.testing.assert_array_equal(_nan_mask(got["out"], od), _nan_mask(ref["out"], od))
        _same_bytes(got["out"][:, cols], clean["out"][:, cols])
    elif quant == QUANT_STATIC_TENSOR:
        _same_bytes(got["out"][:, NAN_COL], ref["out"][:, NAN_COL])
        assert (got["out"][:v, NAN_COL] == 0x7F).all()
        _same_bytes(got["out"][:, cols], clean["out"][:, cols])
    elif quant == QUANT_DYNAMIC_TOKEN:
        # the row maximum skips nothing: every valid row is NaN, scale and codes
        _same_bytes(got["out"], ref["out"])
        _same_bytes(got["out_scale"], ref["out_scale"])
        assert (got["out_scale"][:v].view(np.uint32) == 0x7FC00000).all()
        assert (got["out"][:v] == 0x7F).all()
    else:
        _same_bytes(got["out_scale"][:, 1], ref["out_scale"][:, 1])
        assert (got["out_scale"][:v, 1] == 0xFF).all()
        blk = slice(16, 32) if mode == "mxfp4" else slice(32, 64)
        _same_bytes(got["out"][:, blk], ref["out"][:, blk])
        rest = np.ones(got["out"].shape[1], bool)
        rest[blk] = False
        _same_bytes(got["out"][:, rest], clean["out"][:, rest])
        sc_rest = np.arange(H // 32) != 1
        _same_bytes(got["out_scale"][:, sc_rest], clean["out_scale"][:, sc_rest])


# The maxima run in other code paths for a runtime partial count (tp = 5,
# partials loaded in groups) and for rows of more than 8192 elements (4 or 8
# vectors per thread): the NaN rule must hold there too.
@pytest.mark.parametrize("tp,H", [(5, 1024), (4, 16384), (3, 32768)])
@pytest.mark.parametrize("mode", ["per_token", "per_token_bias", "mxfp8", "static"])
def test_nan_rule_in_every_kernel_shape(dev, tp, H, mode):
    say(f"NaN rule at tp={tp} H={H} mode {mode}")
    quant, out_t, od, bias = MODES[mode]
    S = 6
    w = dataclasses.replace(WORKLOADS["C5"], tp=tp, num_tokens=tp * S - 2, num_tokens_pad=tp * S, hidden=H,
                            quant_mode=quant, out_dtype=out_t, bias=bias, deepstack=True)
    rank = tp - 1
    x = make_inputs(w, rank=rank, device=dev, pad_fill=float("nan"))
    x["partials"][tp - 1, 1, H - 3] = float("nan")   # valid row 1, last partial, near the row's end
    res_out = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((S, H), dtype=torch.uint8, device=dev)
    scale = (torch.tensor([STATIC_SCALE], device=dev) if quant == QUANT_STATIC_TENSOR else
             torch.empty((S,), device=dev) if quant == QUANT_DYNAMIC_TOKEN else
             torch.empty((S, H // 32), dtype=torch.uint8, device=dev))
    sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], x["bias"], 1e-6, quant,
                             x["deepstack"], out, scale, tp_rank=rank, num_tokens=w.num_tokens,
                             residual_out=res_out)
    torch.cuda.synchronize()
    h = {k: to_host(t) for k, t in x.items()}
    ref = oracle.reduce_add_rmsnorm(h["partials"], h["residual"], h["weight"], h["bias"], 1e-6, quant,
                                    h["deepstack"], tp_rank=rank, num_tokens=w.num_tokens, out_dtype=od,
                                    static_scale=STATIC_SCALE, rows=[1])
    _same_bytes(to_host(out)[1], ref["out"][0])
    if quant != QUANT_STATIC_TENSOR:
        _same_bytes(scale.cpu().numpy()[1], ref["out_scale"][0])
    assert np.isnan(bf16_bits_to_f64(to_host(res_out)[1, H - 3]))

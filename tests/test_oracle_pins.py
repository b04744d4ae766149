"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties the oracle to something other than itself: the pages'
worked example and stated equivalences, closed forms, a textbook routine
(torch's rms_norm in float64), library roundings (torch's bf16 and e4m3
casts), format definitions and brute force.  Page tags:
  [SP/FC]    vllm-ascend SP / FlashComm1 / FlashComm2 guide (ai6s.net)
  [SPquant]  vLLM SP / AsyncTP / quantisation notes (beaiera.top)
  [PR18671]  vllm-ascend PR #18671 walkthrough (huashanblogllm.xyz)
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import bf16_bits_to_f64, e4m3_decode, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NONE, STATIC, DYNAMIC = oracle.QUANT_NONE, oracle.QUANT_STATIC_TENSOR, oracle.QUANT_DYNAMIC_TOKEN
MX = oracle.QUANT_MX_BLOCK


def f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


# ---------------------------------------------------------------- formats


def test_e4m3_decode_matches_format_definition():
    # OCP 8-bit floating point spec, E4M3: bias 7, max normal 448, min normal
    # 2^-6, min subnormal 2^-9, S.1111.111 is NaN, no infinities.
    assert oracle.e4m3_to_double(0x38) == 1.0
    assert oracle.e4m3_to_double(0x7E) == 448.0
    assert oracle.e4m3_to_double(0xFE) == -448.0
    assert oracle.e4m3_to_double(0x08) == 2.0 ** -6
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_double(0x07) == 7 / 8 * 2.0 ** -6
    assert oracle.e4m3_to_double(0x78) == 256.0
    assert np.isnan(oracle.e4m3_to_double(0x7F)) and np.isnan(oracle.e4m3_to_double(0xFF))
    vals = [oracle.e4m3_to_double(c) for c in range(256)]
    finite = [v for v in vals if not np.isnan(v)]
    assert len(finite) == 254
    pos = vals[:0x7F]
    assert all(a < b for a, b in zip(pos, pos[1:]))  # magnitude codes are monotone
    # independent decode from the definition, element by element
    ref = e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(ref), np.isnan(vals))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ref[ok], np.asarray(vals)[ok])


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (448.0, 0x7E), (-448.0, 0xFE), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80), (3 * 2.0 ** -10, 0x02),
    (1.0625, 0x38),    # tie between 1.0 (0x38) and 1.125 (0x39): even mantissa
    (1.1875, 0x3A),    # tie between 1.125 (0x39) and 1.25 (0x3A): even mantissa
    (1.0625 + 1e-9, 0x39), (0.0, 0x00), (-0.0, 0x80), (float("nan"), 0x7F),
])
def test_e4m3_encode_fixed_points(x, code):
    assert oracle.e4m3_from_double(x) == code


def test_e4m3_encode_matches_torch_cast_in_range():
    # torch's float8_e4m3fn cast is a library round-to-nearest-even for
    # in-range values; sweep random values, all code values and all midpoints.
    rng = np.random.default_rng(1)
    codes = np.arange(0x7F)
    v = e4m3_decode(codes)
    mids = (v[:-1] + v[1:]) / 2
    x = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000), rng.normal(0, 0.01, 5000),
        v, -v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    x = x.astype(np.float32).astype(np.float64)  # torch casts from float32
    ours = oracle.e4m3_from_double_array(x)
    theirs = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 480.0, 500.0, 1e30, -449.0, -1e30])
    np.testing.assert_array_equal(oracle.e4m3_from_double_array(x),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_bf16_encode_matches_torch_cast_on_float32():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    ties = ((rng.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x32 = np.concatenate([x32, ties, rng.normal(0, 1, 50000).astype(np.float32)])
    ours = oracle.bf16_from_double_array(x32.astype(np.float64))
    np.testing.assert_array_equal(ours, f32_to_bf16_bits(x32))


def test_bf16_encode_rounds_once_from_double():
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7: tie -> even (1.0).
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    # a hair above the midpoint must round up; a float32 detour would lose it
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # 1 + 3*2^-8 is the midpoint between 1+2^-7 (odd) and 1+2^-6 (even)
    assert oracle.bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_from_double(-2.5) == 0xC020
    assert oracle.bf16_from_double(3.0e38 * 1.2) == 0x7F80  # overflow to inf
    assert oracle.bf16_from_double(2.0 ** -133) == 0x0001   # smallest subnormal


# --------------------------------------------------------------- geometry


def test_shard_geometry_matches_worked_example():
    with open(os.path.join(GOLDEN, "shard_geometry.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert oracle.shard_geometry(c["num_tokens"], c["num_tokens_pad"], c["tp"], c["rank"]) == (
            c["shard_rows"], c["local_start"], c["valid_rows"])
    c = g["cases"][0]
    pads = sum(c["num_tokens_pad"] // c["tp"] - oracle.shard_geometry(
        c["num_tokens"], c["num_tokens_pad"], c["tp"], r)[2] for r in range(c["tp"]))
    assert pads == g["pad_rows_total"]


@pytest.mark.parametrize("args", [(10, 12, 5, 0), (13, 12, 4, 0), (10, 12, 4, 4), (10, 12, 4, -1),
                                  (10, 12, 0, 0)])
def test_shard_geometry_rejects_bad_layouts(args):
    with pytest.raises(oracle.OracleError):
        oracle.shard_geometry(*args)


# ------------------------------------------------------------ closed forms


def _run(partials, residual, weight, bias=None, eps=0.0, quant=NONE, deepstack=None, tp_rank=0,
         num_tokens=None, out_dtype=oracle.ORC_F32, static_scale=1.0, rows=None, partial_scale=1.0):
    tp, S, H = np.asarray(partials).shape
    return oracle.reduce_add_rmsnorm(partials, residual, weight, bias, eps, quant, deepstack,
                                     tp_rank=tp_rank,
                                     num_tokens=tp * S if num_tokens is None else num_tokens,
                                     out_dtype=out_dtype, static_scale=static_scale, rows=rows,
                                     partial_scale=partial_scale)


def test_closed_form_rmsnorm_rows():
    # H = 4, two partials, deepstack and residual, eps = 0 unless stated.
    w = f32([1.5, 2.0, -1.0, 0.5])
    b = f32([0.25, -0.5, 0.0, 0.125])
    P = f32([[[1, 0, 0, 0], [-1, -1, -1, -1]],
             [[1, 0, 0, 0], [-2, -2, -2, -2]]])          # [tp=2][S=2][H=4]
    D = f32([[0, 0, 0, 0], [0.5, 0.5, 0.5, 0.5]])
    R = f32([[0, 0, 0, 0], [-1.5, -1.5, -1.5, -1.5]])
    r = _run(P, R, w, b, deepstack=D)
    # row 0: z = (2,0,0,0), mean z^2 = 1, so y = (2w0+b0, b1, b2, b3)
    # row 1: z = -4 everywhere, mean z^2 = 16, rstd = 1/4, so y = -w + b
    np.testing.assert_array_equal(r["residual_out"], [[2, 0, 0, 0], [-4, -4, -4, -4]])
    np.testing.assert_array_equal(r["out"], [[3.25, -0.5, 0.0, 0.125],
                                            [-1.25, -2.5, 1.0, -0.375]])


def test_closed_form_eps_inside_sqrt_and_mean_over_h():
    # z = (1,1,1,1): mean z^2 = 1; with eps = 3, rstd = 1/sqrt(1+3) = 1/2.
    # (eps outside the root, or a divisor of H-1, gives a different value.)
    w = f32([1.0, 2.0, 4.0, -8.0])
    P = f32([[[1, 1, 1, 1]]])
    r = _run(P, f32([[0, 0, 0, 0]]), w, eps=3.0)
    np.testing.assert_array_equal(r["out"], [[0.5, 1.0, 2.0, -4.0]])


def test_closed_form_bf16_output_bits():
    w = f32_to_bf16_bits(np.array([1.5, 2.0, -1.0, 0.5], np.float32))
    b = f32_to_bf16_bits(np.array([0.25, -0.5, 0.0, 0.125], np.float32))
    P = f32([[[1, 0, 0, 0]], [[1, 0, 0, 0]]])
    r = oracle.reduce_add_rmsnorm(P, f32_to_bf16_bits(np.zeros((1, 4), np.float32)), w, b, 0.0,
                                  NONE, tp_rank=0, num_tokens=1, out_dtype=oracle.ORC_BF16)
    np.testing.assert_array_equal(r["out"], f32_to_bf16_bits(np.array([[3.25, -0.5, 0, 0.125]],
                                                                       np.float32)))


def test_textbook_rmsnorm_special_case():
    # tp = 1, no deepstack, zero residual: plain RMSNorm, checked against
    # torch.nn.functional.rms_norm in float64 (a library routine).
    rng = np.random.default_rng(3)
    H = 96
    z = rng.normal(0, 2, (1, 7, H)).astype(np.float32)
    w = rng.normal(1, 0.1, H).astype(np.float32)
    b = rng.normal(0, 0.02, H).astype(np.float32)
    eps = np.float32(1e-6)
    r = _run(z, np.zeros((7, H), np.float32), w, b, eps=float(eps))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(z[0]).double(), (H,),
                                       weight=torch.from_numpy(w).double(), eps=float(eps))
    ref = ref + torch.from_numpy(b).double()
    np.testing.assert_allclose(r["y"], ref.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(r["out"], ref.numpy().astype(np.float32))


def test_multi_partial_sum_is_exact_with_integers():
    # small integers: every partial must be summed exactly once
    rng = np.random.default_rng(4)
    tp, S, H = 5, 3, 16
    P = rng.integers(-8, 9, (tp, S, H)).astype(np.float32)
    R = rng.integers(-8, 9, (S, H)).astype(np.float32)
    D = rng.integers(-8, 9, (S, H)).astype(np.float32)
    r = _run(P, R, np.ones(H, np.float32), deepstack=D)
    np.testing.assert_array_equal(r["residual_out"], P.sum(0) + D + R)


# -------------------------------------------------- the pages' equivalences


def _all_ranks_setup(tp=4, T=10, T_pad=12, H=16, seed=5, deepstack=True):
    rng = np.random.default_rng(seed)
    full = rng.normal(0, 0.5, (tp, T_pad, H)).astype(np.float32)   # rank q's full partial
    R = rng.normal(0, 1, (T_pad, H)).astype(np.float32)
    D = rng.normal(0, 0.3, (T_pad, H)).astype(np.float32) if deepstack else None
    w = rng.normal(1, 0.1, H).astype(np.float32)
    b = rng.normal(0, 0.02, H).astype(np.float32)
    return full, R, D, w, b


@pytest.mark.parametrize("quant,od", [(NONE, oracle.ORC_BF16), (STATIC, oracle.ORC_E4M3),
                                      (DYNAMIC, oracle.ORC_E4M3), (MX, oracle.ORC_E4M3),
                                      (MX, oracle.ORC_E2M1)])
def test_reduce_scatter_plus_all_gather_equals_all_reduce(quant, od):
    # [SP/FC] §2.2: RS followed by AG reproduces AR, and a per-token norm on
    # each shard equals the norm after gathering.  Path A: one shard holding
    # every row (the all-reduce path).  Path B: every rank on its own
    # contiguous slice (replicated residual and full deepstack chunked by
    # rank), concatenated in rank order and unpadded.
    tp, T, T_pad, H = 4, 10, 12, 64
    full, R, D, w, b = _all_ranks_setup(tp, T, T_pad, H)
    S = T_pad // tp
    kw = dict(quant=quant, static_scale=0.01, eps=1e-6, out_dtype=od)
    A = _run(full, R, w, b, deepstack=D, tp_rank=0, num_tokens=T, **kw)
    B = [_run(np.ascontiguousarray(full[:, r * S:(r + 1) * S]), R, w, b, deepstack=D, tp_rank=r,
              num_tokens=T, **kw) for r in range(tp)]
    for key in ["residual_out", "out", "z", "y"] + (["out_scale"] if quant in (DYNAMIC, MX) else []):
        cat = np.concatenate([x[key] for x in B])
        np.testing.assert_array_equal(cat[:T], A[key][:T], err_msg=key)
        assert not np.any(cat[T:]), key  # padding rows of the last rank are zero
    # the same through the oracle's AllGather + unpad ([SP/FC] §3.3)
    for key in ("residual_out", "out"):
        g, _ = oracle.all_gather_unpad([x[key] for x in B], num_tokens=T)
        np.testing.assert_array_equal(g, A[key][:T], err_msg=key)
    if quant in (DYNAMIC, MX):
        g, gs = oracle.all_gather_unpad([x["out"] for x in B], [x["out_scale"] for x in B],
                                        num_tokens=T)
        np.testing.assert_array_equal(g, A["out"][:T])
        np.testing.assert_array_equal(gs, A["out_scale"][:T])


def test_shard_residual_equals_replicated_chunk():
    # maybe_chunk_residual ([SP/FC] §2.3): a replicated residual contributes
    # its block [tp_rank]; passing that block directly gives the same result.
    tp, T, T_pad, H = 4, 12, 12, 8
    full, R, D, w, b = _all_ranks_setup(tp, T, T_pad, H)
    S = T_pad // tp
    for r in range(tp):
        Pr = np.ascontiguousarray(full[:, r * S:(r + 1) * S])
        a = _run(Pr, R, w, b, deepstack=D, tp_rank=r, eps=1e-6)
        c = _run(Pr, np.ascontiguousarray(R[r * S:(r + 1) * S]), w, b,
                 deepstack=np.ascontiguousarray(D[r * S:(r + 1) * S]), tp_rank=r, eps=1e-6)
        for key in ("residual_out", "out", "y"):
            np.testing.assert_array_equal(a[key], c[key])


def test_row_selection_matches_full_run():
    tp, T, T_pad, H = 4, 11, 12, 8
    full, R, D, w, b = _all_ranks_setup(tp, T, T_pad, H)
    S = T_pad // tp
    Pr = np.ascontiguousarray(full[:, 3 * S:])
    a = _run(Pr, R, w, b, deepstack=D, tp_rank=3, num_tokens=T, eps=1e-6, quant=DYNAMIC)
    rows = [2, 0, 1]
    c = _run(Pr, R, w, b, deepstack=D, tp_rank=3, num_tokens=T, eps=1e-6, quant=DYNAMIC,
             rows=rows)
    for key in ("residual_out", "out", "out_scale", "y"):
        np.testing.assert_array_equal(a[key][rows], c[key])


# ------------------------------------------------------------- quantisation


def test_dynamic_per_token_closed_form():
    # z = (1,1,1,1): y = w exactly (eps 0).  amax = 1, scale = 1/448 and the
    # codes encode 448*w: 448 -> 0x7E, -224 -> 0xF6, 112 -> 0x6E, 56 -> 0x66.
    w = f32([1.0, -0.5, 0.25, 0.125])
    P = f32([[[1, 1, 1, 1], [0, 0, 0, 0]]])
    r = _run(P, f32([[0, 0, 0, 0], [0, 0, 0, 0]]), w, quant=DYNAMIC, eps=1e-6,
             out_dtype=oracle.ORC_E4M3)
    r0 = _run(P[:, :1], f32([[0, 0, 0, 0]]), w, quant=DYNAMIC, eps=0.0, out_dtype=oracle.ORC_E4M3)
    np.testing.assert_array_equal(r0["out"][0], [0x7E, 0xF6, 0x6E, 0x66])
    assert r0["out_scale"][0] == np.float32(1.0 / 448.0)
    # an all-zero valid row: scale 0 and zero codes
    assert r["out_scale"][1] == 0.0 and not np.any(r["out"][1])


def test_dynamic_per_token_brute_force():
    # per row: scale = max|y| / 448 found by a linear scan; the argmax
    # element maps to +-448; every code is the nearest e4m3 value to y/scale.
    rng = np.random.default_rng(6)
    tp, S, H = 3, 5, 40
    P = rng.normal(0, 0.5, (tp, S, H)).astype(np.float32)
    R = rng.normal(0, 1, (S, H)).astype(np.float32)
    w = rng.normal(1, 0.1, H).astype(np.float32)
    r = _run(P, R, w, quant=DYNAMIC, eps=1e-6, out_dtype=oracle.ORC_E4M3)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(P.astype(np.float64).sum(0) + R), (H,),
                                       weight=torch.from_numpy(w).double(), eps=1e-6).numpy()
    for s in range(S):
        amax = max(abs(v) for v in ref[s])
        assert abs(r["out_scale"][s] - amax / 448) <= 1e-6 * amax / 448
        t = ref[s] / np.float64(r["out_scale"][s])
        dec = e4m3_decode(r["out"][s])
        k = int(np.argmax(np.abs(ref[s])))
        assert r["out"][s][k] in (0x7E, 0xFE)
        grid = e4m3_decode(np.arange(0x7F))
        for j in range(H):  # nearest by exhaustive search over the grid
            best = grid[np.argmin(np.abs(grid - min(abs(t[j]), 448.0)))]
            assert abs(dec[j]) == best or abs(abs(dec[j]) - abs(t[j])) == abs(best - abs(t[j]))


def test_static_quant_and_saturation():
    rng = np.random.default_rng(7)
    tp, S, H = 2, 4, 32
    P = rng.normal(0, 0.5, (tp, S, H)).astype(np.float32)
    R = rng.normal(0, 1, (S, H)).astype(np.float32)
    w = rng.normal(1, 0.1, H).astype(np.float32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(P.astype(np.float64).sum(0) + R), (H,),
                                       weight=torch.from_numpy(w).double(), eps=1e-6).numpy()
    amax = np.abs(ref).max()
    s = np.float32(amax / 448)
    r = _run(P, R, w, quant=STATIC, eps=1e-6, static_scale=float(s), out_dtype=oracle.ORC_E4M3)
    codes = r["out"]
    k = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    assert codes[k] in (0x7E, 0xFE)
    np.testing.assert_allclose(e4m3_decode(codes), ref / s, rtol=2.0 ** -4, atol=2.0 ** -10)
    # half the calibrated scale: everything above 448 saturates to +-448
    r2 = _run(P, R, w, quant=STATIC, eps=1e-6, static_scale=float(s) / 2, out_dtype=oracle.ORC_E4M3)
    big = np.abs(ref / (s / 2)) > 448
    assert big.any()
    np.testing.assert_array_equal(np.abs(e4m3_decode(r2["out"][big])), 448.0)


# ---------------------------------------------------------------- invariants


def test_power_of_two_scale_invariance():
    # eps = 0: scaling every input by 2^k scales z by 2^k exactly and leaves
    # y, bf16 out, codes and per-token scales unchanged.
    rng = np.random.default_rng(8)
    tp, S, H = 4, 3, 24
    P = rng.normal(0, 0.5, (tp, S, H)).astype(np.float32)
    R = rng.normal(0, 1, (S, H)).astype(np.float32)
    D = rng.normal(0, 0.3, (S, H)).astype(np.float32)
    w = rng.normal(1, 0.1, H).astype(np.float32)
    for quant in (NONE, DYNAMIC):
        od = oracle.ORC_BF16 if quant == NONE else oracle.ORC_E4M3
        a = _run(P, R, w, deepstack=D, quant=quant, out_dtype=od)
        c = _run(P * 8, R * 8, w, deepstack=D * 8, quant=quant, out_dtype=od)
        np.testing.assert_array_equal(c["residual_out"], a["residual_out"] * 8)
        np.testing.assert_array_equal(c["out"], a["out"])
        np.testing.assert_allclose(c["y"], a["y"], rtol=1e-15)


def test_padding_rows_are_zero_and_never_read():
    # [PR18671] §5.2/§5.3: padding rows of the shard are zeroed.  Fill their
    # inputs with NaN: outputs on padding rows must be exactly 0, no NaN anywhere.
    tp, T, T_pad, H = 4, 9, 12, 8
    full, R, D, w, b = _all_ranks_setup(tp, T, T_pad, H)
    S = T_pad // tp
    r = tp - 1
    v = T - r * S  # 0 valid rows on the last rank
    Pr = np.ascontiguousarray(full[:, r * S:])
    Pr[:, v:] = np.nan
    R2, D2 = R.copy(), D.copy()
    R2[r * S + v:] = np.nan
    D2[r * S + v:] = np.nan
    for quant in (NONE, STATIC, DYNAMIC):
        out = _run(Pr, R2, w, b, deepstack=D2, tp_rank=r, num_tokens=T, eps=1e-6, quant=quant,
                   static_scale=0.01, out_dtype=oracle.ORC_BF16 if quant == NONE else oracle.ORC_E4M3)
        for key, val in out.items():
            if val is None:
                continue
            assert not np.any(np.isnan(val.astype(np.float64))), key
            assert not np.any(val[v:]), key


def test_partial_shard_padding():
    tp, T, T_pad, H = 4, 10, 12, 8
    full, R, D, w, b = _all_ranks_setup(tp, T, T_pad, H)
    S = T_pad // tp
    Pr = np.ascontiguousarray(full[:, 3 * S:])
    Pr[:, 1:] = np.nan
    out = _run(Pr, R, w, b, deepstack=D, tp_rank=3, num_tokens=T, eps=1e-6,
               out_dtype=oracle.ORC_BF16)
    assert np.all(np.isfinite(out["y"][0])) and np.any(out["out"][0])
    assert not np.any(out["out"][1:]) and not np.any(out["residual_out"][1:])


# ------------------------------------------------------------------- NaN
#
# The pages say nothing about NaN.  The reading taken: IEEE arithmetic all
# the way, and every NaN reaches the output in the format's own NaN
# encoding -- the OCP e4m3 NaN code S.1111.111 (never a saturated code), the
# E8M0 NaN byte 0xFF of the OCP microscaling format (which makes its whole
# block NaN), IEEE NaN for bf16/f32 and for the per-token scale.  What pins
# it beyond those definitions: a NaN cannot change any output it does not
# feed (rows and, for a gain or bias NaN, columns and blocks elsewhere stay
# bit-identical to a run without it), and one NaN in z reaches every y of its
# row through the sum of squares.

_NAN_MODES = [(NONE, oracle.ORC_BF16), (NONE, oracle.ORC_F32), (STATIC, oracle.ORC_E4M3),
              (DYNAMIC, oracle.ORC_E4M3), (MX, oracle.ORC_E4M3), (MX, oracle.ORC_E2M1)]


def _nan_setup(seed=11, tp=2, S=3, H=64):
    rng = np.random.default_rng(seed)
    P = f32(rng.normal(0, 0.5, (tp, S, H)))
    R = f32(rng.normal(0, 1, (S, H)))
    w = f32(rng.normal(1, 0.1, H))
    b = f32(rng.normal(0, 0.02, H))
    return P, R, w, b


def _is_nan_out(out, od):
    if od == oracle.ORC_BF16:
        return np.isnan(bf16_bits_to_f64(out))
    if od == oracle.ORC_F32:
        return np.isnan(out)
    return None


def _assert_all_nan(res, row, od, quant):
    """Every output of shard row `row` is NaN in its format's encoding."""
    out = res["out"][row]
    if quant == NONE:
        assert _is_nan_out(out, od).all()
    elif quant in (STATIC, DYNAMIC) or (quant == MX and od == oracle.ORC_E4M3):
        assert (out == 0x7F).all()
    else:  # MX e2m1: no NaN code, the 0xFF scale carries it
        assert not out.any()
    if quant == DYNAMIC:
        assert np.isnan(res["out_scale"][row])
    if quant == MX:
        assert (res["out_scale"][row] == 0xFF).all()


@pytest.mark.parametrize("quant,od", _NAN_MODES)
@pytest.mark.parametrize("where", ["partial", "residual", "deepstack"])
def test_nan_input_in_a_valid_row_reaches_every_output_of_that_row(quant, od, where):
    P, R, w, b = _nan_setup()
    D = f32(np.random.default_rng(3).normal(0, 0.3, R.shape))
    clean = _run(P, R, w, b, eps=1e-6, quant=quant, deepstack=D, out_dtype=od, static_scale=0.01)
    P2, R2, D2 = P.copy(), R.copy(), D.copy()
    {"partial": P2[1], "residual": R2, "deepstack": D2}[where][1, 5] = np.nan
    got = _run(P2, R2, w, b, eps=1e-6, quant=quant, deepstack=D2, out_dtype=od, static_scale=0.01)
    # the updated residual is NaN at that element only
    nan_res = np.isnan(got["residual_out"])
    assert nan_res[1, 5] and nan_res.sum() == 1
    keep = np.ones(R.shape, bool)
    keep[1, 5] = False
    np.testing.assert_array_equal(got["residual_out"][keep], clean["residual_out"][keep])
    # the row's sum of squares is NaN, so every y and every output of the row is
    assert np.isnan(got["y"][1]).all()
    _assert_all_nan(got, 1, od, quant)
    # the other rows are untouched by it
    for key in ("out", "out_scale", "residual_out"):
        if key in got:
            for r in (0, 2):
                np.testing.assert_array_equal(got[key][r], clean[key][r])


@pytest.mark.parametrize("quant,od", _NAN_MODES)
@pytest.mark.parametrize("which", ["weight", "bias"])
def test_nan_gain_or_bias_element_reaches_its_column(quant, od, which):
    P, R, w, b = _nan_setup(seed=12)
    h0 = 37  # inside block 1 (elements 32..63)
    clean = _run(P, R, w, b, eps=1e-6, quant=quant, out_dtype=od, static_scale=0.01)
    w2, b2 = w.copy(), b.copy()
    (w2 if which == "weight" else b2)[h0] = np.nan
    got = _run(P, R, w2, b2, eps=1e-6, quant=quant, out_dtype=od, static_scale=0.01)
    # the residual and rstd do not involve the gain or bias
    np.testing.assert_array_equal(got["residual_out"], clean["residual_out"])
    assert np.isnan(got["y"][:, h0]).all()
    others = np.ones(R.shape[1], bool)
    others[h0] = False
    np.testing.assert_array_equal(got["y"][:, others], clean["y"][:, others])
    if quant == NONE:
        assert _is_nan_out(got["out"][:, h0], od).all()
        np.testing.assert_array_equal(got["out"][:, others], clean["out"][:, others])
    elif quant == STATIC:
        assert (got["out"][:, h0] == 0x7F).all()
        np.testing.assert_array_equal(got["out"][:, others], clean["out"][:, others])
    elif quant == DYNAMIC:
        # the row maximum skips nothing: every row's scale is NaN
        for r in range(R.shape[0]):
            _assert_all_nan(got, r, od, quant)
    else:
        # only the block holding h0 is NaN; block 0 is as before
        assert (got["out_scale"][:, 1] == 0xFF).all()
        np.testing.assert_array_equal(got["out_scale"][:, 0], clean["out_scale"][:, 0])
        if od == oracle.ORC_E4M3:
            assert (got["out"][:, 32:64] == 0x7F).all()
            np.testing.assert_array_equal(got["out"][:, :32], clean["out"][:, :32])
        else:
            assert not got["out"][:, 16:32].any()
            np.testing.assert_array_equal(got["out"][:, :16], clean["out"][:, :16])


# ---------------------------------------------------------------- validation


@pytest.mark.parametrize("case", ["rank", "tokens", "residual_rows", "deepstack_rows",
                                  "quant_dyn_tensor", "static_scale_zero", "static_scale_inf"])
def test_oracle_rejects_invalid_problems(case):
    tp, S, H = 2, 3, 8
    P = np.zeros((tp, S, H), np.float32)
    R = np.zeros((S, H), np.float32)
    w = np.ones(H, np.float32)
    kw = dict(tp_rank=0, num_tokens=tp * S, out_dtype=oracle.ORC_F32)
    args = [P, R, w, None, 1e-6, NONE, None]
    if case == "rank":
        kw["tp_rank"] = 2
    elif case == "tokens":
        kw["num_tokens"] = tp * S + 1
    elif case == "residual_rows":
        args[1] = np.zeros((S + 1, H), np.float32)
    elif case == "deepstack_rows":
        args[6] = np.zeros((S + 2, H), np.float32)
    elif case == "quant_dyn_tensor":
        args[5] = 3  # dynamic per-tensor has no shard-local scale
    elif case == "static_scale_zero":
        args[5] = STATIC
        kw["static_scale"] = 0.0
    elif case == "static_scale_inf":
        args[5] = STATIC
        kw["static_scale"] = float("inf")
    with pytest.raises(oracle.OracleError):
        oracle.reduce_add_rmsnorm(*args, **kw)


def test_bf16_inputs_are_decoded_exactly():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], np.uint16)
    np.testing.assert_array_equal(bf16_bits_to_f64(bits),
                                  [oracle.bf16_to_double(int(b)) for b in bits])
    assert oracle.bf16_to_double(0x3F80) == 1.0 and oracle.bf16_to_double(0xC000) == -2.0


def test_all_gather_unpad_worked_example():
    # [PR18671] §2: 3500 tokens padded to 3504 over TP=16, 219 per rank; the
    # gathered, unpadded tensor has 3500 rows, rank 15 contributes its first
    # 215 rows starting at row 3285, and its 4 padding rows are dropped.
    with open(os.path.join(GOLDEN, "shard_geometry.json")) as f:
        g = json.load(f)
    c = g["cases"][-1]
    tp, S, T = c["tp"], c["shard_rows"], c["num_tokens"]
    H = 8
    shards = [np.empty((S, H), np.uint16) for _ in range(tp)]
    for q in range(tp):
        shards[q][:, 0] = q
        shards[q][:, 1] = np.arange(S)
        shards[q][:, 2:] = 7
    scales = [np.full(S, q, np.float32) + np.arange(S, dtype=np.float32) / 1000 for q in range(tp)]
    out, out_scale = oracle.all_gather_unpad(shards, scales, num_tokens=T)
    assert out.shape == (T, H)
    start, valid = c["local_start"], c["valid_rows"]
    np.testing.assert_array_equal(out[start:, 0], tp - 1)
    np.testing.assert_array_equal(out[start:, 1], np.arange(valid))
    assert out[start - 1, 0] == tp - 2 and out[start - 1, 1] == S - 1
    np.testing.assert_array_equal(out[:S, 1], np.arange(S))
    np.testing.assert_array_equal(out_scale[start:], scales[-1][:valid])
    assert T - start == valid and S - valid == g["pad_rows_total"]


def test_all_gather_unpad_of_empty_shards():
    # S = 0 (no tokens in the step): nothing to gather, as the library allows
    for scaled in (False, True):
        shards = [np.empty((0, 16), np.uint8) for _ in range(3)]
        scales = [np.empty((0,), np.float32) for _ in range(3)] if scaled else None
        out, out_scale = oracle.all_gather_unpad(shards, scales, num_tokens=0)
        assert out.shape == (0, 16) and (out_scale is None) == (not scaled)
        assert not scaled or out_scale.shape == (0,)



# ------------------------------------------------ block scaling (MX form)


def test_e2m1_decode_matches_format_definition():
    # OCP FP4 E2M1: bias 1, subnormal m/2, no NaN/inf: 0, .5, 1, 1.5, 2, 3, 4, 6
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [oracle.e2m1_to_double(c) for c in range(8)] == mags
    assert [oracle.e2m1_to_double(c | 8) for c in range(8)] == [-m for m in mags]


@pytest.mark.parametrize("x,code", [
    (0.0, 0), (-0.0, 8), (0.5, 1), (1.0, 2), (6.0, 7), (-6.0, 15), (100.0, 7), (-7.0, 15),
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),   # ties: even
    (0.26, 1), (2.51, 5), (4.99, 6), (5.01, 7), (-1.3, 11),
])
def test_e2m1_encode_fixed_points(x, code):
    assert oracle.e2m1_from_double(x) == code


def test_e2m1_encode_brute_force_sweep():
    grid = np.array([oracle.e2m1_to_double(c) for c in range(8)])
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.uniform(-7, 7, 5000), (grid[:-1] + grid[1:]) / 2])
    codes = oracle.e2m1_from_double_array(x)
    for xi, c in zip(x, codes):
        a = min(abs(xi), 6.0)
        d = np.abs(grid - a)
        assert d[c & 7] == d.min()
        assert (c >> 3) == (1 if np.signbit(xi) else 0)


def _exact_rows(values):
    """Partials/residual/gain such that y equals `values` exactly: z = +-1
    everywhere (mean square 1, eps 0, rstd 1) and w = values * sign."""
    values = np.asarray(values, np.float32)
    n, H = values.shape
    rng = np.random.default_rng(H)
    sign = np.where(rng.random((n, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    # one shared gain: rows differ only through the sign pattern, so give
    # every row its own call
    return [(sign[i:i + 1][None], np.zeros((1, H), np.float32), values[i] * sign[i])
            for i in range(n)]


def _mx_row(values, od):
    (P, R, w), = _exact_rows(np.asarray(values, np.float32)[None])
    r = _run(P, R, w, quant=MX, eps=0.0, out_dtype=od)
    return r


def _e2m1_unpack(packed, H):
    out = np.empty(H, np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out


def test_mx_fp4_closed_form_blocks():
    blk = np.zeros(32, np.float32)
    blk[:8] = [6.0, 3.0, -1.5, 0.5, 0.25, 0.75, -2.5, 5.0]
    vals = np.concatenate([blk, blk * 2.0 ** 5, np.zeros(32, np.float32), blk * 2.0 ** -140])
    r = _mx_row(vals, oracle.ORC_E2M1)
    codes = _e2m1_unpack(r["out"][0], vals.size)
    # block 0: max 6 -> floor(log2 6) - 2 = 0 -> X = 1 -> byte 127
    # block 1: max 6*2^5 -> X = 2^5 -> byte 132, same codes
    # block 2: all zero -> e = -127 -> byte 0, zero codes
    # block 3: max 6*2^-140 -> e = -140 < -127 clamps -> byte 0; y*2^127 ~ 2^-13 -> 0
    np.testing.assert_array_equal(r["out_scale"][0], [127, 132, 0, 0])
    want = [7, 5, 11, 1, 0, 2, 12, 6] + [0] * 24
    np.testing.assert_array_equal(codes[:32], want)
    np.testing.assert_array_equal(codes[32:64], want)
    assert not (codes[64:] & 7).any()


def test_mx_fp8_closed_form_blocks():
    blk = np.zeros(32, np.float32)
    blk[:6] = [448.0, 300.0, -1.0, 0.5, 2.0 ** -9, 464.0 / 2]
    sat = np.zeros(32, np.float32)
    sat[:3] = [500.0, 260.0, -1.0]
    vals = np.concatenate([blk, blk / 256, sat])
    r = _mx_row(vals, oracle.ORC_E4M3)
    # block 0: max 448 -> floor(log2 448) - 8 = 0 -> byte 127, codes of the values
    # block 1: the same / 256 -> e = -8 -> byte 119, same codes
    # block 2: max 500 -> e = 0, 500 saturates to 448
    np.testing.assert_array_equal(r["out_scale"][0], [127, 119, 127])
    c = r["out"][0]
    np.testing.assert_array_equal(c[:6], [0x7E, 0x79, 0xB8, 0x30, 0x01, 0x76])  # 300 -> 288
    np.testing.assert_array_equal(c[32:38], c[:6])
    np.testing.assert_array_equal(c[64:67], [0x7E, 0x78, 0xB8])


def test_mx_block_scale_invariance():
    # scaling a whole row by 2^k moves every E8M0 byte by k and keeps the codes
    rng = np.random.default_rng(10)
    vals = (rng.normal(0, 1, 128) * np.repeat([1.0, 2.0 ** -3, 7.0, 1e-3], 32)).astype(np.float32)
    for od in (oracle.ORC_E4M3, oracle.ORC_E2M1):
        a = _mx_row(vals, od)
        c = _mx_row(vals * 2.0 ** 6, od)
        np.testing.assert_array_equal(c["out"], a["out"])
        np.testing.assert_array_equal(c["out_scale"].astype(int), a["out_scale"].astype(int) + 6)


def test_mx_codes_decode_within_half_a_step():
    # every block: codes decode, times 2^e, to within half an element step of y
    rng = np.random.default_rng(11)
    vals = rng.normal(0, 1, 256).astype(np.float32)
    for od, emax in ((oracle.ORC_E4M3, 8), (oracle.ORC_E2M1, 2)):
        r = _mx_row(vals, od)
        e = r["out_scale"][0].astype(int) - 127
        codes = r["out"][0] if od == oracle.ORC_E4M3 else _e2m1_unpack(r["out"][0], 256)
        dec = e4m3_decode(codes) if od == oracle.ORC_E4M3 else np.array(
            [oracle.e2m1_to_double(c) for c in codes])
        for b in range(8):
            blk = vals[32 * b:32 * b + 32].astype(np.float64)
            assert e[b] == int(np.floor(np.log2(np.abs(blk).max()))) - emax
            t = blk / 2.0 ** e[b]
            if od == oracle.ORC_E4M3:
                step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6))) - 3)
                tmax = 448.0
            else:
                step = np.where(np.abs(t) < 2, 0.5, np.where(np.abs(t) < 4, 1.0, 2.0))
                tmax = 6.0
            d = dec[32 * b:32 * b + 32]
            assert (np.abs(d - np.clip(t, -tmax, tmax)) <= step / 2 + 1e-12).all()



def test_partials_scaled_before_the_sum():
    # [PR18671] §5.3: the o_proj output is multiplied by a factor before the
    # reduction.  Partials (4, 0, 0, 0) and (-2, 2, 0, 0) scaled by 1/2 sum to
    # (1, 1, 0, 0); residual (1, -1, 0, 0) gives z = (2, 0, 0, 0) -> y = (2w0, 0, 0, 0).
    w = f32([1.5, 2.0, -1.0, 0.5])
    P = f32([[[4, 0, 0, 0]], [[-2, 2, 0, 0]]])
    r = _run(P, f32([[1, -1, 0, 0]]), w, partial_scale=0.5)
    np.testing.assert_array_equal(r["residual_out"], [[2, 0, 0, 0]])
    np.testing.assert_array_equal(r["out"], [[3.0, 0, 0, 0]])
    # scaling every partial by c equals feeding c-scaled partials
    rng = np.random.default_rng(12)
    P = rng.normal(0, 0.5, (3, 4, 16)).astype(np.float32)
    R = rng.normal(0, 1, (4, 16)).astype(np.float32)
    a = _run(P, R, np.ones(16, np.float32), partial_scale=0.25, eps=1e-6)
    c = _run(P * np.float32(0.25), R, np.ones(16, np.float32), eps=1e-6)
    np.testing.assert_array_equal(a["z"], c["z"])


# ------------------------------------------------- FlashComm2 regrouping


def test_fc2_regroup_matches_worked_example():
    with open(os.path.join(GOLDEN, "fc2_regroup_example.json")) as f:
        g = json.load(f)
    G, otp = g["global_tp"], g["otp"]
    assert oracle.fc2_batch_ids(G, otp) == g["batch_ids"]
    N, Cc = 8, 3                      # 4 segments of 2 tokens, 3 feature columns per rank
    seg = N // G
    # value = 100*token + 10*rank + column: every element says where it came from
    srcs = [np.array([[100 * n + 10 * q + c for c in range(Cc)] for n in range(N)], np.float32)
            for q in range(G)]
    dsts = oracle.fc2_regroup(srcs, otp)
    letters = g["features"]
    for r, blocks in g["rank_rows"].items():
        d = dsts[int(r)]
        assert d.shape == (N // (G // otp), (G // otp) * Cc)
        for b, (tok, feats) in enumerate(blocks):
            segment = int(tok[1:])
            for u in range(seg):
                row = d[b * seg + u]
                n = segment * seg + u
                want = [100 * n + 10 * letters.index(ch) + c for ch in feats for c in range(Cc)]
                np.testing.assert_array_equal(row, want)


@pytest.mark.parametrize("G,otp", [(8, 2), (8, 4), (16, 4), (6, 3)])
def test_fc2_regroup_then_otp_reduce_gives_sequence_parallel_layout(G, otp):
    # [SP/FC] §4.5-4.6: the OTP group of rank r (same position j) computes
    # o_proj on the same tokens with different feature columns; its
    # reduce-scatter hands rank r token segment r -- the same rows and the
    # same sums as the global-TP reduce-scatter.  Integer data: exact.
    rng = np.random.default_rng(G * 10 + otp)
    N, Cc, Hout = 4 * G, 2, 5
    X = rng.integers(-3, 4, (N, G * Cc)).astype(np.float64)       # all features of all tokens
    W = rng.integers(-3, 4, (G * Cc, Hout)).astype(np.float64)    # o_proj weight
    srcs = [np.ascontiguousarray(X[:, q * Cc:(q + 1) * Cc]) for q in range(G)]
    dsts = oracle.fc2_regroup(srcs, otp)
    odp, seg = G // otp, N // G
    tp_sum = X @ W                                                 # global-TP all-reduce
    for r in range(G):
        gidx, j = divmod(r, odp)
        total = np.zeros((seg, Hout))
        for g2 in range(otp):                                      # OTP group of r
            r2 = g2 * odp + j
            part = dsts[r2] @ W[g2 * odp * Cc:(g2 + 1) * odp * Cc]  # its o_proj partial
            total += part[gidx * seg:(gidx + 1) * seg]             # rows of segment r
        np.testing.assert_array_equal(total, tp_sum[r * seg:(r + 1) * seg])


# ------------------------------------------- DSA-CP o_proj exchange (path B)


@pytest.mark.parametrize("tp,S,D", [(2, 3, 2), (4, 5, 3), (8, 2, 4), (16, 3, 1)])
def test_dsacp_path_b_equals_path_a(tp, S, D):
    # [PR18671] §5.3: path A runs o_proj with the full weight on the rank's
    # own tokens and all heads; path B exchanges heads for tokens, runs the
    # row-parallel o_proj on the rank's heads, scales, reduce-scatters.  Both
    # must hand every rank the same output rows (integers: exact).
    rng = np.random.default_rng(tp * 100 + S)
    Hout = 7
    attn = [rng.integers(-3, 4, (S, tp * D)).astype(np.float64) for _ in range(tp)]
    W = rng.integers(-3, 4, (tp * D, Hout)).astype(np.float64)
    c = 0.5                                             # a power of two keeps it exact
    recv = oracle.dsacp_heads_to_tokens(attn)
    for q in range(tp):
        assert recv[q].shape == (tp * S, D)
    proj = [c * (recv[q] @ W[q * D:(q + 1) * D]) for q in range(tp)]   # [tp*S, Hout] each
    for p in range(tp):
        path_b = sum(proj[q][p * S:(p + 1) * S] for q in range(tp))     # RS: rank p's rows
        path_a = c * (attn[p] @ W)
        np.testing.assert_array_equal(path_b, path_a)


@pytest.mark.parametrize("tp,S,D", [(2, 4, 8), (4, 3, 5), (8, 1, 2)])
def test_dsacp_exchange_is_undone_by_the_plain_all_to_all(tp, S, D):
    # the FC2 regroup with otp = 1 (one ODP group: every rank takes its own
    # token segment with all features) is the inverse permutation
    rng = np.random.default_rng(tp + S + D)
    attn = [rng.integers(0, 1 << 16, (S, tp * D)).astype(np.uint16) for _ in range(tp)]
    back = oracle.fc2_regroup(oracle.dsacp_heads_to_tokens(attn), otp=1)
    for p in range(tp):
        np.testing.assert_array_equal(back[p], attn[p])


# ------------------------------- row-parallel GEMM + scatter (the producer)


def _bf16_bits(a):
    a = np.asarray(a, dtype=np.float32)
    assert np.array_equal(a, (a.view(np.uint32) & 0xFFFF0000).view(np.float32)), "not bf16-exact"
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def test_matmul_scatter_brute_force():
    # every element against a plain triple loop over exact integers and halves
    rng = np.random.default_rng(5)
    tp, S, K, N = 3, 2, 5, 4
    x = rng.integers(-6, 7, (tp * S, K)) / 2.0
    w = rng.integers(-5, 6, (N, K)) / 2.0
    for rank in range(tp):
        dst = oracle.matmul_scatter(_bf16_bits(x), _bf16_bits(w), tp=tp, rank=rank)
        for m in range(tp * S):
            r, s = divmod(m, S)
            for n in range(N):
                want = 0.0
                for k in range(K):
                    want += x[m][k] * w[n][k]
                assert dst[r][rank][s][n] == want, (rank, m, n)
                for q in range(tp):
                    if q != rank:
                        assert dst[r][q][s][n] == 0.0


@pytest.mark.parametrize("tp,S,Kr,N", [(2, 3, 4, 5), (4, 2, 3, 6), (8, 1, 2, 3)])
def test_matmul_reduce_scatter_equals_all_reduce(tp, S, Kr, N):
    # [SPquant] §二 / [SP/FC] §2.2: each rank's K-slice GEMM, scattered by token
    # block and summed on the destination, equals the full GEMM's row block
    rng = np.random.default_rng(tp * 10 + S)
    X = rng.integers(-4, 5, (tp * S, tp * Kr)).astype(np.float32)   # full input
    W = rng.integers(-4, 5, (N, tp * Kr)).astype(np.float32)        # full weight [N, K]
    dst = None
    for q in range(tp):
        dst = oracle.matmul_scatter(_bf16_bits(X[:, q * Kr:(q + 1) * Kr]),
                                    _bf16_bits(W[:, q * Kr:(q + 1) * Kr]), tp=tp, rank=q, dst=dst)
    full = X.astype(np.float64) @ W.T.astype(np.float64)
    for r in range(tp):
        np.testing.assert_array_equal(dst[r].astype(np.float64).sum(0), full[r * S:(r + 1) * S])


def test_matmul_scatter_places_token_blocks_by_destination():
    # x row m carries its token index; w picks it out: element = m.  Rank q's
    # block for destination r must sit in slot q of dst[r] (rows r*S + s)
    tp, S, K, N = 4, 3, 2, 2
    x = np.zeros((tp * S, K), np.float32)
    x[:, 0] = np.arange(tp * S)
    w = np.zeros((N, K), np.float32)
    w[:, 0] = 1.0
    for q in range(tp):
        dst = oracle.matmul_scatter(_bf16_bits(x * (q + 1)), _bf16_bits(w), tp=tp, rank=q)
        for r in range(tp):
            for s in range(S):
                np.testing.assert_array_equal(dst[r][q][s], (q + 1) * (r * S + s))


def test_matmul_scatter_rows_and_bf16_rounding():
    # bf16 output is the once-rounded exact dot product; rows selects tokens
    x = np.array([[1.0, 2.0 ** -8], [3.0, 1.0]], np.float32)     # 1 + 2^-8 is a bf16 tie
    w = np.array([[1.0, 1.0]], np.float32)
    dst = oracle.matmul_scatter(_bf16_bits(x), _bf16_bits(w), tp=1, rank=0,
                                out_dtype=oracle.ORC_BF16, rows=[0])
    assert dst[0][0][0][0] == 0x3F80        # ties to even: 1.0
    assert dst[0][0][1][0] == 0             # row 1 not computed
    d32 = oracle.matmul_scatter(_bf16_bits(x), _bf16_bits(w), tp=1, rank=0)
    assert d32[0][0][0][0] == np.float32(1 + 2.0 ** -8) and d32[0][0][1][0] == 4.0


def test_producer_feeds_the_fused_path():
    # the receive buffer of rank r, reduced by the fused oracle, equals the
    # fused oracle on the AllReduced GEMM output (integers: exact)
    tp, S, Kr, N = 4, 3, 8, 32
    rng = np.random.default_rng(77)
    X = rng.integers(-3, 4, (tp * S, tp * Kr)).astype(np.float32)
    W = rng.integers(-3, 4, (N, tp * Kr)).astype(np.float32)
    R = _bf16_bits(rng.integers(-4, 5, (tp * S, N)).astype(np.float32))
    g = _bf16_bits(np.ones(N, np.float32))
    dst = None
    for q in range(tp):
        dst = oracle.matmul_scatter(_bf16_bits(X[:, q * Kr:(q + 1) * Kr]),
                                    _bf16_bits(W[:, q * Kr:(q + 1) * Kr]), tp=tp, rank=q, dst=dst)
    full = (X.astype(np.float64) @ W.T.astype(np.float64)).astype(np.float32)[None]
    T = tp * S - 2
    for r in range(tp):
        a = oracle.reduce_add_rmsnorm(dst[r], R, g, None, 1e-6, oracle.QUANT_NONE, None,
                                      tp_rank=r, num_tokens=T)
        v = max(0, min(S, T - r * S))
        b = oracle.reduce_add_rmsnorm(full[:, r * S:(r + 1) * S].copy(), R[r * S:(r + 1) * S], g,
                                      None, 1e-6, oracle.QUANT_NONE, None, tp_rank=0, num_tokens=v)
        np.testing.assert_array_equal(a["out"], b["out"])
        np.testing.assert_array_equal(a["residual_out"], b["residual_out"])


def _finite_e4m3_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def test_scaled_matmul_with_unit_scales_equals_bf16_matmul():
    # every finite e4m3 value is exact in bf16, so the FP8 producer on codes
    # equals the (pinned) bf16 producer on their bf16 images
    rng = np.random.default_rng(8)
    tp, S, K, N = 2, 3, 48, 5
    x8 = _finite_e4m3_codes(rng, (tp * S, K))
    w8 = _finite_e4m3_codes(rng, (N, K))
    dec = np.vectorize(oracle.e4m3_to_double)
    xb, wb = _bf16_bits(dec(x8).astype(np.float32)), _bf16_bits(dec(w8).astype(np.float32))
    one = np.ones(1, np.float32)
    for rank in range(tp):
        a = oracle.scaled_matmul_scatter(x8, one, w8, one, tp=tp, rank=rank)
        b = oracle.matmul_scatter(xb, wb, tp=tp, rank=rank)
        for r in range(tp):
            np.testing.assert_array_equal(a[r], b[r])


def test_scaled_matmul_brute_force_with_row_and_column_scales():
    rng = np.random.default_rng(9)
    tp, S, K, N = 2, 2, 6, 3
    x8 = _finite_e4m3_codes(rng, (tp * S, K))
    w8 = _finite_e4m3_codes(rng, (N, K))
    xs = rng.uniform(0.5, 2, tp * S).astype(np.float32)
    ws = rng.uniform(0.5, 2, N).astype(np.float32)
    dst = oracle.scaled_matmul_scatter(x8, xs, w8, ws, tp=tp, rank=1, out_dtype=oracle.ORC_F32)
    for m in range(tp * S):
        r, s = divmod(m, S)
        for n in range(N):
            dot = 0.0
            for k in range(K):
                dot += oracle.e4m3_to_double(int(x8[m, k])) * oracle.e4m3_to_double(int(w8[n, k]))
            want = np.float32(dot * float(xs[m]) * float(ws[n]))
            assert dst[r][1][s][n] == want, (m, n)


def test_scaled_matmul_scale_placement():
    # codes of 1.0 everywhere: P[m][n] = K * x_scale[m] * w_scale[n]; powers of
    # two keep it exact and tell rows from columns
    tp, S, K, N = 2, 4, 16, 6
    x8 = np.full((tp * S, K), 0x38, np.uint8)
    w8 = np.full((N, K), 0x38, np.uint8)
    xs = (2.0 ** (np.arange(tp * S) % 4)).astype(np.float32)
    ws = (2.0 ** -(np.arange(N) % 3)).astype(np.float32)
    for xsc, wsc in ((xs, ws), (xs[:1], ws), (xs, ws[:1]), (xs[:1], ws[:1])):
        dst = oracle.scaled_matmul_scatter(x8, xsc, w8, wsc, tp=tp, rank=0)
        for m in range(tp * S):
            r, s = divmod(m, S)
            want = K * (xsc[0] if xsc.size == 1 else xs[m]) * (wsc if wsc.size > 1 else np.full(N, wsc[0]))
            np.testing.assert_array_equal(dst[r][0][s], want.astype(np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.scaled_matmul_scatter(x8, xs[:3], w8, ws, tp=tp, rank=0)   # neither 1 nor M scales

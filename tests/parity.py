"""GPU-vs-oracle parity driver shared by the GPU tests and the smoke check.

Runs libsprms on seeded inputs (through the C ABI via the binding), runs the
CPU oracle on the same inputs (copied to the host before the call), and
checks every computed row with the rules in helpers.py.  Output buffers are
allocated with a canary row on each side that must come back untouched.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import (bf16_bits_to_f64, bf16_round, e4m3_decode, e4m3_round, to_host,
                     within_rounding, y_error, z_error)
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_NONE, QUANT_STATIC_TENSOR,
                                           Workload, make_inputs)

QUANT_MX_BLOCK = sp.SP_QUANT_MX_BLOCK


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e2m1 decode from the format definition (bias 1, subnormal m/2)."""
    c = codes.astype(np.int64)
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_round(x: np.ndarray) -> np.ndarray:
    return e2m1_decode(oracle.e2m1_from_double_array(x))


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out

CANARY = 0xA5


@dataclasses.dataclass
class Result:
    rows: np.ndarray
    valid: int
    stats: dict


def _host_f64(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _canary_buffer(S: int, H: int, dtype, dev):
    buf = torch.empty(((S + 2) * H,), dtype=torch.uint8 if dtype == torch.uint8 else dtype,
                      device=dev)
    buf.view(torch.uint8).fill_(CANARY)
    return buf.view(S + 2, H), buf.view(S + 2, H)[1:S + 1]


def run_case(w: Workload, rank: int, *, dev, S: Optional[int] = None, T: Optional[int] = None,
             rows: Optional[Sequence[int]] = None, pad_fill: Optional[float] = float("nan"),
             in_place: bool = False, out_dtype: Optional[torch.dtype] = None,
             static_scale: Optional[float] = None, shard_deepstack: bool = False,
             inputs: Optional[dict] = None, base_seed: Optional[int] = None,
             require_exact_frac: float = 0.99, fp4: bool = False,
             partial_scale: float = 1.0, workers: int = 1) -> Result:
    S = w.shard_rows if S is None else S
    T = min(w.num_tokens, w.tp * S) if T is None else T
    kw = {} if base_seed is None else {"base_seed": base_seed}
    x = inputs if inputs is not None else make_inputs(w, rank=rank, device=dev, shard_rows=S,
                                                       num_tokens=T, pad_fill=pad_fill, **kw)
    tp, S_, H = x["partials"].shape
    assert S_ == S
    if shard_deepstack and x["deepstack"] is not None and x["deepstack"].shape[0] != S:
        x["deepstack"] = x["deepstack"][rank * S:(rank + 1) * S].contiguous()
    quant = w.quant_mode
    out_dtype = out_dtype or w.out_dtype
    v = max(0, min(S, T - rank * S))

    # host copies of every input before the call (the residual may be updated in place)
    h = {k: to_host(t) for k, t in x.items()}

    mx = quant == QUANT_MX_BLOCK
    fp4 = fp4 and mx
    out_buf, out = _canary_buffer(S, H // 2 if fp4 else H, out_dtype, dev)
    res_buf = res_out = None
    if not in_place:
        res_buf, res_out = _canary_buffer(S, H, w.act_dtype, dev)
    scale_t = None
    if quant == QUANT_STATIC_TENSOR:
        assert static_scale is not None
        scale_t = torch.tensor([static_scale], dtype=torch.float32, device=dev)
    elif quant == QUANT_DYNAMIC_TOKEN:
        scale_buf = torch.full((S + 2,), float("nan"), dtype=torch.float32, device=dev)
        scale_t = scale_buf[1:S + 1]
    elif mx:
        scale_buf, scale_t = _canary_buffer(S, H // 32, torch.uint8, dev)

    sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], x["bias"], w.eps,
                             quant, x["deepstack"], out, scale_t, tp_rank=rank, num_tokens=T,
                             residual_out=res_out, out_dtype=sp.SP_FP4_E2M1 if fp4 else None,
                             partial_scale=partial_scale)
    torch.cuda.synchronize()

    # ---- canaries and untouched memory (byte-exact)
    ob = out_buf.view(torch.uint8).cpu().numpy().reshape(S + 2, -1)
    assert (ob[0] == CANARY).all() and (ob[-1] == CANARY).all(), "out canary overwritten"
    roff = rank * S if x["residual"].shape[0] == tp * S and tp > 1 else 0
    if res_buf is not None:
        rb = res_buf.view(torch.uint8).cpu().numpy().reshape(S + 2, -1)
        assert (rb[0] == CANARY).all() and (rb[-1] == CANARY).all(), "residual_out canary"
        got_res_full = to_host(res_out)
        # the input residual is read only
        np.testing.assert_array_equal(to_host(x["residual"]).view(np.uint8),
                                      h["residual"].view(np.uint8))
    else:
        res_now = to_host(x["residual"])
        got_res_full = res_now[roff:roff + S]
        # rows of other ranks' blocks are untouched
        mask = np.ones(res_now.shape[0], bool)
        mask[roff:roff + S] = False
        np.testing.assert_array_equal(res_now[mask].view(np.uint8), h["residual"][mask].view(np.uint8))
    if quant == QUANT_DYNAMIC_TOKEN:
        sb = scale_buf.cpu().numpy()
        assert np.isnan(sb[0]) and np.isnan(sb[-1]), "out_scale canary"
    if mx:
        sb = scale_buf.cpu().numpy()
        assert (sb[0] == CANARY).all() and (sb[-1] == CANARY).all(), "out_scale canary"
    for k in ("partials", "weight", "bias", "deepstack"):
        if x[k] is not None:
            np.testing.assert_array_equal(to_host(x[k]).view(np.uint8), h[k].view(np.uint8))

    # ---- oracle and checks on the selected rows, in row chunks on host threads
    if rows is None:
        rows = np.arange(S)
    rows = np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    got_out_full = to_host(out)
    got_scale_full = None if scale_t is None or quant == QUANT_STATIC_TENSOR else scale_t.cpu().numpy()
    ctx = dict(w=w, h=h, rank=rank, T=T, S=S, tp=tp, v=v, roff=roff, quant=quant, mx=mx, fp4=fp4,
               out_dtype=out_dtype, static_scale=static_scale, partial_scale=partial_scale,
               got_res=got_res_full, got_out=got_out_full, got_scale=got_scale_full)
    chunks = [rows] if workers <= 1 else [rows[i:i + CHUNK_ROWS] for i in range(0, len(rows), CHUNK_ROWS)]
    if len(chunks) == 1:
        parts = [_check_rows(ctx, chunks[0])]
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            parts = list(pool.map(lambda c: _check_rows(ctx, c), chunks))
    counts = {}
    for part in parts:
        for k, val in part.items():
            counts[k] = max(counts.get(k, 0.0), val) if k.endswith("_max") else counts.get(k, 0) + val

    stats = {"rows": len(rows), "elements": len(rows) * H}
    for key in ("residual_exact", "out_exact", "codes_exact", "block_scale_exact"):
        if counts.get(key + "_n"):
            stats[key] = counts[key] / counts[key + "_n"]
    if "scale_rel_max" in counts:
        stats["scale_max_rel"] = counts["scale_rel_max"]
    if counts.get("codes_exact_n"):
        frac = 1.0 - stats["codes_exact"]
        assert frac <= 1e-3, f"{frac:.3%} of codes differ from the oracle's"
    # bf16 roundings of fp32 and fp64 values differ only next to a rounding tie
    checks = []
    if w.act_dtype == torch.bfloat16 and counts.get("residual_exact_n"):
        checks.append("residual_exact")
    if quant == QUANT_NONE and out_dtype == torch.bfloat16 and counts.get("out_exact_n"):
        checks.append("out_exact")
    for key in checks:
        assert stats[key] >= require_exact_frac, f"{key}={stats[key]}"
    return Result(rows, v, stats)


# rows per oracle call when the check is split over host threads
CHUNK_ROWS = 256
# host threads for the oracle: at most 16 (a one-GPU share of the host)
DEFAULT_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _check_rows(c, rows):
    """Oracle on `rows` (sorted shard rows) and every check against the GPU's
    outputs on them; returns counts, summed over chunks by the caller."""
    w, h, quant, mx, fp4, out_dtype = c["w"], c["h"], c["quant"], c["mx"], c["fp4"], c["out_dtype"]
    rank, S, tp, v, roff = c["rank"], c["S"], c["tp"], c["v"], c["roff"]
    H = h["partials"].shape[2]
    ref = oracle.reduce_add_rmsnorm(
        h["partials"], h["residual"], h["weight"], h["bias"], w.eps, quant, h["deepstack"],
        tp_rank=rank, num_tokens=c["T"],
        out_dtype=oracle.ORC_E2M1 if fp4 else {torch.bfloat16: oracle.ORC_BF16,
                                                torch.float32: oracle.ORC_F32}.get(
            out_dtype, oracle.ORC_E4M3),
        static_scale=c["static_scale"] if c["static_scale"] is not None else 1.0, rows=rows,
        partial_scale=c["partial_scale"])
    counts = {}
    valid = rows < v
    pad = ~valid
    got_res = c["got_res"][rows]
    got_out = c["got_out"][rows]

    # ---- padding rows: every output byte zero
    if pad.any():
        assert not got_res[pad].view(np.uint8).any(), "residual_out not zero on padding rows"
        assert not got_out[pad].view(np.uint8).any(), "out not zero on padding rows"
        if quant in (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK):
            assert not c["got_scale"][rows[pad]].any(), "out_scale not zero on padding rows"
    if not valid.any():
        return counts

    vr = rows[valid]
    z = ref["z"][valid]
    y = ref["y"][valid]
    P = _host_f64(h["partials"][:, vr, :])
    cs = abs(float(np.float32(c["partial_scale"])))
    A = cs * np.abs(P).sum(0) + np.abs(_host_f64(h["residual"][roff + vr]))
    del P
    if h["deepstack"] is not None:
        doff = rank * S if h["deepstack"].shape[0] == tp * S and tp > 1 else 0
        A += np.abs(_host_f64(h["deepstack"][doff + vr]))
    wv = _host_f64(h["weight"])
    bv = None if h["bias"] is None else _host_f64(h["bias"])
    err_z = z_error(A, tp)
    rstd = 1.0 / np.sqrt((z * z).mean(1) + np.float64(np.float32(w.eps)))
    err_y = y_error(y, bv, err_z, rstd, wv)

    # ---- updated residual
    gr = _host_f64(got_res[valid])
    if w.act_dtype == torch.bfloat16:
        ok = within_rounding(gr, z - err_z, z + err_z, bf16_round)
    else:
        ok = np.abs(gr - z) <= err_z + U_half(z)
    counts["residual_exact"] = int((got_res[valid] == ref["residual_out"][valid]).sum())
    counts["residual_exact_n"] = int(valid.sum()) * H
    assert ok.all(), f"residual_out outside bound at rows {vr[np.argwhere(~ok)[:5, 0]].tolist()}"

    # ---- normalised output
    go = got_out[valid]
    if quant == QUANT_NONE:
        g = _host_f64(go)
        rnd = bf16_round if out_dtype == torch.bfloat16 else (lambda t: t.astype(np.float32).astype(np.float64))
        ok = within_rounding(g, y - err_y, y + err_y, rnd)
        assert ok.all(), f"out outside bound at rows {vr[np.argwhere(~ok)[:5, 0]].tolist()}"
        assert (np.abs(g - y) <= 1e-3 + 2.0 ** -7 * np.abs(y)).all(), "out outside 1e-3 + 2^-7|y|"
        counts["out_exact"] = int((go == ref["out"][valid]).sum())
        counts["out_exact_n"] = go.size
    elif mx:
        _check_mx(counts, go, c["got_scale"][vr], ref["out"][valid], ref["out_scale"][valid],
                  y, err_y, fp4)
    else:
        if quant == QUANT_STATIC_TENSOR:
            sc = np.full(len(vr), np.float64(np.float32(c["static_scale"])))
        else:
            sc_gpu = c["got_scale"][vr].astype(np.float64)
            sc_ref = ref["out_scale"][valid].astype(np.float64)
            rel = np.abs(sc_gpu - sc_ref) / np.maximum(sc_ref, 1e-30)
            assert (rel <= 1e-5).all(), f"per-token scale off by {rel.max():.3g}"
            assert (rel <= 2.0 ** -16).all(), f"per-token scale off by {rel.max():.3g}"
            counts["scale_rel_max"] = float(rel.max())
            sc = sc_gpu
        g = e4m3_decode(go)
        zero = sc == 0  # a row whose max |y| is 0: scale 0 and zero codes
        assert not g[zero].any(), "non-zero codes on a row with scale 0"
        sc_safe = np.where(zero, 1.0, sc)[:, None]
        t = np.where(zero[:, None], 0.0, y / sc_safe)
        err_t = np.where(zero[:, None], 0.0, err_y / sc_safe + 2.0 ** -21 * np.abs(t))
        ok = within_rounding(g, t - err_t, t + err_t, e4m3_round)
        assert ok.all(), f"e4m3 codes outside bound at rows {vr[np.argwhere(~ok)[:5, 0]].tolist()}"
        own = ref["out"][valid]
        diff = go != own
        both_zero = (e4m3_decode(own) == 0) & (g == 0)
        diff &= ~both_zero
        counts["codes_exact"] = int(diff.size - diff.sum())
        counts["codes_exact_n"] = diff.size
        # a differing code is the oracle's neighbour in value order
        assert (np.abs(e4m3_ordinal(go[diff]) - e4m3_ordinal(own[diff])) <= 1).all(), \
            "an e4m3 code more than one step from the oracle's"
    return counts


def U_half(z):
    return 2.0 ** -24 * np.abs(z)


def e4m3_ordinal(codes):
    """Position of an e4m3 code in value order, +0 and -0 both 0: adjacent
    values (one e4m3 step apart) have ordinals that differ by exactly 1."""
    c = codes.astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def e2m1_ordinal(codes):
    c = codes.astype(np.int64)
    return np.where(c & 0x8, -(c & 0x7), c & 0x7)


def _check_mx(stats, got_codes, got_scale, ref_codes, ref_scale, y, err_y, fp4):
    """Block-scaled outputs.  The block exponent is an integer decided by the
    block max: accept the GPU's wherever the max lies within the y error bound
    of a power of two; then every code must be a correct rounding of
    y * 2^-e (the kernel's scaling by 2^-e is exact) within the bound."""
    emax = 2 if fp4 else 8
    n, H = y.shape
    nb = H // 32
    yb = np.abs(y).reshape(n, nb, 32)
    eb = err_y.reshape(n, nb, 32)

    def exp_of(m):
        e = np.where(m > 0, np.floor(np.log2(np.where(m > 0, m, 1.0))) - emax, -127)
        return np.clip(e, -127, 127)

    e_lo = exp_of(np.maximum(yb - eb, 0).max(-1))
    e_hi = exp_of((yb + eb).max(-1))
    e_gpu = got_scale.astype(np.int64) - 127
    ok = (e_gpu >= e_lo) & (e_gpu <= e_hi)
    assert ok.all(), f"block exponents outside the bound at {np.argwhere(~ok)[:5].tolist()}"
    stats["block_scale_exact"] = int((got_scale == ref_scale).sum())
    stats["block_scale_exact_n"] = got_scale.size
    codes = unpack_e2m1(got_codes) if fp4 else got_codes
    own = unpack_e2m1(ref_codes) if fp4 else ref_codes
    dec, rnd = (e2m1_decode, e2m1_round) if fp4 else (e4m3_decode, e4m3_round)
    X = np.repeat(2.0 ** e_gpu, 32, axis=1)
    t = y / X
    err_t = err_y / X
    g = dec(codes)
    ok = within_rounding(g, t - err_t, t + err_t, rnd)
    assert ok.all(), f"block codes outside bound at {np.argwhere(~ok)[:5].tolist()}"
    same_e = np.repeat(got_scale == ref_scale, 32, axis=1)  # blocks on the oracle's exponent
    diff = (codes != own) & ~((dec(own) == 0) & (g == 0)) & same_e
    stats["codes_exact"] = int(diff.size - diff.sum())
    stats["codes_exact_n"] = diff.size
    ordinal = e2m1_ordinal if fp4 else e4m3_ordinal
    assert (np.abs(ordinal(codes[diff]) - ordinal(own[diff])) <= 1).all(), \
        "a block code more than one step from the oracle's"

"""Benchmark of the fused shard path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C5]
                    [--path fused|gather|fc2|dsacp] [--quant mxfp8|mxfp4]

One step = one call of sp_reduce_add_rmsnorm over the whole shard of the
workload's timed rank (every stage of the path in one kernel), inputs
already resident in HBM.  Prints one JSON line: whole-job HBM throughput
over the algorithmic bytes (GB/s), the roofline of the kernel (per-launch
HIP-event durations on the launch stream), and the CPU oracle timed on a
bounded sample of the same shard.  The default run (C5, the headline) also
times C4 with the same protocol, before the headline's inputs are allocated,
and reports it under "also".
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import reduce_add_rmsnorm_amd as sp  # noqa: E402
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK,  # noqa: E402
                                           QUANT_STATIC_TENSOR, WORKLOADS, make_inputs)

METRIC = "achieved HBM GB/s (% of MI355X peak) + shard tokens/s for fused reduce-add-RMSNorm"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published
# sources each measured kernel is built from: the fused kernel, and the
# layout kernels (gather, regroupings)
_CSRC = os.path.join(ROOT, "reduce_add_rmsnorm_amd", "csrc")
KERNEL_SRCS = {"fused": [os.path.join(_CSRC, f) for f in ("sprms.hip", "common.h")],
               "layout": [os.path.join(_CSRC, f) for f in ("layout.hip", "common.h")],
               "gemm": [os.path.join(_CSRC, f) for f in ("gemm.hip", "common.h")]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.md")
QUANT_NAMES = {0: "none (bf16 out)", 1: "static per-tensor e4m3", 2: "dynamic per-token e4m3",
               4: "block-scaled (32-element E8M0 scales)"}


def kernel_hash(kind: str = "fused") -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS[kind]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str = "fused"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current source of the kernel; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"<!--\s*traffic\s+(\{.*?\})\s*-->", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(workload)
    if not rec or rec.get("kernel_sha256_16") != kernel_hash(kind):
        return None
    return int(rec["hbm_bytes_per_launch"])


def static_scale() -> float:
    with open(os.path.join(ROOT, "tests", "golden", "c4_static_scale.json")) as f:
        return float(json.load(f)["scale"])


def setup(w, dev):
    x = make_inputs(w, rank=w.rank, device=dev)
    S, H = w.shard_rows, w.hidden
    out = torch.empty((S, H // 2 if w.fp4 else H), dtype=w.out_dtype, device=dev)
    res_out = torch.empty((S, H), dtype=w.act_dtype, device=dev)
    scale = None
    if w.quant_mode == QUANT_STATIC_TENSOR:
        scale = torch.tensor([static_scale()], dtype=torch.float32, device=dev)
    elif w.quant_mode == QUANT_DYNAMIC_TOKEN:
        scale = torch.empty((S,), dtype=torch.float32, device=dev)
    elif w.quant_mode == QUANT_MX_BLOCK:
        scale = torch.empty((S, H // 32), dtype=torch.uint8, device=dev)
    def make_launch():
        """The call marshalled once, on torch's current stream at this moment."""
        return sp.prepare(x["partials"], x["residual"], x["weight"], x["bias"], w.eps, w.quant_mode,
                          x["deepstack"], out, scale, tp_rank=w.rank, num_tokens=w.num_tokens,
                          residual_out=res_out, out_dtype=sp.SP_FP4_E2M1 if w.fp4 else None)

    launch = make_launch()
    launch.remake = make_launch
    return x, launch, (out, res_out, scale)


def setup_gather(w, dev):
    """Every rank's shard output of the workload (S x H in the output dtype,
    plus per-row scales for quantised outputs), gathered into [T, H]."""
    S, H, T = w.shard_rows, w.hidden, w.num_tokens
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_index)
    if w.out_dtype == torch.uint8:
        shards = [torch.randint(0, 256, (S, H), generator=g, device=dev, dtype=torch.uint8)
                  for _ in range(w.tp)]
    else:
        shards = [torch.randn((S, H), generator=g, device=dev).to(w.out_dtype) for _ in range(w.tp)]
    scaled = w.quant_mode == QUANT_DYNAMIC_TOKEN
    scales = [torch.rand(S, generator=g, device=dev) for _ in range(w.tp)] if scaled else None
    out = torch.empty((T, H), dtype=w.out_dtype, device=dev)
    out_scale = torch.empty((T,), dtype=torch.float32, device=dev) if scaled else None

    def launch():
        sp.sp_all_gather_unpad(shards, scales, out, out_scale, num_tokens=T)

    e = out.element_size()
    nbytes = 2 * T * (H * e + (4 if scaled else 0))  # read and write each gathered byte once
    return (shards, scales, out, out_scale), launch, nbytes, T


FC2_OTP = 2  # the o_proj group size of the FlashComm2 worked example


def setup_fc2(w, dev):
    """FlashComm2 o_proj input regrouping, one rank's share: the workload's
    tp ranks as the FlashComm2 group (G = tp, otp = 2), each holding its
    H/G feature columns of all num_tokens_pad tokens in bf16; rank w.rank
    pulls its [N/odp, odp*H/G] block from the G source buffers."""
    G, N, H = w.tp, w.num_tokens_pad, w.hidden
    Cc = H // G
    odp = G // FC2_OTP
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_index + 1)
    srcs = [torch.randn((N, Cc), generator=g, device=dev).to(torch.bfloat16) for _ in range(G)]
    dsts = [None] * G
    dsts[w.rank] = torch.empty((N // odp, odp * Cc), dtype=torch.bfloat16, device=dev)

    def launch():
        sp.sp_fc2_regroup(srcs, dsts, otp=FC2_OTP, rank=w.rank)

    nbytes = 2 * (N // odp) * odp * Cc * 2  # read and write the block once
    desc = (f"FlashComm2 regroup, rank {w.rank} of G={G}, otp={FC2_OTP}: [{N}, {Cc}] x {G} -> "
            f"[{N // odp}, {odp * Cc}] bf16")
    return (srcs, dsts), launch, nbytes, N // odp, desc


def setup_dsacp(w, dev):
    """DSA-CP o_proj input exchange, one rank's share: the workload's tp
    ranks each hold their S shard tokens with every rank's heads, [S, H] in
    bf16 (H = tp * D); rank w.rank pulls every token's head block, [tp*S, D]."""
    tp, S, H = w.tp, w.shard_rows, w.hidden
    D = H // tp
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_index + 2)
    attn = [torch.randn((S, tp * D), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
    outs = [None] * tp
    outs[w.rank] = torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev)

    def launch():
        sp.sp_dsacp_heads_to_tokens(attn, outs, rank=w.rank)

    nbytes = 2 * tp * S * D * 2
    desc = (f"DSA-CP head-to-token exchange, rank {w.rank} of tp={tp}: [{S}, {tp * D}] x {tp} -> "
            f"[{tp * S}, {D}] bf16")
    return (attn, outs), launch, nbytes, tp * S, desc


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD published


def setup_gemm(w, dev):
    """One rank's producer GEMM at the workload's shape: x [T_pad, H/tp] and
    the weight [H, H/tp] in bf16, bf16 partials written into slot `rank` of
    the tp receive buffers [tp, S, H] (o_proj split along K; K = H/tp)."""
    tp, S, H = w.tp, w.shard_rows, w.hidden
    M, K = tp * S, H // tp
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_index + 3)
    x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    wt = (torch.randn((H, K), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    dsts = [torch.empty((tp, S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]

    def launch():
        sp.sp_matmul_scatter(x, wt, dsts, rank=w.rank)

    desc = (f"producer GEMM of rank {w.rank} of tp={tp}: [{M}, {K}] x [{H}, {K}]^T bf16, fp32 "
            f"accumulation, bf16 partials scattered to {tp} receive buffers")
    return (x, wt, dsts), launch, 2 * M * K * H, M, desc


MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak, AMD published


def setup_gemm_fp8(w, dev):
    """The FP8 producer at the workload's shape: e4m3 codes x [T_pad, H/tp]
    with per-token scales, weight [H, H/tp] with per-column scales, bf16
    partials into the tp receive buffers."""
    tp, S, H = w.tp, w.shard_rows, w.hidden
    M, K = tp * S, H // tp
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_index + 4)
    x8 = torch.randint(0, 256, (M, K), generator=g, device=dev, dtype=torch.uint8)
    w8 = torch.randint(0, 256, (H, K), generator=g, device=dev, dtype=torch.uint8)
    x8[(x8 & 0x7F) == 0x7F] = 0x38   # no NaN codes
    w8[(w8 & 0x7F) == 0x7F] = 0x38
    xs = torch.rand((M,), generator=g, device=dev) * 0.01 + 0.001
    ws = torch.rand((H,), generator=g, device=dev) * 0.01 + 0.001
    dsts = [torch.empty((tp, S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]

    def launch():
        sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, dsts, rank=w.rank)

    desc = (f"FP8 producer GEMM of rank {w.rank} of tp={tp}: e4m3 [{M}, {K}] x [{H}, {K}]^T, "
            f"per-token and per-column fp32 scales, bf16 partials scattered to {tp} receive buffers")
    return (x8, xs, w8, ws, dsts), launch, 2 * M * K * H, M, desc


def library_fp8_gemm_us(x8, xs, w8, ws, steps=20):
    """hipBLASLt through torch._scaled_mm on the same codes and scales, for
    context only; None where this torch build does not offer it."""
    try:
        a = x8.view(torch.float8_e4m3fn)
        b = w8.view(torch.float8_e4m3fn).t()
        call = lambda: torch._scaled_mm(a, b, scale_a=xs.view(-1, 1), scale_b=ws.view(1, -1),
                                        out_dtype=torch.bfloat16)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
    except Exception as e:  # noqa: BLE001 -- context only
        return {"error": type(e).__name__ + ": " + str(e)[:120]}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1000 / steps, 2)


def library_gemm_us(x, wt, steps=20):
    """hipBLASLt (torch's linear) on the same operands, for context only."""
    import torch.nn.functional as F
    for _ in range(3):
        F.linear(x, wt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        F.linear(x, wt)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000 / steps


def _host_bits(t):
    """A device tensor as a host array; bf16 as its uint16 bit patterns."""
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _oracle_legs(units: int, make, call, budget_s: float, threads: int):
    """Time the oracle on units [0, n) of the workload in one thread, n grown
    from a probe until the leg takes about budget_s; when all units take
    less, the call is repeated to fill the budget and timed per call.  Then
    the same code on disjoint unit ranges in `threads` threads at once (the
    oracle's C calls release the interpreter lock), repeated as often.
    make(a, b) builds the host arguments of units [a, b) outside the timed
    region; call runs the oracle on them.  Returns (n, seconds per call,
    repeats, n_parallel, seconds per parallel round, threads used)."""
    import threading

    def run(n):
        args = make(0, n)
        t0 = time.perf_counter()
        call(args)
        return time.perf_counter() - t0

    n = min(units, 8)
    secs = run(n)
    while n < units and secs < 0.25:
        n = min(units, n * 8)
        secs = run(n)
    reps = 1
    if n < units and secs < budget_s:
        n = int(min(units, max(n, n * budget_s / max(secs, 1e-9))))
        secs = run(n)
    elif n == units and secs < budget_s / 2:
        args, reps = make(0, n), 0
        t0 = time.perf_counter()
        while reps < 1000 and time.perf_counter() - t0 < budget_s:
            call(args)
            reps += 1
        secs = (time.perf_counter() - t0) / reps
    n_par = int(min(units, max(threads, threads * budget_s / max(secs / n, 1e-12))))
    bounds = np.linspace(0, n_par, threads + 1).astype(int)
    chunks = [make(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]

    def work(c):
        for _ in range(reps):
            call(c)

    workers = [threading.Thread(target=work, args=(c,)) for c in chunks]
    t0 = time.perf_counter()
    for t_ in workers:
        t_.start()
    for t_ in workers:
        t_.join()
    return n, secs, reps, n_par, (time.perf_counter() - t0) / reps, len(workers)


def _host_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def cpu_baseline(path: str, w, x, budget_s: float, threads: int, *, nbytes=None, fp8_gemm=False):
    """The C oracle on a bounded sample of the same workload, in the unit of
    the path's metric: single-threaded, then the same code on disjoint chunks
    in `threads` threads.  The layout and GEMM oracles compute every rank's
    result of their call; their bytes (flops) count what they computed."""
    import oracle  # CPU checker; only this leg of the benchmark uses it

    S, r, tp = w.shard_rows, w.rank, w.tp
    scale, unit, extra = 1e9, "GB/s", {}
    if path == "fused":
        roff = r * S if w.residual_replicated else 0
        out_dt = (oracle.ORC_E2M1 if w.fp4 else oracle.ORC_BF16 if w.out_dtype == torch.bfloat16
                  else oracle.ORC_E4M3)
        sscale = static_scale() if w.quant_mode == QUANT_STATIC_TENSOR else 1.0
        wt = _host_bits(x["weight"])
        bias = None if x["bias"] is None else _host_bits(x["bias"])

        def make(a, b):  # rows [a, b) of the shard as a compact shard of their own (all valid)
            D = None if x["deepstack"] is None else _host_bits(x["deepstack"][r * S + a:r * S + b])
            return (_host_bits(x["partials"][:, a:b]), _host_bits(x["residual"][roff + a:roff + b]), D)

        def call(arr):
            P, R, D = arr
            oracle.reduce_add_rmsnorm(P, R, wt, bias, w.eps, w.quant_mode, D, tp_rank=r,
                                      num_tokens=tp * P.shape[1], out_dtype=out_dt,
                                      static_scale=sscale, want_debug=False)

        units, per_unit, what = S, w.algorithmic_bytes() / S, f"rows of the rank-{r} shard ({w.name})"
    elif path == "gather":
        shards, scales = x[0], x[1]

        def make(a, b):
            return ([_host_bits(t[a:b]) for t in shards],
                    None if scales is None else [_host_bits(t[a:b]) for t in scales])

        def call(arr):
            oracle.all_gather_unpad(arr[0], arr[1], num_tokens=tp * arr[0][0].shape[0])

        units, per_unit = S, tp * nbytes / w.num_tokens
        what = f"rows of each of the {tp} shards, gathered ({w.name})"
    elif path == "fc2":
        srcs = x[0]
        G = len(srcs)

        def make(a, b):  # tokens [G*a, G*b) of every source
            return [_host_bits(t[G * a:G * b]) for t in srcs]

        def call(arr):
            oracle.fc2_regroup(arr, FC2_OTP)

        units = w.num_tokens_pad // G
        per_unit = G * nbytes / units  # every destination of the group
        what = f"token groups of {G} (all {G} destinations of the group, {w.name})"
    elif path == "dsacp":
        attn = x[0]

        def make(a, b):
            return [_host_bits(t[a:b]) for t in attn]

        def call(arr):
            oracle.dsacp_heads_to_tokens(arr)

        units, per_unit = S, tp * nbytes / S  # every rank's destination
        what = f"rows of each rank's tokens (all {tp} destinations, {w.name})"
    elif path == "gemm":
        scale, unit = 1e12, "TFLOP/s"
        if fp8_gemm:
            x8, xs, w8, ws = x[0], x[1], x[2], x[3]
            wh, wsh = _host_bits(w8), _host_bits(ws)

            def make(a, b):
                return _host_bits(x8[a:b]), _host_bits(xs[a:b] if xs.numel() > 1 else xs)

            def call(arr):
                oracle.scaled_matmul_scatter(arr[0], arr[1], wh, wsh, tp=1, rank=0,
                                             out_dtype=oracle.ORC_BF16)
        else:
            xb, wb = x[0], x[1]
            wh = _host_bits(wb)

            def make(a, b):
                return _host_bits(xb[a:b])

            def call(arr):
                oracle.matmul_scatter(arr, wh, tp=1, rank=0, out_dtype=oracle.ORC_BF16)

        units = x[0].shape[0]
        per_unit = nbytes / units  # flops per token row
        what = f"token rows of x against the whole weight, one destination ({w.name})"
    else:
        raise ValueError(path)

    n, secs, reps, n_par, par_secs, nthr = _oracle_legs(units, make, call, budget_s, threads)
    rep = f" per call, mean of {reps} calls" if reps > 1 else ""
    if path == "fused":
        extra = {"tokens_per_s": round(n / secs, 2)}
    return {
        "value": float(f"{n * per_unit / secs / scale:.4g}"),
        "unit": unit,
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {n} of {units} {what}; {secs:.3g} s{rep}"
                  + (f"; {n / secs:.1f} shard tokens/s" if path == "fused" else ""),
        **extra,
        "seconds": float(f"{secs:.4g}"),
        **({"repeats": reps} if reps > 1 else {}),
        "parallel": {"value": float(f"{n_par * per_unit / par_secs / scale:.4g}"), "unit": unit,
                     "cores": nthr, "seconds": float(f"{par_secs:.4g}"),
                     **({"tokens_per_s": round(n_par / par_secs, 2)} if path == "fused" else {}),
                     "sample": f"first {n_par} of {units} in {nthr} disjoint chunks, one thread each{rep}"},
        "host": {"cpu": _host_model(), "logical_cpus": os.cpu_count()},
    }


def time_plain(launch, stream, steps):
    """K back-to-back launches bracketed by HIP events on the launch stream and
    by the host clock between two synchronisations, then a short pass with an
    event pair per launch for the spread.  Returns (mean kernel ms from the
    events, wall ms per step, per-launch ms list)."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        launch()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = ev0.elapsed_time(ev1) / steps
    n_spread = min(steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread)]
    for i in range(n_spread):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return avg_ms, wall * 1000.0 / steps, [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]


def also_fused(name, args, dev):
    """Another workload's fused kernel, timed with the headline's protocol
    (same warm-up and step count), for the same JSON line."""
    w = WORKLOADS[name]
    x, launch, bufs = setup(w, dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    avg_ms, ms_per_step, per = time_plain(launch, stream, args.steps)
    nbytes = w.algorithmic_bytes()
    achieved = nbytes / (avg_ms / 1000.0) / 1e9
    rec = {
        "workload": f"{w.name}: {w.description}",
        "tp": w.tp, "rank": w.rank, "shard_rows": w.shard_rows, "hidden": w.hidden,
        "quant": QUANT_NAMES[w.quant_mode],
        "algorithmic_bytes": nbytes,
        "ms_per_step": round(ms_per_step, 6),
        "value_gbs": round(nbytes / (ms_per_step / 1000.0) / 1e9, 2),
        "shard_tokens_per_s": round(w.valid_rows() / (ms_per_step / 1000.0), 1),
        "kernel_us": {"mean": round(avg_ms * 1000, 2),
                      "median_single": round(statistics.median(per) * 1000, 2),
                      "p10": round(float(np.percentile(per, 10)) * 1000, 2),
                      "p90": round(float(np.percentile(per, 90)) * 1000, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, "fused")},
    }
    del x, launch, bufs
    torch.cuda.empty_cache()
    return rec


def hbm_ceilings(args, dev):
    """HBM rates that plain streaming kernels of torch and the HIP runtime
    reach on this part, to read the fused kernel's figures against: a
    read-mostly reduction (a sum over the first dim of 64 planes: one byte
    written per 64 read), a write-only fill and a device copy over MIB MiB
    each (far past the 256 MB Infinity Cache), and torch's own sums of C4's
    eight and C5's four partial planes (the fused kernel's reduce step alone,
    tp read streams and one write stream).  HIP events around K launches
    after W warm-up launches."""
    n = args.ceilings << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src64 = src.view(64, -1)
    red = torch.empty((src64.shape[1],), dtype=torch.float32, device=dev)
    cases = {
        "read: torch.sum over the first dim of 64 float32 planes": (
            lambda: torch.sum(src64, dim=0, out=red), n, n // 64),
        "write: fill_ of a float32 tensor": (lambda: dst.fill_(1.0), 0, n),
        "copy: device-to-device copy_": (lambda: dst.copy_(src), n, n),
    }
    for name in ("C4", "C5"):
        w = WORKLOADS[name]
        planes = torch.ones((w.tp, w.shard_rows, w.hidden), dtype=torch.bfloat16, device=dev)
        psum = torch.empty((w.shard_rows, w.hidden), dtype=torch.bfloat16, device=dev)
        pb = planes.numel() * 2
        cases[f"{name} partials: torch.sum over the {w.tp} bf16 planes"] = (
            lambda planes=planes, psum=psum: torch.sum(planes, dim=0, out=psum), pb, pb // w.tp)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, (f, nr, nw) in cases.items():
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / args.steps
        res[name] = {"bytes_read": nr, "bytes_written": nw, "us": round(us, 2),
                     "gbs": round((nr + nw) / us / 1e3, 1),
                     "frac_of_peak": round((nr + nw) / us / 1e3 / HBM_PEAK_GBS, 4)}
    print(json.dumps({"hbm_ceilings": res, "mib": args.ceilings, "steps": args.steps,
                      "warmup": args.warmup}), flush=True)


def copy_calibration(args, dev):
    """A device-to-device copy of known size: every launch reads and writes
    exactly n bytes, which fixes the scale of FETCH_SIZE / WRITE_SIZE."""
    n = args.copy_calibration << 20
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000 / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "gbs": round(2 * n / ms / 1e6, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C5", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for each leg of the CPU baseline, single "
                         "thread and all threads (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=min(os.cpu_count() or 1, 16),
                    help="threads of the parallel CPU-baseline leg (default: the host's, at most 16)")
    ap.add_argument("--graph", type=int, default=0, metavar="N",
                    help="capture N launches in one HIP graph and time back-to-back replays "
                         "(per-launch cost without the host launch path, as in a captured step)")
    ap.add_argument("--cold", action="store_true",
                    help="cache-cold protocol for shards that fit the 256 MB Infinity Cache: "
                         "a 512 MiB read+write scrub before every launch, each launch timed "
                         "by its own event pair, value from the median launch")
    ap.add_argument("--path", default="fused", choices=["fused", "gather", "fc2", "dsacp", "gemm"],
                    help="fused: the shard kernel (the headline); gather: AllGather + unpad of "
                         "every rank's shard output of the workload into [T, H] on this GPU; "
                         "fc2 / dsacp: one rank's share of the FlashComm2 o_proj regroup or of "
                         "the DSA-CP head-to-token exchange at the workload's tp, tokens and H; "
                         "gemm: one rank's producer GEMM (o_proj split along K) with its "
                         "ReduceScatter destinations")
    ap.add_argument("--quant", default=None, choices=["mxfp8", "mxfp4", "fp8"],
                    help="fused path: replace the workload's output quantisation by block "
                         "scaling (32-element E8M0 scales) with e4m3 or e2m1 elements; gemm "
                         "path: fp8 times the e4m3 producer (sp_scaled_matmul_scatter)")
    ap.add_argument("--also", default=None, metavar="W[,W...]",
                    help="fused path: further workloads timed with the same protocol before the "
                         "headline's inputs are allocated, reported under 'also' in the same line (default: C4 "
                         "when the headline is the default C5 run; '' for none)")
    ap.add_argument("--ceilings", type=int, default=0, metavar="MIB",
                    help="time plain streaming kernels (read-only sum, fill, copy over MIB MiB, and "
                         "torch's sum of C4's partial planes) instead of the path, for reference")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the path, time a plain device copy of MIB MiB (the "
                         "reference kernel for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fused shard kernel runs on one rank's shard "
              "and the library has no collective path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.quant == "fp8" and args.path != "gemm":
        ap.error("--quant fp8 goes with --path gemm")
    if args.path == "gemm" and args.quant not in (None, "fp8"):
        ap.error("--path gemm takes --quant fp8 or nothing")
    if args.path in ("gather", "fc2", "dsacp") and args.quant:
        ap.error(f"--path {args.path} takes no --quant")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(args, dev)
        return
    if args.ceilings:
        hbm_ceilings(args, dev)
        return
    w = WORKLOADS[args.workload]
    fp8_gemm = args.path == "gemm" and args.quant == "fp8"
    if args.quant and not args.path == "gemm":
        w = dataclasses.replace(w, quant_mode=QUANT_MX_BLOCK, out_dtype=torch.uint8,
                                fp4=args.quant == "mxfp4")
    sp.load()
    also = args.also
    if also is None:
        also = ("C4" if args.path == "fused" and args.workload == "C5" and not args.quant
                and not args.graph and not args.cold else "")
    if also and (args.path != "fused" or args.quant or args.graph or args.cold):
        ap.error("--also goes with the plain fused path")
    # the other workloads first, each on a heap with no other workload's
    # tensors, as in a run of its own (timed after the headline's tensors had
    # been allocated, C4 read about half a point of peak lower)
    also_recs = {n: also_fused(n, args, dev) for n in also.split(",") if n}
    desc = None
    if args.path == "gather":
        x, launch, nbytes, tokens = setup_gather(w, dev)
        desc = (f"{w.name} AllGather + unpad of all {w.tp} shard outputs into "
                f"[{w.num_tokens}, {w.hidden}] (+ per-row scales)")
    elif args.path == "fc2":
        x, launch, nbytes, tokens, desc = setup_fc2(w, dev)
        desc = f"{w.name} {desc}"
    elif args.path == "dsacp":
        x, launch, nbytes, tokens, desc = setup_dsacp(w, dev)
        desc = f"{w.name} {desc}"
    elif args.path == "gemm":
        x, launch, nbytes, tokens, desc = (setup_gemm_fp8 if fp8_gemm else setup_gemm)(w, dev)
        desc = f"{w.name} {desc}"  # nbytes holds the flops here
    else:
        x, launch, _ = setup(w, dev)
        nbytes, tokens = w.algorithmic_bytes(), w.valid_rows()
    stream = torch.cuda.current_stream(dev)
    print(f"# {w.name}: {w.description}; rank {w.rank}; S={w.shard_rows} H={w.hidden} "
          f"tp={w.tp}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    if args.graph and args.cold:
        ap.error("--graph and --cold are separate protocols")
    if args.graph:
        # N launches captured once (side-stream warm-up first, as capture
        # requires), then ceil(K / N) replays timed by one event pair
        # a prepared launch holds the stream it was made on: remake it on the
        # side and capture streams (the other paths read the current stream)
        remake = getattr(launch, "remake", lambda: launch)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            remake()()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            captured = remake()
            for _ in range(args.graph):
                captured()
        replays = -(-args.steps // args.graph)
        for _ in range(3):
            graph.replay()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(replays):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        n_launch = replays * args.graph
        avg_ms = ev0.elapsed_time(ev1) / n_launch
        ms_per_step = wall * 1000.0 / n_launch
        per_launch_ms = [avg_ms]
    elif not args.cold:
        # timed region: K back-to-back launches, HIP events on the launch stream
        # at both ends, host clock between two synchronisations
        avg_ms, ms_per_step, per_launch_ms = time_plain(launch, stream, args.steps)
    else:
        # cache-cold: before every launch a read+write pass over 512 MiB (twice
        # the Infinity Cache) on the same stream, outside the launch's events
        scrub = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            scrub.add_(1)
            starts[i].record(stream)
            launch()
            ends[i].record(stream)
        torch.cuda.synchronize()
        per_launch_ms = [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]
        avg_ms = ms_per_step = statistics.median(per_launch_ms)
        del scrub
    gemm = args.path == "gemm"
    scale = 1e12 if gemm else 1e9   # TFLOP/s for the GEMM, GB/s for the rest
    peak = (MFMA_FP8_PEAK_TFLOPS if fp8_gemm else MFMA_BF16_PEAK_TFLOPS) if gemm else HBM_PEAK_GBS
    value = nbytes / (ms_per_step / 1000.0) / scale
    achieved = nbytes / (avg_ms / 1000.0) / scale
    traffic = measured_traffic(w.name if args.path == "fused" and not args.quant else
                               f"{w.name}-{args.path}-{args.quant}",
                               {"fused": "fused", "gemm": "gemm"}.get(args.path, "layout"))

    result = {
        "metric": METRIC if args.path == "fused" else
        (f"achieved {'fp8' if fp8_gemm else 'bf16'} TFLOP/s (% of MI355X dense MFMA peak) for the "
         "producer GEMM") if gemm else
        f"achieved HBM GB/s (% of MI355X peak) for {args.path} (one rank's share)",
        "value": round(value, 2),
        "unit": "TFLOP/s" if gemm else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the fused path computes in fp32; the layout paths move elements unchanged
        "dtype": ("f32" if args.path == "fused" else "e4m3" if fp8_gemm else
                  "bf16" if args.path in ("fc2", "dsacp", "gemm")
                  else {torch.uint8: "u8", torch.bfloat16: "bf16"}.get(w.out_dtype, "f32")),
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}" if args.path == "fused" else desc,
            "path": {"fused": "sp_reduce_add_rmsnorm", "gather": "sp_all_gather_unpad",
                     "fc2": "sp_fc2_regroup", "dsacp": "sp_dsacp_heads_to_tokens",
                     "gemm": "sp_scaled_matmul_scatter" if fp8_gemm else "sp_matmul_scatter"}[args.path],
            "tp": w.tp, "rank": w.rank, "num_tokens": w.num_tokens,
            "shard_rows": w.shard_rows, "hidden": w.hidden,
            "quant": QUANT_NAMES[w.quant_mode] + (
                (" e2m1" if w.fp4 else " e4m3") if w.quant_mode == QUANT_MX_BLOCK else ""),
            "deepstack": w.deepstack, "bias": w.bias,
            **({"protocol": "cache-cold: 512 MiB read+write scrub before each launch; value and "
                            "roofline from the median per-launch HIP-event time"} if args.cold else {}),
            **({"protocol": f"HIP graph of {args.graph} launches, replayed back to back"}
               if args.graph else {}),
            ("algorithmic_flops" if gemm else "algorithmic_bytes"): nbytes,
            # the GEMM moves x, w and its output once each
            **({"algorithmic_bytes": (1 if fp8_gemm else 2) * (w.num_tokens_pad * (w.hidden // w.tp)
                                                                + w.hidden * (w.hidden // w.tp))
                                     + 2 * w.num_tokens_pad * w.hidden}
               if gemm else {}),
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "shard_tokens_per_s": round(tokens / (ms_per_step / 1000.0), 1),
        "kernel_us": {
            "mean": round((statistics.mean(per_launch_ms) if args.cold else avg_ms) * 1000, 2),
            "median_single": round(statistics.median(per_launch_ms) * 1000, 2),
            "p10": round(float(np.percentile(per_launch_ms, 10)) * 1000, 2),
            "p90": round(float(np.percentile(per_launch_ms, 90)) * 1000, 2),
        },
        "roofline": {
            "bound": "mfma" if gemm else "hbm",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s" if gemm else "GB/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if also_recs:
        result["also"] = also_recs
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(args.path, w, x, args.cpu_budget, max(1, args.cpu_threads),
                                              nbytes=nbytes, fp8_gemm=fp8_gemm)
    if gemm and fp8_gemm:
        result["context"] = {"hipblaslt_scaled_mm_us": library_fp8_gemm_us(x[0], x[1], x[2], x[3]),
                             "note": "torch._scaled_mm (hipBLASLt) on the same codes and scales, "
                                     "one [M, H] bf16 output, no scatter"}
    elif gemm:
        result["context"] = {"hipblaslt_linear_us": round(library_gemm_us(x[0], x[1]), 2),
                             "note": "torch's linear (hipBLASLt) on the same operands, "
                                     "one [M, H] output, no scatter"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

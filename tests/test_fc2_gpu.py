"""FlashComm2 on one GPU: the o_proj input regrouping against the oracle
(bit-exact), and the whole FC2 tail -- regroup, o_proj partials of each OTP
group, the fused reduce + add + RMSNorm on those partials -- against the
global-TP path on the same tokens (vllm-ascend SP / FlashComm guide,
§4.3-4.6: the OTP group's reduce-scatter leaves rank r with token segment r,
so the fused call sees the same sums as under global TP).  The partial
scale (a dequantisation factor applied to every partial) is checked against
the oracle here too."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import bf16_bits_to_f64, to_host
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_NONE, WORKLOADS,
                                           make_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _srcs(G, N, Cc, dtype, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if dtype == torch.uint8:
        return [torch.randint(0, 256, (N, Cc), generator=g, device=dev, dtype=torch.uint8)
                for _ in range(G)]
    return [torch.randn((N, Cc), generator=g, device=dev).to(dtype) for _ in range(G)]


@pytest.mark.parametrize("G,otp,N,Cc,dtype", [
    (4, 2, 4 * 16, 512, torch.bfloat16),        # the worked example's grouping
    (8, 2, 8 * 37, 1024, torch.bfloat16),       # H=8192 over 8 ranks, 37-token segments
    (16, 4, 3504, 512, torch.bfloat16),         # 3504 padded tokens, H=8192 over 16 ranks
    (8, 4, 8 * 5, 3, torch.float32),            # 12-byte pieces: 4-byte path
    (6, 3, 6 * 7, 20, torch.uint8),             # e4m3 codes, 20-byte pieces
    (4, 1, 4 * 9, 64, torch.bfloat16),          # otp=1: one ODP group, plain all-to-all
    (64, 32, 64 * 2, 8, torch.bfloat16),        # the largest group
    (4, 2, 0, 64, torch.bfloat16),              # empty
])
def test_fc2_regroup_matches_oracle(dev, G, otp, N, Cc, dtype):
    say(f"fc2 regroup G={G} otp={otp} N={N} C={Cc} {dtype}")
    srcs = _srcs(G, N, Cc, dtype, dev, seed=G * 100 + otp)
    odp = G // otp
    bufs = []
    for _ in range(G):
        b = torch.empty((N // odp + 2, odp * Cc), dtype=dtype, device=dev)
        b.view(torch.uint8).fill_(0xA5)
        bufs.append(b)
    dsts = [b[1:N // odp + 1] for b in bufs]
    sp.sp_fc2_regroup(srcs, dsts, otp=otp)
    torch.cuda.synchronize()
    ref = oracle.fc2_regroup([to_host(t) for t in srcs], otp)
    for r in range(G):
        np.testing.assert_array_equal(to_host(dsts[r]).view(np.uint8), ref[r].view(np.uint8))
        ob = bufs[r].view(torch.uint8).cpu().numpy()
        assert (ob[0] == 0xA5).all() and (ob[-1] == 0xA5).all(), f"dst[{r}] canary"


def test_fc2_regroup_rejects_overlap(dev):
    srcs = _srcs(4, 16, 64, torch.bfloat16, dev, 3)
    dsts = [torch.empty((8, 128), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    bad = list(dsts)
    bad[3] = dsts[0]
    with pytest.raises(sp.SprmsError) as e:
        sp.sp_fc2_regroup(srcs, bad, otp=2)
    assert e.value.status == sp.SP_ERR_SHAPE


@pytest.mark.parametrize("quant", [QUANT_NONE, QUANT_DYNAMIC_TOKEN])
@pytest.mark.parametrize("G,otp", [(8, 2), (8, 4), (16, 4)])
def test_fc2_tail_equals_global_tp(dev, G, otp, quant):
    """Integer-valued activations and weights keep every sum exact in fp32,
    so the fused call on the FC2 partials (tp = otp, strided rows of the OTP
    group's o_proj outputs) must give bit-identical outputs to the call on
    the global-TP partials (tp = G) for every rank."""
    odp, seg, Cc, Hout = G // otp, 24, 64, 1024
    N = G * seg
    say(f"fc2 tail G={G} otp={otp} N={N} C={Cc} Hout={Hout} quant={quant}")
    rng = np.random.default_rng(G * 7 + otp)
    X = rng.integers(-2, 3, (N, G * Cc)).astype(np.float64)      # attention output, all features
    W = rng.integers(-2, 3, (G * Cc, Hout)).astype(np.float64)   # o_proj weight
    srcs = [torch.from_numpy(np.ascontiguousarray(X[:, q * Cc:(q + 1) * Cc])).to(
        torch.bfloat16).to(dev) for q in range(G)]
    dsts = [torch.empty((N // odp, odp * Cc), dtype=torch.bfloat16, device=dev) for _ in range(G)]
    sp.sp_fc2_regroup(srcs, dsts, otp=otp)
    torch.cuda.synchronize()
    # o_proj partials (integers, exact in f64 and in f32)
    fc2_part = np.stack([bf16_bits_to_f64(to_host(dsts[r])) for r in range(G)])
    fc2_out = np.empty((G, N // odp, Hout))
    for r in range(G):
        g = r // odp
        fc2_out[r] = fc2_part[r] @ W[g * odp * Cc:(g + 1) * odp * Cc]
    tp_out = np.stack([X[:, q * Cc:(q + 1) * Cc] @ W[q * Cc:(q + 1) * Cc] for q in range(G)])
    assert np.abs(tp_out).max() < 2 ** 24 and np.abs(fc2_out).max() < 2 ** 24
    tp_parts = torch.from_numpy(tp_out.astype(np.float32)).to(dev)          # [G, N, Hout]
    gsz = torch.Generator(device=dev)
    gsz.manual_seed(G + otp)
    resid = torch.randint(-4, 5, (N, Hout), generator=gsz, device=dev).to(torch.bfloat16)
    wt = (torch.randn((Hout,), generator=gsz, device=dev) * 0.1 + 1).to(torch.bfloat16)
    bs = (torch.randn((Hout,), generator=gsz, device=dev) * 0.02).to(torch.bfloat16)
    odt = torch.bfloat16 if quant == QUANT_NONE else torch.uint8
    for r in range(G):
        g, j = divmod(r, odp)
        # OTP group of r: ranks g2*odp + j; stacked, rank r's rows are block g
        grp = torch.from_numpy(np.stack([fc2_out[g2 * odp + j] for g2 in range(otp)]).astype(
            np.float32)).to(dev)                                         # [otp, N/odp, Hout]
        parts_fc2 = grp[:, g * seg:(g + 1) * seg]
        parts_tp = tp_parts[:, r * seg:(r + 1) * seg]
        res_chunk = resid[r * seg:(r + 1) * seg]
        outs = []
        for parts, tp_rank, T, rin in ((parts_fc2, g, otp * seg, res_chunk),
                                       (parts_tp, r, N, resid)):
            out = torch.empty((seg, Hout), dtype=odt, device=dev)
            ro = torch.empty((seg, Hout), dtype=torch.bfloat16, device=dev)
            sc = torch.empty((seg,), device=dev) if quant == QUANT_DYNAMIC_TOKEN else None
            sp.sp_reduce_add_rmsnorm(parts, rin, wt, bs, 1e-6, quant, None, out, sc,
                                     tp_rank=tp_rank, num_tokens=T, residual_out=ro)
            outs.append((out, ro, sc))
        torch.cuda.synchronize()
        (o1, r1, s1), (o2, r2, s2) = outs
        assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), f"rank {r}: out differs"
        assert torch.equal(r1.view(torch.int16), r2.view(torch.int16)), f"rank {r}: residual differs"
        if s1 is not None:
            assert torch.equal(s1, s2), f"rank {r}: scales differ"
        if r == G - 1:
            # and the FC2 call itself against the oracle
            w = dataclasses.replace(WORKLOADS["C2"], tp=otp, num_tokens=otp * seg,
                                    num_tokens_pad=otp * seg, hidden=Hout,
                                    partial_dtype=torch.float32, quant_mode=quant, out_dtype=odt,
                                    residual_replicated=False, deepstack=False, bias=True)
            run_case(w, g, dev=dev, inputs={"partials": parts_fc2, "residual": res_chunk,
                                            "weight": wt, "bias": bs, "deepstack": None},
                     require_exact_frac=0.98)


@pytest.mark.parametrize("c", [0.5, -1.0, 0.0078125, 3.3e-3])
def test_partial_scale_matches_oracle(dev, c):
    # e.g. int8-GEMM partials dequantised by one per-tensor factor
    w = WORKLOADS["C2"]
    say(f"partial_scale={c} on C2 rank 7 (24 padding rows)")
    x = make_inputs(w, rank=7, device=dev)
    x["partials"] = (x["partials"].float() / c).to(w.partial_dtype)
    run_case(w, 7, dev=dev, inputs=x, partial_scale=c)


def test_partial_scale_power_of_two_is_exact_scaling(dev):
    # c = 2^-k scales every product exactly: same outputs as pre-scaled partials
    w = WORKLOADS["C3"]
    x = make_inputs(w, rank=15, device=dev)
    big = (x["partials"].float() * 64).to(torch.bfloat16)
    assert torch.equal((big.float() / 64).to(torch.bfloat16).view(torch.int16),
                       x["partials"].view(torch.int16))
    outs = []
    for parts, c in ((x["partials"], 1.0), (big, 1.0 / 64)):
        out = torch.empty((w.shard_rows, w.hidden), dtype=torch.bfloat16, device=dev)
        ro = torch.empty_like(out)
        sp.sp_reduce_add_rmsnorm(parts, x["residual"], x["weight"], x["bias"], w.eps, QUANT_NONE,
                                 x["deepstack"], out, None, tp_rank=15, num_tokens=w.num_tokens,
                                 residual_out=ro, partial_scale=c)
        outs.append((out, ro))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_prepared_launch_equals_the_direct_call(dev):
    # the marshalled launcher the benchmark times, with every option set
    w = WORKLOADS["C2"]
    x = make_inputs(w, rank=7, device=dev)
    outs = []
    for prepared in (False, True):
        out = torch.full((w.shard_rows, w.hidden), 0x3F, dtype=torch.uint8, device=dev)
        ro = torch.full((w.shard_rows, w.hidden), 2.0, dtype=torch.bfloat16, device=dev)
        sc = torch.full((w.shard_rows,), -1.0, device=dev)
        kw = dict(tp_rank=7, num_tokens=w.num_tokens, residual_out=ro, valid_rows_only=True,
                  partial_scale=0.75)
        args = (x["partials"], x["residual"], x["weight"], None, w.eps, QUANT_DYNAMIC_TOKEN, None, out, sc)
        if prepared:
            launch = sp.prepare(*args, **kw)
            launch()
            launch()   # repeat: same bytes
        else:
            sp.sp_reduce_add_rmsnorm(*args, **kw)
        torch.cuda.synchronize()
        outs.append((out, ro, sc))
    (o1, r1, s1), (o2, r2, s2) = outs
    assert torch.equal(o1, o2) and torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    assert torch.equal(s1, s2)
    v = w.num_tokens - 7 * w.shard_rows
    assert (o2[v:] == 0x3F).all() and (s2[v:] == -1.0).all()   # padding rows untouched

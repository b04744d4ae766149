"""DSA-CP's o_proj input exchange on one GPU, against the oracle (bit-exact),
and the whole path-B tail -- exchange, row-parallel o_proj on each rank's
heads, output scale before the reduce, the fused reduce + add + RMSNorm --
against path A, which multiplies the full weight on the rank's own tokens
and needs no exchange (vllm-ascend PR #18671 walkthrough, §5.3).  Also the
single-rank mode of both regroupings against the all-ranks call."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import bf16_bits_to_f64, to_host
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import QUANT_DYNAMIC_TOKEN, QUANT_NONE, WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _rand(shape, dtype, dev, g):
    if dtype == torch.uint8:
        return torch.randint(0, 256, shape, generator=g, device=dev, dtype=torch.uint8)
    return torch.randn(shape, generator=g, device=dev).to(dtype)


@pytest.mark.parametrize("tp,S,D,dtype", [
    (16, 219, 1024, torch.bfloat16),   # 3504 tokens over 16 ranks, 8 heads x 128 per rank
    (8, 128, 512, torch.bfloat16),
    (4, 33, 6, torch.float32),          # 24-byte pieces: 4-byte path
    (3, 7, 20, torch.uint8),            # e4m3 codes, 20-byte pieces
    (1, 5, 64, torch.bfloat16),         # one rank: a copy
    (64, 2, 8, torch.bfloat16),         # the largest group
    (2, 0, 64, torch.bfloat16),         # empty
])
def test_dsacp_exchange_matches_oracle(dev, tp, S, D, dtype):
    say(f"dsacp exchange tp={tp} S={S} D={D} {dtype}")
    g = torch.Generator(device=dev)
    g.manual_seed(tp * 1000 + S)
    attn = [_rand((S, tp * D), dtype, dev, g) for _ in range(tp)]
    bufs = []
    for _ in range(tp):
        b = torch.empty((tp * S + 2, D), dtype=dtype, device=dev)
        b.view(torch.uint8).fill_(0xA5)
        bufs.append(b)
    outs = [b[1:tp * S + 1] for b in bufs]
    sp.sp_dsacp_heads_to_tokens(attn, outs)
    torch.cuda.synchronize()
    ref = oracle.dsacp_heads_to_tokens([to_host(t) for t in attn])
    for q in range(tp):
        np.testing.assert_array_equal(to_host(outs[q]).view(np.uint8), ref[q].view(np.uint8))
        ob = bufs[q].view(torch.uint8).cpu().numpy()
        assert (ob[0] == 0xA5).all() and (ob[-1] == 0xA5).all(), f"out[{q}] canary"


def test_single_rank_calls_match_the_group_call(dev):
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    tp, S, D = 8, 40, 256
    attn = [_rand((S, tp * D), torch.bfloat16, dev, g) for _ in range(tp)]
    whole = [torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_dsacp_heads_to_tokens(attn, whole)
    G, otp, N, Cc = 8, 2, 8 * 24, 384
    srcs = [_rand((N, Cc), torch.bfloat16, dev, g) for _ in range(G)]
    odp = G // otp
    fc2_whole = [torch.empty((N // odp, odp * Cc), dtype=torch.bfloat16, device=dev)
                 for _ in range(G)]
    sp.sp_fc2_regroup(srcs, fc2_whole, otp=otp)
    for r in range(tp):
        say(f"rank {r} alone")
        mine = [None] * tp
        mine[r] = torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev)
        sp.sp_dsacp_heads_to_tokens(attn, mine, rank=r)
        fmine = [None] * G
        fmine[r] = torch.empty((N // odp, odp * Cc), dtype=torch.bfloat16, device=dev)
        sp.sp_fc2_regroup(srcs, fmine, otp=otp, rank=r)
        torch.cuda.synchronize()
        assert torch.equal(mine[r].view(torch.int16), whole[r].view(torch.int16))
        assert torch.equal(fmine[r].view(torch.int16), fc2_whole[r].view(torch.int16))


@pytest.mark.parametrize("quant", [QUANT_NONE, QUANT_DYNAMIC_TOKEN])
@pytest.mark.parametrize("tp,S,T", [(4, 48, 4 * 48 - 5), (8, 24, 8 * 24), (16, 12, 16 * 12 - 13)])
def test_path_b_tail_equals_path_a(dev, tp, S, T, quant):
    """Integer activations and weights with output scale 1/2 keep every sum
    exact in fp32: the fused call on path B's reduce-scatter partials (tp
    partials, strided, partial_scale = 1/2) must equal the call on path A's
    full-weight product (one partial, same scale) bit for bit, on every rank,
    padding rows included."""
    D, Hout, c = 64, 1024, 0.5
    say(f"dsacp tail tp={tp} S={S} T={T} quant={quant}")
    rng = np.random.default_rng(tp * 31 + S)
    attn_h = [rng.integers(-2, 3, (S, tp * D)).astype(np.float64) for _ in range(tp)]
    W = rng.integers(-2, 3, (tp * D, Hout)).astype(np.float64)
    attn = [torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in attn_h]
    recv = [torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_dsacp_heads_to_tokens(attn, recv)
    torch.cuda.synchronize()
    proj = np.stack([bf16_bits_to_f64(to_host(recv[q])) @ W[q * D:(q + 1) * D]
                     for q in range(tp)])                                  # [tp, tp*S, Hout]
    assert np.abs(proj).max() < 2 ** 24
    proj_t = torch.from_numpy(proj.astype(np.float32)).to(dev)
    gz = torch.Generator(device=dev)
    gz.manual_seed(tp + S)
    resid = torch.randint(-4, 5, (tp * S, Hout), generator=gz, device=dev).to(torch.bfloat16)
    wt = (torch.randn((Hout,), generator=gz, device=dev) * 0.1 + 1).to(torch.bfloat16)
    odt = torch.bfloat16 if quant == QUANT_NONE else torch.uint8
    for p in range(tp):
        v = max(0, min(S, T - p * S))
        full = torch.from_numpy((attn_h[p] @ W).astype(np.float32)).to(dev)[None]   # [1, S, Hout]
        res_chunk = resid[p * S:(p + 1) * S]
        outs = []
        for parts, tp_, rank, T_, rin in ((proj_t[:, p * S:(p + 1) * S], tp, p, T, resid),
                                          (full, 1, 0, v, res_chunk)):
            out = torch.empty((S, Hout), dtype=odt, device=dev)
            ro = torch.empty((S, Hout), dtype=torch.bfloat16, device=dev)
            sc = torch.empty((S,), device=dev) if quant == QUANT_DYNAMIC_TOKEN else None
            sp.sp_reduce_add_rmsnorm(parts, rin, wt, None, 1e-6, quant, None, out, sc,
                                     tp_rank=rank, num_tokens=T_, residual_out=ro,
                                     partial_scale=c)
            outs.append((out, ro, sc))
        torch.cuda.synchronize()
        (o1, r1, s1), (o2, r2, s2) = outs
        assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), f"rank {p}: out differs"
        assert torch.equal(r1.view(torch.int16), r2.view(torch.int16)), f"rank {p}: residual differs"
        if s1 is not None:
            assert torch.equal(s1, s2), f"rank {p}: scales differ"
        assert not o1[v:].view(torch.uint8).any() and not r1[v:].view(torch.int16).any()


def test_path_b_with_fp16_guard_scale_matches_oracle(dev):
    # 1 / routed_scaling_factor (2.5 here) is not a power of two: the sums
    # round, so the fused call on path B's partials is held to the oracle
    tp, S, T, D, Hout = 8, 32, 8 * 32 - 9, 128, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    attn = [(torch.randn((S, tp * D), generator=g, device=dev) * 0.5).to(torch.bfloat16)
            for _ in range(tp)]
    W = (torch.randn((tp * D, Hout), generator=g, device=dev) / 16).to(torch.float32)
    recv = [torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_dsacp_heads_to_tokens(attn, recv)
    proj = torch.stack([recv[q].double().cpu() @ W[q * D:(q + 1) * D].double().cpu()
                        for q in range(tp)]).float().to(dev)                  # [tp, tp*S, Hout]
    resid = torch.randn((tp * S, Hout), generator=g, device=dev).to(torch.bfloat16)
    wt = (torch.randn((Hout,), generator=g, device=dev) * 0.1 + 1).to(torch.bfloat16)
    w = dataclasses.replace(WORKLOADS["C2"], tp=tp, num_tokens=T, num_tokens_pad=tp * S,
                            hidden=Hout, partial_dtype=torch.float32, quant_mode=QUANT_NONE,
                            out_dtype=torch.bfloat16, residual_replicated=True, deepstack=False,
                            bias=False)
    for p in (0, tp - 1):
        say(f"path B, output scale 0.4, rank {p}")
        run_case(w, p, dev=dev, inputs={"partials": proj[:, p * S:(p + 1) * S], "residual": resid,
                                        "weight": wt, "bias": None, "deepstack": None},
                 partial_scale=0.4)

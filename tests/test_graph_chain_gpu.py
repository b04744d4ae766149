"""The one-GPU layer tail captured as one HIP graph: every rank's producer
GEMM into the receive buffers, every rank's fused reduce + add + RMSNorm +
dynamic FP8 call, then the AllGather + unpad of the codes and scales.  The
calls allocate nothing and record no memset, so the captured graph must
replay to the eager results bit for bit, with eager work and
synchronisations between replays."""

import numpy as np
import pytest
import torch

import reduce_add_rmsnorm_amd as sp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def _bits(t):
    return t.view(torch.uint8).clone()


@pytest.mark.parametrize("fp8_producer", [False, True])
def test_layer_tail_graph_replays_match_eager(dev, fp8_producer):
    tp, S, Kr, H = 4, 48, 128, 512
    T = tp * S - 5                      # the last rank holds 5 padding rows
    print(f"graph chain: tp={tp} S={S} K/rank={Kr} H={H} T={T} fp8 producer={fp8_producer}", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    if fp8_producer:
        codes = torch.tensor([0x00, 0x30, 0x38, 0x3C, 0x40, 0xB0, 0xB8, 0xBC, 0xC0], dtype=torch.uint8,
                             device=dev)
        xs = [codes[torch.randint(0, 9, (tp * S, Kr), generator=g, device=dev)] for _ in range(tp)]
        ws = [codes[torch.randint(0, 9, (H, Kr), generator=g, device=dev)] for _ in range(tp)]
        x_scale = torch.rand((tp * S,), generator=g, device=dev) * 0.5 + 0.25
        w_scale = torch.rand((H,), generator=g, device=dev) * 0.5 + 0.25
    else:
        xs = [torch.randn((tp * S, Kr), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
        ws = [(torch.randn((H, Kr), generator=g, device=dev) * 0.1).to(torch.bfloat16) for _ in range(tp)]
    recv = [torch.empty((tp, S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    resid = [torch.randn((S, H), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
    weight = (1.0 + 0.1 * torch.randn((H,), generator=g, device=dev)).to(torch.bfloat16)
    res_out = [torch.empty((S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    out = [torch.empty((S, H), dtype=torch.uint8, device=dev) for _ in range(tp)]
    scale = [torch.empty((S,), dtype=torch.float32, device=dev) for _ in range(tp)]
    gathered = torch.empty((T, H), dtype=torch.uint8, device=dev)
    gathered_scale = torch.empty((T,), dtype=torch.float32, device=dev)
    outputs = recv + res_out + out + scale + [gathered, gathered_scale]

    def tail():
        for q in range(tp):
            if fp8_producer:
                sp.sp_scaled_matmul_scatter(xs[q], x_scale, ws[q], w_scale, recv, rank=q)
            else:
                sp.sp_matmul_scatter(xs[q], ws[q], recv, rank=q)
        for r in range(tp):
            sp.sp_reduce_add_rmsnorm(recv[r], resid[r], weight, None, 1e-6, sp.SP_QUANT_DYNAMIC_TOKEN, None,
                                     out[r], scale[r], tp_rank=r, num_tokens=T, residual_out=res_out[r])
        sp.sp_all_gather_unpad(out, scale, gathered, gathered_scale, num_tokens=T)

    tail()
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outputs]
    # the gather is a pure layout step: rows in shard order, padding rows dropped
    want = torch.cat(out)[:T]
    assert torch.equal(gathered, want) and torch.equal(gathered_scale, torch.cat(scale)[:T])
    assert bool((out[-1][S - 5:] == 0).all()) and bool((scale[-1][S - 5:] == 0).all())
    assert bool(torch.isfinite(torch.cat(scale)).all()) and float(torch.cat(scale)[:T].min()) > 0.0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tail()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tail()
    for it in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, t) in enumerate(zip(ref, outputs)):
            assert torch.equal(a, _bits(t)), f"replay {it}: output {k} differs from the eager chain"
    # inputs changed between replays are read at replay time
    resid[0].mul_(2.0)
    graph.replay()
    torch.cuda.synchronize()
    replay_res = _bits(res_out[0])
    tail()
    torch.cuda.synchronize()
    assert torch.equal(replay_res, _bits(res_out[0]))
    assert not torch.equal(replay_res, ref[tp])
    print(f"graph chain ok: {tp} producer + {tp} fused + 1 gather launches per replay", flush=True)


def test_regroupings_graph_replays_match_eager(dev):
    # FlashComm2's o_proj input regrouping (G = 4, otp = 2) and DSA-CP's
    # head-to-token exchange (tp = 4), every rank, captured together
    G, otp, N, C = 4, 2, 64, 96
    tp, S, D = 4, 24, 40
    print(f"graph regroupings: fc2 G={G} otp={otp} N={N} C={C}; dsacp tp={tp} S={S} D={D}", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    odp = G // otp
    srcs = [torch.randn((N, C), generator=g, device=dev).to(torch.bfloat16) for _ in range(G)]
    dsts = [torch.empty((N // odp, odp * C), dtype=torch.bfloat16, device=dev) for _ in range(G)]
    attn = [torch.randn((S, tp * D), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
    outs = [torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    outputs = dsts + outs

    def regroup():
        sp.sp_fc2_regroup(srcs, dsts, otp=otp)
        sp.sp_dsacp_heads_to_tokens(attn, outs)

    regroup()
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outputs]
    # DSA-CP: rank q's output row p*S + s is head block q of rank p's token s
    for q in range(tp):
        want = torch.cat([attn[p][:, q * D:(q + 1) * D] for p in range(tp)])
        assert torch.equal(outs[q], want)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        regroup()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        regroup()
    for it in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, t) in enumerate(zip(ref, outputs)):
            assert torch.equal(a, _bits(t)), f"replay {it}: output {k} differs from the eager calls"
    # inputs changed between replays are read at replay time
    srcs[1].neg_()
    attn[2].neg_()
    graph.replay()
    torch.cuda.synchronize()
    replayed = [_bits(t) for t in outputs]
    regroup()
    torch.cuda.synchronize()
    assert all(torch.equal(a, _bits(t)) for a, t in zip(replayed, outputs))
    assert any(not torch.equal(a, b) for a, b in zip(replayed, ref))
    print("graph regroupings ok", flush=True)


def test_calls_follow_the_given_stream(dev):
    """A call given a side stream through `stream` runs there, after the work
    enqueued on that stream just before it (here the product it reads)."""
    tp, S, H = 2, 64, 256
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    part = torch.randn((tp, S, H), generator=g, device=dev).to(torch.bfloat16)
    resid = torch.randn((S, H), generator=g, device=dev).to(torch.bfloat16)
    weight = torch.ones((H,), dtype=torch.bfloat16, device=dev)
    out_a = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    out_b = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
    res_a = torch.empty_like(resid)
    res_b = torch.empty_like(resid)
    sp.sp_reduce_add_rmsnorm(part, resid, weight, None, 1e-6, sp.SP_QUANT_NONE, None, out_a, None,
                             tp_rank=0, num_tokens=tp * S, residual_out=res_a)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # the side stream scales the partials, then the call (given `side`
        # explicitly) must see the scaled values
        part2 = part * 2
    sp.sp_reduce_add_rmsnorm(part2, resid, weight, None, 1e-6, sp.SP_QUANT_NONE, None, out_b, None,
                             tp_rank=0, num_tokens=tp * S, residual_out=res_b, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    z = part.float().sum(0)
    z2 = part2.float().sum(0)
    assert not torch.equal(res_a, res_b)
    ref_b = (z2 + resid.float()).to(torch.bfloat16)
    assert torch.equal(res_b, ref_b)
    assert torch.equal(res_a, (z + resid.float()).to(torch.bfloat16))
    np.testing.assert_array_equal(out_b.isfinite().cpu().numpy(), True)


def test_concurrent_streams_match_sequential_calls(dev):
    """Every rank's fused call enqueued on its own stream at once gives the same
    bytes as the calls made one after another: the library holds no scratch
    or other state that concurrent calls could share."""
    tp, S, H = 4, 256, 2048
    T = tp * S - 9
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    parts = [torch.randn((tp, S, H), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
    resid = [torch.randn((S, H), generator=g, device=dev).to(torch.bfloat16) for _ in range(tp)]
    deep = torch.randn((tp * S, H), generator=g, device=dev).to(torch.bfloat16)
    weight = (1.0 + 0.1 * torch.randn((H,), generator=g, device=dev)).to(torch.bfloat16)

    def outputs():
        return ([torch.empty((S, H), dtype=torch.uint8, device=dev) for _ in range(tp)],
                [torch.empty((S,), dtype=torch.float32, device=dev) for _ in range(tp)],
                [torch.empty((S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)])

    def call(r, out, sc, ro, stream=None):
        sp.sp_reduce_add_rmsnorm(parts[r], resid[r], weight, None, 1e-6, sp.SP_QUANT_DYNAMIC_TOKEN, deep,
                                 out[r], sc[r], tp_rank=r, num_tokens=T, residual_out=ro[r], stream=stream)

    seq = outputs()
    for r in range(tp):
        call(r, *seq)
    torch.cuda.synchronize()
    con = outputs()
    streams = [torch.cuda.Stream() for _ in range(tp)]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for r in range(tp):
            call(r, *con, stream=streams[r])
    for s_ in streams:
        torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    for a, b in zip(seq, con):
        for r in range(tp):
            assert torch.equal(_bits(a[r]), _bits(b[r])), f"rank {r} differs"

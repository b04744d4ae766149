"""AllGather + unpad on the GPU, the valid-rows-only and strided-partials
modes of the fused call, and the whole sequence-parallel tail on one GPU:
every rank's fused kernel followed by the gather must equal the oracle's
AllReduce path on every token (vllm-ascend SP / FlashComm guide §2.2: RS + AG
equals AR, and a per-token norm on shards equals the norm after gathering)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import bf16_bits_to_f64, bf16_round, to_host, within_rounding, y_error, z_error
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import QUANT_DYNAMIC_TOKEN, QUANT_NONE, WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _rand_shards(tp, S, H, dtype, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if dtype == torch.uint8:
        return [torch.randint(0, 256, (S, H), generator=g, device=dev, dtype=torch.uint8)
                for _ in range(tp)]
    return [torch.randn((S, H), generator=g, device=dev).to(dtype) for _ in range(tp)]


@pytest.mark.parametrize("tp,S,H,T,dtype,scales", [
    (16, 219, 8192, 3500, torch.bfloat16, False),   # the worked example's shape
    (8, 128, 4096, 1000, torch.bfloat16, False),
    (4, 64, 5120, 4 * 64, torch.uint8, True),        # e4m3 payload + per-token scales
    (4, 33, 520, 4 * 33 - 17, torch.uint8, True),    # rows of 520 bytes: 8-byte path
    (3, 10, 64, 21, torch.float32, False),
    (5, 7, 8, 0, torch.bfloat16, False),             # empty
])
def test_gather_unpad_matches_oracle(dev, tp, S, H, T, dtype, scales):
    say(f"gather tp={tp} S={S} H={H} T={T} {dtype} scales={scales}")
    shards = _rand_shards(tp, S, H, dtype, dev, seed=tp * 1000 + H)
    sc = [torch.rand(S, device=dev) for _ in range(tp)] if scales else None
    out_buf = torch.full((T + 2, H), 0, dtype=dtype, device=dev)
    out_buf.view(torch.uint8).fill_(0xA5)
    out = out_buf[1:T + 1]
    osc_buf = torch.full((T + 2,), float("nan"), device=dev) if scales else None
    osc = osc_buf[1:T + 1] if scales else None
    sp.sp_all_gather_unpad(shards, sc, out, osc, num_tokens=T)
    torch.cuda.synchronize()
    ref, ref_sc = oracle.all_gather_unpad([to_host(t) for t in shards],
                                          None if sc is None else [t.cpu().numpy() for t in sc],
                                          num_tokens=T)
    ob = out_buf.view(torch.uint8).cpu().numpy().reshape(T + 2, -1)
    assert (ob[0] == 0xA5).all() and (ob[-1] == 0xA5).all()
    np.testing.assert_array_equal(to_host(out).view(np.uint8), ref.view(np.uint8))
    if scales:
        np.testing.assert_array_equal(osc.cpu().numpy(), ref_sc)
        b = osc_buf.cpu().numpy()
        assert np.isnan(b[0]) and np.isnan(b[-1])


def test_gather_rejects_bad_calls(dev):
    shards = _rand_shards(2, 4, 16, torch.bfloat16, dev, 1)
    out = torch.empty((9, 16), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sp.SprmsError) as e:   # T > tp*S
        sp.sp_all_gather_unpad(shards, None, out, None, num_tokens=9)
    assert e.value.status == sp.SP_ERR_SHAPE
    with pytest.raises(sp.SprmsError) as e:   # out on top of a shard
        sp.sp_all_gather_unpad(shards, None, shards[1], None, num_tokens=4)
    assert e.value.status == sp.SP_ERR_SHAPE
    with pytest.raises(sp.SprmsError) as e:   # scales given without out_scale
        sp.sp_all_gather_unpad(shards, [torch.ones(4, device=dev)] * 2, out[:8], None, num_tokens=8)
    assert e.value.status == sp.SP_ERR_NULL


def test_valid_rows_only_leaves_padding_rows_untouched(dev):
    w = dataclasses.replace(WORKLOADS["C5"], num_tokens=4 * 48 - 11, num_tokens_pad=4 * 48)
    say("valid_rows_only: rank 3 with 11 padding rows, dynamic e4m3")
    x = make_inputs(w, rank=3, device=dev, shard_rows=48, num_tokens=w.num_tokens)
    out = torch.full((48, w.hidden), 0x5A, dtype=torch.uint8, device=dev)
    res = torch.full((48, w.hidden), 3.0, dtype=torch.bfloat16, device=dev)
    sc = torch.full((48,), -1.0, device=dev)
    sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], None, w.eps,
                             QUANT_DYNAMIC_TOKEN, x["deepstack"], out, sc, tp_rank=3,
                             num_tokens=w.num_tokens, residual_out=res, valid_rows_only=True)
    torch.cuda.synchronize()
    v = 48 - 11
    assert (out[v:] == 0x5A).all() and (res[v:].float() == 3.0).all() and (sc[v:] == -1.0).all()
    # the valid rows equal those of the ordinary call
    out2 = torch.empty_like(out)
    res2 = torch.empty_like(res)
    sc2 = torch.empty_like(sc)
    sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], None, w.eps,
                             QUANT_DYNAMIC_TOKEN, x["deepstack"], out2, sc2, tp_rank=3,
                             num_tokens=w.num_tokens, residual_out=res2)
    torch.cuda.synchronize()
    assert torch.equal(out[:v], out2[:v]) and torch.equal(sc[:v], sc2[:v])
    assert torch.equal(res[:v].view(torch.int16), res2[:v].view(torch.int16))


def test_strided_partials_match_packed(dev):
    # rank r's rows of tp full [T_pad, H] partials held in one [tp, T_pad, H] buffer
    w = WORKLOADS["C2"]
    tp, S, H = w.tp, w.shard_rows, w.hidden
    say("strided partials: rows [r*S, (r+1)*S) of a [8, 1024, 4096] buffer, every rank")
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    full = (torch.randn((tp, tp * S, H), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    for r in range(tp):
        x = make_inputs(w, rank=r, device=dev)
        x["partials"] = full[:, r * S:(r + 1) * S]          # a strided view
        run_case(w, r, dev=dev, inputs=x)


def test_sequence_parallel_tail_equals_all_reduce_path(dev):
    """C3's shape end to end: 16 ranks, each rank's fused kernel reading its
    row block of the 16 full partials (strided) and chunk of the replicated
    residual, writing its valid rows straight into the gathered, unpadded
    [3500, 8192] outputs; the result must match the oracle's AllReduce path
    (all 16 partials summed over all 3500 tokens, then add + RMSNorm) on
    every token.  The same outputs gathered from per-rank buffers with
    sp_all_gather_unpad must be bit-identical."""
    w = dataclasses.replace(WORKLOADS["C3"], residual_replicated=True)
    tp, T, Tp, H = w.tp, w.num_tokens, w.num_tokens_pad, w.hidden
    S = Tp // tp
    say(f"SP tail: tp={tp} T={T} T_pad={Tp} H={H}")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    full = (torch.randn((tp, Tp, H), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    full[:, T:] = float("nan")                                  # graph padding rows
    resid = torch.randn((Tp, H), generator=g, device=dev).to(torch.bfloat16)
    resid[T:] = float("nan")
    wt = (torch.randn((H,), generator=g, device=dev) * 0.1 + 1).to(torch.bfloat16)
    bs = (torch.randn((H,), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    shard_out = [torch.empty((S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    shard_res = [torch.empty((S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    for r in range(tp):
        v = max(0, min(S, T - r * S))
        parts = full[:, r * S:(r + 1) * S]
        sp.sp_reduce_add_rmsnorm(parts, resid, wt, bs, w.eps, QUANT_NONE, None, out[r * S:r * S + v],
                                 None, tp_rank=r, num_tokens=T, residual_out=res_out[r * S:r * S + v],
                                 valid_rows_only=True)
        sp.sp_reduce_add_rmsnorm(parts, resid, wt, bs, w.eps, QUANT_NONE, None, shard_out[r], None,
                                 tp_rank=r, num_tokens=T, residual_out=shard_res[r])
    gathered = torch.empty_like(out)
    gathered_res = torch.empty_like(res_out)
    sp.sp_all_gather_unpad(shard_out, None, gathered, None, num_tokens=T)
    sp.sp_all_gather_unpad(shard_res, None, gathered_res, None, num_tokens=T)
    torch.cuda.synchronize()
    assert torch.equal(gathered.view(torch.int16), out.view(torch.int16))
    assert torch.equal(gathered_res.view(torch.int16), res_out.view(torch.int16))

    # oracle AllReduce path: one "shard" holding every token, the 16 full partials
    hP, hR = to_host(full), to_host(resid)
    ref = oracle.reduce_add_rmsnorm(hP, hR, to_host(wt), to_host(bs), w.eps, oracle.QUANT_NONE,
                                    None, tp_rank=0, num_tokens=T, out_dtype=oracle.ORC_BF16,
                                    rows=np.arange(T))
    z, y = ref["z"], ref["y"]
    A = np.abs(bf16_bits_to_f64(hR[:T]))
    for q in range(tp):
        A += np.abs(bf16_bits_to_f64(hP[q, :T]))
    err_z = z_error(A, tp)
    rstd = 1.0 / np.sqrt((z * z).mean(1) + np.float64(np.float32(w.eps)))
    err_y = y_error(y, bf16_bits_to_f64(to_host(bs)), err_z, rstd, bf16_bits_to_f64(to_host(wt)))
    got_r = bf16_bits_to_f64(to_host(res_out))
    got_o = bf16_bits_to_f64(to_host(out))
    assert within_rounding(got_r, z - err_z, z + err_z, bf16_round).all()
    assert within_rounding(got_o, y - err_y, y + err_y, bf16_round).all()
    assert (to_host(out) == ref["out"]).mean() >= 0.99
    assert np.isfinite(got_o).all()


@pytest.mark.parametrize("tp,S,H,T", [
    (4, 40, 160, 4 * 40 - 7),      # 5 E8M0 bytes per row: byte-wise scale copy
    (4, 40, 5120, 4 * 40 - 7),     # 160 bytes per row: word-wise scale copy
    (3, 9, 96, 25),                # 3 bytes per row
])
def test_gather_block_scales_match_oracle(dev, tp, S, H, T):
    say(f"gather with E8M0 block scales tp={tp} S={S} H={H} T={T}")
    g = torch.Generator(device=dev)
    g.manual_seed(H + T)
    shards = [torch.randint(0, 256, (S, H), generator=g, device=dev, dtype=torch.uint8)
              for _ in range(tp)]
    sc = [torch.randint(0, 256, (S, H // 32), generator=g, device=dev, dtype=torch.uint8)
          for _ in range(tp)]
    out = torch.empty((T, H), dtype=torch.uint8, device=dev)
    osc_buf = torch.full((T * (H // 32) + 2,), 0xA5, dtype=torch.uint8, device=dev)
    osc = osc_buf[1:T * (H // 32) + 1].view(T, H // 32)   # 1-byte offset: byte-wise copy
    osc_al = torch.full((T, H // 32), 0xA5, dtype=torch.uint8, device=dev)
    sp.sp_all_gather_unpad(shards, sc, out, osc, num_tokens=T)
    sp.sp_all_gather_unpad(shards, sc, out, osc_al, num_tokens=T)
    torch.cuda.synchronize()
    ref, ref_sc = oracle.all_gather_unpad([t.cpu().numpy() for t in shards],
                                          [t.cpu().numpy() for t in sc], num_tokens=T)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    np.testing.assert_array_equal(osc.cpu().numpy(), ref_sc)
    np.testing.assert_array_equal(osc_al.cpu().numpy(), ref_sc)
    b = osc_buf.cpu().numpy()
    assert b[0] == 0xA5 and b[-1] == 0xA5

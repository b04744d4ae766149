"""Block-scaled (OCP microscaling form) outputs of the fused call on the GPU:
MXFP8 (e4m3 elements) and MXFP4 (e2m1 elements, two per byte) with one E8M0
scale per 32 elements, against the CPU oracle; exact conversion sweeps of the
element encoders through the product path; gathering the block scales."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import to_host
from parity import run_case, unpack_e2m1
from reduce_add_rmsnorm_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
MX = sp.SP_QUANT_MX_BLOCK


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def mx(name, **kw):
    return dataclasses.replace(WORKLOADS[name], quant_mode=MX, out_dtype=torch.uint8, **kw)


def sample_rows(S, n=40, seed=0):
    rng = np.random.default_rng(seed)
    return sorted(set(rng.choice(S, size=min(n, S), replace=False).tolist()) | {0, S - 1})


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("name,rank", [("C5", 3), ("C4", 7)])
def test_mx_full_size_sampled_rows(dev, name, rank, fp4):
    w = mx(name)
    say(f"{name} rank {rank} block-scaled {'e2m1' if fp4 else 'e4m3'}: full size, sampled rows")
    r = run_case(w, rank, dev=dev, rows=sample_rows(w.shard_rows, seed=rank), pad_fill=None, fp4=fp4)
    say(r.stats)


@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("tp,H,bias,act", [(16, 8192, True, torch.bfloat16), (3, 1024, False, torch.float32),
                                           (1, 32, True, torch.bfloat16), (8, 16384, False, torch.bfloat16)])
def test_mx_small_shapes_every_row(dev, fp4, tp, H, bias, act):
    w = mx("C3", tp=tp, hidden=H, bias=bias, act_dtype=act, partial_dtype=torch.bfloat16,
           num_tokens=tp * 12 - 5, num_tokens_pad=tp * 12)
    say(f"block-scaled {'e2m1' if fp4 else 'e4m3'} tp={tp} H={H} bias={bias} act={act} S=12 rank {tp - 1}")
    run_case(w, tp - 1, dev=dev, fp4=fp4)


def test_mx_rejects_bad_hidden(dev):
    w = WORKLOADS["C2"]
    x = make_inputs(w, rank=0, device=dev, shard_rows=4)
    x["partials"] = x["partials"][:, :, :4088].contiguous()
    out = torch.empty((4, 4088), dtype=torch.uint8, device=dev)
    sc = torch.empty((4, 128), dtype=torch.uint8, device=dev)
    with pytest.raises(sp.SprmsError) as e:
        sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"][:, :4088].contiguous(),
                                 x["weight"][:4088].contiguous(), None, w.eps, MX, None, out, sc,
                                 tp_rank=0, num_tokens=32)
    assert e.value.status == sp.SP_ERR_SHAPE


def _exact_call(dev, values, fp4):
    """One row whose y equals `values` exactly (tp=1, +-1 partials, zero
    residual, eps 0: rstd = 1 and y = (+-1 * w) * 1)."""
    H = values.shape[0]
    rng = np.random.default_rng(H + int(fp4))
    sign = np.where(rng.random(H) < 0.5, -1.0, 1.0).astype(np.float32)
    P = torch.from_numpy(sign.reshape(1, 1, H)).to(dev)
    R = torch.zeros((1, H), dtype=torch.float32, device=dev)
    wt = torch.from_numpy(np.ascontiguousarray(values.astype(np.float32) * sign)).to(dev)
    out = torch.empty((1, H // 2 if fp4 else H), dtype=torch.uint8, device=dev)
    sc = torch.empty((1, H // 32), dtype=torch.uint8, device=dev)
    sp.sp_reduce_add_rmsnorm(P, R, wt, None, 0.0, MX, None, out, sc, tp_rank=0, num_tokens=1,
                             residual_out=torch.empty_like(R),
                             out_dtype=sp.SP_FP4_E2M1 if fp4 else None)
    torch.cuda.synchronize()
    return out.cpu().numpy()[0], sc.cpu().numpy()[0]


@pytest.mark.parametrize("fp4", [False, True])
def test_block_element_conversion_sweep_exact(dev, fp4):
    # Every block starts with +-(max element value), so its exponent is 0 and
    # the other 31 elements are converted as they are: all element values,
    # all midpoints (ties), their fp32 neighbours and a dense random sweep,
    # bit-identical to the oracle's brute-force encoders.
    say(f"block element conversion sweep ({'e2m1' if fp4 else 'e4m3'})")
    top = 6.0 if fp4 else 448.0
    if fp4:
        grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    else:
        from helpers import e4m3_decode
        grid = e4m3_decode(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    base = np.concatenate([grid, -grid, mids, -mids]).astype(np.float32)
    near = np.concatenate([np.nextafter(base, np.float32(1e9)), np.nextafter(base, np.float32(-1e9))])
    # values below 2^(emax+1) keep the block exponent at 0; those between the
    # largest element value and that bound exercise saturation
    lim = 8.0 if fp4 else 512.0
    rng = np.random.default_rng(3)
    rand = rng.uniform(-lim, lim, 60000).astype(np.float32)
    vals = np.concatenate([base, near, rand]).astype(np.float32)
    vals = vals[np.abs(vals) < lim]
    per = 31
    nblk = -(-len(vals) // per)
    blocks = np.zeros((nblk, 32), np.float32)
    flat = np.zeros(nblk * per, np.float32)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(nblk, per)
    blocks[:, 0] = np.where(np.arange(nblk) % 2 == 0, top, -top)
    rows = blocks.reshape(-1)
    pad = (-rows.size) % 32768
    rows = np.concatenate([rows, np.tile(np.r_[top, np.zeros(31)], pad // 32).astype(np.float32)])
    enc = oracle.e2m1_from_double_array if fp4 else oracle.e4m3_from_double_array
    for chunk in rows.reshape(-1, 32768):
        codes, scales = _exact_call(dev, chunk, fp4)
        assert (scales == 127).all()
        got = unpack_e2m1(codes) if fp4 else codes
        want = enc(chunk.astype(np.float64))
        zero_mask = 7 if fp4 else 0x7F
        both_zero = ((got & zero_mask) == 0) & ((want & zero_mask) == 0)
        np.testing.assert_array_equal(np.where(both_zero, 0, got), np.where(both_zero, 0, want))


def test_gather_block_scaled_outputs(dev):
    w = mx("C5", num_tokens=4 * 40 - 13, num_tokens_pad=4 * 40)
    S, H, tp, T = 40, w.hidden, w.tp, w.num_tokens
    say("gather block-scaled e2m1 outputs + E8M0 scales of 4 ranks, 13 padding rows")
    outs, scs = [], []
    for r in range(tp):
        x = make_inputs(w, rank=r, device=dev, shard_rows=S, num_tokens=T)
        o = torch.empty((S, H // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((S, H // 32), dtype=torch.uint8, device=dev)
        sp.sp_reduce_add_rmsnorm(x["partials"], x["residual"], x["weight"], None, w.eps, MX,
                                 x["deepstack"], o, sc, tp_rank=r, num_tokens=T,
                                 residual_out=torch.empty_like(x["residual"]),
                                 out_dtype=sp.SP_FP4_E2M1)
        outs.append(o)
        scs.append(sc)
    g = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
    gs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    sp.sp_all_gather_unpad(outs, scs, g, gs, num_tokens=T, dtype=sp.SP_FP4_E2M1)
    torch.cuda.synchronize()
    ref, ref_s = oracle.all_gather_unpad([to_host(o) for o in outs], [to_host(c) for c in scs],
                                         num_tokens=T)
    np.testing.assert_array_equal(to_host(g), ref)
    np.testing.assert_array_equal(to_host(gs), ref_s)

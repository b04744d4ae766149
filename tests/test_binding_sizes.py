"""The Python binding's size checks, on the CPU.  The C ABI receives only
pointers, so a tensor too small for the descriptor the binding builds would
let a kernel read or write past its allocation; the binding must refuse it
before anything reaches the library.  Host tensors are used: a call whose
sizes are right gets past these checks and stops at the device check, which
is how the tests tell the two apart."""

import pytest
import torch

import reduce_add_rmsnorm_amd as sp

tp, S, H = 4, 8, 64
BF, F32, U8 = torch.bfloat16, torch.float32, torch.uint8


def fused_args(**over):
    a = dict(partials=torch.zeros((tp, S, H), dtype=BF), residual=torch.zeros((S, H), dtype=BF),
             weight=torch.zeros((H,), dtype=BF), bias=None, eps=1e-6,
             quant_mode=sp.SP_QUANT_DYNAMIC_TOKEN, deepstack=None,
             out=torch.zeros((S, H), dtype=U8), out_scale=torch.zeros((S,), dtype=F32))
    kw = dict(tp_rank=1, num_tokens=tp * S, residual_out=torch.zeros((S, H), dtype=BF))
    for k, v in over.items():
        (a if k in a else kw)[k] = v
    return a, kw


def call(fn, **over):
    a, kw = fused_args(**over)
    return fn(*a.values(), **kw)


@pytest.mark.parametrize("fn", [sp.sp_reduce_add_rmsnorm, sp.prepare])
def test_right_sizes_reach_the_device_check(fn):
    with pytest.raises(ValueError, match="device tensors only"):
        call(fn)
    with pytest.raises(ValueError, match="device tensors only"):   # replicated residual, deepstack, bias
        call(fn, residual=torch.zeros((tp * S, H), dtype=BF), deepstack=torch.zeros((S, H), dtype=BF),
             bias=torch.zeros((H,), dtype=BF))
    with pytest.raises(ValueError, match="device tensors only"):   # block-scaled e2m1
        call(fn, quant_mode=sp.SP_QUANT_MX_BLOCK, out=torch.zeros((S, H // 2), dtype=U8),
             out_dtype=sp.SP_FP4_E2M1, out_scale=torch.zeros((S, H // 32), dtype=U8))


@pytest.mark.parametrize("fn", [sp.sp_reduce_add_rmsnorm, sp.prepare])
@pytest.mark.parametrize("over,msg", [
    (dict(out=torch.zeros((S - 1, H), dtype=U8)), "out has 7 rows"),
    (dict(out=torch.zeros((S, H // 2), dtype=U8)), "out rows must be 64 bytes"),
    (dict(quant_mode=sp.SP_QUANT_NONE, out=torch.zeros((S, H // 2), dtype=BF)), "out rows must be 128 bytes"),
    (dict(out_scale=torch.zeros((S - 1,), dtype=F32)), "out_scale must be float32 with at least 8"),
    (dict(out_scale=torch.zeros((S,), dtype=BF)), "out_scale must be float32"),
    (dict(quant_mode=sp.SP_QUANT_STATIC_TENSOR, out_scale=torch.zeros((0,), dtype=F32)), "at least 1"),
    (dict(quant_mode=sp.SP_QUANT_MX_BLOCK, out_dtype=sp.SP_FP8_E4M3,
          out_scale=torch.zeros((S, 1), dtype=U8)), "E8M0 bytes"),
    (dict(weight=torch.zeros((H - 8,), dtype=BF)), "weight must hold H=64"),
    (dict(weight=torch.zeros((H,), dtype=F32)), "weight must have the residual's dtype"),
    (dict(bias=torch.zeros((H + 8,), dtype=BF)), "bias must hold H=64"),
    (dict(residual=torch.zeros((S, H - 8), dtype=BF)), r"residual must be \[rows, H=64\]"),
    (dict(residual=torch.zeros((2 * S, H), dtype=BF)), "residual must have 8 or 32 rows"),
    (dict(deepstack=torch.zeros((S + 1, H), dtype=BF)), "deepstack must have 8 or 32 rows"),
    (dict(deepstack=torch.zeros((S, H), dtype=F32)), "deepstack must have the residual's dtype"),
    (dict(residual_out=torch.zeros((S - 2, H), dtype=BF)), "residual_out has 6 rows"),
    (dict(residual_out=torch.zeros((S, H // 2), dtype=BF)), r"residual_out must be \[rows, H=64\]"),
])
def test_wrong_sizes_are_refused(fn, over, msg):
    with pytest.raises(ValueError, match=msg):
        call(fn, **over)


def test_valid_rows_only_needs_only_the_valid_rows():
    # rank 3 of tp=4 with T = 3*S + 5: five valid rows, so a 5-row block of
    # the gathered tensor is enough, four rows are not
    T = 3 * S + 5
    with pytest.raises(ValueError, match="device tensors only"):
        call(sp.sp_reduce_add_rmsnorm, tp_rank=3, num_tokens=T, valid_rows_only=True,
             out=torch.zeros((5, H), dtype=U8), out_scale=torch.zeros((5,), dtype=F32),
             residual_out=torch.zeros((5, H), dtype=BF))
    with pytest.raises(ValueError, match="out has 4 rows, the call writes 5"):
        call(sp.sp_reduce_add_rmsnorm, tp_rank=3, num_tokens=T, valid_rows_only=True,
             out=torch.zeros((4, H), dtype=U8), out_scale=torch.zeros((5,), dtype=F32),
             residual_out=torch.zeros((5, H), dtype=BF))
    with pytest.raises(ValueError, match="out has 5 rows, the call writes 8"):   # without the flag
        call(sp.sp_reduce_add_rmsnorm, tp_rank=3, num_tokens=T,
             out=torch.zeros((5, H), dtype=U8), residual_out=torch.zeros((S, H), dtype=BF))


def test_gather_sizes():
    shards = [torch.zeros((S, H), dtype=U8) for _ in range(tp)]
    scales = [torch.zeros((S,), dtype=F32) for _ in range(tp)]
    T = tp * S - 3
    ok = dict(num_tokens=T)
    with pytest.raises(ValueError, match="device tensors only"):
        sp.sp_all_gather_unpad(shards, scales, torch.zeros((T, H), dtype=U8), torch.zeros((T,), dtype=F32), **ok)
    with pytest.raises(ValueError, match=f"out has {T - 1} rows"):
        sp.sp_all_gather_unpad(shards, scales, torch.zeros((T - 1, H), dtype=U8), torch.zeros((T,), dtype=F32), **ok)
    with pytest.raises(ValueError, match="as wide as the shards"):
        sp.sp_all_gather_unpad(shards, scales, torch.zeros((T, H), dtype=BF), torch.zeros((T,), dtype=F32), **ok)
    with pytest.raises(ValueError, match="out_scale must hold"):
        sp.sp_all_gather_unpad(shards, scales, torch.zeros((T, H), dtype=U8), torch.zeros((T - 1,), dtype=F32), **ok)
    with pytest.raises(ValueError, match="one size"):
        bad = scales[:-1] + [torch.zeros((S - 1,), dtype=F32)]
        sp.sp_all_gather_unpad(shards, bad, torch.zeros((T, H), dtype=U8), torch.zeros((T,), dtype=F32), **ok)
    with pytest.raises(ValueError, match="one scale tensor per shard"):
        sp.sp_all_gather_unpad(shards, scales[:2], torch.zeros((T, H), dtype=U8), torch.zeros((T,), dtype=F32), **ok)


def test_regrouping_destination_sizes():
    srcs = [torch.zeros((16, 32), dtype=BF) for _ in range(4)]
    with pytest.raises(ValueError, match="device tensors only"):
        sp.sp_fc2_regroup(srcs, [torch.zeros((8, 64), dtype=BF) for _ in range(4)], otp=2)
    with pytest.raises(ValueError, match=r"dsts\[2\] must hold 512 elements"):
        sp.sp_fc2_regroup(srcs, [torch.zeros((8, 64), dtype=BF)] * 2 + [torch.zeros((8, 32), dtype=BF)] * 2,
                          otp=2)
    with pytest.raises(ValueError, match=r"dsts\[0\] must hold 512 elements of torch.bfloat16"):
        sp.sp_fc2_regroup(srcs, [torch.zeros((8, 64), dtype=F32)] + [None] * 3, otp=2, rank=0)
    attn = [torch.zeros((8, 4 * 16), dtype=BF) for _ in range(4)]
    with pytest.raises(ValueError, match="device tensors only"):
        sp.sp_dsacp_heads_to_tokens(attn, [torch.zeros((32, 16), dtype=BF) for _ in range(4)])
    with pytest.raises(ValueError, match=r"outs\[1\] must be \[32, 16\]"):
        sp.sp_dsacp_heads_to_tokens(attn, [None, torch.zeros((16, 32), dtype=BF), None, None], rank=1)

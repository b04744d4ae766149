"""Seeded random configurations of the fused call against the oracle: every
combination the descriptor allows (tp, S, H, partial and activation dtypes,
output mode, bias, deepstack shard- or full-sized, replicated or shard
residual, in place or not, partial scale, rank, valid tokens), small enough
that each case runs in well under a second, compared on every row with the
same bars as the other parity tests (tests/parity.py)."""

import dataclasses

import numpy as np
import pytest
import torch

import reduce_add_rmsnorm_amd as sp
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import (QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK, QUANT_NONE,
                                           QUANT_STATIC_TENSOR, WORKLOADS)

N_CASES = 64


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def draw(i):
    rng = np.random.default_rng(1000 + i)
    tp = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    S = int(rng.integers(1, 41))
    quant = int(rng.choice([QUANT_NONE, QUANT_STATIC_TENSOR, QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK]))
    H = 32 * int(rng.integers(1, 65)) if quant == QUANT_MX_BLOCK else 8 * int(rng.integers(1, 257))
    pdt = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    adt = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    if quant == QUANT_NONE:
        odt = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    else:
        odt = torch.uint8
    T = int(rng.integers(0, tp * S + 1)) if rng.random() < 0.5 else tp * S
    case = dict(
        tp=tp, S=S, H=H, quant=quant, pdt=pdt, adt=adt, odt=odt, T=T,
        rank=int(rng.integers(0, tp)),
        bias=bool(rng.random() < 0.4), deepstack=bool(rng.random() < 0.4),
        replicated=bool(rng.random() < 0.4), shard_deepstack=bool(rng.random() < 0.5),
        in_place=bool(rng.random() < 0.3), fp4=quant == QUANT_MX_BLOCK and bool(rng.random() < 0.5),
        partial_scale=float(rng.choice([1.0, 1.0, 0.5, 0.75, -1.0])),
        sigma=float(rng.choice([0.05, 0.5, 2.0])),
        static_scale=float(rng.uniform(0.005, 0.05)),
        seed=int(rng.integers(0, 2 ** 31)),
    )
    return case


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(dev, i):
    c = draw(i)
    print(f"case {i}: " + ", ".join(f"{k}={v}" for k, v in c.items()), flush=True)
    w = dataclasses.replace(
        WORKLOADS["C2"], tp=c["tp"], num_tokens=c["T"], num_tokens_pad=c["tp"] * c["S"],
        hidden=c["H"], partial_dtype=c["pdt"], act_dtype=c["adt"], quant_mode=c["quant"],
        out_dtype=c["odt"], residual_replicated=c["replicated"], deepstack=c["deepstack"],
        bias=c["bias"], rank=c["rank"], partial_sigma=c["sigma"], fp4=c["fp4"])
    res = run_case(w, c["rank"], dev=dev, S=c["S"], T=c["T"], in_place=c["in_place"],
                   static_scale=c["static_scale"] if c["quant"] == QUANT_STATIC_TENSOR else None,
                   shard_deepstack=c["shard_deepstack"], base_seed=c["seed"], fp4=c["fp4"],
                   partial_scale=c["partial_scale"])
    print(f"  ok: {res.stats}", flush=True)


def test_the_draws_cover_every_option():
    """CPU: the seeded draws reach every option of the descriptor."""
    cases = [draw(i) for i in range(N_CASES)]
    assert {c["quant"] for c in cases} == {QUANT_NONE, QUANT_STATIC_TENSOR, QUANT_DYNAMIC_TOKEN, QUANT_MX_BLOCK}
    assert any(c["fp4"] for c in cases) and any(c["quant"] == QUANT_MX_BLOCK and not c["fp4"] for c in cases)
    for k in ("bias", "deepstack", "replicated", "in_place", "shard_deepstack"):
        assert any(c[k] for c in cases) and not all(c[k] for c in cases), k
    assert {c["pdt"] for c in cases} == {torch.float32, torch.bfloat16}
    assert {c["adt"] for c in cases} == {torch.float32, torch.bfloat16}
    assert any(c["T"] < c["tp"] * c["S"] for c in cases) and any(c["T"] == 0 for c in cases)
    assert any(max(0, min(c["S"], c["T"] - c["rank"] * c["S"])) == 0 for c in cases)   # a rank with no valid row
    assert any(c["partial_scale"] != 1.0 for c in cases) and any(c["tp"] == 1 for c in cases)

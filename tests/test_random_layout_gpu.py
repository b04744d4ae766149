"""Seeded random configurations of the other entry points against the
oracle: the gather + unpad (every row width and scale layout), the FC2
regrouping and the DSA-CP exchange (group sizes, piece widths, dtypes, one
rank or all) bit for bit with canaries around every destination, and both
producer GEMMs (shapes, ranks, output dtypes, scale layouts) within the
bounds of tests/test_matmul_gpu.py."""

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import to_host
from test_matmul_gpu import (_check, _check_fp8, _e4m3_codes, _operands, _receive_buffers,
                             _slots_untouched)

N_CASES = 32
CANARY = 0xA5


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


def _framed(rows, cols, dtype, dev):
    """A [rows, cols] view with one canary row on each side."""
    b = torch.empty((rows + 2, cols), dtype=dtype, device=dev)
    b.view(torch.uint8).fill_(CANARY)
    return b, b[1:rows + 1]


def _frame_intact(b):
    ob = b.view(torch.uint8).cpu().numpy().reshape(b.shape[0], -1)
    return bool((ob[0] == CANARY).all() and (ob[-1] == CANARY).all())


DTYPES = [torch.bfloat16, torch.float32, torch.uint8]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_gather(dev, i):
    rng = np.random.default_rng(2000 + i)
    tp, S = int(rng.integers(1, 17)), int(rng.integers(0, 41))
    kind = str(rng.choice(["bf16", "f32", "e4m3", "e2m1"]))
    H = 16 * int(rng.integers(1, 129)) if kind == "e2m1" else 8 * int(rng.integers(1, 257))
    scales = str(rng.choice(["none", "token", "block"])) if H % 32 == 0 else str(rng.choice(["none", "token"]))
    T = int(rng.integers(0, tp * S + 1))
    say(f"gather case {i}: tp={tp} S={S} H={H} {kind} scales={scales} T={T}")
    g = torch.Generator(device=dev)
    g.manual_seed(i)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}.get(kind, torch.uint8)
    W = H // 2 if kind == "e2m1" else H
    shards = [_rand((S, W), dt, dev, g) for _ in range(tp)]
    sc = None
    if scales == "token":
        sc = [torch.rand((S,), generator=g, device=dev) for _ in range(tp)]
    elif scales == "block":
        sc = [_rand((S, H // 32), torch.uint8, dev, g) for _ in range(tp)]
    ob, out = _framed(T, W, dt, dev)
    osb, osc = (None, None)
    if sc is not None:
        osb, osc = _framed(T, 1 if scales == "token" else H // 32,
                           torch.float32 if scales == "token" else torch.uint8, dev)
        osc = osc.reshape(-1) if scales == "token" else osc
    sp.sp_all_gather_unpad(shards, sc, out, osc, num_tokens=T,
                           dtype=sp.SP_FP4_E2M1 if kind == "e2m1" else None)
    torch.cuda.synchronize()
    ref, ref_sc = oracle.all_gather_unpad([to_host(t) for t in shards],
                                          None if sc is None else [to_host(t) for t in sc], num_tokens=T)
    np.testing.assert_array_equal(to_host(out).view(np.uint8), ref.view(np.uint8))
    assert _frame_intact(ob), "out canary"
    if sc is not None:
        np.testing.assert_array_equal(to_host(osc).view(np.uint8).reshape(-1),
                                      ref_sc.view(np.uint8).reshape(-1))
        assert _frame_intact(osb), "out_scale canary"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fc2_regroup(dev, i):
    rng = np.random.default_rng(3000 + i)
    G = int(rng.choice([2, 3, 4, 6, 8, 12, 16]))
    otp = int(rng.choice([d for d in range(1, G) if G % d == 0]))
    odp = G // otp
    dt = DTYPES[int(rng.integers(0, 3))]
    e = torch.tensor([], dtype=dt).element_size()
    Cc = int(rng.integers(1, 97)) * (4 // e if e < 4 else 1)
    N = G * int(rng.integers(0, 9))
    rank = int(rng.integers(-1, G))
    say(f"fc2 case {i}: G={G} otp={otp} N={N} C={Cc} {dt} rank={rank}")
    g = torch.Generator(device=dev)
    g.manual_seed(i)
    srcs = [_rand((N, Cc), dt, dev, g) for _ in range(G)]
    framed = [_framed(N // odp, odp * Cc, dt, dev) if rank in (-1, r) else (None, None) for r in range(G)]
    sp.sp_fc2_regroup(srcs, [d for _, d in framed], otp=otp, rank=rank)
    torch.cuda.synchronize()
    ref = oracle.fc2_regroup([to_host(t) for t in srcs], otp)
    for r, (b, d) in enumerate(framed):
        if d is None:
            continue
        np.testing.assert_array_equal(to_host(d).view(np.uint8), ref[r].view(np.uint8))
        assert _frame_intact(b), f"dst[{r}] canary"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_dsacp_exchange(dev, i):
    rng = np.random.default_rng(4000 + i)
    tp, S = int(rng.integers(1, 17)), int(rng.integers(0, 21))
    dt = DTYPES[int(rng.integers(0, 3))]
    e = torch.tensor([], dtype=dt).element_size()
    D = int(rng.integers(1, 65)) * (4 // e if e < 4 else 1)
    rank = int(rng.integers(-1, tp))
    say(f"dsacp case {i}: tp={tp} S={S} D={D} {dt} rank={rank}")
    g = torch.Generator(device=dev)
    g.manual_seed(i)
    attn = [_rand((S, tp * D), dt, dev, g) for _ in range(tp)]
    framed = [_framed(tp * S, D, dt, dev) if rank in (-1, q) else (None, None) for q in range(tp)]
    sp.sp_dsacp_heads_to_tokens(attn, [d for _, d in framed], rank=rank)
    torch.cuda.synchronize()
    ref = oracle.dsacp_heads_to_tokens([to_host(t) for t in attn])
    for q, (b, d) in enumerate(framed):
        if d is None:
            continue
        np.testing.assert_array_equal(to_host(d).view(np.uint8), ref[q].view(np.uint8))
        assert _frame_intact(b), f"out[{q}] canary"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_random_matmul_scatter(dev, i):
    rng = np.random.default_rng(5000 + i)
    tp, S = int(rng.integers(1, 9)), int(rng.integers(1, 81))
    K, N = 8 * int(rng.integers(1, 66)), 8 * int(rng.integers(1, 76))
    dt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    rank = int(rng.integers(0, tp))
    say(f"matmul case {i}: tp={tp} S={S} K={K} N={N} {dt} rank={rank}")
    x, w = _operands(tp * S, K, N, dev, seed=i)
    dsts = _receive_buffers(tp, S, N, dt, dev)
    sp.sp_matmul_scatter(x, w, dsts, rank=rank)
    torch.cuda.synchronize()
    _check(x, w, dsts, rank)
    _slots_untouched(dsts, rank)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_random_scaled_matmul_scatter(dev, i):
    rng = np.random.default_rng(6000 + i)
    tp, S = int(rng.integers(1, 9)), int(rng.integers(1, 81))
    K, N = 16 * int(rng.integers(1, 34)), 8 * int(rng.integers(1, 76))
    dt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    per_token, per_col = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    rank = int(rng.integers(0, tp))
    say(f"scaled matmul case {i}: tp={tp} S={S} K={K} N={N} {dt} token={per_token} col={per_col} rank={rank}")
    g = torch.Generator(device=dev)
    g.manual_seed(i)
    M = tp * S
    x8, w8 = _e4m3_codes((M, K), dev, g), _e4m3_codes((N, K), dev, g)
    xs = torch.rand((M if per_token else 1,), generator=g, device=dev) * 0.02 + 0.001
    ws = torch.rand((N if per_col else 1,), generator=g, device=dev) * 0.02 + 0.001
    dsts = _receive_buffers(tp, S, N, dt, dev)
    sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, dsts, rank=rank)
    torch.cuda.synchronize()
    _check_fp8(x8, xs, w8, ws, dsts, rank)
    _slots_untouched(dsts, rank)

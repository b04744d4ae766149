"""The producer GEMM (sp_matmul_scatter) against the oracle, and the chain
producer -> fused shard kernel against the oracle's chain (vLLM SP /
AsyncTP / quantisation notes, §2: GEMM + ReduceScatter at a block's exit).

Tolerance: the GPU sums K bf16 products in fp32 on the matrix cores; the
oracle sums them exactly (fp64) and rounds once.  With A = sum_k |x_k w_k|,
the fp32 sum differs from the exact one by at most (K + 2) 2^-24 A; the
oracle's f32 value adds 2^-24 of itself.  A bf16 output must lie between the
bf16 roundings of the interval's ends (rounding is monotone)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import bf16_bits_to_f64, bf16_round, e4m3_decode, to_host, within_rounding
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import QUANT_DYNAMIC_TOKEN, QUANT_NONE, WORKLOADS

pytestmark = pytest.mark.gpu

CANARY = 0xA5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _operands(M, K, N, dev, seed, integers=False):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if integers:
        x = torch.randint(-3, 4, (M, K), generator=g, device=dev).to(torch.bfloat16)
        w = torch.randint(-3, 4, (N, K), generator=g, device=dev).to(torch.bfloat16)
    else:
        x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        w = (torch.randn((N, K), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    return x, w


def _receive_buffers(tp, S, N, dtype, dev):
    bufs = []
    for _ in range(tp):
        b = torch.empty((tp, S, N), dtype=dtype, device=dev)
        b.view(torch.uint8).fill_(CANARY)
        bufs.append(b)
    return bufs


def _check(x, w, dsts, rank, rows=None):
    """Rows m (default all) of rank's partial, read back from slot `rank` of
    their destinations, against the oracle."""
    tp = len(dsts)
    M, K = x.shape
    N = w.shape[0]
    S = M // tp
    f32 = dsts[0].dtype == torch.float32
    rows = np.arange(M) if rows is None else np.asarray(sorted(set(int(m) for m in rows)))
    hx, hw = to_host(x), to_host(w)
    ref32 = oracle.matmul_scatter(hx, hw, tp=tp, rank=rank, out_dtype=oracle.ORC_F32, rows=rows)
    ref16 = None if f32 else oracle.matmul_scatter(hx, hw, tp=tp, rank=rank,
                                                   out_dtype=oracle.ORC_BF16, rows=rows)
    ax = np.abs(bf16_bits_to_f64(hx[rows]))
    aw = np.abs(bf16_bits_to_f64(hw))
    A = ax @ aw.T                                   # sum_k |x_k w_k|, for the bound only
    exact_eq = []
    for i, m in enumerate(rows):
        r, s = divmod(int(m), S)
        want = ref32[r][rank][s].astype(np.float64)
        E = (K + 2) * 2.0 ** -24 * A[i] + 2.0 ** -24 * np.abs(want)
        got_t = dsts[r][rank, s]
        if f32:
            got = got_t.cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= E).all(), f"row {m}: f32 partial outside the bound"
        else:
            bits = to_host(got_t)
            got = bf16_bits_to_f64(bits)
            ok = within_rounding(got, want - E, want + E, bf16_round)
            assert ok.all(), f"row {m}: bf16 partial outside the bound at {np.argwhere(~ok)[:4].tolist()}"
            exact_eq.append((bits == ref16[r][rank][s]).mean())
    if exact_eq:
        assert np.mean(exact_eq) >= 0.99, f"only {np.mean(exact_eq):.4f} of bf16 partials equal the oracle's"


def _slots_untouched(dsts, rank):
    for r, d in enumerate(dsts):
        b = d.view(torch.uint8)
        for q in range(d.shape[0]):
            if q != rank:
                assert bool((b[q] == CANARY).all()), f"dst[{r}] slot {q} was written"


@pytest.mark.parametrize("tp,S,K,N,dtype", [
    (2, 300, 136, 520, torch.float32),   # 3 x 3 tiles, ragged M, N and a K tail of 8
    (2, 300, 136, 520, torch.bfloat16),
    (4, 64, 64, 256, torch.bfloat16),    # exactly one tile
    (2, 70, 128, 264, torch.bfloat16),   # exactly two K stages
    (1, 40, 72, 136, torch.float32),     # two K stages, the second a tail of 8
    (2, 130, 192, 256, torch.bfloat16),  # exactly three K stages
    (1, 5, 8, 8, torch.float32),         # smallest
    (8, 33, 896, 1024, torch.bfloat16),  # K of one rank at hidden 7168 over 8 ranks
    (3, 100, 1288, 264, torch.float32),  # long K with a tail, N just past a tile
])
def test_matmul_scatter_matches_oracle(dev, tp, S, K, N, dtype):
    M = tp * S
    say(f"matmul_scatter tp={tp} S={S} K={K} N={N} {dtype}")
    x, w = _operands(M, K, N, dev, seed=M + K + N)
    for rank in sorted({0, tp - 1}):
        dsts = _receive_buffers(tp, S, N, dtype, dev)
        sp.sp_matmul_scatter(x, w, dsts, rank=rank)
        torch.cuda.synchronize()
        _check(x, w, dsts, rank)
        _slots_untouched(dsts, rank)


def test_matmul_scatter_integer_inputs_are_exact(dev):
    tp, S, K, N = 4, 130, 320, 384
    x, w = _operands(tp * S, K, N, dev, seed=3, integers=True)
    for dtype, od in ((torch.float32, oracle.ORC_F32), (torch.bfloat16, oracle.ORC_BF16)):
        dsts = _receive_buffers(tp, S, N, dtype, dev)
        sp.sp_matmul_scatter(x, w, dsts, rank=2)
        torch.cuda.synchronize()
        ref = oracle.matmul_scatter(to_host(x), to_host(w), tp=tp, rank=2, out_dtype=od)
        for r in range(tp):
            np.testing.assert_array_equal(to_host(dsts[r][2]).view(np.uint8), ref[r][2].view(np.uint8))


@pytest.mark.parametrize("name", ["C4", "C5"])
def test_matmul_scatter_full_size_sampled_rows(dev, name):
    # the benchmark's shape and launch: M = T_pad tokens, K = H / tp, N = H,
    # bf16 partials, the timed rank
    w_ = WORKLOADS[name]
    tp, S, H = w_.tp, w_.shard_rows, w_.hidden
    M, K = tp * S, H // tp
    say(f"matmul_scatter {name}: M={M} K={K} N={H} rank {w_.rank}, sampled rows")
    x, w = _operands(M, K, H, dev, seed=11)
    dsts = [torch.empty((tp, S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_matmul_scatter(x, w, dsts, rank=w_.rank)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = [0, 1, 255, 256, 257, S - 1, S, M - 256, M - 1] + list(rng.integers(0, M, 24))
    _check(x, w, dsts, w_.rank, rows=rows)


@pytest.mark.parametrize("quant", [QUANT_NONE, QUANT_DYNAMIC_TOKEN])
def test_producer_then_fused_kernel(dev, quant):
    """Every rank's GEMM writes its slot; each rank's receive buffer then goes
    through the fused kernel.  Integer operands: the GPU's receive buffers
    equal the oracle's bit for bit, and the fused outputs match the oracle's
    fused call on the oracle's buffers."""
    tp, S, Kr, N = 4, 96, 128, 1024
    T = tp * S - 10
    say(f"producer -> fused: tp={tp} S={S} K/rank={Kr} N={N} T={T} quant={quant}")
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    X = torch.randint(-2, 3, (tp * S, tp * Kr), generator=g, device=dev).to(torch.bfloat16)
    W = torch.randint(-2, 3, (N, tp * Kr), generator=g, device=dev).to(torch.bfloat16)
    resid = torch.randint(-4, 5, (tp * S, N), generator=g, device=dev).to(torch.bfloat16)
    wt = (torch.randn((N,), generator=g, device=dev) * 0.1 + 1).to(torch.bfloat16)
    dsts = [torch.empty((tp, S, N), dtype=torch.float32, device=dev) for _ in range(tp)]
    ref = None
    for q in range(tp):
        xq = X[:, q * Kr:(q + 1) * Kr].contiguous()
        wq = W[:, q * Kr:(q + 1) * Kr].contiguous()
        sp.sp_matmul_scatter(xq, wq, dsts, rank=q)
        ref = oracle.matmul_scatter(to_host(xq), to_host(wq), tp=tp, rank=q, dst=ref)
    torch.cuda.synchronize()
    odt = torch.bfloat16 if quant == QUANT_NONE else torch.uint8
    w = dataclasses.replace(WORKLOADS["C2"], tp=tp, num_tokens=T, num_tokens_pad=tp * S, hidden=N,
                            partial_dtype=torch.float32, quant_mode=quant, out_dtype=odt,
                            residual_replicated=True, deepstack=False, bias=False)
    for r in range(tp):
        np.testing.assert_array_equal(dsts[r].cpu().numpy(), ref[r])
        say(f"fused call of rank {r} on its receive buffer")
        run_case(w, r, dev=dev, inputs={"partials": torch.from_numpy(ref[r]).to(dev),
                                        "residual": resid, "weight": wt, "bias": None,
                                        "deepstack": None})
        # and the kernel reading the producer's buffer directly gives the same bytes
        outs = []
        for parts in (dsts[r], torch.from_numpy(ref[r]).to(dev)):
            out = torch.empty((S, N), dtype=odt, device=dev)
            ro = torch.empty((S, N), dtype=torch.bfloat16, device=dev)
            sc = torch.empty((S,), device=dev) if quant == QUANT_DYNAMIC_TOKEN else None
            sp.sp_reduce_add_rmsnorm(parts, resid, wt, None, 1e-6, quant, None, out, sc,
                                     tp_rank=r, num_tokens=T, residual_out=ro)
            outs.append((out, ro))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0].view(torch.uint8), outs[1][0].view(torch.uint8))
        assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_matmul_scatter_rejects_bad_calls(dev):
    x, w = _operands(8, 16, 16, dev, seed=1)
    dsts = [torch.empty((2, 4, 16), dtype=torch.float32, device=dev) for _ in range(2)]
    with pytest.raises(sp.SprmsError) as e:
        sp.sp_matmul_scatter(x, w, dsts, rank=2)
    assert e.value.status == sp.SP_ERR_SHAPE
    with pytest.raises(sp.SprmsError) as e:
        sp.sp_matmul_scatter(x, w, [dsts[0], dsts[0]], rank=0)   # slots overlap
    assert e.value.status == sp.SP_ERR_SHAPE
    with pytest.raises(ValueError):
        sp.sp_matmul_scatter(x, w.cpu(), dsts, rank=0)


# ------------------------------------------------------------- FP8 producer


def _e4m3_codes(shape, dev, g):
    c = torch.randint(0, 256, shape, generator=g, device=dev, dtype=torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38       # no NaN codes
    return c


def _check_fp8(x8, xs, w8, ws, dsts, rank, rows=None):
    tp = len(dsts)
    M, K = x8.shape
    N = w8.shape[0]
    S = M // tp
    f32 = dsts[0].dtype == torch.float32
    rows = np.arange(M) if rows is None else np.asarray(sorted(set(int(m) for m in rows)))
    hx, hw = x8.cpu().numpy(), w8.cpu().numpy()
    hxs, hws = xs.cpu().numpy(), ws.cpu().numpy()
    ref32 = oracle.scaled_matmul_scatter(hx, hxs, hw, hws, tp=tp, rank=rank, out_dtype=oracle.ORC_F32,
                                         rows=rows)
    ax = np.abs(e4m3_decode(hx[rows])).astype(np.float32)   # e4m3 products are exact in fp32
    aw = np.abs(e4m3_decode(hw)).astype(np.float32)
    A = ax.astype(np.float64) @ aw.T.astype(np.float64)      # sum_k |x_k w_k|, for the bound only
    sw = np.abs(hws.astype(np.float64)) if hws.size > 1 else np.full(N, abs(float(hws[0])))
    steps = -(-K // 64)
    for i, m in enumerate(rows):
        r, s = divmod(int(m), S)
        sx = abs(float(hxs[m if hxs.size > 1 else 0]))
        want = ref32[r][rank][s].astype(np.float64)
        pmax = (ax[i][None, :] * aw).max(axis=1).astype(np.float64)   # max_k |x_k w_k|
        # the e4m3 MFMA sums each step of 64 products (zero-padded past K)
        # to within a fraction of the largest of them -- measured on the
        # device over 1.3 million random single-step sums at up to 2^-10.76 --
        # and the steps are added in fp32
        E = (steps * 2.0 ** -10 * pmax + (steps + 2) * 2.0 ** -24 * A[i]) * sx * sw + 3 * 2.0 ** -24 * np.abs(want)
        got_t = dsts[r][rank, s]
        if f32:
            got = got_t.cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= E).all(), f"row {m}: f32 partial outside the bound"
        else:
            bits = to_host(got_t)
            ok = within_rounding(bf16_bits_to_f64(bits), want - E, want + E, bf16_round)
            assert ok.all(), f"row {m}: bf16 partial outside the bound at {np.argwhere(~ok)[:4].tolist()}"


@pytest.mark.gpu
def test_fp8_step_error_is_a_fraction_of_the_largest_product(dev):
    """The property the e4m3 bound above rests on, on many more sums than the
    parity cases: one step of 64 e4m3 products with unit scales, against the
    exact sum (decoded values, float64, exact here), over 20 random code
    matrices of 256 x 256 dots.  The largest error measured is 2^-10.76 of
    the step's largest |product|; the bound uses 2^-10."""
    M = N = 256
    K = 64
    worst = 0.0
    one = torch.ones(1, device=dev)
    for trial in range(20):
        g = torch.Generator(device=dev)
        g.manual_seed(64000 + trial)
        x8, w8 = _e4m3_codes((M, K), dev, g), _e4m3_codes((N, K), dev, g)
        dst = [torch.zeros((1, M, N), dtype=torch.float32, device=dev)]
        sp.sp_scaled_matmul_scatter(x8, one, w8, one, dst, rank=0)
        torch.cuda.synchronize()
        got = dst[0][0].cpu().numpy().astype(np.float64)
        dx = e4m3_decode(x8.cpu().numpy()).astype(np.float64)
        dw = e4m3_decode(w8.cpu().numpy()).astype(np.float64)
        pmax = np.abs(dx[:, None, :] * dw[None, :, :]).max(axis=2)
        worst = max(worst, float((np.abs(got - dx @ dw.T) / np.maximum(pmax, 1e-300)).max()))
    say(f"worst single-step error: 2^{np.log2(worst):.2f} of the largest product")
    assert worst <= 2.0 ** -10


@pytest.mark.parametrize("tp,S,K,N,dtype,per_token,per_col", [
    (2, 300, 144, 520, torch.float32, True, True),    # ragged M, N, a K tail of 16
    (2, 300, 144, 520, torch.bfloat16, False, True),
    (4, 64, 128, 256, torch.bfloat16, True, False),   # one tile, one K stage
    (1, 5, 16, 8, torch.float32, False, False),       # smallest
    (8, 33, 896, 1024, torch.bfloat16, True, True),
])
def test_scaled_matmul_scatter_matches_oracle(dev, tp, S, K, N, dtype, per_token, per_col):
    M = tp * S
    say(f"scaled_matmul_scatter tp={tp} S={S} K={K} N={N} {dtype} token={per_token} col={per_col}")
    g = torch.Generator(device=dev)
    g.manual_seed(M + K + N)
    x8, w8 = _e4m3_codes((M, K), dev, g), _e4m3_codes((N, K), dev, g)
    xs = torch.rand((M if per_token else 1,), generator=g, device=dev) * 0.02 + 0.001
    ws = torch.rand((N if per_col else 1,), generator=g, device=dev) * 0.02 + 0.001
    for rank in sorted({0, tp - 1}):
        dsts = _receive_buffers(tp, S, N, dtype, dev)
        sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, dsts, rank=rank)
        torch.cuda.synchronize()
        _check_fp8(x8, xs, w8, ws, dsts, rank)
        _slots_untouched(dsts, rank)


def test_scaled_matmul_scatter_exact_on_integer_codes(dev):
    # codes of small integers and power-of-two scales: every step exact
    tp, S, K, N = 2, 96, 256, 384
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    table = torch.tensor([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0xC8], dtype=torch.uint8,
                         device=dev)                 # 0, 1, 2, 3, 4, -1, -2, -3, -4
    x8 = table[torch.randint(0, 9, (tp * S, K), generator=g, device=dev)]
    w8 = table[torch.randint(0, 9, (N, K), generator=g, device=dev)]
    xs = 2.0 ** -torch.randint(0, 4, (tp * S,), generator=g, device=dev).float()
    ws = 2.0 ** -torch.randint(0, 4, (N,), generator=g, device=dev).float()
    dsts = _receive_buffers(tp, S, N, torch.float32, dev)
    sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, dsts, rank=1)
    torch.cuda.synchronize()
    ref = oracle.scaled_matmul_scatter(x8.cpu().numpy(), xs.cpu().numpy(), w8.cpu().numpy(),
                                       ws.cpu().numpy(), tp=tp, rank=1)
    for r in range(tp):
        np.testing.assert_array_equal(dsts[r][1].cpu().numpy(), ref[r][1])


@pytest.mark.parametrize("name", ["C4", "C5"])
def test_scaled_matmul_scatter_full_size_sampled_rows(dev, name):
    w_ = WORKLOADS[name]
    tp, S, H = w_.tp, w_.shard_rows, w_.hidden
    M, K = tp * S, H // tp
    say(f"scaled_matmul_scatter {name}: M={M} K={K} N={H} rank {w_.rank}, sampled rows")
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    x8, w8 = _e4m3_codes((M, K), dev, g), _e4m3_codes((H, K), dev, g)
    xs = torch.rand((M,), generator=g, device=dev) * 0.01 + 0.001
    ws = torch.rand((1,), generator=g, device=dev) * 0.01 + 0.001
    dsts = [torch.empty((tp, S, H), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, dsts, rank=w_.rank)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = [0, 255, 256, S - 1, S, M - 1] + list(rng.integers(0, M, 16))
    _check_fp8(x8, xs, w8, ws, dsts, w_.rank, rows=rows)


@pytest.mark.parametrize("tp,S,K,N", [(64, 3, 64, 64), (3, 1, 16, 8)])
def test_producers_at_group_and_size_extremes(dev, tp, S, K, N):
    # 64 destinations inside one tile; a 3-token problem
    M = tp * S
    say(f"producers at extremes: tp={tp} S={S} K={K} N={N}")
    g = torch.Generator(device=dev)
    g.manual_seed(tp + S)
    x, w = _operands(M, K, N, dev, seed=tp * 7 + S, integers=True)
    dsts = _receive_buffers(tp, S, N, torch.float32, dev)
    sp.sp_matmul_scatter(x, w, dsts, rank=tp - 1)
    x8, w8 = _e4m3_codes((M, K), dev, g), _e4m3_codes((N, K), dev, g)
    xs = torch.rand((M,), generator=g, device=dev) + 0.5
    ws = torch.rand((N,), generator=g, device=dev) + 0.5
    d8 = _receive_buffers(tp, S, N, torch.bfloat16, dev)
    sp.sp_scaled_matmul_scatter(x8, xs, w8, ws, d8, rank=0)
    torch.cuda.synchronize()
    ref = oracle.matmul_scatter(to_host(x), to_host(w), tp=tp, rank=tp - 1)
    for r in range(tp):
        np.testing.assert_array_equal(dsts[r][tp - 1].cpu().numpy(), ref[r][tp - 1])
    _slots_untouched(dsts, tp - 1)
    _check_fp8(x8, xs, w8, ws, d8, 0)
    _slots_untouched(d8, 0)

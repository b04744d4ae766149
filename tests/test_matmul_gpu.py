"""The producer GEMM (sp_matmul_scatter) against the oracle, and the chain
producer -> fused shard kernel against the oracle's chain (vLLM SP /
AsyncTP / quantisation notes, §2: GEMM + ReduceScatter at a block's exit).

Tolerance: the GPU sums K bf16 products on the matrix cores; the oracle sums
them exactly (fp64) and rounds once.  One v_mfma_f32_16x16x32_bf16 step of 32
products (probed with constructed operands: one product 2^16, the others
equal powers of two at every offset below it, and subsets of the slots) sums
4 groups of 8 consecutive k, each product truncated toward zero to a multiple
of 2^(E_g - 24) of its group's largest exponent sum (loss < 7 * 2^-24 of the
group's largest product), then adds the group sums and the accumulator in
fp32, rounding to nearest (4 roundings).  Per step that is at most
11 * 2^-24 (|acc| + sum |p|), so with A = sum_k |x_k w_k| the result is within
11 * ceil(K/32) * 2^-24 * A of the exact sum, inside the (K + 2) 2^-24 A used
here for every K >= 32; the oracle's f32 value adds 2^-24 of itself.  A bf16
output must lie between the bf16 roundings of the interval's ends (rounding
is monotone).  The e4m3 instruction's rule is stated with its tests below."""

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


def _bf16_bits(v):
    v = np.asarray(v, np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert ((bits.astype(np.uint32) << 16).view(np.float32) == v).all(), "value not exact in bf16"
    return bits


def _bf16_step_gpu(xv, wv, dev):
    """x [M, K], w [N, K] (exact bf16 values) through sp_matmul_scatter with f32
    partials; returns the [M, N] result."""
    xt = torch.from_numpy(_bf16_bits(xv).view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(_bf16_bits(wv).view(np.int16)).to(dev).view(torch.bfloat16)
    dst = [torch.zeros((1, xv.shape[0], wv.shape[0]), dtype=torch.float32, device=dev)]
    sp.sp_matmul_scatter(xt, wt, dst, rank=0)
    torch.cuda.synchronize()
    return dst[0][0].cpu().numpy().astype(np.float64)


def _bf16_group_model(xv, wv):
    """The bf16 instruction's rule written out: per 32-product step, 4 groups
    of 8 consecutive k; products truncated toward zero to multiples of
    2^(E_g - 24) of the group's largest exponent sum; each group sum rounded
    to fp32 and added to the accumulator in group order, rounding to nearest."""
    def bexp(v):
        u = (np.asarray(v, np.float32).view(np.uint32) >> 23) & 0xFF
        return np.where(u == 0, -126, u.astype(np.int64) - 127)
    M, K = xv.shape
    N = wv.shape[0]
    p = xv[:, None, :].astype(np.float64) * wv[None, :, :]
    es = (bexp(xv)[:, None, :] + bexp(wv)[None, :, :]).reshape(M, N, K // 8, 8)
    unit = np.exp2(es.max(axis=3, keepdims=True) - 24)
    g = (np.trunc(p.reshape(M, N, K // 8, 8) / unit) * unit).sum(axis=3)
    acc = np.zeros((M, N), np.float32)
    for i in range(K // 8):
        acc = (acc + g[:, :, i].astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


@pytest.mark.gpu
def test_bf16_step_follows_the_group_model(dev):
    """Constructed 32-product steps: 2^16 at k = 0 and equal powers of two
    (both signs) at every offset from 2^-40 to 2^23 below and above it in all
    other slots, or in chosen subsets of them (one slot, a group, several
    groups, every other slot): bit-exact to the model, which is what puts the
    instruction inside the (K + 2) 2^-24 sum|xw| bound."""
    K = 32
    x = np.zeros((64, K), np.float32)
    r = 0
    for a in (-24, -12, 0):
        for sg in (1, -1):
            x[r, 0] = 256
            x[r, 1:] = sg * 2.0 ** a
            r += 1
    for S in ([1], list(range(1, 8)), list(range(8, 16)), list(range(16, 32)), [1, 2, 3],
              [4, 5, 6, 7], list(range(1, 32, 2)), [1, 8, 16, 24]):
        for a in (-12, 0):
            x[r, 0] = 256
            x[r, S] = 2.0 ** a
            r += 1
    x[r:, 0] = 256
    w = np.zeros((64, K), np.float32)
    w[:, 0] = 256
    w[:, 1:] = (2.0 ** (np.arange(64) - 40.0))[:, None]
    got = _bf16_step_gpu(x, w, dev)
    np.testing.assert_array_equal(got, _bf16_group_model(x, w))
    # the worst case of the rule: 7 same-sign products just under each group's
    # grid 2^-8 (255/128 * 2^-9), all truncated away, against the bound
    xw = np.full((8, K), 255 / 128 * 2.0 ** -9, np.float32)
    xw[:, 0::8] = 256
    ww = np.ones((8, K), np.float32)
    ww[:, 0::8] = 256
    got = _bf16_step_gpu(xw, ww, dev)
    np.testing.assert_array_equal(got, _bf16_group_model(xw, ww))
    exact = xw.astype(np.float64) @ ww.astype(np.float64).T
    A = np.abs(xw.astype(np.float64)) @ np.abs(ww.astype(np.float64)).T
    assert (np.abs(got - exact) > 0).all() and (np.abs(got - exact) <= (K + 2) * 2.0 ** -24 * A).all()


def e4m3_exponent(codes):
    """Unbiased exponent of e4m3 codes as the matrix instruction aligns them:
    the exponent field minus 7, and -6 for subnormals and zero."""
    e = (np.asarray(codes).astype(np.int64) >> 3) & 0xF
    return np.where(e == 0, -6, e - 7)


# How one step of v_mfma_scale_f32_32x32x64_f8f6f4 (64 products) sums, found
# with constructed operands (the tests below keep it pinned): the 64 products
# form 8 groups of 8 consecutive k; inside a group every product is aligned
# to the group's largest exponent sum E_g = max(e_x + e_w) (the codes'
# exponents, not the products' magnitudes) and truncated toward zero to a
# multiple of 2^(E_g - 13); the 8 group sums and the accumulator are then
# combined in fp32, which was seen to add at most 2 ulps of the result.
# Derived bound, per step: a group loses less than 7 * 2^(E_g - 13) (the
# product with the largest exponent sum loses nothing), and the combination
# is allowed 16 * 2^-24 * (|acc| + sum |p|), four times the largest combination
# error seen; over T steps |acc| <= sum_k |p_k| = A.
FP8_GROUP, FP8_GRID_BITS, FP8_COMBINE = 8, 13, 16


def fp8_truncation_bound(xe_row, we):
    """Sum over steps and groups of 7 * 2^(E_g - 13) for one token row
    (exponents xe_row [K]) against every weight row (we [N, K])."""
    N, K = we.shape
    es = (xe_row[None, :] + we).reshape(N, K // FP8_GROUP, FP8_GROUP)
    return ((FP8_GROUP - 1) * np.exp2(es.max(axis=2) - FP8_GRID_BITS)).sum(axis=1)


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
    xe, we = e4m3_exponent(hx[rows]), e4m3_exponent(hw)
    sw = np.abs(hws.astype(np.float64)) if hws.size > 1 else np.full(N, abs(float(hws[0])))
    steps = -(-K // 64)
    for i, m in enumerate(rows):
        r, s = divmod(int(m), S)
        sx = abs(float(hxs[m if hxs.size > 1 else 0]))
        want = ref32[r][rank][s].astype(np.float64)
        acc_bound = (fp8_truncation_bound(xe[i], we)
                     + FP8_COMBINE * steps * 2.0 ** -24 * A[i] * (1 + 2.0 ** -10))
        E = acc_bound * sx * sw + 3 * 2.0 ** -24 * np.abs(want)   # + the two scale products
        got_t = dsts[r][rank, s]
        if f32:
            got = got_t.cpu().numpy().astype(np.float64)
            assert (np.abs(got - want) <= E).all(), f"row {m}: f32 partial outside the bound"
        else:
            bits = to_host(got_t)
            ok = within_rounding(bf16_bits_to_f64(bits), want - E, want + E, bf16_round)
            assert ok.all(), f"row {m}: bf16 partial outside the bound at {np.argwhere(~ok)[:4].tolist()}"


def _encode_e4m3(v):
    """Codes of values that e4m3 represents exactly (checked by decoding)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = (a >= 2.0 ** -6)
    mant = np.where(normal, a / np.exp2(e) - 1, a / 2.0 ** -9)
    field = np.where(normal, ((e + 7) << 3) | np.round(mant * 8).astype(np.int64),
                     np.round(mant).astype(np.int64))
    codes = (np.where(a > 0, field, 0) | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    assert (e4m3_decode(codes) == v).all(), "value not exact in e4m3"
    return codes


def _one_step(xv, wv, dev):
    """x [M, K] and w [N, K] (exact e4m3 values) through sp_scaled_matmul_scatter
    with unit scales and f32 partials; returns the [M, N] result."""
    xc, wc = _encode_e4m3(xv), _encode_e4m3(wv)
    one = torch.ones(1, device=dev)
    dst = [torch.zeros((1, xv.shape[0], wv.shape[0]), dtype=torch.float32, device=dev)]
    sp.sp_scaled_matmul_scatter(torch.from_numpy(xc).to(dev), one, torch.from_numpy(wc).to(dev), one,
                                dst, rank=0)
    torch.cuda.synchronize()
    return dst[0][0].cpu().numpy().astype(np.float64), xc, wc


def _group_model(xv, wv, xc, wc):
    """The group truncation rule written out: per step of 64 and group of 8
    consecutive k, products truncated toward zero to multiples of
    2^(E_g - 13); the group sums added exactly; one rounding to fp32."""
    xe, we = e4m3_exponent(xc), e4m3_exponent(wc)
    M, K = xv.shape
    N = wv.shape[0]
    p = xv[:, None, :] * wv[None, :, :]                     # [M, N, K], exact
    es = (xe[:, None, :] + we[None, :, :]).reshape(M, N, K // 8, 8)
    unit = np.exp2(es.max(axis=3, keepdims=True) - 13)
    t = np.trunc(p.reshape(M, N, K // 8, 8) / unit) * unit
    return t.sum(axis=(2, 3)).astype(np.float32).astype(np.float64)


@pytest.mark.gpu
def test_fp8_step_truncation_follows_the_group_model(dev):
    """Constructed single-step sums: one product of exponent sum 12 at k = 0
    and 63 equal products 2^(12-d) (1 + m/8) with d = -2 .. 27 (across the
    grid), every mantissa, both signs, a negative largest product, alternating
    signs.  The model predicts every result to within the fp32 combination
    (2 ulps) and most of them exactly; its truncation is what decides them."""
    K = 64
    x = np.zeros((64, K))
    r = 0
    for a in (-6, 0, 6):
        for m in range(8):
            for sg in (1, -1):
                x[r, 0] = 64
                x[r, 1:] = sg * (1 + m / 8) * 2.0 ** a
                r += 1
    for m in range(8):
        x[r, 0] = -64
        x[r, 1:] = 1 + m / 8
        r += 1
    for m in range(8):
        x[r, 0] = 64
        x[r, 1:] = (1 + m / 8) * np.where(np.arange(1, K) % 2, 1, -1)
        r += 1
    w = np.zeros((32, K))
    for n in range(18):
        w[n, 0] = 64
        w[n, 1:] = 2.0 ** (n - 9)
    for j, cnt in enumerate([1, 2, 3, 4, 7, 8, 15, 16, 31, 32, 48, 62, 63, 63]):
        w[18 + j, 0] = 64
        w[18 + j, 1:1 + cnt] = 2.0 ** (-4 if j < 13 else 2)
    got, xc, wc = _one_step(x, w, dev)
    pred = _group_model(x, w, xc, wc)
    exact = x @ w.T
    ulp = np.spacing(np.abs(got).astype(np.float32)).astype(np.float64)
    assert (np.abs(got - pred) <= 2 * ulp).all()
    frac = float((got == pred).mean())
    truncated = np.abs(exact - pred) > 2 * ulp   # where the truncation moves the result
    say(f"group model exact on {frac:.1%} of {got.size} sums; truncation decides {truncated.sum()}")
    assert frac >= 0.95 and truncated.sum() > 500


@pytest.mark.gpu
def test_fp8_worst_case_step_meets_the_derived_bound(dev):
    """The worst case of the rule: every group holds one product 2^12 and 7
    products of the same sign just under the group's grid 2^-1
    (0.46875 = 1.875 * 2^-2), all of which are truncated away: each step loses
    56 * 0.46875 = 26.25, 2^-7.3 of the largest product, where random codes
    never lose more than about 2^-10.8 of it.  Results are bit-exact to the
    model and inside the derived bound, over one and two steps."""
    for K, sign in ((64, 1), (64, -1), (128, 1)):
        x = np.full((32, K), sign * 0.46875)
        x[:, 0::8] = 64
        w = np.ones((32, K))
        w[:, 0::8] = 64
        got, xc, wc = _one_step(x, w, dev)
        exact = x @ w.T
        steps = K // 64
        assert (got == 4096.0 * 8 * steps).all()                  # the model, bit for bit
        err = np.abs(got - exact)
        assert np.allclose(err, 56 * 0.46875 * steps)
        A = np.abs(x) @ np.abs(w).T
        bound = fp8_truncation_bound(e4m3_exponent(xc[0]), e4m3_exponent(wc))[0] \
            + FP8_COMBINE * steps * 2.0 ** -24 * A[0, 0]
        assert (err <= bound).all()
        say(f"K={K} sign={sign:+d}: error {err.max():.4g} = 2^{np.log2(err.max() / 4096):.2f} of the "
            f"largest product per {steps} step(s); derived bound {bound:.4g}")


@pytest.mark.gpu
def test_fp8_derived_bound_holds_on_random_codes(dev):
    """Single steps of 64 random e4m3 products (unit scales) against the exact
    sums: every error inside the derived bound (20 code matrices of 256 x 256
    dot products)."""
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
        hx, hw = x8.cpu().numpy(), w8.cpu().numpy()
        dx, dw = e4m3_decode(hx).astype(np.float64), e4m3_decode(hw).astype(np.float64)
        A = np.abs(dx) @ np.abs(dw).T
        xe, we = e4m3_exponent(hx), e4m3_exponent(hw)
        bound = np.stack([fp8_truncation_bound(xe[i], we) for i in range(M)]) + FP8_COMBINE * 2.0 ** -24 * A
        ratio = np.abs(got - dx @ dw.T) / bound
        worst = max(worst, float(ratio.max()))
    say(f"largest error / derived bound over random steps: {worst:.3f}")
    assert worst <= 1.0


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

"""Buffers past 4 GiB: every kernel forms its row addresses in 64-bit
arithmetic, so rows whose byte offset from the buffer start exceeds 2^32
must come out as right as the first rows.  Each case places sampled rows on
both sides of that boundary and checks them against the oracle (fused call,
producer GEMM, the two regroupings) or byte for byte (gather), with sizes a
288 GB part holds easily (10-18 GB of device memory per case)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import reduce_add_rmsnorm_amd as sp
from helpers import to_host
from parity import run_case
from reduce_add_rmsnorm_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu
GiB4 = 1 << 32


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def spread(n_lo, n_hi, lo_end, hi_start, hi_end, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(4)) | set(range(hi_end - 12, hi_end))
    rows |= set(rng.integers(0, lo_end, n_lo).tolist()) | set(rng.integers(hi_start, hi_end, n_hi).tolist())
    return sorted(rows)


def test_fused_rows_past_4gib(dev):
    """C5's structure (bf16 partials, deepstack, per-token FP8) at H=4096 and a
    140000-row shard: partial 3 of rank 3 spans 3.4-4.6 GB into the partials
    buffer and rank 3's deepstack block the same range of the deepstack
    buffer; the last 9 rows are padding."""
    S, H, tp = 140000, 4096, 4
    w = dataclasses.replace(WORKLOADS["C5"], hidden=H, num_tokens=tp * S - 9, num_tokens_pad=tp * S)
    first_high = -(-(GiB4 - 3 * S * H * 2) // (H * 2))   # first row of partial 3 past 4 GiB
    assert 0 < first_high < S - 100
    rows = spread(24, 40, first_high, first_high, S, seed=3)
    say(f"fused past 4 GiB: tp={tp} S={S} H={H} rank 3, {len(rows)} sampled rows, "
        f"rows >= {first_high} of partial 3 beyond 4 GiB")
    res = run_case(w, 3, dev=dev, S=S, rows=rows)
    say(f"  ok: {res.stats}")
    torch.cuda.empty_cache()


def test_producer_gemm_slot_past_4gib(dev):
    """Rank 1 of tp=2 writes slot 1 of each [2, 300000, 4096] bf16 receive
    buffer: slot 1 spans 2.5-4.9 GB.  Integer operands keep every sum exact
    (bf16 holds the integers up to 256), so the rows must equal the oracle's."""
    tp, S, K, N, rank = 2, 300000, 64, 4096, 1
    first_high = -(-(GiB4 - rank * S * N * 2) // (N * 2))
    assert 0 < first_high < S - 100
    say(f"GEMM slot past 4 GiB: tp={tp} S={S} K={K} N={N} rank {rank}, slot rows >= {first_high} beyond 4 GiB")
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    x = torch.randint(-2, 3, (tp * S, K), generator=g, device=dev).to(torch.bfloat16)
    wt = torch.randint(-2, 3, (N, K), generator=g, device=dev).to(torch.bfloat16)
    dsts = [torch.full((tp, S, N), -7.0, dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_matmul_scatter(x, wt, dsts, rank=rank)
    torch.cuda.synchronize()
    srows = spread(16, 24, first_high, first_high, S, seed=4)
    n = len(srows)
    idx = torch.tensor(srows, device=dev)
    # compact problem for the oracle: the sampled rows of each destination
    xc = torch.cat([x[idx], x[S + idx]])
    ref = oracle.matmul_scatter(to_host(xc), to_host(wt), tp=tp, rank=rank, out_dtype=oracle.ORC_BF16)
    for r in range(tp):
        got = to_host(dsts[r][rank][idx])
        np.testing.assert_array_equal(got, ref[r][rank][:n], err_msg=f"destination {r}")
        other = to_host(dsts[r][1 - rank][idx])
        assert (other == to_host(torch.tensor([-7.0], dtype=torch.bfloat16))[0]).all(), "slot 0 was written"
    say(f"  ok: {n} rows in each of {tp} destinations equal the oracle's")
    del x, wt, dsts
    torch.cuda.empty_cache()


def test_gather_rows_past_4gib(dev):
    """Two 2.4M-row e4m3 shards of 1 KiB rows gathered into a [T, 1024] tensor
    of 4.9 GB (T = 2S - 7): rows of shard 1 land past 4 GiB; scales travel
    with them; nothing is written past row T."""
    tp, S, H = 2, 2_400_000, 1024
    T = tp * S - 7
    say(f"gather past 4 GiB: tp={tp} S={S} H={H} T={T}")
    g = torch.Generator(device=dev)
    g.manual_seed(22)
    shards = [torch.randint(0, 256, (S, H), generator=g, device=dev, dtype=torch.uint8) for _ in range(tp)]
    scales = [torch.rand((S,), generator=g, device=dev) for _ in range(tp)]
    out_buf = torch.full((T + 1, H), 0x5A, dtype=torch.uint8, device=dev)
    osc_buf = torch.full((T + 1,), -1.0, dtype=torch.float32, device=dev)
    sp.sp_all_gather_unpad(shards, scales, out_buf[:T], osc_buf[:T], num_tokens=T)
    torch.cuda.synchronize()
    first_high = -(-GiB4 // H)
    rows = spread(16, 32, S, first_high, T, seed=5)
    for m in rows:
        q, s = divmod(m, S)
        assert torch.equal(out_buf[m], shards[q][s]), f"row {m}"
        assert float(osc_buf[m]) == float(scales[q][s]), f"scale of row {m}"
    assert bool((out_buf[T] == 0x5A).all()) and float(osc_buf[T]) == -1.0, "written past row T"
    say(f"  ok: {len(rows)} rows, {sum(r >= first_high for r in rows)} of them past 4 GiB")
    del shards, scales, out_buf, osc_buf
    torch.cuda.empty_cache()


def test_fc2_regroup_past_4gib(dev):
    """FlashComm2 regrouping of G=2 ranks (otp=1, odp=2) with 4.4 GB sources
    and destinations, every rank's destination at once, against the oracle."""
    G, N, Cc = 2, 1_080_000, 2048
    assert N * Cc * 2 > GiB4
    say(f"FC2 regroup past 4 GiB: G={G} otp=1 N={N} C={Cc} bf16")
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    srcs = [torch.randint(-30000, 30000, (N, Cc), generator=g, device=dev, dtype=torch.int16).view(torch.bfloat16)
            for _ in range(G)]
    dsts = [torch.empty((N // 2, 2 * Cc), dtype=torch.bfloat16, device=dev) for _ in range(G)]
    sp.sp_fc2_regroup(srcs, dsts, otp=1)
    torch.cuda.synchronize()
    want = oracle.fc2_regroup([to_host(t) for t in srcs], 1)
    first_high = -(-GiB4 // (2 * Cc * 2))
    rows = spread(16, 32, first_high, first_high, N // 2, seed=6)
    idx = torch.tensor(rows, device=dev)
    for r in range(G):
        np.testing.assert_array_equal(to_host(dsts[r][idx]), want[r][rows], err_msg=f"rank {r}")
    say(f"  ok: {len(rows)} rows of each destination, rows >= {first_high} past 4 GiB")
    del srcs, dsts, want
    torch.cuda.empty_cache()


def test_dsacp_exchange_past_4gib(dev):
    """DSA-CP head-to-token exchange of tp=2 ranks with 4.4 GB inputs and
    outputs, against the oracle."""
    tp, S, D = 2, 1_080_000, 1024
    assert S * tp * D * 2 > GiB4
    say(f"DSA-CP exchange past 4 GiB: tp={tp} S={S} D={D} bf16")
    g = torch.Generator(device=dev)
    g.manual_seed(24)
    attn = [torch.randint(-30000, 30000, (S, tp * D), generator=g, device=dev, dtype=torch.int16).view(torch.bfloat16)
            for _ in range(tp)]
    outs = [torch.empty((tp * S, D), dtype=torch.bfloat16, device=dev) for _ in range(tp)]
    sp.sp_dsacp_heads_to_tokens(attn, outs)
    torch.cuda.synchronize()
    want = oracle.dsacp_heads_to_tokens([to_host(t) for t in attn])
    first_high = -(-GiB4 // (D * 2))
    rows = spread(16, 32, first_high, first_high, tp * S, seed=7)
    idx = torch.tensor(rows, device=dev)
    for q in range(tp):
        np.testing.assert_array_equal(to_host(outs[q][idx]), want[q][rows], err_msg=f"rank {q}")
    say(f"  ok: {len(rows)} rows of each output, rows >= {first_high} past 4 GiB")
    del attn, outs, want
    torch.cuda.empty_cache()

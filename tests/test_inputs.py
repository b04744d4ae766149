"""The seeded synthetic inputs (reduce_add_rmsnorm_amd/inputs.py), on the CPU:
deterministic, rank-dependent only where the method says so, the shapes and
dtypes each workload states, padding rows filled when asked, value
distributions as stated, and the algorithmic byte counts the benchmark
divides by."""

import dataclasses

import numpy as np
import pytest
import torch

from reduce_add_rmsnorm_amd.inputs import WORKLOADS, make_inputs


def _small(name):
    # the workload's dtypes, flags and tp at a size the CPU draws in milliseconds
    w = WORKLOADS[name]
    S = 12
    return dataclasses.replace(w, num_tokens=min(w.num_tokens, w.tp * S - (5 if name in ("C2", "C3") else 0)),
                               num_tokens_pad=w.tp * S, hidden=min(w.hidden, 256))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_same_seed_same_inputs(name):
    w = _small(name)
    a, b = make_inputs(w, rank=w.tp - 1), make_inputs(w, rank=w.tp - 1)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert torch.equal(a[k].view(torch.uint8) if a[k].dtype != torch.float32 else a[k].view(torch.int32),
                               b[k].view(torch.uint8) if b[k].dtype != torch.float32 else b[k].view(torch.int32)), k


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_ranks_differ_but_gain_and_bias_are_replicated(name):
    w = _small(name)
    a, b = make_inputs(w, rank=0), make_inputs(w, rank=1)
    assert not torch.equal(a["partials"], b["partials"])
    # a replicated residual is the same full tensor on every rank; a shard
    # residual holds the rank's own rows
    assert torch.equal(a["residual"], b["residual"]) == w.residual_replicated
    assert torch.equal(a["weight"], b["weight"])
    if w.bias:
        assert torch.equal(a["bias"], b["bias"])
    c = make_inputs(w, rank=0, base_seed=7)
    assert not torch.equal(a["partials"], c["partials"])


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_shapes_and_dtypes_follow_the_workload(name):
    w = _small(name)
    x = make_inputs(w)
    S, H, tp = w.shard_rows, w.hidden, w.tp
    assert x["partials"].shape == (tp, S, H) and x["partials"].dtype == w.partial_dtype
    assert x["residual"].shape == ((tp * S if w.residual_replicated else S), H)
    assert x["residual"].dtype == w.act_dtype
    assert x["weight"].shape == (H,) and x["weight"].dtype == w.act_dtype
    assert (x["bias"] is not None) == w.bias
    assert (x["deepstack"] is not None) == w.deepstack
    if w.deepstack:
        assert x["deepstack"].shape == (tp * S, H)


def test_padding_rows_take_the_fill_and_nothing_else_does():
    w = _small("C2")                       # last rank: 5 padding rows
    r = w.tp - 1
    v = w.num_tokens - r * w.shard_rows
    x = make_inputs(w, rank=r, pad_fill=float("nan"))
    clean = make_inputs(w, rank=r)
    assert torch.isnan(x["partials"][:, v:].float()).all()
    assert not torch.isnan(x["partials"][:, :v].float()).any()
    assert torch.equal(x["partials"][:, :v], clean["partials"][:, :v])
    assert torch.isnan(x["residual"][v:].float()).all() and not torch.isnan(x["residual"][:v].float()).any()
    w5 = dataclasses.replace(_small("C5"), num_tokens=_small("C5").num_tokens_pad - 3)
    x5 = make_inputs(w5, rank=w5.tp - 1, pad_fill=float("nan"))
    S = w5.shard_rows
    d = x5["deepstack"][(w5.tp - 1) * S:]
    assert torch.isnan(d[S - 3:].float()).all() and not torch.isnan(d[:S - 3].float()).any()
    assert not torch.isnan(x5["deepstack"][:(w5.tp - 1) * S].float()).any()   # other ranks' rows


def test_value_distributions_are_as_stated():
    w = dataclasses.replace(WORKLOADS["C3"], num_tokens=16 * 64, num_tokens_pad=16 * 64, hidden=4096)
    x = make_inputs(w)
    p = x["partials"].float().numpy()
    r = x["residual"].float().numpy()
    g = x["weight"].float().numpy()
    b = x["bias"].float().numpy()
    assert abs(p.mean()) < 0.01 and abs(p.std() - w.partial_sigma) < 0.01
    assert abs(r.mean()) < 0.02 and abs(r.std() - w.residual_sigma) < 0.02
    assert abs(g.mean() - w.weight_mu) < 0.01 and abs(g.std() - w.weight_sigma) < 0.01
    assert abs(b.std() - w.bias_sigma) < 0.002
    # one rounding to bf16: every value is exactly representable
    assert np.array_equal(x["partials"].float().to(torch.bfloat16).view(torch.int16).numpy(),
                          x["partials"].view(torch.int16).numpy())


def test_algorithmic_bytes_of_the_timed_workloads():
    # reads: tp partial rows + residual (+ deepstack) for the valid rows, gain
    # (+ bias) once, the static scale; writes: residual_out + out for every
    # row (+ the per-token scales)
    c4, c5 = WORKLOADS["C4"], WORKLOADS["C5"]
    S4, H4 = 8192, 7168
    assert c4.algorithmic_bytes() == S4 * H4 * (8 * 2 + 2) + H4 * 2 + 4 + S4 * H4 * (2 + 1)
    S5, H5 = 32768, 5120
    assert c5.algorithmic_bytes() == S5 * H5 * (4 * 2 + 2 + 2) + H5 * 2 + S5 * (H5 * (2 + 1) + 4)
    assert c4.algorithmic_bytes() == 1_233_139_716 and c5.algorithmic_bytes() == 2_516_723_712
    # padding rows are not read but are written
    c2 = WORKLOADS["C2"]
    S2, H2, v2 = 128, 4096, 1000 - 7 * 128
    assert c2.algorithmic_bytes() == v2 * H2 * (8 * 2 + 2) + H2 * 2 + S2 * H2 * (2 + 2)


# ------------------------------------------------ the counter-based generator

from reduce_add_rmsnorm_amd import inputs as I  # noqa: E402

M64 = (1 << 64) - 1


def _mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _reference_value(seed, tensor, source, row, col, cols, mu, sigma):
    """The recipe of inputs_gen.c restated in Python (integers exact, the
    transcendental part in double, so equal to the single-precision draw to
    ~1e-6)."""
    import math
    key = _mix64((_mix64(seed) + tensor * 0xD1B54A32D192ED03 + source * 0xABC98388FB8FAC03) & M64)
    e = row * cols + col
    u = _mix64((key + ((e >> 1) + 1) * 0x9E3779B97F4A7C15) & M64)
    u1 = ((u >> 40) + 1) / 2.0 ** 24
    u2 = (u & 0xFFFFFF) / 2.0 ** 24
    r = math.sqrt(-2.0 * math.log(u1))
    z = r * (math.sin(2 * math.pi * u2) if e & 1 else math.cos(2 * math.pi * u2))
    return mu + sigma * z


def test_generator_follows_its_stated_recipe():
    seed, cols = 20261206, 40
    t = I.draw(seed, 1, 3, 1000, 5, cols, 0.25, 0.5, torch.float32)
    for row in range(5):
        for col in (0, 1, 2, 17, 38, 39):
            want = _reference_value(seed, 1, 3, 1000 + row, col, cols, 0.25, 0.5)
            assert abs(float(t[row, col]) - want) < 2e-5, (row, col)
    # bf16 storage is the f32 draw rounded to nearest even
    b = I.draw(seed, 1, 3, 1000, 5, cols, 0.25, 0.5, torch.bfloat16)
    assert torch.equal(b, t.to(torch.bfloat16))


def test_generator_rows_are_independent_of_the_call():
    # any row range, any thread count: the same bytes for the same positions
    full = I.draw(7, 2, 0, 0, 300, 64, 0.0, 1.0, torch.bfloat16)
    part = I.draw(7, 2, 0, 123, 77, 64, 0.0, 1.0, torch.bfloat16)
    assert torch.equal(part.view(torch.int16), full[123:200].view(torch.int16))
    saved = I.GEN_THREADS
    try:
        I.GEN_THREADS = 1
        one = I.draw(7, 2, 0, 0, 300, 64, 0.0, 1.0, torch.bfloat16)
    finally:
        I.GEN_THREADS = saved
    assert torch.equal(one.view(torch.int16), full.view(torch.int16))
    # another tensor id, source or seed: another stream
    assert not torch.equal(I.draw(7, 3, 0, 0, 300, 64, 0.0, 1.0, torch.bfloat16), full)
    assert not torch.equal(I.draw(7, 2, 1, 0, 300, 64, 0.0, 1.0, torch.bfloat16), full)
    assert not torch.equal(I.draw(8, 2, 0, 0, 300, 64, 0.0, 1.0, torch.bfloat16), full)


@pytest.mark.parametrize("name", ["C2", "C5"])
def test_rank_shards_are_slices_of_the_full_tensors(name):
    # partial q of rank r is rows [r*S, (r+1)*S) of partial q's full tensor, so
    # the ranks' shards of one workload fit together into the whole layer
    w = _small(name)
    S, H, tp = w.shard_rows, w.hidden, w.tp
    full = {q: I.draw(I.BASE_SEED + w.seed_index, 1, q, 0, tp * S, H, 0.0, w.partial_sigma, w.partial_dtype)
            for q in range(tp)}
    for r in (0, tp - 1):
        x = make_inputs(w, rank=r)
        for q in range(tp):
            assert torch.equal(x["partials"][q].view(torch.int16), full[q][r * S:(r + 1) * S].view(torch.int16))
        if w.deepstack:   # the full deepstack is the same on every rank
            assert torch.equal(x["deepstack"], make_inputs(w, rank=0)["deepstack"])


@pytest.mark.parametrize("name", ["C2", "C5"])
def test_an_empty_shard_has_row_major_strides(name):
    # S = 0: the tensors are empty but strided like any [tp][S][H] block, which
    # the binding checks before it hands pointers to the library
    w = _small(name)
    x = make_inputs(w, rank=0, shard_rows=0, num_tokens=0)
    assert x["partials"].shape == (w.tp, 0, w.hidden)
    assert x["partials"].stride() == torch.empty((w.tp, 0, w.hidden)).stride()
    assert x["residual"].stride() == torch.empty((0, w.hidden)).stride()

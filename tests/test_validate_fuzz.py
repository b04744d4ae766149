"""CPU: seeded perturbations of valid descriptors through sp_validate (host
checks only, fake device addresses).  Every call returns a status, and
every call the library accepts satisfies the rules include/sprms.h states
for sp_reduce_add_rmsnorm's arguments -- including, with pointers moved into
each other's buffers, that no byte the call writes is read by it or written
twice (the in-place residual update excepted) and that the partials span at
most 2^47 bytes."""

import ctypes as C
import math
import random

import pytest

import reduce_add_rmsnorm_amd as sp

N_CALLS = 20000
BIG = [0, 1, 2, 7, 8, 16, 31, 32, 33, 64, 4096, 8192, 32768, 32776, 65536, 2 ** 31 - 1, 2 ** 31,
       2 ** 32, 2 ** 62, -1, -8]
SMALL = [0, 1, 2, 3, 4, 5, 8, 16, 63, 64, 65, 2 ** 31 - 1, -1, -2]
WIDE = ("shard_rows", "hidden", "num_tokens", "residual_rows", "deepstack_rows", "partial_stride")
FIELDS = WIDE + ("tp", "tp_rank", "partial_dtype", "act_dtype", "out_dtype", "flags")


def _valid(R):
    tp = R.choice([1, 2, 3, 4, 8, 16, 64])
    S = R.choice([0, 1, 5, 128, 219, 8192])
    q = R.choice([0, 1, 2, 4])
    H = 8 * R.randint(1, 4096)
    if q == 4:
        H = 32 * max(1, H // 32)
    p = sp.sp_problem()
    p.tp, p.tp_rank, p.shard_rows, p.hidden = tp, R.randrange(tp), S, H
    p.num_tokens = R.randint(0, tp * S)
    p.partial_dtype, p.act_dtype = R.choice([0, 1]), R.choice([0, 1])
    p.out_dtype = R.choice([0, 1]) if q == 0 else (2 if q in (1, 2) else R.choice([2, 3]))
    p.residual_rows = R.choice([S, tp * S])
    p.deepstack_rows = R.choice([0, S, tp * S])
    p.residual_out = 0x7F1000000000 if R.random() < 0.5 else None
    p.partial_stride = R.choice([0, S * H * R.choice([1, 2])])
    p.flags = R.choice([0, 1])
    p.partial_scale = R.choice([1.0, 0.5, 0.0])
    return p, q


def _check_spans(p, q, ptr):
    """The header's overlap and span rules, restated from its text."""
    S, H, tp, r = p.shard_rows, p.hidden, p.tp, p.tp_rank
    pe = 4 if p.partial_dtype == 0 else 2
    ae = 4 if p.act_dtype == 0 else 2
    stride = p.partial_stride or S * H
    span = ((tp - 1) * stride + S * H) * pe
    assert span <= 2 ** 47
    v = max(0, min(S, p.num_tokens - r * S))
    rows = v if p.flags & 1 else S
    used = ptr["residual"] + (r * S if p.residual_rows == tp * S else 0) * H * ae
    res_w = p.residual_out or used
    in_place = res_w == used
    orow = H // 2 if p.out_dtype == 3 else H * {0: 4, 1: 2, 2: 1}[p.out_dtype]
    srow = 4 if q == 2 else (H // 32 if q == 4 else 0)
    ins = {"partials": (ptr["partials"], span), "weight": (ptr["weight"], H * ae),
           "bias": (ptr["bias"], H * ae if ptr["bias"] else 0),
           "deepstack": (ptr["ds"], p.deepstack_rows * H * ae if ptr["ds"] else 0),
           "residual": (ptr["residual"], p.residual_rows * H * ae),
           "static scale": (ptr["osc"], 4 if q == 1 else 0)}
    outs = {"residual written": (res_w, rows * H * ae), "out": (ptr["out"], rows * orow),
            "out_scale": (ptr["osc"], rows * srow)}

    def meet(a, b):
        return bool(a[0] and b[0] and a[1] and b[1] and a[0] < b[0] + b[1] and b[0] < a[0] + a[1])

    for o, ospan in outs.items():
        for i, ispan in ins.items():
            if o == "residual written" and i == "residual" and in_place:
                continue
            assert not meet(ospan, ispan), (o, i)
    names = list(outs)
    for a in range(3):
        for b in range(a + 1, 3):
            assert not meet(outs[names[a]], outs[names[b]]), (names[a], names[b])


@pytest.mark.parametrize("seed", [1, 2])
def test_accepted_calls_obey_the_header(seed):
    lib = sp.load()
    R = random.Random(seed)
    accepted = 0
    for _ in range(N_CALLS):
        p, q = _valid(R)
        for _ in range(R.choice([0, 0, 1, 2])):  # break up to two fields
            f = R.choice(FIELDS + ("quant", "scale"))
            if f == "quant":
                q = R.randint(-1, 6)
            elif f == "scale":
                p.partial_scale = R.choice([float("inf"), float("nan"), -1.0, 1e-30])
            else:
                pool = BIG if f in WIDE else SMALL
                setattr(p, f, R.choice(pool) if R.random() < 0.7 else R.randint(-5, 40000))
        partials = None if R.random() < 0.05 else 0x7F0000000000
        bias = 0x7F3800000000 if R.random() < 0.5 else None
        ds = 0x7F4000000000 if p.deepstack_rows else None
        if R.random() < 0.05:
            ds = None if ds else 0x7F4000000000
        out = 0x7F5000000000 + (R.choice([1, 2, 4, 8]) if R.random() < 0.05 else 0)
        osc = 0x7F6000000000 if q != 0 else None
        eps = R.choice([0.0, 1e-6, 1e-6, -1.0, float("nan")])
        ptr = dict(partials=partials, residual=0x7F2000000000, weight=0x7F3000000000, bias=bias,
                   ds=ds, out=out, osc=osc)
        if R.random() < 0.3:  # move one pointer into another buffer
            k = R.choice(["residual", "weight", "bias", "ds", "out", "osc", "residual_out"])
            base = R.choice([0x7F0000000000, 0x7F1000000000, 0x7F2000000000, 0x7F3000000000,
                             0x7F4000000000, 0x7F5000000000, 0x7F6000000000])
            at = base + 64 * R.choice([0, 1, 7, 1024, 1 << 20, 1 << 26])
            if k == "residual_out":
                p.residual_out = at
            elif ptr[k] is not None:
                ptr[k] = at
        rc = lib.sp_validate(C.byref(p), ptr["partials"], ptr["residual"], ptr["weight"], ptr["bias"],
                             C.c_float(eps), q, ptr["ds"], ptr["out"], ptr["osc"])
        assert rc in (0, -1, -2, -3, -4, -5), rc
        if rc != 0:
            continue
        accepted += 1
        assert 1 <= p.tp <= 64 and 0 <= p.tp_rank < p.tp
        assert 8 <= p.hidden <= 32768 and p.hidden % 8 == 0
        assert 0 <= p.shard_rows <= 2 ** 31 - 1 and 0 <= p.num_tokens <= p.tp * p.shard_rows
        assert p.residual_rows in (p.shard_rows, p.tp * p.shard_rows)
        assert p.deepstack_rows in ((0,) if ds is None else (p.shard_rows, p.tp * p.shard_rows))
        assert q in (0, 1, 2, 4) and p.flags in (0, 1)
        assert eps >= 0 and math.isfinite(eps) and math.isfinite(p.partial_scale)
        assert p.partial_stride == 0 or p.partial_stride >= p.shard_rows * p.hidden
        assert ptr["partials"] is not None or p.shard_rows == 0  # S == 0 enqueues nothing
        assert q != 4 or p.hidden % 32 == 0
        _check_spans(p, q, ptr)
    assert accepted > N_CALLS // 10

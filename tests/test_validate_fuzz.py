"""CPU: seeded perturbations of valid descriptors through sp_validate (host
checks only, fake device addresses).  Every call returns a status, and
every call the library accepts satisfies the rules include/sprms.h states
for sp_reduce_add_rmsnorm's arguments."""

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
        rc = lib.sp_validate(C.byref(p), partials, 0x7F2000000000, 0x7F3000000000, bias, C.c_float(eps), q,
                             ds, out, osc)
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
        assert partials is not None or p.shard_rows == 0  # S == 0 enqueues nothing
        assert q != 4 or p.hidden % 32 == 0
    assert accepted > N_CALLS // 10

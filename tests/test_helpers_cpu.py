"""CPU: the comparison helpers used by the GPU parity checks agree with the
pinned oracle's encoders (the helpers are faster restatements of the same
rounding rule, so every bound they compute is the one the oracle implies)."""

import numpy as np

import oracle
from helpers import E4M3_TABLE, e4m3_decode, e4m3_round


def test_e4m3_table_matches_the_oracle_decoder():
    for c in range(256):
        want = oracle.e4m3_to_double(c)
        got = E4M3_TABLE[c]
        assert (np.isnan(want) and np.isnan(got)) or want == got, c
    np.testing.assert_array_equal(e4m3_decode(np.array([0x38, 0x7E, 0xFE, 0x01])),
                                  [1.0, 448.0, -448.0, 2.0 ** -9])


def test_e4m3_round_matches_the_oracle_encoder_on_a_dense_sweep():
    rng = np.random.default_rng(0)
    finite = E4M3_TABLE[np.isfinite(E4M3_TABLE)]
    mids = (finite[:-1] + finite[1:]) / 2  # not all adjacent in the table, still useful points
    pos = np.sort(np.abs(finite))
    ties = (pos[:-1] + pos[1:]) / 2
    near = np.concatenate([ties * (1 + 2.0 ** -40), ties * (1 - 2.0 ** -40)])
    x = np.concatenate([finite, mids, ties, -ties, near, -near,
                        rng.uniform(-500, 500, 400000), rng.normal(0, 1, 400000),
                        rng.normal(0, 2.0 ** -8, 200000), [0.0, -0.0, 448.0, 464.0, 1e30, -1e30,
                                                           2.0 ** -10, 2.0 ** -11, np.nan]])
    want = e4m3_decode(oracle.e4m3_from_double_array(x))
    got = e4m3_round(x)
    both_nan = np.isnan(want) & np.isnan(got)
    assert (both_nan | (want == got)).all(), x[~(both_nan | (want == got))][:10]
    assert (np.signbit(got) == np.signbit(want))[~both_nan].all()

"""CPU checks of the parity helpers' derived FP8-datapath bound (tests.parity):
the group-maximum sum against a brute-force loop, and the bound's relation to
sum |a b|."""

import numpy as np

from tests.parity import ACC_REL, FP8_GROUP_UNIT, fp8_group_max_sum, fp8_path_bound


def test_group_max_sum_brute_force():
    rng = np.random.default_rng(5)
    M, K, N = 4, 21, 3  # a ragged last group of 5
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N))
    got = fp8_group_max_sum(a, b)
    for i in range(M):
        for j in range(N):
            exp = 0.0
            for g in range(0, K, 8):
                exp += max(abs(a[i, k] * b[k, j]) for k in range(g, min(K, g + 8)))
            assert abs(got[i, j] - exp) <= 1e-12 * exp


def test_bound_between_group_max_and_sum_abs():
    """sum_g max_g <= sum|ab| <= 8 sum_g max_g, so the bound is at most
    (2^-10 + 1e-5) sum|ab| and at least 2^-13 sum|ab|."""
    rng = np.random.default_rng(6)
    a = rng.standard_normal((16, 64))
    b = rng.standard_normal((64, 12))
    sum_abs = np.abs(a) @ np.abs(b)
    gm = fp8_group_max_sum(a, b)
    assert (gm <= sum_abs * (1 + 1e-12)).all() and (sum_abs <= 8 * gm * (1 + 1e-12)).all()
    bound = fp8_path_bound(a, b, sum_abs)
    assert (bound <= (8 * FP8_GROUP_UNIT + ACC_REL) * sum_abs * (1 + 1e-12)).all()
    assert (bound >= FP8_GROUP_UNIT * sum_abs).all()

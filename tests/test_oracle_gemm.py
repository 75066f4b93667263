"""Pins of the oracle's exact GEMM, BF16 rounding and dequant (CPU only)."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import bf16, fp8, gemm
from oracle.fp8 import E4M3, E5M2
from oracle.gemm import OP_N, OP_T

# ----------------------------------------------------------------------------- bf16


def _torch_bf16_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_fp32_inputs():
    """For fp32 inputs, rounding to bf16 is torch's fp32 -> bf16 conversion."""
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 300_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45], np.float32)])
    got = bf16.round_to_bf16_vec(x.astype(np.float64))
    assert np.array_equal(got, _torch_bf16_bits(x))
    small = x[:3000]
    assert np.array_equal(bf16.round_to_bf16(small.astype(np.float64)), got[:3000])


def test_bf16_exhaustive_round_trip():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.widen(pats).astype(np.float64)
    back = bf16.round_to_bf16_vec(vals)
    ok = ~np.isnan(vals)
    assert np.array_equal(back[ok], pats[ok])
    assert np.all((back[~ok] & 0x7FFF) == 0x7FC0)


def test_bf16_ties_and_overflow():
    r = lambda v: int(bf16.round_to_bf16_vec(np.array([v]))[0])
    assert r(1.0 + 2.0**-8) == 0x3F80  # tie -> even (1.0)
    assert r(1.0 + 3 * 2.0**-8) == 0x3F82  # tie -> even (1 + 2^-6)
    assert r(1.0 + 2.0**-8 + 2.0**-40) == 0x3F81  # just above the tie (fp64 input)
    bmax = (2 - 2.0**-7) * 2.0**127
    assert r(bmax) == 0x7F7F
    assert r(2.0**128 - 2.0**119) == 0x7F80  # midpoint to 2^128 rounds to even -> inf
    assert r(2.0**128 - 2.0**119 - 2.0**100) == 0x7F7F
    assert r(-(2.0**-133)) == 0x8001  # smallest subnormal
    assert r(2.0**-134) == 0x0000  # half of it: tie -> even (0)


# ----------------------------------------------------------------------------- GEMM


def _ints_to_codes(ints, fmt):
    codes = fp8.encode(ints.astype(np.float32), fmt)
    assert np.array_equal(fp8.decode(codes, fmt), ints.astype(np.float64))
    return codes


def _stored(a, op):
    return np.ascontiguousarray(a if op == OP_N else a.T)


@pytest.mark.parametrize("opa,opb", [(OP_N, OP_N), (OP_N, OP_T), (OP_T, OP_N)])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
def test_small_integer_gemm_is_int_matmul(opa, opb, fa, fb):
    """Integers in [-16,16] (E4M3) / [-8,8] (E5M2) are exact FP8 values; the product
    is then numpy's int64 matmul, the textbook routine."""
    rng = np.random.default_rng(opa * 10 + opb + 3 * fa + 7 * fb)
    M, N, K = 37, 29, 70
    ra = 16 if fa == E4M3 else 8
    rb = 16 if fb == E4M3 else 8
    ia = rng.integers(-ra, ra + 1, (M, K))
    ib = rng.integers(-rb, rb + 1, (K, N))
    ca = _stored(_ints_to_codes(ia, fa), opa)
    cb = _stored(_ints_to_codes(ib, fb), opb)
    acc, sum_abs = gemm.gemm_exact(ca, fa, opa, cb, fb, opb)
    assert np.array_equal(acc, (ia @ ib).astype(np.float64))
    assert np.array_equal(sum_abs, (np.abs(ia) @ np.abs(ib)).astype(np.float64))
    ex, q = gemm.gemm_int_exact(ca, fa, opa, cb, fb, opb)
    assert np.array_equal(np.ldexp(ex.astype(np.float64), q), acc)


def test_op_semantics_hand_example():
    # A = [[1,2],[3,4]] (op N); B = [[1,0],[2,1]]; A@B = [[5,2],[11,4]]
    A = np.array([[1, 2], [3, 4]])
    B = np.array([[1, 0], [2, 1]])
    ca = _ints_to_codes(A, E4M3)
    cb = _ints_to_codes(B, E4M3)
    acc, _ = gemm.gemm_exact(ca, E4M3, OP_N, cb, E4M3, OP_N)
    assert acc.tolist() == [[5, 2], [11, 4]]
    # T on A: the stored array is A^T -> same product
    acc_t, _ = gemm.gemm_exact(np.ascontiguousarray(ca.T), E4M3, OP_T, cb, E4M3, OP_N)
    assert acc_t.tolist() == [[5, 2], [11, 4]]
    # T on B: stored B^T
    acc_bt, _ = gemm.gemm_exact(ca, E4M3, OP_N, np.ascontiguousarray(cb.T), E4M3, OP_T)
    assert acc_bt.tolist() == [[5, 2], [11, 4]]
    # and N on a stored transpose gives a different product
    acc_wrong, _ = gemm.gemm_exact(np.ascontiguousarray(ca.T), E4M3, OP_N, cb, E4M3, OP_N)
    assert acc_wrong.tolist() != [[5, 2], [11, 4]]


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_code_pair_table(fa, fb):
    """Row i of A holds code i at k=0, column j of B code j: C[i,j] = value(i) * value(j),
    checked against Python float products of the decoded table."""
    K = 128
    A = np.zeros((256, K), np.uint8)
    A[:, 0] = np.arange(256)
    B = np.zeros((K, 256), np.uint8)
    B[0, :] = np.arange(256)
    acc, _ = gemm.gemm_exact(A, fa, OP_N, B, fb, OP_N)
    ta, tb = fp8.decode_table(fa), fp8.decode_table(fb)
    for i in range(256):
        for j in range(256):
            if math.isfinite(ta[i]) and math.isfinite(tb[j]):
                assert acc[i, j] == ta[i] * tb[j]


def test_brute_force_triple_loop():
    rng = np.random.default_rng(9)
    M, N, K = 9, 11, 40
    for fa, fb in ((E4M3, E4M3), (E5M2, E4M3)):
        ca = rng.integers(0, 256, (M, K)).astype(np.uint8)
        cb = rng.integers(0, 256, (K, N)).astype(np.uint8)
        # keep finite codes only
        ca[np.isnan(fp8.decode(ca, fa)) | np.isinf(fp8.decode(ca, fa))] = 0x30
        cb[np.isnan(fp8.decode(cb, fb)) | np.isinf(fp8.decode(cb, fb))] = 0x30
        acc, _ = gemm.gemm_exact(ca, fa, OP_N, cb, fb, OP_N)
        for i in range(M):
            for j in range(N):
                s = 0
                from fractions import Fraction
                for k in range(K):
                    s += Fraction(fp8.decode_one(ca[i, k], fa)) * Fraction(fp8.decode_one(cb[k, j], fb))
                assert abs(Fraction(acc[i, j]) - s) <= Fraction(K) * Fraction(2) ** -53 * abs(
                    Fraction(float(np.abs(fp8.decode(ca[i], fa)) @ np.abs(fp8.decode(cb[:, j], fb)))))


def test_e4m3_fp64_sum_is_exact():
    """E4M3 x E4M3 sums are exact in fp64 for K <= 2^14: compare with int64."""
    rng = np.random.default_rng(10)
    ca = rng.integers(0, 256, (8, 4096)).astype(np.uint8)
    cb = rng.integers(0, 256, (4096, 8)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x7E
    cb[(cb & 0x7F) == 0x7F] = 0x7E
    acc, _ = gemm.gemm_exact(ca, E4M3, OP_N, cb, E4M3, OP_N)
    ex, q = gemm.gemm_int_exact(ca, E4M3, OP_N, cb, E4M3, OP_N)
    assert np.array_equal(np.ldexp(ex.astype(np.float64), q), acc)


def test_dequant_power_of_two_scales_exact():
    """With power-of-two scales and small integer sums the BF16 output is exact."""
    rng = np.random.default_rng(12)
    ia = rng.integers(-4, 5, (16, 8))
    ib = rng.integers(-4, 5, (8, 16))
    ca, cb = _ints_to_codes(ia, E4M3), _ints_to_codes(ib, E4M3)
    acc, _ = gemm.gemm_exact(ca, E4M3, OP_N, cb, E4M3, OP_N)
    y = gemm.dequant_to_bf16(acc, 4.0, 0.5)  # divide by 2
    exp = (ia @ ib) / 2.0
    assert np.array_equal(bf16.widen(y).astype(np.float64), exp)
    assert gemm.output_amax(y) == np.max(np.abs(exp))
    # the dequant divides (not multiplies) by the scale product
    y2 = gemm.dequant_to_bf16(acc, 8.0, 1.0)
    assert np.array_equal(bf16.widen(y2).astype(np.float64), (ia @ ib) / 8.0)


def test_dequant_scale_product_is_fp32():
    sa, sb = np.float32(1.1), np.float32(3.3)
    assert gemm.dequant_scale(sa, sb) == np.float32(sa * sb)
    assert float(gemm.dequant_scale(sa, sb)) != float(sa) * float(sb)

"""Pins of the MXFP8 oracle (oracle/mx.py): hand-worked blocks, the E8M0 code
values, power-of-two shifts, the largest element's binade, a brute-force
nearest-value check of every element, block independence, degenerate blocks, and
the MX GEMM against the plain GEMM (unit scales) and an exact-fraction triple
loop."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8 as ofp8
from oracle import gemm as ogemm
from oracle import mx as omx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")
FMTS = {"e4m3": ofp8.E4M3, "e5m2": ofp8.E5M2}


def _golden():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        f, vals, sc, codes = (p.strip() for p in line.split("|"))
        v = np.zeros(32, np.float32)
        for tok in vals.split():
            i, x = tok.split(":")
            v[int(i)] = np.float32(float(x))
        c = np.zeros(32, np.uint8)
        for tok in codes.split():
            i, x = tok.split(":")
            if i == "*":
                c[:] = int(x, 16)
            else:
                c[int(i)] = int(x, 16)
        out.append((FMTS[f], v, int(sc, 16), c))
    return out


def test_golden_blocks():
    cases = _golden()
    assert len(cases) == 6
    for fmt, v, sc, c in cases:
        codes, s = omx.quantize_block(v, fmt)
        assert s == sc
        np.testing.assert_array_equal(codes, c)


def test_e8m0_values():
    assert omx.e8m0_value(127) == 1.0
    assert omx.e8m0_value(0) == 2.0**-127
    assert omx.e8m0_value(254) == 2.0**127
    assert omx.e8m0_value(128) == 2.0
    assert np.isnan(omx.e8m0_value(255))


@pytest.mark.parametrize("fmt", [ofp8.E4M3, ofp8.E5M2])
def test_power_of_two_shift(fmt):
    rng = np.random.default_rng(5)
    v = rng.standard_normal(32).astype(np.float32)
    c0, s0 = omx.quantize_block(v, fmt)
    for k in (-20, -3, -1, 1, 7, 30):
        c, s = omx.quantize_block(np.ldexp(v, k).astype(np.float32), fmt)
        np.testing.assert_array_equal(c, c0)
        assert s == s0 + k


@pytest.mark.parametrize("fmt,lo,hi", [(ofp8.E4M3, 0x78, 0x7E), (ofp8.E5M2, 0x78, 0x7B)])
def test_largest_element_in_top_binade(fmt, lo, hi):
    rng = np.random.default_rng(6)
    for _ in range(200):
        v = (rng.standard_normal(32) * np.exp(rng.uniform(-20, 20))).astype(np.float32)
        c, _ = omx.quantize_block(v, fmt)
        top = c[np.argmax(np.abs(v))] & 0x7F
        assert lo <= top <= hi


@pytest.mark.parametrize("fmt", [ofp8.E4M3, ofp8.E5M2])
def test_elements_are_nearest_scaled_values(fmt):
    """Every element code is the nearest of the 256 table values to V / X
    (brute force over the table; exact ties are skipped, saturation clamps)."""
    table = ofp8.decode_table(fmt)
    finite = np.isfinite(table)
    rng = np.random.default_rng(7)
    vmax = ofp8.fmt_max(fmt)
    for _ in range(100):
        v = (rng.standard_normal(32) * np.exp(rng.uniform(-8, 8))).astype(np.float32)
        c, s = omx.quantize_block(v, fmt)
        X = omx.e8m0_value(s)
        for i in range(32):
            t = float(v[i]) / X
            t = max(-vmax, min(vmax, t))
            d = np.where(finite, np.abs(table - t), np.inf)
            best = np.flatnonzero(d == d.min())
            if len(best) > 1 and table[best].min() != table[best].max():
                continue  # an exact tie between two values
            assert table[c[i]] == table[best[0]]


def test_blocks_are_independent():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    c0, s0 = omx.mx_cast(x, ofp8.E4M3)
    y = x.copy()
    y[1, 32:64] *= 1000.0
    c1, s1 = omx.mx_cast(y, ofp8.E4M3)
    mask = np.ones_like(c0, bool)
    mask[1, 32:64] = False
    np.testing.assert_array_equal(c0[mask], c1[mask])
    smask = np.ones_like(s0, bool)
    smask[1, 1] = False
    np.testing.assert_array_equal(s0[smask], s1[smask])
    assert s1[1, 1] == s0[1, 1] + 9 or s1[1, 1] == s0[1, 1] + 10  # 1000 = 2^9.97


def test_degenerate_blocks():
    z = np.zeros(32, np.float32)
    c, s = omx.quantize_block(z, ofp8.E5M2)
    assert s == 0 and not c.any()
    v = np.ones(32, np.float32)
    v[4] = np.inf
    c, s = omx.quantize_block(v, ofp8.E4M3)
    assert s == 0xFF and (c == 0x7F).all()
    v[4] = -np.nan
    c, s = omx.quantize_block(v, ofp8.E5M2)
    assert s == 0xFF and (c == 0x7F).all()
    d = omx.mx_dequant(c[None, :], np.array([[s]], np.uint8), ofp8.E5M2)
    assert np.isnan(d).all()


@pytest.mark.parametrize("fa,fb", [(ofp8.E4M3, ofp8.E4M3), (ofp8.E5M2, ofp8.E4M3)])
def test_gemm_unit_scales_is_plain_gemm(fa, fb):
    rng = np.random.default_rng(9)
    a = rng.integers(0, 256, (16, 64), dtype=np.uint8)
    b = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    a[(a & 0x7F) >= (0x7F if fa == ofp8.E4M3 else 0x7C)] = 0x11
    b[(b & 0x7F) >= (0x7F if fb == ofp8.E4M3 else 0x7C)] = 0x22
    ones_a = np.full((16, 2), 127, np.uint8)
    ones_b = np.full((8, 2), 127, np.uint8)
    acc, sa = omx.mx_gemm_nt(a, ones_a, fa, b, ones_b, fb)
    ref, rs = ogemm.gemm_exact(a, fa, ogemm.OP_N, b, fb, ogemm.OP_T)
    np.testing.assert_array_equal(acc, ref)
    np.testing.assert_array_equal(sa, rs)


def test_gemm_brute_force_fractions():
    rng = np.random.default_rng(10)
    M, N, K = 3, 4, 64
    a = rng.integers(0, 0x7F, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    b = rng.integers(0, 0x7C, (N, K), dtype=np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    sa = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    acc, _ = omx.mx_gemm_nt(a, sa, ofp8.E4M3, b, sb, ofp8.E5M2)
    fa = {int(c): Fraction(ofp8.decode_one(int(c), ofp8.E4M3)) for c in np.unique(a)}
    fb = {int(c): Fraction(ofp8.decode_one(int(c), ofp8.E5M2)) for c in np.unique(b)}
    for i in range(M):
        for j in range(N):
            tot = Fraction(0)
            for k in range(K):
                tot += (fa[a[i, k]] * Fraction(2) ** (int(sa[i, k // 32]) - 127) *
                        fb[b[j, k]] * Fraction(2) ** (int(sb[j, k // 32]) - 127))
            assert abs(Fraction(acc[i, j]) - tot) <= abs(tot) * Fraction(1, 2**50) + Fraction(1, 2**200)


@pytest.mark.parametrize("fmt", [ofp8.E4M3, ofp8.E5M2])
def test_array_cast_equals_blockwise_definition(fmt):
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((9, 256)) *
         np.repeat(2.0 ** rng.integers(-140, 120, (9, 8)), 32, axis=1)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 40] = np.inf
    x[2, 70] = -np.nan
    x[3, 100] = np.float32(1.9 * 2**7)
    codes, scales = omx.mx_cast(x, fmt)
    for r in range(9):
        for b in range(8):
            c, s = omx.quantize_block(x[r, 32 * b:32 * (b + 1)], fmt)
            assert scales[r, b] == s
            np.testing.assert_array_equal(codes[r, 32 * b:32 * (b + 1)], c)

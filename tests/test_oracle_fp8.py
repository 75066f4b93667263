"""Pins of the oracle's FP8 codec and scaled cast against what the pages and the
mathematics fix (CPU only)."""

import math
import os
import random

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.fp8 import E4M3, E5M2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split()
        out[k] = v
    return out


def f32(x):
    return np.array([x], dtype=np.float32)


def enc1(x, fmt):
    return int(fp8.encode(f32(x), fmt)[0])


def test_page_constants():
    g = _golden("fp8_page_constants.txt")
    assert fp8.fmt_max(E4M3) == float(g["e4m3_max"]) == fp8.decode_one(0x7E, E4M3)
    assert fp8.fmt_max(E5M2) == float(g["e5m2_max"]) == fp8.decode_one(0x7B, E5M2)
    # exponent field == bias encodes 1.0 (implicit leading one, mantissa 0)
    b4, b5 = int(g["e4m3_bias"]), int(g["e5m2_bias"])
    assert fp8.decode_one(b4 << int(g["e4m3_mantissa_bits"]), E4M3) == 1.0
    assert fp8.decode_one(b5 << int(g["e5m2_mantissa_bits"]), E5M2) == 1.0
    assert fp8.decode_one(0x38, E4M3) == 1.0
    assert fp8.decode_one(0x39, E4M3) - 1.0 == float(g["e4m3_step_near_one"])
    assert fp8.decode_one(0x3C, E5M2) == 1.0
    assert fp8.decode_one(0x3D, E5M2) == 1.25


def test_code_classes():
    t4 = fp8.decode_table(E4M3)
    t5 = fp8.decode_table(E5M2)
    assert np.isfinite(t4).sum() == 254 and np.isnan(t4).sum() == 2
    assert np.isfinite(t5).sum() == 248 and np.isinf(t5).sum() == 2 and np.isnan(t5).sum() == 6
    assert np.isnan(t4[0x7F]) and np.isnan(t4[0xFF])
    assert t5[0x7C] == np.inf and t5[0xFC] == -np.inf
    # smallest subnormals and normals
    assert t4[0x01] == 2.0**-9 and t4[0x08] == 2.0**-6
    assert t5[0x01] == 2.0**-16 and t5[0x04] == 2.0**-14
    # sign symmetry
    for t in (t4, t5):
        fin = np.isfinite(t[:128])
        assert np.array_equal(t[128:][fin], -t[:128][fin])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_all_codes_round_trip(fmt):
    vals = fp8.decode_table(fmt)
    codes = np.arange(256, dtype=np.uint8)
    back = fp8.encode(vals.astype(np.float32), fmt)
    fin = np.isfinite(vals)
    assert np.array_equal(back[fin], codes[fin])
    nan = np.isnan(vals)
    sign = (codes[nan] >> 7).astype(np.uint32)
    signed_nan = (np.uint32(0x7FC00000) | (sign << 31)).view(np.float32)
    assert np.array_equal(fp8.encode(signed_nan, fmt), (0x7F | (sign << 7)).astype(np.uint8))
    if fmt == E5M2:
        assert back[0x7C] == 0x7B and back[0xFC] == 0xFB


def test_saturation_cases():
    for v in (448.0, 449.0, 463.99, 464.0, 465.0, 1e30, math.inf):
        assert enc1(v, E4M3) == 0x7E, v
        assert enc1(-v, E4M3) == 0xFE, v
    for v in (57344.0, 61440.0, 1e30, math.inf):
        assert enc1(v, E5M2) == 0x7B, v
        assert enc1(-v, E5M2) == 0xFB, v


def test_underflow_and_sign():
    assert enc1(2.0**-10, E4M3) == 0x00  # half the smallest subnormal: tie to even (0)
    nxt = float(np.nextafter(np.float32(2.0**-10), np.float32(1.0)))
    assert enc1(nxt, E4M3) == 0x01
    assert enc1(-(2.0**-11), E4M3) == 0x80  # keeps the sign
    assert enc1(3 * 2.0**-10, E4M3) == 0x02  # tie between codes 1 and 2 -> even
    assert enc1(-0.0, E4M3) == 0x80 and enc1(0.0, E5M2) == 0x00
    assert enc1(2.0**-17, E5M2) == 0x00 and enc1(-(2.0**-17) * 1.5, E5M2) == 0x81


def test_nan_input():
    assert enc1(math.nan, E4M3) == 0x7F
    assert enc1(math.nan, E5M2) == 0x7F
    neg_nan = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)
    assert fp8.encode(neg_nan, E4M3)[0] == 0xFF


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_midpoints_and_neighbours(fmt):
    """Every midpoint between adjacent finite values goes to the even code; one
    fp32 ulp either side goes to the nearer value (the definition of RNE)."""
    vals = fp8.decode_table(fmt)
    max_code = 0x7E if fmt == E4M3 else 0x7B
    for c in range(max_code):
        lo, hi = vals[c], vals[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # midpoints are exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert enc1(mid, fmt) == even
        assert enc1(np.nextafter(mid, np.float32(np.inf)), fmt) == c + 1
        assert enc1(np.nextafter(mid, np.float32(-np.inf)), fmt) == c
        assert enc1(-mid, fmt) == even | 0x80


def _torch_codes(x, fmt):
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    return torch.from_numpy(x).to(dt).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_matches_torch_in_range(fmt):
    """Inside the finite range, saturation is inactive and the encoding is plain
    round-to-nearest-even: torch's fp32 -> fp8 conversion is the library routine."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= fp8.fmt_max(fmt))]
    # all bf16 patterns as well
    b = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b) & (np.abs(b) <= fp8.fmt_max(fmt))]
    # values near the representable range, densely
    d = rng.uniform(-2 * fp8.fmt_max(fmt), 2 * fp8.fmt_max(fmt), 500_000).astype(np.float32)
    d = d[np.abs(d) <= fp8.fmt_max(fmt)]
    s = (rng.standard_normal(500_000) * 2.0 ** rng.integers(-20, 4, 500_000)).astype(np.float32)
    for arr in (x, b, d, s):
        assert np.array_equal(fp8.encode(arr, fmt), _torch_codes(arr, fmt))


def _brute_one(v, fmt):
    """Pure-Python nearest finite value with the even-code tie rule."""
    vals = fp8.decode_table(fmt)
    if math.isnan(v):
        return 0x7F | (0x80 if math.copysign(1, v) < 0 else 0)
    best, bestd = None, None
    for c in range(256):
        t = vals[c]
        if not math.isfinite(t):
            continue
        if (t == 0 and math.copysign(1, t) != math.copysign(1, v)):
            continue
        if t != 0 and (t > 0) != (v > 0):
            continue
        dist = abs(float(v) - t)
        if best is None or dist < bestd or (dist == bestd and c % 2 == 0):
            best, bestd = c, dist
    if abs(v) > fp8.fmt_max(fmt):
        return (0x7E if fmt == E4M3 else 0x7B) | (0x80 if v < 0 else 0)
    return best


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_brute_force_sample(fmt):
    random.seed(11)
    xs = []
    for _ in range(1500):
        e = random.randint(-30, 18)
        xs.append(random.choice([-1, 1]) * random.random() * 2.0**e)
    xs = np.array(xs, dtype=np.float32)
    got = fp8.encode(xs, fmt)
    for v, g in zip(xs, got):
        assert g == _brute_one(float(v), fmt), (float(v), g)


def test_scaled_cast_reduces_to_encode():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000).astype(np.float32) * 30
    for fmt in (E4M3, E5M2):
        codes, _ = fp8.cast(x, 1.0, fmt)
        assert np.array_equal(codes, fp8.encode(x, fmt))
        # power-of-two scale: the fp32 product is exact
        for k in (-3, 2, 5):
            codes, _ = fp8.cast(x, 2.0**k, fmt)
            exact = (x.astype(np.float64) * 2.0**k).astype(np.float32)
            assert np.array_equal(codes, fp8.encode(exact, fmt))


def test_double_rounding_is_part_of_the_definition():
    """The product is rounded to fp32 first, then to FP8.  Search for x, s whose
    exact product lies strictly above the E4M3 midpoint 1.0625 (between codes 0x38
    and 0x39) while fl32(x * s) is the midpoint itself: the cast must then take the
    tie rule (even code 0x38), not the exact product's nearest code (0x39)."""
    mid = 1.0625
    s = np.float32(3.0)
    found = 0
    x0 = np.float32(mid / 3.0)
    x = x0
    for _ in range(64):
        exact = float(x) * float(s)  # exact in fp64 (24 x 24 bits)
        if exact > mid and float(np.float32(x * s)) == mid:
            codes, _ = fp8.cast(np.array([x], dtype=np.float32), s, E4M3)
            assert codes[0] == 0x38
            assert fp8.encode(np.array([mid], dtype=np.float32), E4M3)[0] == 0x38
            found += 1
        x = np.nextafter(x, np.float32(2.0))
    assert found >= 1


def test_saturation_count():
    x = np.array([0.0, 1.0, 448.0, 449.0, -1000.0, np.inf, -np.inf, np.nan, 57344.0, 60000.0],
                 dtype=np.float32)
    _, n4 = fp8.cast(x, 1.0, E4M3)
    _, n5 = fp8.cast(x, 1.0, E5M2)
    assert n4 == 6  # 449, -1000, +inf, -inf, 57344, 60000
    assert n5 == 3  # +inf, -inf, 60000
    _, n4s = fp8.cast(x, 0.5, E4M3)
    assert n4s == 5  # 449*0.5 fits; -1000*0.5 = -500 does not

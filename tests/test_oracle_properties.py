"""Property-based pins of the oracle (hypothesis): the FP8 encoder is a
monotone, sign-symmetric nearest-value rounding within the format's half-spacing;
amax is the largest magnitude whatever the order; the scale maps the window value
onto FP8_MAX / 2^margin within one fp32 rounding; an MX block reconstructs each
unsaturated element within the element format's half-spacing."""

import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import amax as oamax
from oracle import fp8 as ofp8
from oracle import mx as omx
from oracle.scaling import scale_from_window

FINITE32 = st.floats(allow_nan=False, allow_infinity=False, width=32)
FMTS = st.sampled_from([ofp8.E4M3, ofp8.E5M2])
# (mantissa bits, smallest normal exponent) of each format
SPEC = {ofp8.E4M3: (3, -6), ofp8.E5M2: (2, -14)}


def half_spacing(v: float, fmt: int) -> float:
    """Half the distance between neighbouring FP8 values around |v|."""
    mbits, emin = SPEC[fmt]
    e = max(math.frexp(abs(v))[1] - 1, emin) if v != 0 else emin
    return math.ldexp(1.0, e - mbits - 1)


@settings(max_examples=400, deadline=None)
@given(FINITE32, FMTS)
def test_encode_is_nearest_within_half_spacing(x, fmt):
    vmax = ofp8.fmt_max(fmt)
    code = ofp8.encode(np.array([x], np.float32), fmt)[0]
    got = float(ofp8.decode(np.array([code], np.uint8), fmt)[0])
    target = max(-vmax, min(vmax, x))
    assert abs(got - target) <= half_spacing(target, fmt)
    assert (code >> 7) == (1 if math.copysign(1.0, x) < 0 else 0)


@settings(max_examples=300, deadline=None)
@given(FINITE32, FINITE32, FMTS)
def test_encode_is_monotone_and_sign_symmetric(x, y, fmt):
    lo, hi = sorted((x, y))
    c = ofp8.encode(np.array([lo, hi, -lo], np.float32), fmt)
    d = ofp8.decode(c, fmt)
    assert d[0] <= d[1]
    assert c[2] == c[0] ^ 0x80


@settings(max_examples=200, deadline=None)
@given(st.lists(FINITE32, min_size=1, max_size=64), st.randoms(use_true_random=False))
def test_amax_is_the_largest_magnitude_in_any_order(xs, rnd):
    a = np.array(xs, np.float32)
    m = oamax.amax(a)
    assert m == np.float32(max(abs(v) for v in xs))
    perm = list(xs)
    rnd.shuffle(perm)
    assert oamax.amax(np.array(perm, np.float32)) == m


@settings(max_examples=300, deadline=None)
@given(st.floats(min_value=float(np.float32(1e-30)), max_value=float(np.float32(1e30)), width=32),
       FMTS, st.integers(0, 4))
def test_scale_maps_the_window_onto_max(w, fmt, margin):
    s = float(scale_from_window(np.float32(w), fmt, margin))
    target = ofp8.fmt_max(fmt) / 2.0**margin
    assert abs(s * w - target) <= target * 2.0**-23


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(min_value=-1e6, max_value=1e6, width=32), min_size=32, max_size=32),
       FMTS)
def test_mx_block_reconstructs_within_half_spacing(xs, fmt):
    v = np.array(xs, np.float32)
    codes, sc = omx.quantize_block(v, fmt)
    if sc == 0 and not v.any():
        assert not (codes & 0x7F).any()
        return
    X = omx.e8m0_value(sc)
    vals = ofp8.decode(codes, fmt) * X
    vmax = ofp8.fmt_max(fmt)
    for i in range(32):
        q = float(v[i]) / X
        if abs(q) > vmax:  # saturated: the block maximum rounded above the format maximum
            assert abs(vals[i]) == vmax * X
            continue
        assert abs(vals[i] - float(v[i])) <= half_spacing(q, fmt) * X

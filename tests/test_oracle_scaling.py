"""Pins of the oracle's amax, scale formula and history window (CPU only)."""

import math
from collections import deque
from fractions import Fraction

import numpy as np
import pytest

from oracle import amax as amax_mod
from oracle import fp8, scaling
from oracle.fp8 import E4M3, E5M2
from oracle.scaling import ALGO_MAX, ALGO_MOST_RECENT, ScalingState

# ----------------------------------------------------------------------------- amax


def test_amax_matches_numpy_and_invariants():
    rng = np.random.default_rng(1)
    for n in (1, 7, 1000, 65537):
        x = (rng.standard_normal(n) * 10).astype(np.float32)
        a = amax_mod.amax(x)
        assert a == np.max(np.abs(x))
        assert np.all(np.abs(x) <= a) and np.any(np.abs(x) == a)


def test_amax_special_cases():
    assert amax_mod.amax(np.zeros(0, np.float32)) == 0.0
    z = amax_mod.amax(np.array([-0.0, -0.0], np.float32))
    assert z == 0.0 and not math.copysign(1.0, float(z)) < 0
    assert amax_mod.amax(np.array([1.0, -np.inf], np.float32)) == np.inf
    n = amax_mod.amax(np.array([1.0, np.nan, -np.inf], np.float32))
    assert np.array([n], np.float32).view(np.uint32)[0] == 0x7FC00000
    assert amax_mod.amax(np.array([-5.0, 3.0], np.float32)) == 5.0


# ----------------------------------------------------------------------------- scale formula


@pytest.mark.parametrize(
    "fmt,w,margin,expected",
    [
        # exact by hand: (MAX / w) / 2**margin with power-of-two-friendly quotients
        (E4M3, 448.0, 0, 1.0),
        (E4M3, 1.0, 0, 448.0),
        (E4M3, 4.0, 0, 112.0),
        (E4M3, 7.0, 2, 16.0),  # 448/7 = 64, /4 = 16: margin divides
        (E4M3, 0.5, 0, 896.0),
        (E5M2, 448.0, 0, 128.0),
        (E5M2, 57344.0, 0, 1.0),
        (E5M2, 7.0, 3, 1024.0),  # 57344/7 = 8192, /8
    ],
)
def test_scale_exact_cases(fmt, w, margin, expected):
    assert scaling.scale_from_window(np.float32(w), fmt, margin) == np.float32(expected)


def test_scale_is_correctly_rounded_quotient():
    """The fp32 scale is the fp32 number nearest the real (MAX / w) / 2**margin
    (checked with exact rationals against both fp32 neighbours)."""
    rng = np.random.default_rng(2)
    ws = np.concatenate([
        (rng.random(3000) * 2.0 ** rng.integers(-20, 20, 3000)).astype(np.float32),
        np.array([3.0, 100.0, 1000.0, 0.1, 1e-3, 12345.678], np.float32),
    ])
    for fmt in (E4M3, E5M2):
        for w in ws:
            if w <= 0:
                continue
            for margin in (0, 1, 3):
                s = scaling.scale_from_window(w, fmt, margin)
                exact = Fraction(int(fp8.fmt_max(fmt))) / Fraction(float(w)) / 2**margin
                if not (2.0**-126 <= float(exact) < 3.0e38):
                    continue
                err = abs(Fraction(float(s)) - exact)
                up = np.nextafter(s, np.float32(np.inf))
                dn = np.nextafter(s, np.float32(0))
                assert err <= abs(Fraction(float(up)) - exact)
                assert err <= abs(Fraction(float(dn)) - exact)


def test_scale_worked_values_bits():
    """Quotients that are not exact: the fp32 bits of the nearest value, found by
    exact rational rounding, not by the formula in fp32."""

    def nearest_f32(fr):
        c = np.float32(float(fr))
        best = min([c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))],
                   key=lambda v: abs(Fraction(float(v)) - fr))
        return best

    for fmt, w, margin in [(E4M3, 3.0, 0), (E4M3, 100.0, 0), (E4M3, 1000.0, 0), (E4M3, 1000.0, 1),
                           (E5M2, 100.0, 0), (E5M2, 1000.0, 0), (E5M2, 3.0, 0)]:
        fr = Fraction(int(fp8.fmt_max(fmt))) / Fraction(w) / 2**margin
        assert scaling.scale_from_window(np.float32(w), fmt, margin) == nearest_f32(fr)


def test_scale_fallback():
    for w in (0.0, np.nan, np.inf, -1.0):
        assert scaling.scale_from_window(np.float32(w), E4M3, 0) == 1.0
    # amax so small that MAX / amax overflows fp32 -> fallback
    assert scaling.scale_from_window(np.float32(1e-40), E4M3, 0) == 1.0
    # huge margin underflows to 0 -> fallback
    assert scaling.scale_from_window(np.float32(1.0), E4M3, 200) == 1.0


# ----------------------------------------------------------------------------- history


def _brute_window(amaxes, L, algo, fmt, margin):
    """Scale after each step, from a plain list of the last L values (zeros first)."""
    win = deque([0.0] * L, maxlen=L)
    out = []
    for a in amaxes:
        win.append(float(a))
        w = max(win) if algo == ALGO_MAX else float(a)
        if any(math.isnan(v) for v in win) and algo == ALGO_MAX:
            w = math.nan
        if not math.isfinite(w) or w <= 0:
            out.append(1.0)
            continue
        q = float(np.float32(np.float32(fp8.fmt_max(fmt)) / np.float32(w)))
        s = math.ldexp(q, -margin)
        out.append(s if math.isfinite(s) and s > 0 else 1.0)
    return out


@pytest.mark.parametrize("L", [1, 3, 16, 1024])
@pytest.mark.parametrize("algo", [ALGO_MAX, ALGO_MOST_RECENT])
def test_history_matches_brute_force(L, algo):
    rng = np.random.default_rng(L * 10 + algo)
    amaxes = (rng.random(60) * 2.0 ** rng.integers(-5, 10, 60)).astype(np.float32)
    amaxes[17] = 0.0
    for fmt in (E4M3, E5M2):
        st = ScalingState(fmt, L)
        got = [float(st.update(a, algo, 1)) for a in amaxes]
        assert got == _brute_window(amaxes, L, algo, fmt, 1)


def test_len_one_max_equals_most_recent():
    rng = np.random.default_rng(5)
    amaxes = (rng.random(40) * 100).astype(np.float32)
    a, b = ScalingState(E4M3, 1), ScalingState(E4M3, 1)
    for v in amaxes:
        assert a.update(v, ALGO_MAX, 0) == b.update(v, ALGO_MOST_RECENT, 0)


def test_long_window_is_cumulative_max():
    rng = np.random.default_rng(6)
    amaxes = (rng.random(10) * 100).astype(np.float32)
    st = ScalingState(E5M2, 16)
    for t, v in enumerate(amaxes):
        s = st.update(v, ALGO_MAX, 0)
        assert s == scaling.scale_from_window(np.max(amaxes[: t + 1]), E5M2, 0)


def test_outlier_step_behaviour():
    """A 50x batch at step 6: under max it sets the scale for every later step of a
    16-long window; under most_recent the scale recovers one step later."""
    amaxes = [4.0 * (1 + 2 * t / 9) for t in range(10)]
    amaxes[6] *= 50
    smax, srec = ScalingState(E4M3, 16), ScalingState(E4M3, 16)
    after_max, after_rec = [], []
    for v in amaxes:
        after_max.append(smax.update(np.float32(v), ALGO_MAX, 0))
        after_rec.append(srec.update(np.float32(v), ALGO_MOST_RECENT, 0))
    out_scale = scaling.scale_from_window(np.float32(amaxes[6]), E4M3, 0)
    assert all(s == out_scale for s in after_max[6:])
    assert after_rec[6] == out_scale and after_rec[7] != out_scale
    assert after_rec[7] == scaling.scale_from_window(np.float32(amaxes[7]), E4M3, 0)


def test_nan_in_window_falls_back_then_persists():
    st = ScalingState(E4M3, 4)
    st.update(np.float32(2.0), ALGO_MAX, 0)
    assert st.update(np.float32(np.nan), ALGO_MAX, 0) == 1.0
    for _ in range(3):  # NaN still inside the window of 4
        assert st.update(np.float32(2.0), ALGO_MAX, 0) == 1.0
    assert st.update(np.float32(2.0), ALGO_MAX, 0) == 224.0  # NaN has left the window


def test_cursor_wraps():
    st = ScalingState(E4M3, 3)
    for i in range(7):
        st.update(np.float32(i + 1), ALGO_MAX, 0)
    assert st.cursor == 7 % 3
    assert sorted(st.history.tolist()) == [5.0, 6.0, 7.0]

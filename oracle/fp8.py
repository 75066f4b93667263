"""FP8 E4M3 / E5M2 codec and the scaled saturating cast (oracle; test infrastructure only).

Formats ([P2] §一 "FP8 格式设计", [P3] §核心原理 "E4M3 与 E5M2 承担不同职责"):

* E4M3: 1 sign, 4 exponent, 3 mantissa bits, exponent bias 7, largest magnitude 448.
* E5M2: 1 sign, 5 exponent, 2 mantissa bits, exponent bias 15, largest magnitude 57344.

The pages fix only the field widths, the biases and the largest magnitudes.  The
special values follow [OCP] (E4M3 is the finite-only "fn" variant, the dtype name
``float8_e4m3fn`` used in [P2] §五):

* E4M3: exponent field 15 with mantissa 7 is NaN; there is no infinity.
* E5M2: exponent field 31 with mantissa 0 is +-inf, with mantissa != 0 NaN.
* Exponent field 0 encodes subnormals (no implicit leading one).

The cast ([P2] §四 "动态缩放", the quantize step: multiply by the scale, clamp to
the format range, convert) is ``code = encode(fl32(x * s))``: one IEEE fp32
multiply with round-to-nearest-even, then a saturating round-to-nearest-even
conversion to the nearest finite FP8 value.  Reading taken where the pages are
silent: a NaN input becomes the canonical NaN code ``0x7F | sign << 7`` in both
formats; a magnitude above the format maximum (infinity included) becomes the
largest finite code of that sign; the sign is kept on underflow to zero.
"""

from __future__ import annotations

import numpy as np

E4M3 = 0
E5M2 = 1

# (exponent bits, mantissa bits, bias, max finite value, code of max finite value)
_SPEC = {
    E4M3: (4, 3, 7, 448.0, 0x7E),
    E5M2: (5, 2, 15, 57344.0, 0x7B),
}

FORMAT_NAMES = {E4M3: "e4m3", E5M2: "e5m2"}


def fmt_max(fmt: int) -> float:
    """Largest finite magnitude of ``fmt`` ([P2] §一; [P2] §四 constants)."""
    return _SPEC[fmt][3]


def decode_one(code: int, fmt: int) -> float:
    """Value of one FP8 code as a Python float (fp64); NaN codes give nan.

    Straight from the field definition: sign, biased exponent, mantissa.
    """
    ebits, mbits, bias, _, _ = _SPEC[fmt]
    code = int(code) & 0xFF
    sign = -1.0 if code >> 7 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if fmt == E4M3 and e == emax_field and m == (1 << mbits) - 1:
        return float("nan")
    if fmt == E5M2 and e == emax_field:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


def decode_table(fmt: int) -> np.ndarray:
    """All 256 codes decoded, as fp64 (index = code)."""
    return np.array([decode_one(c, fmt) for c in range(256)], dtype=np.float64)


_TABLES = {f: decode_table(f) for f in (E4M3, E5M2)}


def decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Decode an array of uint8 codes to fp64 values."""
    return _TABLES[fmt][np.asarray(codes, dtype=np.uint8)]


def _positive_finite(fmt: int):
    """Non-negative finite codes in increasing value order, and their values.

    For both formats the codes 0 .. max_code are exactly the non-negative finite
    values and they increase with the code number.
    """
    max_code = _SPEC[fmt][4]
    codes = np.arange(max_code + 1, dtype=np.int64)
    vals = _TABLES[fmt][: max_code + 1]
    assert np.all(np.diff(vals) > 0)
    return codes, vals


def encode(v: np.ndarray, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even conversion of fp32 values to FP8 codes.

    Nearest-value search over the table of finite values, with the tie rule
    written out: ``2|v|`` is compared with ``lo + hi`` (both exact in fp64), and an
    exact tie picks the code with the even mantissa, i.e. the even code number.
    """
    v = np.asarray(v, dtype=np.float32)
    codes, vals = _positive_finite(fmt)
    vmax = _SPEC[fmt][3]
    max_code = _SPEC[fmt][4]

    bits = v.view(np.uint32)
    sign = (bits >> 31).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(v)
    a_clean = np.where(nan, 0.0, a)
    sat = a_clean > vmax

    # hi = index of the smallest table value >= a; lo = largest value <= a.
    a_in = np.minimum(a_clean, vmax)
    hi = np.searchsorted(vals, a_in, side="left")
    exact = vals[hi] == a_in
    lo = np.where(exact, hi, hi - 1)
    lo = np.maximum(lo, 0)
    twice = 2.0 * a_in
    mid = vals[lo] + vals[hi]
    pick_hi = (twice > mid) | ((twice == mid) & (codes[hi] % 2 == 0))
    mag = np.where(exact, codes[hi], np.where(pick_hi, codes[hi], codes[lo]))
    mag = np.where(sat, max_code, mag)
    out = (mag | (sign.astype(np.int64) << 7)).astype(np.uint8)
    out = np.where(nan, (0x7F | (sign.astype(np.int64) << 7)).astype(np.uint8), out)
    return out.astype(np.uint8)


def scaled_product_f32(x: np.ndarray, scale: np.float32) -> np.ndarray:
    """``fl32(x * s)``: one IEEE fp32 multiply, round-to-nearest-even.

    ``x`` is the unscaled tensor widened exactly to fp32 (from bf16 or fp32).
    numpy's float32 multiply is the IEEE operation with subnormals kept.
    """
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return (x32 * np.float32(scale)).astype(np.float32)


def cast(x: np.ndarray, scale, fmt: int):
    """Scaled saturating cast ([P2] §四 quantize; [P2] §五 the fp8 linear op).

    Returns ``(codes uint8, saturation count)``.  The saturation count is the
    number of elements with ``|fl32(x * s)| > max`` (infinities counted, NaN not).
    """
    y = scaled_product_f32(x, np.float32(scale))
    return encode(y, fmt), _count_above_max(y, fmt)


def _count_above_max(y: np.ndarray, fmt: int) -> int:
    with np.errstate(invalid="ignore"):
        return int(np.count_nonzero(np.abs(y.astype(np.float64)) > fmt_max(fmt)))


def saturation_count(x: np.ndarray, scale, fmt: int) -> int:
    """The saturation count of :func:`cast` alone (no encoding): ``#{|fl32(x*s)| > max}``."""
    return _count_above_max(scaled_product_f32(x, np.float32(scale)), fmt)

"""Quantization-health counts of one scaled cast (oracle; test infrastructure only).

[P3] "第四步：建立 Amax 与低精度异常画像" asks every converted module for
quantization-quality metrics (the share of values near the FP8 upper limit, the
share of zeros after quantization) and gradient-health counts (NaN / Inf /
overflow); [P2] §七 "陷阱 1：NaN/Inf 难以定位" checks each tensor for NaN and
infinity.  The pages name these quantities without fixing their arithmetic; the
readings taken here (all counts over the elements of one cast):

* ``saturated``: elements with ``|fl32(x * s)| > max`` (infinities counted, NaN
  not): the overflow count, the same quantity as the cast's saturation count.
* ``nan``: input elements that are NaN.
* ``inf``: input elements that are +-infinity.
* ``zero``: elements whose FP8 code is +-0 (underflow to zero and exact zeros).
* ``near_max``: elements whose FP8 code is finite and lies in the format's top
  binade ``[2^emax, max]``: [256, 448] for E4M3, [32768, 57344] for E5M2
  (saturated elements included).

The counts are taken from the codes of :func:`oracle.fp8.cast` and from the
decoded values, never from the GPU's packed byte tests.
"""

from __future__ import annotations

import numpy as np

from . import fp8 as ofp8

NAMES = ("saturated", "nan", "inf", "zero", "near_max")

# smallest magnitude of the top binade of each format (2^emax)
TOP_BINADE = {ofp8.E4M3: 256.0, ofp8.E5M2: 32768.0}


def cast_health(x: np.ndarray, scale, fmt: int) -> dict:
    """Counts of :data:`NAMES` for the cast of ``x`` (values widened exactly to
    fp32) with ``scale`` into ``fmt``."""
    x32 = np.asarray(x, dtype=np.float32).ravel()
    codes, saturated = ofp8.cast(x32, scale, fmt)
    vals = ofp8.decode(codes, fmt).astype(np.float64)
    finite = np.isfinite(vals)
    mag = np.abs(np.where(finite, vals, 0.0))
    return {
        "saturated": int(saturated),
        "nan": int(np.count_nonzero(np.isnan(x32))),
        "inf": int(np.count_nonzero(np.isinf(x32))),
        "zero": int(np.count_nonzero(finite & (mag == 0.0))),
        "near_max": int(np.count_nonzero(finite & (mag >= TOP_BINADE[fmt]))),
    }

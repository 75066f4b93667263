"""amax of the unscaled tensor (oracle; test infrastructure only).

[P2] §四 "动态缩放": the quantize step first takes the maximum absolute value of
the high-precision tensor.  [P3] §核心原理 "Scale 决定数值是否进入可表示区间"
defines amax the same way (the largest absolute value of the tensor).

Rules where the pages are silent, following the behaviour of ``max(abs(x))`` over
a tensor as written on [P2]: any NaN makes the result NaN (returned as the
canonical quiet NaN 0x7FC00000), otherwise any infinity gives +inf; an empty
tensor gives 0.0; ``|-0| = +0``.
"""

from __future__ import annotations

import numpy as np

CANONICAL_NAN_BITS = 0x7FC00000


def amax(x: np.ndarray) -> np.float32:
    """``max_i |x_i|`` as fp32 (exact: the maximum is one of the inputs)."""
    x = np.asarray(x)
    if x.size == 0:
        return np.float32(0.0)
    xf = x.astype(np.float64).ravel()
    if np.isnan(xf).any():
        return np.array([CANONICAL_NAN_BITS], dtype=np.uint32).view(np.float32)[0]
    return np.float32(np.max(np.abs(xf)))

"""GPU parity: every fp32 bit pattern the FP8 encoders can round to a finite
non-zero code (plus two binades below, which round to zero), both signs, cast at
scale 1 and compared byte for byte with the oracle's encoder.

The casts encode with gfx950's packed FP8 converts after a clamp to the format's
range; this sweep is the evidence that those converts round every in-range
fp32 value to nearest even exactly as the saturating encoder of the OCP formats
does ([P2] "FP8 混合精度训练工程实践" §一 "FP8 格式设计": E4M3 bias 7 and max 448,
E5M2 bias 15 and max 57344).  Values above the top binade are clamped to the
format's maximum before the convert; NaN inputs take the software encoder; both
are covered by the bf16-pattern and special-value tests of test_gpu_cast.py.

E4M3: |v| in [2^-13, 2^9)   -- 22 binades x 2^23 patterns x 2 signs = 369M values.
E5M2: |v| in [2^-20, 2^16)  -- 36 binades x 2^23 patterns x 2 signs = 604M values.
The oracle's encoder runs over the same bit patterns in threads (numpy releases
the interpreter lock), a chunk of 2^24 patterns at a time."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 1 << 24
SUB = 1 << 21
RANGES = {dsg.E4M3: (-13, 9), dsg.E5M2: (-20, 16)}


def _oracle_codes(start: int, stop: int, sign: int) -> np.ndarray:
    bits = (np.arange(start, stop, dtype=np.uint32) | np.uint32(sign)).view(np.float32)
    return bits


@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
def test_every_in_range_fp32_pattern(fmt):
    lo, hi = RANGES[fmt]
    first, last = (lo + 127) << 23, (hi + 127) << 23
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    q = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    sat = torch.zeros(1, dtype=torch.int64, device=DEV)
    checked = 0
    with ThreadPoolExecutor(8) as pool:
        for sign in (0, 0x80000000):
            for start in range(first, last, CHUNK):
                stop = min(start + CHUNK, last)
                n = stop - start
                # the same bit patterns on the device (int64 arithmetic, then the
                # low 32 bits reinterpreted as fp32)
                b = torch.arange(start, stop, dtype=torch.int64, device=DEV) | sign
                b = torch.where(b >= 2**31, b - 2**32, b).to(torch.int32)
                x = b.view(torch.float32)
                dsg.fp8ds_cast(x, fmt, one, q[:n], sat_count=sat)
                got = q[:n].cpu().numpy()

                def oracle(s0, s=sign):
                    v = _oracle_codes(s0, min(s0 + SUB, stop), s)
                    return s0, ofp8.encode(v, fmt), int(np.count_nonzero(
                        np.abs(v.astype(np.float64)) > ofp8.fmt_max(fmt)))

                n_sat = 0
                for s0, exp, ns in pool.map(oracle, range(start, stop, SUB)):
                    seg = got[s0 - start:s0 - start + exp.size]
                    if not np.array_equal(seg, exp):
                        bad = np.flatnonzero(seg != exp)[0]
                        pat = (s0 + bad) | sign
                        pytest.fail(f"pattern 0x{pat:08x}: gpu 0x{seg[bad]:02x} "
                                    f"oracle 0x{exp[bad]:02x}")
                    n_sat += ns
                assert int(sat.item()) == n_sat, (hex(start | sign), int(sat.item()), n_sat)
                checked += n
    assert checked == 2 * (last - first)

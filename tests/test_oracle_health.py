"""Pins of the quantization-health counts (oracle/health.py): hand-computed
cases from the definitions (round-to-nearest-even values worked out by hand)."""

import numpy as np

from oracle import fp8 as ofp8
from oracle import health as ohealth


def test_e4m3_hand_case():
    x = np.array([0.0, -0.0, 1e-10,
                  2.0**-10,      # halfway between 0 and the smallest subnormal 2^-9: ties to 0
                  2.0**-9,       # smallest subnormal: not zero
                  np.nan, np.inf, -np.inf,
                  448.0, 500.0,  # max; saturates to 448
                  256.0,         # bottom of the top binade [256, 448]
                  255.0,         # rounds up to 256 (step 16 below 256)
                  240.0,         # stays 240: below the top binade
                  -300.0,        # rounds to -288 (step 32 above 256)
                  1.0], dtype=np.float32)
    got = ohealth.cast_health(x, 1.0, ofp8.E4M3)
    assert got == {"saturated": 3,   # +inf, -inf, 500
                   "nan": 1, "inf": 2,
                   "zero": 4,        # 0, -0, 1e-10, 2^-10
                   "near_max": 7}    # +-inf, 448, 500, 256, 255, -300


def test_e5m2_hand_case():
    x = np.array([65536.0,   # saturates to 57344
                  57344.0,   # max
                  40000.0,   # rounds to 40960 (step 8192 in [32768, 65536))
                  30000.0,   # rounds to 28672 (step 4096 below 32768): not near max
                  32767.0,   # rounds up to 32768
                  1e-8,      # below half the smallest subnormal 2^-16: zero
                  np.nan, -np.inf], dtype=np.float32)
    got = ohealth.cast_health(x, 1.0, ofp8.E5M2)
    assert got == {"saturated": 2, "nan": 1, "inf": 1, "zero": 1, "near_max": 5}


def test_scale_moves_values_into_the_top_binade():
    x = np.array([1.0, 2.0, 0.5, 2.0**-20], dtype=np.float32)
    # times 256: 256 (top binade), 512 (saturates), 128 (not), 2^-12 (zero in E4M3)
    got = ohealth.cast_health(x, 256.0, ofp8.E4M3)
    assert got == {"saturated": 1, "nan": 0, "inf": 0, "zero": 1, "near_max": 2}


def test_counts_match_brute_force_over_all_bf16_patterns():
    """Over every bf16 bit pattern at scale 1: the counts equal per-element
    classification of each pattern's own cast (NaN and inf by the input bits)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    for fmt in (ofp8.E4M3, ofp8.E5M2):
        got = ohealth.cast_health(x, 1.0, fmt)
        exp_abs = bits & 0x7FFF
        assert got["nan"] == int(np.count_nonzero(exp_abs > 0x7F80))   # 2 * 127 payloads
        assert got["inf"] == 2
        assert got["nan"] == 2 * 127
        codes, _ = ofp8.cast(x, 1.0, fmt)
        mag = codes & 0x7F
        nan_code = 0x7F if fmt == ofp8.E4M3 else 0x7D
        finite = (mag < nan_code) if fmt == ofp8.E4M3 else (mag < 0x7C)
        assert got["zero"] == int(np.count_nonzero(mag == 0))
        assert got["near_max"] == int(np.count_nonzero(finite & (mag >= 0x78)))

"""Host-side health logic (delayed_scaling_gemm_amd/health.py): the spike rule's
boundaries, the alert levels and the override table."""

import json

from delayed_scaling_gemm_amd import health as H


def test_spike_rule_needs_more_than_ten_values_and_is_strict():
    d = H.AmaxSpikeDetector()
    for _ in range(9):
        assert not d.push("x", 1.0)
    assert not d.push("x", 100.0)        # 10th value: not checked yet
    d2 = H.AmaxSpikeDetector()
    for _ in range(10):
        d2.push("x", 1.0)
    assert not d2.push("x", 3.0)         # mean of the previous 9 is 1: 3 is not above 3x
    # the previous nine are now eight 1.0 and the 3.0: mean 11/9, threshold 3.67
    assert not d2.push("x", 3.6)         # 3.6 < 3.67
    # previous nine: seven 1.0, 3.0 and 3.6: mean 13.6/9, threshold 4.53
    assert not d2.push("x", 4.5)
    d3 = H.AmaxSpikeDetector()
    for v in [1.0] * 10 + [3.0, 3.6]:
        d3.push("x", v)
    assert d3.push("x", 4.6)


def test_spike_rule_flags_a_jump():
    d = H.AmaxSpikeDetector()
    for _ in range(10):
        d.push("w", 2.0)
    assert d.push("w", 6.01)             # > 3 x 2.0
    assert not d.push("other", 1e9)      # series are per tensor


def test_levels():
    m = H.HealthMonitor(sat_fraction=1e-3, sat_checks=3)
    c0 = {"saturated": 0, "nan": 0, "inf": 0, "zero": 10, "near_max": 0}
    assert m.check("x", 1.0, c0, 1000).level == H.OK
    assert m.check("x", 1.0, dict(c0, nan=1), 1000).level == H.STOP
    assert m.check("x", 1.0, dict(c0, inf=2), 1000).level == H.STOP
    sat = dict(c0, saturated=5)                      # 5e-3 > 1e-3
    assert m.check("y", 1.0, sat, 1000).level == H.OK
    assert m.check("y", 1.0, sat, 1000).level == H.OK
    v = m.check("y", 1.0, sat, 1000)
    assert v.level == H.DEGRADE and "saturation" in v.reasons[0]
    assert m.check("y", 1.0, c0, 1000).level == H.OK  # the run is broken
    assert m.check("y", 1.0, sat, 1000).level == H.OK


def test_zero_share_jump_is_observed():
    m = H.HealthMonitor()
    c = {"saturated": 0, "nan": 0, "inf": 0, "zero": 10, "near_max": 0}
    for _ in range(9):
        assert m.check("g", 1.0, c, 1000).level == H.OK
    assert m.check("g", 1.0, dict(c, zero=20), 1000).level == H.OK       # 2x is not above 2x
    assert m.check("g", 1.0, dict(c, zero=40), 1000).level == H.OBSERVE


def test_override_table():
    t = H.PrecisionOverrides()
    t.activate("model.layers.17.mlp.down_proj", 18240, "persistent saturation",
               metric="saturated", threshold="1e-3 x 3 checks")
    t.activate("model.layers.17.mlp.down_proj", 19000, "again")       # first activation kept
    assert t.lookup("model.layers.17.mlp.down_proj").activated_at_step == 18240
    assert t.lookup("model.layers.0.mlp.up_proj") is None
    d = json.loads(json.dumps(t.to_dict()))
    t2 = H.PrecisionOverrides.from_dict(d)
    assert t2.to_dict() == t.to_dict()

"""fp8ds_adamw against the oracle (oracle/adamw.py): the fp32 update is one fixed
sequence of correctly rounded fp32 operations on both sides, so w, m and v are
compared bit for bit; the FP8 copies, amax, saturation count and scale
snapshot are bit-exact too (integer results of the same fp32 values)."""

import numpy as np
import pytest
import torch

import delayed_scaling_gemm_amd as dsg
import workloads
from oracle import adamw as oadam
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _assert_same_f32(got, exp, what):
    g, e = _bits(got), _bits(exp)
    bad = g != e
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} differ; e.g. gpu "
                           f"{got.ravel()[bad.ravel()][:3]} oracle {exp.ravel()[bad.ravel()][:3]}")


def _state(rows, cols, step=0):
    w, m, v, gbits = workloads.adamw_state(rows, cols, step)
    g32 = (gbits.astype(np.uint32) << 16).view(np.float32)  # the values the GPU reads
    return w, m, v, gbits, g32


def _dev_grad(gbits, g32, gdtype):
    if gdtype == torch.bfloat16:
        return torch.from_numpy(gbits.view(np.int16)).to(DEV).view(torch.bfloat16), g32
    return torch.from_numpy(np.ascontiguousarray(g32)).to(DEV), g32


def _run(w, m, v, gd, t, fmt, scale, transposed, grad_amax=None, grad_scale=1.0, cast=True,
         flat=False):
    rows, cols = w.shape
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(DEV)
    md = torch.from_numpy(np.ascontiguousarray(m)).to(DEV)
    vd = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    if flat:
        wd, md, vd, gd = wd.reshape(-1), md.reshape(-1), vd.reshape(-1), gd.reshape(-1)
    out = dict(w=wd, m=md, v=vd)
    kw = {}
    if cast:
        out.update(q=torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV),
                   q_t=(torch.full((rows * cols,), 0xCD, dtype=torch.uint8, device=DEV)
                        if transposed else None),
                   scale=torch.tensor([scale], device=DEV),
                   scale_used=torch.zeros(1, device=DEV),
                   amax=torch.full((1,), -1.0, device=DEV),
                   sat=torch.full((1,), 777, dtype=torch.int64, device=DEV))
        kw = dict(fmt=fmt, scale=out["scale"], q=out["q"], q_t=out["q_t"],
                  scale_used=out["scale_used"], amax=out["amax"], sat_count=out["sat"])
    ga = None if grad_amax is None else torch.tensor([grad_amax], device=DEV)
    dsg.fp8ds_adamw(wd, gd, md, vd, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                    HP["weight_decay"], t, grad_scale=grad_scale, grad_amax=ga, **kw)
    torch.cuda.synchronize()
    return {k: (x.cpu().numpy() if x is not None else None) for k, x in out.items()}


def _check(got, exp, rows, cols, scale, transposed, cast=True):
    _assert_same_f32(got["w"].reshape(rows, cols), exp["w"], "w")
    _assert_same_f32(got["m"].reshape(rows, cols), exp["m"], "m")
    _assert_same_f32(got["v"].reshape(rows, cols), exp["v"], "v")
    if not cast:
        return
    np.testing.assert_array_equal(got["q"].reshape(rows, cols), exp["q"])
    if transposed:
        np.testing.assert_array_equal(got["q_t"].reshape(cols, rows), exp["q_t"])
    assert _bits(got["amax"])[0] == _bits(np.float32(exp["amax"]))[0]
    assert int(got["sat"][0]) == exp["sat"]
    assert got["scale_used"][0] == np.float32(scale)


def _consts(t, grad_scale=1.0):
    return oadam.step_constants(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                                HP["weight_decay"], grad_scale, t)


@pytest.mark.parametrize("gdtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("shape,transposed,flat", [
    ((1, 1000), False, True),         # 62 pieces + a ragged tail of 8
    ((1, 16 * 4096 + 5), False, True),
    ((37, 512), False, False),        # 2-D, no transposed copy
    ((256, 384), True, False),        # whole tiles
    ((130, 200), True, False),        # ragged tiles, cols % 16 != 0: element path
    ((272, 144), True, False),        # rows, cols % 16 == 0 with partial tiles
    ((16, 16), True, False),
])
def test_adamw_cast_matches_oracle(gdtype, fmt, shape, transposed, flat):
    rows, cols = shape
    w, m, v, gbits, g32 = _state(rows, cols)
    gd, gval = _dev_grad(gbits, g32, gdtype)
    scale = np.float32(448.0 / 0.04 if fmt == dsg.E4M3 else 57344.0 / 0.04)  # ~5% saturate
    t = 3
    got = _run(w, m, v, gd, t, fmt, scale, transposed, flat=flat)
    exp = oadam.adamw_cast(w, gval, m, v, _consts(t), scale, fmt)
    assert not exp["skipped"] and exp["sat"] > 0
    _check(got, exp, rows, cols, scale, transposed)


def test_adamw_three_steps_in_a_row():
    rows, cols = 256, 256
    w, m, v, _, _ = _state(rows, cols)
    wd = torch.from_numpy(w.copy()).to(DEV)
    md = torch.from_numpy(m.copy()).to(DEV)
    vd = torch.from_numpy(v.copy()).to(DEV)
    q = torch.empty(rows * cols, dtype=torch.uint8, device=DEV)
    qt = torch.empty_like(q)
    s = torch.tensor([2000.0], device=DEV)
    for t in (1, 2, 3):
        _, _, _, gbits, g32 = _state(rows, cols, step=t)
        gd = torch.from_numpy(gbits.view(np.int16)).to(DEV).view(torch.bfloat16)
        dsg.fp8ds_adamw(wd, gd, md, vd, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                        HP["weight_decay"], t, grad_scale=0.5, fmt=dsg.E4M3, scale=s, q=q,
                        q_t=qt)
        exp = oadam.adamw_cast(w, g32, m, v, _consts(t, 0.5), np.float32(2000.0), dsg.E4M3)
        w, m, v = exp["w"], exp["m"], exp["v"]
    torch.cuda.synchronize()
    _assert_same_f32(wd.cpu().numpy(), w, "w")
    _assert_same_f32(md.cpu().numpy(), m, "m")
    _assert_same_f32(vd.cpu().numpy(), v, "v")
    np.testing.assert_array_equal(q.cpu().numpy().reshape(rows, cols), exp["q"])
    np.testing.assert_array_equal(qt.cpu().numpy().reshape(cols, rows), exp["q_t"])


@pytest.mark.parametrize("bad", [float("inf"), float("nan")])
@pytest.mark.parametrize("transposed", [False, True])
def test_nonfinite_grad_amax_skips_the_update(bad, transposed):
    rows, cols = 128, 256
    w, m, v, gbits, g32 = _state(rows, cols)
    g32 = g32.copy()
    g32[5, 7] = bad  # the gradient the amax describes
    gd = torch.from_numpy(g32).to(DEV)
    got = _run(w, m, v, gd, 2, dsg.E4M3, np.float32(1000.0), transposed, grad_amax=bad)
    exp = oadam.adamw_cast(w, g32, m, v, _consts(2), np.float32(1000.0), dsg.E4M3)
    assert exp["skipped"]
    _check(got, exp, rows, cols, np.float32(1000.0), transposed)


def test_finite_grad_amax_updates():
    rows, cols = 64, 128
    w, m, v, gbits, g32 = _state(rows, cols)
    gd = torch.from_numpy(gbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    got = _run(w, m, v, gd, 1, dsg.E4M3, np.float32(1000.0), True,
               grad_amax=float(np.abs(g32).max()))
    exp = oadam.adamw_cast(w, g32, m, v, _consts(1), np.float32(1000.0), dsg.E4M3)
    _check(got, exp, rows, cols, np.float32(1000.0), True)


@pytest.mark.parametrize("shape", [(1, 4099), (64, 80)])
def test_update_without_cast(shape):
    rows, cols = shape
    w, m, v, gbits, g32 = _state(rows, cols)
    gd = torch.from_numpy(gbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    got = _run(w, m, v, gd, 5, dsg.E4M3, np.float32(1.0), False, cast=False)
    w1, m1, v1 = oadam.adamw_update(w, g32, m, v, _consts(5))
    _check(got, dict(w=w1, m=m1, v=v1), rows, cols, None, False, cast=False)


def test_empty_writes_scalar_outputs():
    e = torch.empty(0, device=DEV)
    q = torch.empty(0, dtype=torch.uint8, device=DEV)
    s = torch.tensor([3.0], device=DEV)
    su = torch.zeros(1, device=DEV)
    am = torch.full((1,), 5.0, device=DEV)
    sat = torch.full((1,), 9, dtype=torch.int64, device=DEV)
    dsg.fp8ds_adamw(e.reshape(0, 16), e, e, e, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, fmt=dsg.E4M3,
                    scale=s, q=q, q_t=q, scale_used=su, amax=am, sat_count=sat)
    torch.cuda.synchronize()
    assert su.item() == 3.0 and am.item() == 0.0 and sat.item() == 0


def test_full_size_weight_4096():
    """The 4096 x 4096 weight of the benchmarked Linear, BF16 dW, E4M3 with q and
    q_t: the launch configuration the benchmark times, compared in full."""
    rows = cols = 4096
    w, m, v, gbits, g32 = _state(rows, cols)
    gd = torch.from_numpy(gbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    scale = np.float32(448.0 / 0.1)
    got = _run(w, m, v, gd, 10, dsg.E4M3, scale, True)
    exp = oadam.adamw_cast(w, g32, m, v, _consts(10), scale, dsg.E4M3)
    _check(got, exp, rows, cols, scale, True)

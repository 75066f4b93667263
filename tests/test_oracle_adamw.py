"""Pins of the AdamW oracle (oracle/adamw.py) against things other than itself:
torch.optim.AdamW in float64 (a different implementation and formulation),
closed forms of the first step, of zero and of constant gradients, an exact
decimal evaluation of one step, and the skip rule."""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import adamw as oadam
from oracle import fp8 as ofp8

f32 = np.float32
ULP = 2.0 ** -23


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(f32)


def test_step_constants_dyadic():
    # beta1 = 1/2: 1 - beta1^t = 1 - 2^-t exactly; beta2 = 3/4 at t = 1: 1/sqrt(1/4) = 2
    for t in (1, 2, 5, 30):
        c = oadam.step_constants(0.25, 0.5, 0.75, 1e-8, 0.5, 1.0, t)
        assert c.step_size == f32(0.25 / (1.0 - 2.0 ** -t))
        assert c.decay == f32(0.875)
        assert c.one_minus_beta1 == f32(0.5) and c.one_minus_beta2 == f32(0.25)
    assert oadam.step_constants(0.25, 0.5, 0.75, 0, 0, 1, 1).inv_sqrt_bc2 == f32(2.0)
    # late steps: the corrections vanish
    c = oadam.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 10 ** 6)
    assert c.step_size == f32(1e-3) and c.inv_sqrt_bc2 == f32(1.0)
    with pytest.raises(ValueError):
        oadam.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 0)


def test_first_step_is_lr_times_sign():
    # At t = 1 the bias-corrected moments are g and g^2, so (eps = 0) the step is
    # lr * sign(g).  Dyadic settings make every fp32 operation exact.
    g = np.array([1.0, -2.0, 3.0, -0.5, 1.5, -12.0, 2.0 ** -20], dtype=f32)
    w = np.array([2.0, 2.0, -1.0, 0.5, 0.0, 4.0, -3.0], dtype=f32)
    c = oadam.step_constants(0.25, 0.5, 0.75, 0.0, 0.5, 1.0, 1)
    w1, m1, v1 = oadam.adamw_update(w, g, np.zeros_like(w), np.zeros_like(w), c)
    np.testing.assert_array_equal(w1, w * f32(0.875) - f32(0.25) * np.sign(g))
    np.testing.assert_array_equal(m1, 0.5 * g)
    np.testing.assert_array_equal(v1, 0.25 * g * g)


def test_zero_gradient_is_pure_decay():
    w = _rand(64, 1)
    c = oadam.step_constants(1e-2, 0.9, 0.999, 1e-8, 0.1, 1.0, 1)
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    ref = w.astype(np.float64)
    for t in range(1, 11):
        c = oadam.step_constants(1e-2, 0.9, 0.999, 1e-8, 0.1, 1.0, t)
        w, m, v = oadam.adamw_update(w, np.zeros_like(w), m, v, c)
        ref = ref * (1.0 - 1e-2 * float(f32(0.1)))
    assert not m.any() and not v.any()
    # one rounding of the decay constant and one per step
    np.testing.assert_allclose(w, ref, rtol=12 * ULP, atol=0)


def test_constant_gradient_moves_linearly():
    # m_hat = g and v_hat = g^2 at every step in exact arithmetic, so without
    # weight decay w_t = w_0 - t * lr * g / (|g| + eps)
    g = np.array([0.3, -1e-3, 5.0, -7.25], dtype=f32)
    w0 = np.array([1.0, -2.0, 0.5, 3.0], dtype=f32)
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    lr, eps, T = 1e-3, 1e-8, 50
    for t in range(1, T + 1):
        c = oadam.step_constants(lr, 0.9, 0.999, eps, 0.0, 1.0, t)
        w, m, v = oadam.adamw_update(w, g, m, v, c)
    g64 = g.astype(np.float64)
    ref = w0.astype(np.float64) - T * float(f32(lr)) * g64 / (np.abs(g64) + float(f32(eps)))
    np.testing.assert_allclose(w, ref, rtol=0, atol=T * (4 * ULP * 3.0 + 1e-5 * lr))


def _exact_step(w, g, m, v, lr, b1, b2, eps, wd, gs, t):
    """One step in 50-digit decimal arithmetic from the fp32 inputs."""
    getcontext().prec = 50
    D = lambda x: Decimal(float(x))  # noqa: E731  (fp32 -> exact decimal)
    lr, b1, b2, eps, wd, gs = (D(f32(x)) for x in (lr, b1, b2, eps, wd, gs))
    gg = D(g) * gs
    m1 = b1 * D(m) + (1 - b1) * gg
    v1 = b2 * D(v) + (1 - b2) * gg * gg
    bc1 = 1 - b1 ** t
    bc2 = 1 - b2 ** t
    den = (v1 / bc2).sqrt() + eps
    w1 = D(w) * (1 - lr * wd) - lr * (m1 / bc1) / den
    return float(w1), float(m1), float(v1), float(lr * (m1 / bc1) / den)


def test_one_step_against_exact_decimal():
    rng = np.random.default_rng(7)
    n = 200
    w = rng.standard_normal(n).astype(f32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1, n)).astype(f32)
    m = (rng.standard_normal(n) * 1e-2).astype(f32)
    v = (rng.uniform(0, 1e-3, n)).astype(f32)
    hp = (3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 1024, 7)
    c = oadam.step_constants(*hp[:6], hp[6])
    w1, m1, v1 = oadam.adamw_update(w, g, m, v, c)
    for i in range(n):
        ew, em, ev, eu = _exact_step(w[i], g[i], m[i], v[i], *hp)
        # m: 3 roundings, v: 4 roundings of terms of the same sign as the result
        assert abs(float(m1[i]) - em) <= 3 * ULP * (abs(0.9 * float(m[i])) + abs(em) + 1e-30)
        assert abs(float(v1[i]) - ev) <= 4 * ULP * abs(ev) + 1e-45
        # w: two roundings on w, and the update term within ~12 roundings
        assert abs(float(w1[i]) - ew) <= 2 * ULP * abs(ew) + 12 * ULP * abs(eu) + 1e-45


@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_against_torch_adamw_float64(wd):
    rng = np.random.default_rng(11)
    n, T = 300, 25
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    w0 = rng.standard_normal(n).astype(f32)
    grads = [(rng.standard_normal(n) * 0.1).astype(f32) for _ in range(T)]
    p = torch.nn.Parameter(torch.tensor(w0.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=float(f32(lr)), betas=(float(f32(b1)), float(f32(b2))),
                            eps=float(f32(eps)), weight_decay=float(f32(wd)), foreach=False)
    w, m, v = w0, np.zeros(n, f32), np.zeros(n, f32)
    for t in range(1, T + 1):
        c = oadam.step_constants(lr, b1, b2, eps, wd, 1.0, t)
        w, m, v = oadam.adamw_update(w, grads[t - 1], m, v, c)
        p.grad = torch.tensor(grads[t - 1].astype(np.float64))
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(w, p.detach().numpy(), rtol=0, atol=T * (4 * ULP * 4 + 1e-5 * lr))
    # m sums terms of both signs: its error scales with the largest gradient
    gmax = max(float(np.max(np.abs(g))) for g in grads)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=0, atol=T * 4 * ULP * gmax)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=T * 4 * ULP, atol=1e-15)


def test_grad_scale_unscales():
    g = _rand(100, 3)
    w, m, v = _rand(100, 4), _rand(100, 5, 1e-2), np.abs(_rand(100, 6, 1e-3))
    c1 = oadam.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 3)
    c2 = oadam.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0 / 1024, 3)
    a = oadam.adamw_update(w, g, m, v, c1)
    b = oadam.adamw_update(w, g * f32(1024), m, v, c2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_nonfinite_gradient_skips_the_step(bad):
    w = _rand((8, 16), 8)
    g = _rand((8, 16), 9)
    g[3, 5] = bad
    m, v = _rand((8, 16), 10, 1e-2), np.abs(_rand((8, 16), 11, 1e-3))
    c = oadam.step_constants(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 2)
    out = oadam.adamw_cast(w, g, m, v, c, f32(64.0), ofp8.E4M3)
    assert out["skipped"]
    np.testing.assert_array_equal(out["w"], w)
    np.testing.assert_array_equal(out["m"], m)
    np.testing.assert_array_equal(out["v"], v)
    np.testing.assert_array_equal(out["q"], ofp8.cast(w, f32(64.0), ofp8.E4M3)[0].reshape(8, 16))


def test_fused_cast_is_the_next_forward_cast():
    w = _rand((24, 40), 12)
    g = _rand((24, 40), 13, 1e-2)
    m, v = np.zeros_like(w), np.zeros_like(w)
    c = oadam.step_constants(1e-2, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    out = oadam.adamw_cast(w, g, m, v, c, f32(300.0), ofp8.E4M3)
    assert not out["skipped"]
    q, sat = ofp8.cast(out["w"], f32(300.0), ofp8.E4M3)
    np.testing.assert_array_equal(out["q"], q.reshape(24, 40))
    np.testing.assert_array_equal(out["q_t"], q.reshape(24, 40).T)
    assert out["sat"] == sat > 0  # |w| > 448/300 exists among 960 normal draws
    assert out["amax"] == np.max(np.abs(out["w"]))

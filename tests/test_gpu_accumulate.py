"""GPU checks of the accumulating entry points (fp8ds_cast_acc, fp8ds_gemm_acc,
fp8ds_scale_update_clear): from zeroed accumulators they give exactly what the
resetting calls give; over two calls the amax is the maximum and the counts the
sum; the scale update's clear zeroes exactly the given bytes.  Parity against the
oracle follows from the identity with the resetting calls (which the other GPU
tests compare with the oracle) and is also checked directly on the casts."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from oracle import amax as oamax  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from tests.parity import f32_bits  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    x.ravel()[rng.choice(x.size, 7, replace=False)] = 3.0e4  # saturate E4M3 at s = 1/8
    return x


@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("shape", [(256, 384), (129, 200)])
def test_cast_acc_equals_cast_and_accumulates(fmt, transpose, shape):
    rng = np.random.default_rng(shape[0] + 3 * fmt + 7 * transpose)
    x1, x2 = _rand(rng, shape, 2.0), _rand(rng, shape, 5.0)
    s = torch.tensor([0.125], device=DEV)
    n = x1.size
    outs = {}
    for name, fn in (("plain", dsg.fp8ds_cast), ("acc", dsg.fp8ds_cast_acc)):
        q = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)
        qt = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV) if transpose else None
        su = torch.full((1,), -1.0, device=DEV)
        am = torch.zeros(1, device=DEV)
        sat = torch.zeros(1, dtype=torch.int64, device=DEV)
        fn(torch.from_numpy(x1).to(DEV), fmt, s, q, qt, su, am, sat)
        torch.cuda.synchronize()
        outs[name] = (q.cpu().numpy(), None if qt is None else qt.cpu().numpy(), su.item(),
                      f32_bits(am.item()), sat.item())
        if name == "acc":  # a second call combines into the same accumulators
            fn(torch.from_numpy(x2).to(DEV), fmt, s, q, qt, su, am, sat)
            torch.cuda.synchronize()
            a12 = max(oamax.amax(x1), oamax.amax(x2))
            assert f32_bits(am.item()) == f32_bits(a12)
            assert sat.item() == (ofp8.saturation_count(x1, np.float32(0.125), fmt) +
                                  ofp8.saturation_count(x2, np.float32(0.125), fmt))
            codes, _ = ofp8.cast(x2.ravel(), np.float32(0.125), fmt)
            assert np.array_equal(q.cpu().numpy(), codes)
    p, a = outs["plain"], outs["acc"]
    assert np.array_equal(p[0], a[0]) and (p[1] is None or np.array_equal(p[1], a[1]))
    assert p[2:] == a[2:]
    codes, sat1 = ofp8.cast(x1.ravel(), np.float32(0.125), fmt)
    assert np.array_equal(a[0], codes) and a[4] == sat1 and a[2] == 0.125
    assert a[3] == f32_bits(oamax.amax(x1))


def test_cast_acc_empty_writes_the_snapshot():
    x = torch.zeros(0, dtype=torch.float32, device=DEV)
    q = torch.zeros(16, dtype=torch.uint8, device=DEV)
    s = torch.tensor([3.5], device=DEV)
    su = torch.zeros(1, device=DEV)
    am = torch.full((1,), 2.0, device=DEV)
    dsg.fp8ds_cast_acc(x, dsg.E4M3, s, q, None, su, am)
    torch.cuda.synchronize()
    assert su.item() == 3.5 and am.item() == 2.0  # nothing combined into amax


@pytest.mark.parametrize("mma", [dsg.MMA_EXACT, dsg.MMA_FP8])
def test_gemm_acc_equals_gemm_and_accumulates(mma):
    rng = np.random.default_rng(5 + mma)
    M, N, K = 300, 264, 512
    a = torch.from_numpy(rng.integers(0, 0x70, (M, K), dtype=np.uint8)).to(DEV)
    b = torch.from_numpy(rng.integers(0, 0x70, (N, K), dtype=np.uint8)).to(DEV)
    one = torch.ones(1, device=DEV)
    two = torch.tensor([2.0], device=DEV)
    c1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    c2 = torch.empty_like(c1)
    am1 = torch.full((1,), 7.0, device=DEV)
    am2 = torch.zeros(1, device=DEV)
    dsg.fp8ds_gemm(0, 1, M, N, K, a, 0, K, one, b, 0, K, one, c1, N, am1, mma=mma)
    dsg.fp8ds_gemm_acc(0, 1, M, N, K, a, 0, K, one, b, 0, K, one, c2, N, am2, mma=mma)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    assert am1.item() == am2.item() == c1.float().abs().max().item()
    # a second product dequantized by 1/2: the accumulated amax stays the first one's
    dsg.fp8ds_gemm_acc(0, 1, M, N, K, a, 0, K, one, b, 0, K, two, c2, N, am2, mma=mma)
    torch.cuda.synchronize()
    assert am2.item() == am1.item() and c2.float().abs().max().item() == am1.item() / 2


def test_scale_update_clear_zeroes_exactly_the_given_bytes():
    n, L = 3, 16
    hist = torch.rand(n, L, device=DEV)
    cur = torch.tensor([0, 5, 15], dtype=torch.int32, device=DEV)
    amax = torch.tensor([3.0, 100.0, 0.0], device=DEV)
    s1, s2 = torch.ones(n, device=DEV), torch.ones(n, device=DEV)
    buf = torch.full((64,), -1, dtype=torch.int32, device=DEV)
    h1, c1 = hist.clone(), cur.clone()
    fmts = [dsg.E4M3, dsg.E4M3, dsg.E5M2]
    dsg.fp8ds_scale_update(h1, c1, amax, fmts, dsg.ALGO_MAX, 0, s1)
    dsg.fp8ds_scale_update_clear(hist, cur, amax, fmts, dsg.ALGO_MAX, 0, s2, buf[8:40])
    torch.cuda.synchronize()
    assert torch.equal(h1, hist) and torch.equal(c1, cur) and torch.equal(s1, s2)
    b = buf.cpu().numpy()
    assert (b[8:40] == 0).all() and (b[:8] == -1).all() and (b[40:] == -1).all()

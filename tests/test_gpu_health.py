"""Quantization-health counts of fp8ds_cast_health against the oracle
(oracle/health.py), bit-exact, with the codes themselves compared too."""

import numpy as np
import pytest
import torch

import delayed_scaling_gemm_amd as dsg
import workloads
from oracle import fp8 as ofp8
from oracle import health as ohealth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def special_input(rng, n, scale_hint):
    """Normal values of spread `scale_hint` with NaN, +-inf, zeros, tiny values and
    values around the formats' top binades sprinkled in."""
    x = rng.normal(0.0, scale_hint, n).astype(np.float32)
    k = max(1, n // 50)
    for vals in ([np.nan, -np.nan], [np.inf, -np.inf], [0.0, -0.0], [1e-12, -3e-9],
                 [250.0, 300.0, 448.0, 500.0, -1000.0], [30000.0, 40000.0, 60000.0, -1e6]):
        pos = rng.choice(n, k, replace=False)
        x[pos] = rng.choice(np.array(vals, np.float32), k)
    return x


def to_dev(x32, dtype):
    if dtype == torch.bfloat16:
        bits = workloads.to_bf16_bits(x32)
        xw = (bits.astype(np.uint32) << 16).view(np.float32)  # the values the GPU sees
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16), xw
    return torch.from_numpy(x32).to(DEV), x32


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("shape,transposed", [((1, 1000), False), ((1, 16 * 4096 + 7), False),
                                              ((37, 512), False), ((256, 384), True),
                                              ((130, 200), True), ((16, 16), True)])
def test_health_counts_match_oracle(dtype, fmt, shape, transposed):
    rows, cols = shape
    rng = np.random.default_rng(rows * 1000 + cols + 7 * fmt + (dtype == torch.float32))
    scale_hint = 30.0 if fmt == dsg.E4M3 else 3000.0
    x32 = special_input(rng, rows * cols, scale_hint).reshape(rows, cols)
    xd, xw = to_dev(x32, dtype)
    if rows == 1:
        xd = xd.reshape(-1)
    scale = np.float32(1.5 if fmt == dsg.E4M3 else 2.0)
    s = torch.tensor([scale], device=DEV)
    q = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    qt = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV) if transposed else None
    counts = torch.full((dsg.HEALTH_COUNTS,), 12345, dtype=torch.int64, device=DEV)
    amax = torch.zeros(1, device=DEV)
    dsg.fp8ds_cast_health(xd if rows > 1 else xd, fmt, s, q, counts, q_t=qt, amax=amax)
    torch.cuda.synchronize()
    exp = ohealth.cast_health(xw.ravel(), scale, fmt)
    got = dict(zip(dsg.HEALTH_NAMES, counts.cpu().numpy().tolist()))
    assert got == exp
    codes, _ = ofp8.cast(xw.ravel(), scale, fmt)
    assert np.array_equal(q.cpu().numpy(), codes)
    if transposed:
        assert np.array_equal(qt.cpu().numpy().reshape(cols, rows), codes.reshape(rows, cols).T)


def test_health_counts_are_reset_each_call():
    x = torch.tensor([np.nan, 1.0, 0.0, 448.0] * 8, dtype=torch.float32, device=DEV)
    q = torch.zeros(32, dtype=torch.uint8, device=DEV)
    s = torch.ones(1, device=DEV)
    counts = torch.zeros(dsg.HEALTH_COUNTS, dtype=torch.int64, device=DEV)
    for _ in range(3):
        dsg.fp8ds_cast_health(x, dsg.E4M3, s, q, counts)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().tolist() == [0, 8, 0, 8, 8]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("scale", [1.0, -1.5, 2.0**-6])
def test_health_counts_at_the_group_bounds(dtype, fmt, scale):
    """Groups of 16 built around the values where the count changes: ties to
    zero, the smallest subnormal, the binade below the top, values that round
    into the top binade; negative and small scales included."""
    top = 256.0 if fmt == dsg.E4M3 else 32768.0
    sub = 2.0**-9 if fmt == dsg.E4M3 else 2.0**-16
    edge = np.array([sub / 2, sub, sub * 0.75, sub * 1.25, top / 2, top * 0.97, top * 0.9,
                     top - 1, top, 0.0, -sub / 2, 1.0, top * 1.75, top / 2 - 1, 3.0, -top],
                    np.float32)
    rng = np.random.default_rng(int(abs(scale) * 1e6) + fmt)
    groups = [np.abs(rng.normal(1.0, 0.1, 16)).astype(np.float32) for _ in range(30)]
    for i in range(30):
        groups[i][rng.integers(0, 16)] = edge[i % len(edge)] / np.float32(abs(scale))
    x32 = np.concatenate(groups)
    xd, xw = to_dev(x32, dtype)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    q = torch.zeros(x32.size, dtype=torch.uint8, device=DEV)
    counts = torch.zeros(dsg.HEALTH_COUNTS, dtype=torch.int64, device=DEV)
    dsg.fp8ds_cast_health(xd, fmt, s, q, counts)
    torch.cuda.synchronize()
    exp = ohealth.cast_health(xw, np.float32(scale), fmt)
    assert dict(zip(dsg.HEALTH_NAMES, counts.cpu().numpy().tolist())) == exp
    codes, _ = ofp8.cast(xw, np.float32(scale), fmt)
    assert np.array_equal(q.cpu().numpy(), codes)

"""A seeded sweep of random shapes against the oracle: casts of random sizes,
dtypes, formats and scales (bytes, amax and saturation count bit-exact), and
GEMMs of random shapes, layouts, formats and scales on the exact datapath
(accumulator bound on FP32 output, +1 BF16 ulp on BF16 output).  Shapes are
drawn to land on and off every tile, piece and stage boundary."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from oracle import amax as oamax  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from tests.parity import bf16_bits, check_acc, check_bf16_out, f32_bits  # noqa: E402
from tests.test_gpu_gemm import finite_codes, run_gemm, stored_shape  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("case", range(24))
def test_random_cast(case):
    rng = np.random.default_rng(10_000 + case)
    n = int(rng.choice([rng.integers(1, 200), rng.integers(200, 70_000),
                        rng.integers(70_000, 3_000_000)]))
    bf16 = bool(rng.integers(0, 2))
    fmt = int(rng.integers(0, 2))
    scale = np.float32(2.0 ** rng.uniform(-12, 12))
    x = (rng.standard_normal(n) * 2.0 ** rng.uniform(-6, 6)).astype(np.float32)
    if n > 10:
        x[rng.choice(n, max(1, n // 1000), replace=False)] *= np.float32(1e4)  # saturating outliers
    print(f"[random cast] case={case} n={n} bf16={bf16} fmt={fmt} scale={scale}", flush=True)
    if bf16:
        xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
        xw = xt.float().cpu().numpy()  # the exact bf16 values (torch rounds to nearest even)
    else:
        xt = torch.from_numpy(x).to(DEV)
        xw = x
    q = torch.empty(n, dtype=torch.uint8, device=DEV)
    s = torch.tensor([scale], device=DEV)
    am = torch.zeros(1, device=DEV)
    sat = torch.zeros(1, dtype=torch.int64, device=DEV)
    dsg.fp8ds_cast(xt, fmt, s, q, None, None, am, sat)
    torch.cuda.synchronize()
    codes, osat = ofp8.cast(xw, scale, fmt)
    np.testing.assert_array_equal(q.cpu().numpy(), codes)
    assert int(sat.item()) == osat
    assert f32_bits(am.item()) == f32_bits(oamax.amax(xw))


LAYOUTS = [(dsg.OP_N, dsg.OP_T), (dsg.OP_N, dsg.OP_N), (dsg.OP_T, dsg.OP_N)]


@pytest.mark.parametrize("case", range(24))
def test_random_gemm(case):
    rng = np.random.default_rng(20_000 + case)
    M, N = (int(v) for v in rng.integers(1, 700, 2))
    K = int(rng.choice([rng.integers(1, 300), rng.integers(300, 1500)]))
    opa, opb = LAYOUTS[case % 3]
    fa, fb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    sa = float(np.float32(2.0 ** rng.uniform(-8, 8)))
    sb = float(np.float32(2.0 ** rng.uniform(-8, 8)))
    print(f"[random gemm] case={case} M={M} N={N} K={K} ops={opa}{opb} fmts={fa}{fb}", flush=True)
    a_st = finite_codes(rng, stored_shape(opa, M, K), fa)
    b_st = finite_codes(rng, stored_shape(opb, K, N), fb)
    acc, sum_abs = ogemm.gemm_exact(a_st, fa, opa, b_st, fb, opb)
    C32, _ = run_gemm(opa, opb, a_st, fa, b_st, fb, M, N, K)
    check_acc(C32.cpu().numpy(), acc, sum_abs, f"case {case} fp32")
    C16, am = run_gemm(opa, opb, a_st, fa, b_st, fb, M, N, K, sa=sa, sb=sb, out=torch.bfloat16)
    y = bf16_bits(C16)
    d = 1.0 / float(ogemm.dequant_scale(sa, sb))
    check_bf16_out(y, acc, sum_abs, ogemm.dequant_to_bf16(acc, sa, sb), d, f"case {case} bf16")
    assert am == f32_bits(ogemm.output_amax(y))

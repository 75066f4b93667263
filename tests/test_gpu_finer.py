"""GPU parity of finer-grained scaling against the oracle (oracle/finer.py):
per-row and per-tensor current scaling (codes, scales, inverse scales and amax
bit-exact), and the GEMM with per-row / per-column scales (accumulator bound
plus one BF16 ulp, as the per-tensor GEMM; bit-identical to fp8ds_gemm where the
scales are powers of two)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import finer as ofin  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from tests.parity import ACC_REL, bf16_bits, bf16_ulp  # noqa: E402
from tests.test_gpu_gemm import finite_codes, pad16, stored_shape, to_dev_padded  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _input(rows, cols, seed, bf16, specials=False):
    x = workloads.normal(rows * cols, seed, 3.0).reshape(rows, cols)
    # rows of very different ranges: per-row scales differ by orders of magnitude
    x *= np.float32(10.0) ** np.linspace(-3, 3, rows, dtype=np.float32)[:, None]
    if specials and rows >= 4 and cols >= 4:
        x[1] = 0.0                    # all-zero row: scale 1.0
        x[2, cols // 2] = np.inf      # infinite amax: scale 1.0, saturates
        x[3, 1] = np.nan              # NaN amax: scale 1.0, NaN code
    if bf16:
        bits = workloads.to_bf16_bits(x)
        return (torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16),
                obf16.widen(bits).reshape(rows, cols))
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV), x


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("shape", [(1, 4096), (37, 4096), (16, 8200), (9, 12000), (5, 33),
                                   (64, 24), (3, 0)])
@pytest.mark.parametrize("margin", [0, 2])
def test_rowwise_cast_matches_oracle(bf16, fmt, shape, margin):
    rows, cols = shape
    xd, xw = _input(rows, cols, 1000 * rows + cols, bf16, specials=True)
    q = torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    s = torch.full((rows,), -1.0, device=DEV)
    si = torch.full((rows,), -1.0, device=DEV)
    am = torch.full((rows,), -1.0, device=DEV)
    dsg.fp8ds_cast_rowwise(xd, fmt, margin, q, s, si, am)
    torch.cuda.synchronize()
    codes, scale, sinv, amax = ofin.rowwise_cast(xw, fmt, margin)
    np.testing.assert_array_equal(q.cpu().numpy().reshape(rows, cols), codes)
    np.testing.assert_array_equal(_bits(s.cpu().numpy()), _bits(scale))
    np.testing.assert_array_equal(_bits(si.cpu().numpy()), _bits(sinv))
    np.testing.assert_array_equal(_bits(am.cpu().numpy()), _bits(amax))


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape,transposed", [((256, 384), True), ((1, 10000), False),
                                              ((130, 200), True)])
@pytest.mark.parametrize("margin", [0, -1])
def test_current_cast_matches_oracle(bf16, shape, transposed, margin):
    rows, cols = shape
    xd, xw = _input(rows, cols, rows + 7 * cols, bf16)
    q = torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    qt = torch.full((rows * cols,), 0xCD, dtype=torch.uint8, device=DEV) if transposed else None
    s, si, am = (torch.full((1,), -1.0, device=DEV) for _ in range(3))
    sat = torch.full((1,), 99, dtype=torch.int64, device=DEV)
    dsg.fp8ds_cast_current(xd if rows > 1 else xd.reshape(-1), dsg.E4M3, margin, q, s, am, qt, si,
                           sat)
    torch.cuda.synchronize()
    codes, scale, amax, nsat = ofin.current_cast(xw, dsg.E4M3, margin)
    np.testing.assert_array_equal(q.cpu().numpy().reshape(rows, cols), codes)
    if transposed:
        np.testing.assert_array_equal(qt.cpu().numpy().reshape(cols, rows), codes.T)
    assert _bits(s.cpu().numpy())[0] == _bits(scale)[0]
    assert _bits(si.cpu().numpy())[0] == _bits(ofin.inv_scale(scale))[0]
    assert _bits(am.cpu().numpy())[0] == _bits(amax)[0]
    assert int(sat.item()) == nsat  # the row maximum may round one ulp above FP8_MAX


def _run_rowcol(opa, opb, a_st, fa, b_st, fb, M, N, K, ia, ib, out=torch.bfloat16):
    A, lda = to_dev_padded(a_st)
    B, ldb = to_dev_padded(b_st)
    ldc = pad16(N)
    C = torch.full((M, ldc), float("nan"), dtype=out, device=DEV)
    ia_d = torch.from_numpy(ia).to(DEV)
    ib_d = torch.from_numpy(ib).to(DEV)
    am = torch.full((1,), -1.0, device=DEV)
    dsg.fp8ds_gemm_rowcol(opa, opb, M, N, K, A, fa, lda, ia_d, B, fb, ldb, ib_d, C, ldc, am)
    torch.cuda.synchronize()
    return C[:, :N].contiguous(), float(am.item())


def _scales(rng, n):
    """Scales spanning several binades, not powers of two, and the inverse scales
    fl32(1 / s) a cast hands to the GEMM."""
    s = (rng.uniform(0.5, 2.0, n) * 2.0 ** rng.integers(-8, 9, n)).astype(np.float32)
    return s, np.array([ofin.inv_scale(v) for v in s], np.float32)


@pytest.mark.parametrize("opa,opb", [(dsg.OP_N, dsg.OP_T), (dsg.OP_N, dsg.OP_N),
                                     (dsg.OP_T, dsg.OP_N)])
@pytest.mark.parametrize("fa,fb", [(dsg.E4M3, dsg.E4M3), (dsg.E5M2, dsg.E4M3)])
@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (100, 70, 200), (520, 264, 128)])
def test_rowcol_gemm_matches_oracle(opa, opb, fa, fb, M, N, K):
    rng = np.random.default_rng(M + N + K + 10 * opa + opb)
    a_st = finite_codes(rng, stored_shape(opa, M, K), fa)
    b_st = finite_codes(rng, stored_shape(opb, K, N), fb)
    (sa, ia), (sb, ib) = _scales(rng, M), _scales(rng, N)
    y, amax = _run_rowcol(opa, opb, a_st, fa, b_st, fb, M, N, K, ia, ib)
    acc, sum_abs = ogemm.gemm_exact(a_st, fa, opa, b_st, fb, opb)
    ref = ofin.dequant_vec_to_bf16(acc, sa, sb)
    yg = obf16.widen(bf16_bits(y)).astype(np.float64)
    yr = obf16.widen(ref).astype(np.float64)
    fac = ia.astype(np.float64)[:, None] * ib.astype(np.float64)[None, :]
    bound = bf16_ulp(yr) + ACC_REL * fac * sum_abs
    bad = np.abs(yg - yr) > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside the bound"
    assert amax == np.abs(yg).max()


@pytest.mark.parametrize("M,N,K", [(512, 512, 256), (100, 70, 200)])
def test_rowcol_fp32_output(M, N, K):
    rng = np.random.default_rng(M * N)
    a_st = finite_codes(rng, (M, K), dsg.E4M3)
    b_st = finite_codes(rng, (N, K), dsg.E4M3)
    (_, ia), (_, ib) = _scales(rng, M), _scales(rng, N)
    y, _ = _run_rowcol(dsg.OP_N, dsg.OP_T, a_st, dsg.E4M3, b_st, dsg.E4M3, M, N, K, ia, ib,
                       out=torch.float32)
    acc, sum_abs = ogemm.gemm_exact(a_st, dsg.E4M3, dsg.OP_N, b_st, dsg.E4M3, dsg.OP_T)
    fac = ia.astype(np.float64)[:, None] * ib.astype(np.float64)[None, :]
    err = np.abs(y.cpu().numpy().astype(np.float64) - acc * fac)
    # accumulator bound plus the two fp32 roundings of the two products
    assert (err <= ACC_REL * fac * sum_abs + 2 ** -23 * np.abs(acc * fac)).all()


def test_power_of_two_scales_equal_the_per_tensor_gemm():
    rng = np.random.default_rng(4)
    M, N, K = 512, 384, 1024
    a_st = finite_codes(rng, (M, K), dsg.E4M3)
    b_st = finite_codes(rng, (N, K), dsg.E4M3)
    ia = np.full(M, 2.0 ** -6, np.float32)
    ib = np.full(N, 2.0 ** 3, np.float32)
    y, am = _run_rowcol(dsg.OP_N, dsg.OP_T, a_st, dsg.E4M3, b_st, dsg.E4M3, M, N, K, ia, ib)
    A, lda = to_dev_padded(a_st)
    B, ldb = to_dev_padded(b_st)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    am2 = torch.zeros(1, device=DEV)
    dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, M, N, K, A, dsg.E4M3, lda,
                   torch.tensor([64.0], device=DEV), B, dsg.E4M3, ldb,
                   torch.tensor([0.125], device=DEV), C, N, am2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), C.view(torch.int16))
    assert am == am2.item()


def test_per_token_per_channel_forward_full_size_sampled():
    """The 4096-hidden forward at M = 16384 with per-token X and per-channel W:
    rowwise casts of X and W^T, then the scaled NT GEMM, in the launch
    configuration of the benchmark; 48 sampled rows checked against the
    oracle's exact products."""
    M, K, N = 16384, 4096, 4096
    xb, wb, _ = workloads.fwd_bwd_4096()
    x = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    wt = torch.from_numpy(np.ascontiguousarray(wb.T).view(np.int16)).to(DEV).view(torch.bfloat16)
    xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    wq = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    sx, six = torch.empty(M, device=DEV), torch.empty(M, device=DEV)
    sw, siw = torch.empty(N, device=DEV), torch.empty(N, device=DEV)
    dsg.fp8ds_cast_rowwise(x, dsg.E4M3, 0, xq, sx, six)
    dsg.fp8ds_cast_rowwise(wt, dsg.E4M3, 0, wq, sw, siw)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dsg.fp8ds_gemm_rowcol(dsg.OP_N, dsg.OP_T, M, N, K, xq, dsg.E4M3, K, six, wq, dsg.E4M3, K, siw,
                          y, N)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 48, replace=False)
    xw = obf16.widen(xb[rows]).reshape(48, K)
    codes_x, s_x, sinv_x, _ = ofin.rowwise_cast(xw, dsg.E4M3, 0)
    codes_w, s_w, sinv_w, _ = ofin.rowwise_cast(obf16.widen(wb.T.copy()).reshape(N, K), dsg.E4M3, 0)
    np.testing.assert_array_equal(xq.cpu().numpy()[rows], codes_x)
    np.testing.assert_array_equal(wq.cpu().numpy(), codes_w)
    np.testing.assert_array_equal(_bits(six.cpu().numpy()[rows]), _bits(sinv_x))
    acc, sum_abs = ogemm.gemm_exact(codes_x, dsg.E4M3, dsg.OP_N, codes_w, dsg.E4M3, dsg.OP_T)
    ref = obf16.widen(ofin.dequant_vec_to_bf16(acc, s_x, s_w)).astype(np.float64)
    yg = obf16.widen(bf16_bits(y)[rows]).astype(np.float64)
    fac = sinv_x.astype(np.float64)[:, None] * sinv_w.astype(np.float64)[None, :]
    assert (np.abs(yg - ref) <= bf16_ulp(ref) + ACC_REL * fac * sum_abs).all()

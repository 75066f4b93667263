"""Argument checks of the Python binding on device tensors, and strided GEMM
operands addressed through their leading dimensions."""

import numpy as np
import pytest
import torch

import delayed_scaling_gemm_amd as dsg
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_undersized_and_strided_arguments_raise():
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    s = torch.ones(1, device=DEV)
    with pytest.raises(ValueError, match="at least"):
        dsg.fp8ds_cast(x, dsg.E4M3, s, torch.zeros(64 * 128 - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="contiguous"):
        dsg.fp8ds_cast(x[:, :64], dsg.E4M3, s, torch.zeros(64 * 64, dtype=torch.uint8, device=DEV))
    with pytest.raises(TypeError):
        dsg.fp8ds_cast(x, dsg.E4M3, s, torch.zeros(64 * 128, dtype=torch.int8, device=DEV))
    a = torch.zeros(64, 128, dtype=torch.uint8, device=DEV)
    c = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    small_b = torch.zeros(32, 128, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="at least"):  # B needs 64 x 128
        dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, 64, 64, 128, a, dsg.E4M3, 128, s, small_b, dsg.E4M3,
                       128, s, c, 64)
    with pytest.raises(ValueError, match="at least"):  # C too small for ldc
        dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, 64, 64, 128, a, dsg.E4M3, 128, s, a, dsg.E4M3, 128,
                       s, c, 80)
    torch.cuda.synchronize()


def test_submatrix_operands_through_leading_dimensions():
    """Operands that are column slices of wider arrays (lda > K) give the same
    result as contiguous copies."""
    rng = np.random.default_rng(5)
    M, N, K, ld = 192, 160, 256, 384
    ints_a = rng.integers(-8, 9, (M, ld))
    ints_b = rng.integers(-8, 9, (N, ld))
    wa = torch.from_numpy(ofp8.encode(ints_a.astype(np.float32), ofp8.E4M3)).to(DEV)
    wb = torch.from_numpy(ofp8.encode(ints_b.astype(np.float32), ofp8.E4M3)).to(DEV)
    one = torch.ones(1, device=DEV)
    c1 = torch.zeros(M, N, dtype=torch.float32, device=DEV)
    c2 = torch.zeros_like(c1)
    dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, M, N, K, wa[:, 16:16 + K], dsg.E4M3, ld, one,
                   wb[:, 16:16 + K], dsg.E4M3, ld, one, c1, N)
    ca = wa[:, 16:16 + K].contiguous()
    cb = wb[:, 16:16 + K].contiguous()
    dsg.fp8ds_gemm(dsg.OP_N, dsg.OP_T, M, N, K, ca, dsg.E4M3, K, one, cb, dsg.E4M3, K, one, c2, N)
    torch.cuda.synchronize()
    exp = (ints_a[:, 16:16 + K] @ ints_b[:, 16:16 + K].T).astype(np.float32)
    assert np.array_equal(c1.cpu().numpy(), exp)
    assert np.array_equal(c2.cpu().numpy(), exp)

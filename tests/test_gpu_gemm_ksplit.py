"""GPU parity of the GEMM tile choices for narrow and mid-size shapes.

* Two K halves per workgroup: grids of 128 x 128 output tiles that leave each CU
  at most one tile (the k/v-projection weight gradient, 4096 x 1024 with K = 8192
  tokens, is one), K a multiple of 256 and at least 1024, operands fit for direct
  loads.  Each half's FP32 sums meet in LDS.  Checked: the sums on every element
  (1e-5 * sum|ab| on the exact datapath, the derived bound on the FP8 one),
  bit-exact small-integer products (the split must drop or double no product),
  ragged tile edges, batches, and the full-size weight gradient on sampled rows.
* 256 x 256 tiles from K = 2048 on: a 4096 x 4096 x 2048 product on sampled rows
  of every tile band, in the three layouts."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import gemm as ogemm  # noqa: E402
from tests.parity import (ACC_REL, band_rows, bf16_bits, check_acc_bound,  # noqa: E402
                          check_bf16_out_bound, f32_bits, fp8_path_bound)
from tests.test_gpu_gemm import finite_codes, int_codes, run_gemm  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
LAYOUTS = [(dsg.OP_N, dsg.OP_N), (dsg.OP_N, dsg.OP_T), (dsg.OP_T, dsg.OP_N)]


def stored(op, c):
    return c if op == dsg.OP_N else np.ascontiguousarray(c.T)


@pytest.mark.parametrize("mma", [dsg.MMA_EXACT, dsg.MMA_FP8])
@pytest.mark.parametrize("opa,opb", LAYOUTS)
@pytest.mark.parametrize("shape", [(1024, 1024, 2048), (1040, 528, 1280), (256, 4096, 1024)])
def test_split_k_within_tolerance(opa, opb, shape, mma):
    M, N, K = shape
    print(f"[ksplit] {shape} ops {opa}{opb} mma {mma}", flush=True)
    rng = np.random.default_rng(M + 3 * N + 7 * K + 11 * opa + 13 * opb + mma)
    fa, fb = dsg.E4M3, dsg.E5M2
    ca = finite_codes(rng, (M, K), fa)
    cb = finite_codes(rng, (K, N), fb)
    a_st, b_st = stored(opa, ca), stored(opb, cb)
    acc, sum_abs = ogemm.gemm_exact(a_st, fa, opa, b_st, fb, opb)
    bound = ACC_REL * sum_abs if mma == dsg.MMA_EXACT else fp8_path_bound(
        ofp8.decode(ca, fa), ofp8.decode(cb, fb), sum_abs)
    C, _ = run_gemm(opa, opb, a_st, fa, b_st, fb, M, N, K, mma=mma)
    check_acc_bound(C.cpu().numpy(), acc, bound, f"acc {shape}")
    sa, sb = np.float32(3.75), np.float32(0.0625)
    Y, am = run_gemm(opa, opb, a_st, fa, b_st, fb, M, N, K, sa, sb, out=torch.bfloat16, mma=mma)
    yb = bf16_bits(Y)
    check_bf16_out_bound(yb, ogemm.dequant_to_bf16(acc, sa, sb), bound,
                         1.0 / float(ogemm.dequant_scale(sa, sb)), f"bf16 {shape}")
    assert am == f32_bits(ogemm.output_amax(yb))


@pytest.mark.parametrize("mma", [dsg.MMA_EXACT, dsg.MMA_FP8])
@pytest.mark.parametrize("opa,opb", LAYOUTS)
def test_split_k_small_integers_exact(opa, opb, mma):
    """Small integers: every partial and total sum is exact, so the result must
    equal the exact product bit for bit (a dropped or doubled stage would not)."""
    M, N, K = 1024, 512, 4096
    rng = np.random.default_rng(41 + 3 * opa + opb + 5 * mma)
    ca, ia = int_codes(rng, (M, K), dsg.E4M3)
    cb, ib = int_codes(rng, (K, N), dsg.E4M3)
    C, am = run_gemm(opa, opb, stored(opa, ca), dsg.E4M3, stored(opb, cb), dsg.E4M3, M, N, K,
                     mma=mma)
    exp = (ia.astype(np.float64) @ ib.astype(np.float64)).astype(np.float32)
    got = C.cpu().numpy()
    assert np.array_equal(got, exp), f"{np.count_nonzero(got != exp)} differ"
    assert am == f32_bits(np.max(np.abs(exp)))


def test_split_k_batched():
    """Batched problems whose tiles together still fit the CUs."""
    B, M, N, K = 3, 512, 256, 2048
    rng = np.random.default_rng(7)
    ca = [finite_codes(rng, (M, K), dsg.E4M3) for _ in range(B)]
    cb = [finite_codes(rng, (N, K), dsg.E4M3) for _ in range(B)]
    A = torch.from_numpy(np.stack(ca)).to(DEV)
    Bt = torch.from_numpy(np.stack(cb)).to(DEV)
    C = torch.empty(B, M, N, dtype=torch.float32, device=DEV)
    one = torch.ones(B, dtype=torch.float32, device=DEV)
    am = torch.zeros(B, dtype=torch.float32, device=DEV)
    dsg.fp8ds_gemm_batched(dsg.OP_N, dsg.OP_T, M, N, K, B, A, dsg.E4M3, K, M * K, one, Bt,
                           dsg.E4M3, K, N * K, one, C, N, M * N, am)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    for b in range(B):
        acc, sum_abs = ogemm.gemm_exact(ca[b], 0, 0, cb[b], 0, 1)
        check_acc_bound(got[b], acc, ACC_REL * sum_abs, f"batch {b}")


@pytest.mark.parametrize("mma", [dsg.MMA_EXACT, dsg.MMA_FP8])
def test_kv_projection_weight_gradient_full_size(mma):
    """dW = X^T dY at 4096 x 1024 with K = 8192 (TN, E4M3 x E5M2): sampled rows
    of every 128-row tile band, every column, against the oracle."""
    M, N, K = 4096, 1024, 8192
    rng = np.random.default_rng(99 + mma)
    x = finite_codes(rng, (K, M), dsg.E4M3)      # X codes [tokens x in]
    dy = finite_codes(rng, (K, N), dsg.E5M2)     # dY codes [tokens x out]
    C, _ = run_gemm(dsg.OP_T, dsg.OP_N, x, dsg.E4M3, dy, dsg.E5M2, M, N, K, mma=mma)
    got = C.cpu().numpy()
    rows = band_rows(M, 128)
    a = np.ascontiguousarray(x[:, rows].T)
    acc, sum_abs = ogemm.gemm_exact(a, dsg.E4M3, 0, dy, dsg.E5M2, 0)
    bound = ACC_REL * sum_abs if mma == dsg.MMA_EXACT else fp8_path_bound(
        ofp8.decode(a, dsg.E4M3), ofp8.decode(dy, dsg.E5M2), sum_abs)
    check_acc_bound(got[rows], acc, bound, "dW rows")


@pytest.mark.parametrize("opa,opb", LAYOUTS)
def test_big_tiles_at_k2048(opa, opb):
    """4096 x 4096 x 2048 runs on 256 x 256 tiles (every CU one tile, K at the
    threshold of the larger tiles): sampled rows of every tile band."""
    M, N, K = 4096, 4096, 2048
    rng = np.random.default_rng(2048 + 3 * opa + opb)
    ca = finite_codes(rng, (M, K), dsg.E5M2)
    cb = finite_codes(rng, (K, N), dsg.E4M3)
    C, _ = run_gemm(opa, opb, stored(opa, ca), dsg.E5M2, stored(opb, cb), dsg.E4M3, M, N, K)
    got = C.cpu().numpy()
    rows = band_rows(M, 256)
    acc, sum_abs = ogemm.gemm_exact(ca[rows], dsg.E5M2, 0, cb, dsg.E4M3, 0)
    check_acc_bound(got[rows], acc, ACC_REL * sum_abs, "rows")

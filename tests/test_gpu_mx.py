"""GPU parity of MXFP8 against the oracle (oracle/mx.py): the block cast and its
transposed copy (element codes and E8M0 scale codes bit-exact, zero / NaN / Inf /
tiny blocks included), the MX GEMM (accumulator bound on FP32 output, plus one
BF16 ulp on BF16 output; a NaN block poisons exactly its row), and a whole MX
training step (three casts with transposed copies, three NT GEMMs)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import mx as omx  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from tests.parity import (bf16_bits, check_acc, check_acc_bound, check_bf16_out,  # noqa: E402
                          fp8_path_bound)
from tests.test_gpu_gemm import finite_codes, int_codes  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _input(rows, cols, seed, bf16, specials=False):
    """Rows and 32-element blocks of very different magnitudes."""
    x = workloads.normal(rows * cols, seed, 1.0).reshape(rows, cols)
    nb = cols // 32
    rng = np.random.default_rng(seed)
    mag = np.float32(2.0) ** rng.integers(-40, 41, (rows, nb)).astype(np.float32)
    x *= np.repeat(mag, 32, axis=1)
    if specials and rows >= 5 and nb >= 2:
        x[0, 0:32] = 0.0                       # zero block: scale code 0
        x[1, 32 + 3] = np.inf                  # Inf: NaN block
        x[2, 5] = np.nan                       # NaN: NaN block
        x[3, 32:64] *= np.float32(2.0**-90)    # tiny block: scale clamps to code 0
        x[4, 0:32] = np.float32(1.9) * np.float32(2.0**7)  # 486.4 after scaling: saturates
    if bf16:
        bits = workloads.to_bf16_bits(x)
        return (torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16),
                obf16.widen(bits).reshape(rows, cols))
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV), x


def _cast(x, fmt):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    dsg.fp8ds_cast_mx(x, fmt, q, s)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("shape", [(1, 32), (5, 64), (37, 4096), (3, 8192 + 96), (700, 96)])
def test_mx_cast_matches_oracle(bf16, fmt, shape):
    rows, cols = shape
    x, xw = _input(rows, cols, 1000 * rows + cols + fmt, bf16, specials=True)
    q, s = _cast(x, fmt)
    codes, scales = omx.mx_cast(xw, fmt)
    np.testing.assert_array_equal(s.cpu().numpy(), scales)
    np.testing.assert_array_equal(q.cpu().numpy(), codes)


def test_mx_cast_full_size_sampled():
    """X of the 4096-hidden Linear at M = 16384: 64 sampled rows bit-exact."""
    xb, _, _ = workloads.fwd_bwd_4096()
    x = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    q, s = _cast(x, dsg.E4M3)
    rows = np.random.default_rng(1).choice(xb.shape[0], 64, replace=False)
    codes, scales = omx.mx_cast(obf16.widen(xb[rows]).reshape(64, -1), dsg.E4M3)
    np.testing.assert_array_equal(s.cpu().numpy()[rows], scales)
    np.testing.assert_array_equal(q.cpu().numpy()[rows], codes)


def _gemm(a, sa, fa, b, sb, fb, out=torch.bfloat16, mma=dsg.MMA_EXACT):
    M, K = a.shape
    N = b.shape[0]
    A, B = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    SA, SB = torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV)
    ldc = (N + 7) // 8 * 8  # 16-byte rows for BF16 and FP32 outputs
    C = torch.empty((M, ldc), dtype=out, device=DEV)
    am = torch.zeros(1, device=DEV)
    dsg.fp8ds_gemm_mx(M, N, K, A, fa, K, SA, K // 32, B, fb, K, SB, K // 32, C, ldc, am, mma=mma)
    torch.cuda.synchronize()
    return C[:, :N], float(am.item())


FMT_PAIRS = [(dsg.E4M3, dsg.E4M3), (dsg.E5M2, dsg.E4M3), (dsg.E4M3, dsg.E5M2)]


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (100, 70, 256), (520, 264, 128),
                                   (300, 600, 1024)])
def test_mx_gemm_matches_oracle(fa, fb, M, N, K):
    rng = np.random.default_rng(M + 7 * N + K + fa)
    a, b = finite_codes(rng, (M, K), fa), finite_codes(rng, (N, K), fb)
    sa = rng.integers(112, 143, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(112, 143, (N, K // 32)).astype(np.uint8)
    acc, sum_abs = omx.mx_gemm_nt(a, sa, fa, b, sb, fb)
    c32, _ = _gemm(a, sa, fa, b, sb, fb, out=torch.float32)
    check_acc(c32.cpu().numpy(), acc, sum_abs, "mx fp32")
    c16, am = _gemm(a, sa, fa, b, sb, fb)
    y = bf16_bits(c16)
    check_bf16_out(y, acc, sum_abs, omx.to_bf16(acc), 1.0, "mx bf16")
    assert am == np.abs(obf16.widen(y).astype(np.float64)).max()


def test_mx_gemm_wide_scale_range():
    """Block scales from 2^-100 to 2^100 that pair up to moderate products: the
    scaled BF16 widening across the exponent range."""
    rng = np.random.default_rng(11)
    M, N, K = 256, 256, 1024
    a, b = finite_codes(rng, (M, K), dsg.E4M3), finite_codes(rng, (N, K), dsg.E5M2)
    shift = rng.integers(-100, 101, K // 32)
    sa = (127 + shift[None, :] + rng.integers(-8, 9, (M, 1))).astype(np.uint8)
    sb = (127 - shift[None, :] + rng.integers(-8, 9, (N, 1))).astype(np.uint8)
    acc, sum_abs = omx.mx_gemm_nt(a, sa, dsg.E4M3, b, sb, dsg.E5M2)
    c32, _ = _gemm(a, sa, dsg.E4M3, b, sb, dsg.E5M2, out=torch.float32)
    check_acc(c32.cpu().numpy(), acc, sum_abs, "mx wide scales")


def test_mx_gemm_nan_block_poisons_its_row():
    rng = np.random.default_rng(12)
    M, N, K = 128, 256, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[7, 40] = np.nan
    w = rng.standard_normal((N, K)).astype(np.float32)
    xa, xs = _cast(torch.from_numpy(x).to(DEV), dsg.E4M3)
    wa, ws = _cast(torch.from_numpy(w).to(DEV), dsg.E4M3)
    assert xs.cpu().numpy()[7, 1] == 0xFF
    c, _ = _gemm(*(t.cpu().numpy() for t in (xa, xs)), dsg.E4M3,
                 *(t.cpu().numpy() for t in (wa, ws)), dsg.E4M3, out=torch.float32)
    c = c.cpu().numpy()
    assert np.isnan(c[7]).all()
    others = np.delete(c, 7, axis=0)
    assert np.isfinite(others).all()
    acc, sum_abs = omx.mx_gemm_nt(xa.cpu().numpy(), xs.cpu().numpy(), dsg.E4M3,
                                  wa.cpu().numpy(), ws.cpu().numpy(), dsg.E4M3)
    check_acc(others, np.delete(acc, 7, axis=0), np.delete(sum_abs, 7, axis=0), "mx nan rows")


def test_mx_forward_full_size_sampled():
    """The 4096-hidden forward at M = 16384 in MXFP8: X cast along its rows, W^T
    along its rows (blocks along K for both), then the MX GEMM; 32 sampled rows
    against the oracle."""
    M, K, N = 16384, 4096, 4096
    xb, wb, _ = workloads.fwd_bwd_4096()
    x = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    wt = torch.from_numpy(np.ascontiguousarray(wb.T).view(np.int16)).to(DEV).view(torch.bfloat16)
    xq, xs = _cast(x, dsg.E4M3)
    wq, ws = _cast(wt, dsg.E4M3)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dsg.fp8ds_gemm_mx(M, N, K, xq, dsg.E4M3, K, xs, K // 32, wq, dsg.E4M3, K, ws, K // 32, y, N)
    torch.cuda.synchronize()
    rows = np.random.default_rng(2).choice(M, 32, replace=False)
    cx, sx = omx.mx_cast(obf16.widen(xb[rows]).reshape(32, K), dsg.E4M3)
    cw, sw = omx.mx_cast(obf16.widen(np.ascontiguousarray(wb.T)).reshape(N, K), dsg.E4M3)
    np.testing.assert_array_equal(wq.cpu().numpy(), cw)
    np.testing.assert_array_equal(ws.cpu().numpy(), sw)
    acc, sum_abs = omx.mx_gemm_nt(cx, sx, dsg.E4M3, cw, sw, dsg.E4M3)
    check_bf16_out(bf16_bits(y)[rows], acc, sum_abs, omx.to_bf16(acc), 1.0, "mx forward")


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("fmt", [dsg.E4M3, dsg.E5M2])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 128)])
def test_mx_cast_transpose_matches_oracle(bf16, fmt, shape):
    rows, cols = shape
    x, xw = _input(rows, cols, 7 * rows + cols + fmt, bf16, specials=True)
    xw = np.array(xw)  # add column specials: a zero, an Inf, a NaN and a tiny column block
    xw[40:72, 9] = 0.0
    xw[70, 17] = np.inf
    xw[100, 30] = np.nan
    xw[0:32, 50] *= np.float32(2.0**-100)
    if bf16:
        bits = workloads.to_bf16_bits(xw)
        x = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        xw = obf16.widen(bits).reshape(rows, cols)
    else:
        x = torch.from_numpy(np.ascontiguousarray(xw)).to(DEV)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    qt = torch.empty((cols, rows), dtype=torch.uint8, device=DEV)
    st = torch.empty((cols, rows // 32), dtype=torch.uint8, device=DEV)
    dsg.fp8ds_cast_mx(x, fmt, q, s, qt, st)
    torch.cuda.synchronize()
    codes, scales = omx.mx_cast(xw, fmt)
    codes_t, scales_t = omx.mx_cast(np.ascontiguousarray(xw.T), fmt)
    np.testing.assert_array_equal(s.cpu().numpy(), scales)
    np.testing.assert_array_equal(q.cpu().numpy(), codes)
    np.testing.assert_array_equal(st.cpu().numpy(), scales_t)
    np.testing.assert_array_equal(qt.cpu().numpy(), codes_t)


def test_mx_training_step():
    """Y = X W, dX = dY W^T, dW = X^T dY in MXFP8 (E4M3 forward, E5M2 gradient):
    one transposing cast per tensor, three NT GEMMs, every output element against
    the oracle's exact sums."""
    M, K, N = 1024, 512, 256
    x = workloads.normal(M * K, 301, 1.0).reshape(M, K)
    w = workloads.normal(K * N, 302, 0.02).reshape(K, N)
    dy = workloads.heavy_tail_grad(M * N, 303).reshape(M, N)
    dev = {}
    ref = {}
    for name, a, fmt in (("x", x, dsg.E4M3), ("w", w, dsg.E4M3), ("dy", dy, dsg.E5M2)):
        bits = workloads.to_bf16_bits(a)
        t = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        r, c = a.shape
        q = torch.empty((r, c), dtype=torch.uint8, device=DEV)
        s = torch.empty((r, c // 32), dtype=torch.uint8, device=DEV)
        qt = torch.empty((c, r), dtype=torch.uint8, device=DEV)
        st = torch.empty((c, r // 32), dtype=torch.uint8, device=DEV)
        dsg.fp8ds_cast_mx(t, fmt, q, s, qt, st)
        dev[name] = (q, s, qt, st, fmt)
        aw = obf16.widen(bits).reshape(r, c)
        ref[name] = omx.mx_cast(aw, fmt) + omx.mx_cast(np.ascontiguousarray(aw.T), fmt) + (fmt,)

    def run(m, n, k, a, sa, fa, b, sb, fb):
        c = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        dsg.fp8ds_gemm_mx(m, n, k, a, fa, k, sa, k // 32, b, fb, k, sb, k // 32, c, n)
        return c

    X, W, D = dev["x"], dev["w"], dev["dy"]
    y = run(M, N, K, X[0], X[1], X[4], W[2], W[3], W[4])      # X . (W^T blocked along K)
    dx = run(M, K, N, D[0], D[1], D[4], W[0], W[1], W[4])     # dY . W  (blocked along N)
    dw = run(K, N, M, X[2], X[3], X[4], D[2], D[3], D[4])     # X^T . dY^T (blocked along M)
    torch.cuda.synchronize()
    for name in ("x", "w", "dy"):
        q, s, qt, st, _ = dev[name]
        rc, rs, rct, rst, _ = ref[name]
        for g, r in ((q, rc), (s, rs), (qt, rct), (st, rst)):
            np.testing.assert_array_equal(g.cpu().numpy(), r)
    X, W, D = ref["x"], ref["w"], ref["dy"]
    for out, (a, sa, fa), (b, sb, fb), what in (
            (y, (X[0], X[1], X[4]), (W[2], W[3], W[4]), "y"),
            (dx, (D[0], D[1], D[4]), (W[0], W[1], W[4]), "dx"),
            (dw, (X[2], X[3], X[4]), (D[2], D[3], D[4]), "dw")):
        acc, sum_abs = omx.mx_gemm_nt(a, sa, fa, b, sb, fb)
        check_bf16_out(bf16_bits(out), acc, sum_abs, omx.to_bf16(acc), 1.0, what)


# ---------------------------------------------------------------- FP8 datapath (opt-in)
# gfx950's block-scaled FP8 MFMA: exact where no product falls out of its
# summation window, otherwise within the FP8 datapath's derived bound
# (tests.parity.fp8_path_bound on the block-scaled decoded operands).

@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("M,N", [(256, 256), (100, 200)])
def test_mx_fp8_path_small_integers_exact(fa, fb, M, N):
    """Small integers with block scales 2^-2 .. 2^2: every product, group sum and
    FP32 total is exact, so the result equals the oracle bit for bit (this also
    pins which byte of the scale register belongs to which block)."""
    K = 128
    rng = np.random.default_rng(M + N + fa + 2 * fb)
    a, _ = int_codes(rng, (M, K), fa)
    b, _ = int_codes(rng, (N, K), fb)
    sa = rng.integers(125, 130, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(125, 130, (N, K // 32)).astype(np.uint8)
    acc, _ = omx.mx_gemm_nt(a, sa, fa, b, sb, fb)
    c, _ = _gemm(a, sa, fa, b, sb, fb, out=torch.float32, mma=dsg.MMA_FP8)
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), acc)


@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (300, 600, 1024)])
def test_mx_fp8_path_within_bound(fa, fb, M, N, K):
    rng = np.random.default_rng(3 * M + N + K + fa)
    a, b = finite_codes(rng, (M, K), fa), finite_codes(rng, (N, K), fb)
    sa = rng.integers(112, 143, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(112, 143, (N, K // 32)).astype(np.uint8)
    acc, sum_abs = omx.mx_gemm_nt(a, sa, fa, b, sb, fb)
    c32, _ = _gemm(a, sa, fa, b, sb, fb, out=torch.float32, mma=dsg.MMA_FP8)

    def scaled(codes, scales, fmt):  # decoded elements times their block scales
        return ofp8.decode(codes, fmt) * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127,
                                                                  32, axis=1))
    bound = fp8_path_bound(scaled(a, sa, fa), scaled(b, sb, fb).T, sum_abs)
    check_acc_bound(c32.cpu().numpy(), acc, bound, "mx fp8 path")


def test_mx_linear_matches_the_raw_calls():
    """MXLinear.step issues exactly the casts and GEMMs of test_mx_training_step:
    its outputs equal those of the C-ABI calls made one by one, bit for bit."""
    from delayed_scaling_gemm_amd.linear import MXLinear

    M, K, N = 512, 256, 384
    x = torch.randn(M, K, device=DEV).to(torch.bfloat16)
    w = (0.02 * torch.randn(K, N, device=DEV)).to(torch.bfloat16)
    dy = (1e-3 * torch.randn(M, N, device=DEV)).to(torch.bfloat16)
    out = MXLinear(device=DEV).step(x, w, dy)
    torch.cuda.synchronize()
    casts = {}
    for name, t, fmt in (("x", x, dsg.E4M3), ("w", w, dsg.E4M3), ("dy", dy, dsg.E5M2)):
        r, c = t.shape
        q, s = _cast(t, fmt)
        qt = torch.empty((c, r), dtype=torch.uint8, device=DEV)
        st = torch.empty((c, r // 32), dtype=torch.uint8, device=DEV)
        q2 = torch.empty_like(q)
        s2 = torch.empty_like(s)
        dsg.fp8ds_cast_mx(t, fmt, q2, s2, qt, st)
        torch.cuda.synchronize()
        assert torch.equal(q, q2) and torch.equal(s, s2)
        casts[name] = (q, s, qt, st, fmt)
    X, W, D = casts["x"], casts["w"], casts["dy"]
    for key, (m, n, k, a, b) in {"y": (M, N, K, (X[0], X[1], X[4]), (W[2], W[3], W[4])),
                                 "dx": (M, K, N, (D[0], D[1], D[4]), (W[0], W[1], W[4])),
                                 "dw": (K, N, M, (X[2], X[3], X[4]), (D[2], D[3], D[4]))}.items():
        c = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        dsg.fp8ds_gemm_mx(m, n, k, a[0], a[2], k, a[1], k // 32, b[0], b[2], k, b[1], k // 32, c, n)
        torch.cuda.synchronize()
        assert torch.equal(out[key].view(torch.int16), c.view(torch.int16)), key


def test_mx_degenerate_shapes():
    """K = 0 writes zeros (and amax 0); M = 0 only resets the output amax; an
    empty cast is a no-op."""
    c = torch.full((64, 64), 7.0, dtype=torch.float32, device=DEV)
    am = torch.full((1,), 5.0, device=DEV)
    u8 = torch.zeros(1, dtype=torch.uint8, device=DEV)
    dsg.fp8ds_gemm_mx(64, 64, 0, u8, dsg.E4M3, 16, None, 4, u8, dsg.E4M3, 16, None, 4, c, 64, am)
    torch.cuda.synchronize()
    assert not c.any() and am.item() == 0.0
    am.fill_(5.0)
    b = torch.zeros(64, 128, dtype=torch.uint8, device=DEV)
    sb = torch.full((64, 4), 127, dtype=torch.uint8, device=DEV)
    dsg.fp8ds_gemm_mx(0, 64, 128, u8, dsg.E4M3, 128, u8, 4, b, dsg.E4M3, 128, sb, 4, c, 64, am)
    torch.cuda.synchronize()
    assert am.item() == 0.0
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    dsg.fp8ds_cast_mx(x, dsg.E4M3, torch.zeros(0, dtype=torch.uint8, device=DEV),
                      torch.zeros(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()

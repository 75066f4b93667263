"""GPU parity: amax and the fused amax + saturating cast against the oracle
(bit-exact bytes, amax bits and saturation counts)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import delayed_scaling_gemm_amd as dsg  # noqa: E402
import workloads  # noqa: E402
from oracle import amax as oamax  # noqa: E402
from oracle import bf16 as obf16  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from tests.parity import f32_bits  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"
FMTS = [dsg.E4M3, dsg.E5M2]
SCALES = [1.0, np.float32(448.0) / np.float32(3.7), 2.0**-3, 1e-3, 3.0e4, 1e30, 2.0**100]


def dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def run_cast(x_dev, fmt, scale, rows=None, cols=None, transpose=False):
    n = x_dev.numel()
    if rows is not None:
        x_dev = x_dev.view(rows, cols)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    q = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)
    qt = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV) if transpose else None
    su = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    am = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    sat = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    dsg.fp8ds_cast(x_dev, fmt, s, q, qt, su, am, sat)
    torch.cuda.synchronize()
    return (q.cpu().numpy(), None if qt is None else qt.cpu().numpy(), su.item(),
            am.cpu().numpy().view(np.uint32)[0], int(sat.item()))


def oracle_cast(x32, fmt, scale):
    codes, sat = ofp8.cast(x32, np.float32(scale), fmt)
    a = np.array([oamax.amax(x32)], dtype=np.float32).view(np.uint32)[0]
    return codes, int(a), sat


@pytest.mark.parametrize("fmt", FMTS)
def test_all_bf16_patterns(fmt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = dev_bf16(bits)
    x32 = obf16.widen(bits)
    for s in SCALES:
        q, _, su, am, sat = run_cast(x, fmt, s)
        codes, oa, osat = oracle_cast(x32, fmt, s)
        assert np.array_equal(q, codes), f"scale {s}: {np.count_nonzero(q != codes)} bytes differ"
        assert am == oa and sat == osat and su == np.float32(s)


@pytest.mark.parametrize("fmt", FMTS)
def test_random_fp32_patterns(fmt):
    rng = np.random.default_rng(17 + fmt)
    bits = rng.integers(0, 2**32, (1 << 20) + 13, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x = dev_f32(x32)
    for s in (1.0, 2.0**-40, 2.0**40, 0.7):
        q, _, su, am, sat = run_cast(x, fmt, s)
        codes, oa, osat = oracle_cast(x32, fmt, s)
        assert np.array_equal(q, codes) and am == oa and sat == osat


@pytest.mark.parametrize("fmt", FMTS)
def test_midpoints_and_neighbours(fmt):
    vals = ofp8.decode_table(fmt)
    max_code = 0x7E if fmt == dsg.E4M3 else 0x7B
    pts = []
    for c in range(max_code):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        pts += [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts])
    x = dev_f32(pts)
    for s in (1.0, 4.0, 0.25):
        # x / s is exact for powers of two, so fl32(x*s) lands on the same points
        xs = (pts / np.float32(s)).astype(np.float32)
        q, _, _, _, _ = run_cast(dev_f32(xs), fmt, s)
        codes, _, _ = oracle_cast(xs, fmt, s)
        assert np.array_equal(q, codes)
    q, _, _, _, _ = run_cast(x, fmt, 1.0)
    assert np.array_equal(q, ofp8.encode(pts, fmt))


# A tensor of at most 65536 elements is one workgroup of 1024 threads whose 16-byte
# pieces (8 BF16 / 4 FP32 elements) form 16-element groups with partners 1024
# pieces apart; larger tensors take workgroups of 256 threads and 8192 elements,
# partners 256 pieces apart.  The sizes cover both shapes and the switch between
# them (65536, 65537), partial last workgroups whose last pieces lack partners
# (3 * 65536 + 12345), and sub-piece tails.
@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 255, 4099, 65536, 65537, 65536 + 9,
                               65536 + 8 * 1024 + 5, 3 * 65536 + 12345, (1 << 20) + 3])
@pytest.mark.parametrize("bf16", [True, False])
def test_small_and_ragged_sizes(n, bf16):
    rng = np.random.default_rng(n)
    x32 = (rng.standard_normal(n) * 100).astype(np.float32)
    if bf16:
        bits = workloads.to_bf16_bits(x32)
        x, x32 = dev_bf16(bits), obf16.widen(bits)
    else:
        x = dev_f32(x32)
    for fmt in FMTS:
        q, _, su, am, sat = run_cast(x, fmt, 3.0)
        codes, oa, osat = oracle_cast(x32, fmt, 3.0)
        assert np.array_equal(q, codes) and am == oa and sat == osat and su == 3.0


def test_standalone_amax():
    cases = [
        np.zeros(0, np.float32),
        np.array([-0.0, -0.0], np.float32),
        np.array([1.0, -7.5, 3.0] * 11, np.float32),
        np.array([1.0, -np.inf, 2.0] * 7, np.float32),
        np.array([1.0, np.nan, -np.inf] * 7, np.float32),
        (np.random.default_rng(1).standard_normal(100_003) * 5).astype(np.float32),
    ]
    for x32 in cases:
        for bf16 in (False, True):
            if bf16:
                bits = workloads.to_bf16_bits(x32)
                xd, xr = dev_bf16(bits), obf16.widen(bits)
            else:
                xd, xr = dev_f32(x32), x32
            am = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
            dsg.fp8ds_amax(xd, am)
            torch.cuda.synchronize()
            got = am.cpu().numpy().view(np.uint32)[0]
            assert got == f32_bits(oamax.amax(xr)), (x32[:4], bf16)


@pytest.mark.parametrize("shape", [(130, 70), (64, 64), (1, 100), (100, 1), (257, 513),
                                   (256, 384), (384, 128), (272, 400), (128, 2048), (1024, 1040)])
@pytest.mark.parametrize("bf16", [True, False])
def test_cast_with_transposed_copy(shape, bf16):
    """q and its transpose q_t: full 128 x 128 tiles of aligned shapes take the
    vector path, other tiles the element-wise path; both must match the oracle."""
    rows, cols = shape
    rng = np.random.default_rng(rows * 1000 + cols + bf16)
    x32 = (rng.standard_normal(rows * cols) * 200).astype(np.float32)
    x32[rng.choice(x32.size, min(5, x32.size), replace=False)] = 7.0e4  # saturate both formats
    if bf16:
        bits = workloads.to_bf16_bits(x32)
        xd, xr = dev_bf16(bits), obf16.widen(bits)
    else:
        xd, xr = dev_f32(x32), x32
    for fmt in FMTS:
        q, qt, su, am, sat = run_cast(xd, fmt, 1.5, rows, cols, transpose=True)
        codes, oa, osat = oracle_cast(xr, fmt, 1.5)
        assert np.array_equal(q, codes)
        assert np.array_equal(qt.reshape(cols, rows), codes.reshape(rows, cols).T)
        assert am == oa and sat == osat and su == 1.5


def test_cast_batched():
    rng = np.random.default_rng(5)
    B, n = 7, 4099
    x32 = (rng.standard_normal((B, n)) * rng.uniform(0.1, 100, (B, 1))).astype(np.float32)
    xs = dev_f32(x32)
    scales = np.array([1.0, 2.0, 448 / 3.3, 1e-3, 5.0, 1e5, 0.5], np.float32)
    s = dev_f32(scales)
    q = torch.zeros((B, (n + 15) // 16 * 16), dtype=torch.uint8, device=DEV)
    su = torch.zeros(B, dtype=torch.float32, device=DEV)
    am = torch.zeros(B, dtype=torch.float32, device=DEV)
    sat = torch.zeros(B, dtype=torch.int64, device=DEV)
    # tensors padded to a 16-element stride for alignment
    xp = torch.zeros((B, (n + 15) // 16 * 16), dtype=torch.float32, device=DEV)
    xp[:, :n] = xs
    L = dsg.lib()
    dsg._check(L.fp8ds_cast_batched(xp.data_ptr(), dsg.F32, B, n, xp.stride(0), dsg.E4M3,
                                    s.data_ptr(), q.data_ptr(), q.stride(0), su.data_ptr(),
                                    am.data_ptr(), sat.data_ptr(), dsg._stream(None)))
    torch.cuda.synchronize()
    qn, amn, satn = q.cpu().numpy(), am.cpu().numpy(), sat.cpu().numpy()
    for b in range(B):
        codes, oa, osat = oracle_cast(x32[b], dsg.E4M3, scales[b])
        assert np.array_equal(qn[b, :n], codes)
        assert amn.view(np.uint32)[b] == oa and satn[b] == osat
    assert np.array_equal(su.cpu().numpy(), scales)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [65536, 65531, 65537, 70000])
def test_cast_batched_one_workgroup_boundary(fmt, n):
    """Batched bf16 casts on both sides of 64 Ki elements per tensor: up to it one
    workgroup covers a tensor and stores amax, saturation count and the scale
    snapshot itself; beyond it the outputs are reset by a prologue and reduced
    atomically.  The outputs start as garbage and the call runs twice: nothing
    may carry over.  Tensors hold NaN, Inf and saturating values."""
    rng = np.random.default_rng(n + fmt)
    B = 5
    stride = (n + 15) // 16 * 16
    x32 = (rng.standard_normal((B, n)) * rng.uniform(0.1, 100, (B, 1))).astype(np.float32)
    x32[1, n // 3] = np.inf
    x32[2, 7] = np.nan
    x32[3, n - 1] = -1e6  # saturates at any scale here
    bits = obf16.round_to_bf16_vec(x32.astype(np.float64)).reshape(B, n)
    xw = obf16.widen(bits.ravel()).reshape(B, n)
    xp = np.zeros((B, stride), dtype=np.uint16)
    xp[:, :n] = bits
    xd = dev_bf16(xp)
    scales = np.array([1.0, 448 / 3.3, 2.0**-3, 5.0, 1e-3], np.float32)
    s = dev_f32(scales)
    q = torch.full((B, stride), 0xAB, dtype=torch.uint8, device=DEV)
    su = torch.full((B,), -7.0, dtype=torch.float32, device=DEV)
    am = torch.full((B,), 12345.0, dtype=torch.float32, device=DEV)
    sat = torch.full((B,), 999, dtype=torch.int64, device=DEV)
    L = dsg.lib()
    for _ in range(2):
        dsg._check(L.fp8ds_cast_batched(xd.data_ptr(), dsg.BF16, B, n, stride, fmt, s.data_ptr(),
                                        q.data_ptr(), stride, su.data_ptr(), am.data_ptr(),
                                        sat.data_ptr(), dsg._stream(None)))
    torch.cuda.synchronize()
    qn, amn, satn = q.cpu().numpy(), am.cpu().numpy().view(np.uint32), sat.cpu().numpy()
    for b in range(B):
        codes, oa, osat = oracle_cast(xw[b], fmt, scales[b])
        assert np.array_equal(qn[b, :n], codes), b
        assert amn[b] == oa and satn[b] == osat, (b, hex(amn[b]), hex(oa), satn[b], osat)
    assert np.array_equal(su.cpu().numpy(), scales)


@pytest.mark.parametrize("fmt", FMTS)
def test_stress_tensor_full_size(fmt):
    """The bandwidth-stress workload at its full size (2^30 bf16 elements): amax and
    saturation count exact over the whole tensor, bytes exact on a sample that
    includes every injected outlier."""
    n = 1 << 30
    print(f"[stress cast] fmt={fmt} n={n}", flush=True)
    bits = workloads.big_cast_input(n)
    x = dev_bf16(bits)
    s = 1.0
    q, _, su, am, sat = run_cast(x, fmt, s)
    del x
    torch.cuda.empty_cache()
    # exact amax and saturation count over everything (oracle, chunked)
    amax_all = np.float32(0.0)
    osat = 0
    step = 1 << 26
    for lo in range(0, n, step):
        xr = obf16.widen(bits[lo:lo + step])
        amax_all = max(amax_all, oamax.amax(xr))
        osat += ofp8.saturation_count(xr, s, fmt)
    assert am == f32_bits(amax_all)
    assert sat == osat
    if fmt == dsg.E4M3:
        assert osat == round(1e-5 * n)
    else:
        assert osat == 0
    rng = np.random.default_rng(99)
    pos = rng.choice(n, 1 << 20, replace=False)
    big = np.flatnonzero((bits & 0x7FFF) == 0x447A)  # the +-1000 outliers (bf16 0x447A = 1000)
    pos = np.unique(np.concatenate([pos, big, np.arange(64), np.arange(n - 64, n)]))
    codes, _ = ofp8.cast(obf16.widen(bits[pos]), np.float32(s), fmt)
    assert np.array_equal(q[pos], codes)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("base", [(1 << 28) - 4110, (1 << 28) + 12345])
def test_large_ragged_cast(bf16, base):
    """Tensors just below and past 2^28 elements, where the cast switches from
    workgroups of 8192 elements to its large-tensor shape (32768), with a ragged
    tail (not a whole number of pieces or workgroups): amax and saturation count
    exact over everything, bytes exact on a sample that includes both ends and
    every saturating element."""
    n = base + (3 if bf16 else 1)
    print(f"[large ragged cast] bf16={bf16} n={n}", flush=True)
    x = workloads.normal(n, 4242, 1.0)
    x[np.random.default_rng(5).choice(n, 997, replace=False)] = 1000.0  # saturate at s = 1
    scale = 1.0
    if bf16:
        bits = workloads.to_bf16_bits(x)
        q, _, su, am, sat = run_cast(dev_bf16(bits), dsg.E4M3, scale)
        get = lambda idx: obf16.widen(bits[idx])
    else:
        q, _, su, am, sat = run_cast(dev_f32(x), dsg.E4M3, scale)
        get = lambda idx: x[idx]
    assert su == scale
    assert sat == 997
    step = 1 << 24
    amax_all = max(oamax.amax(get(np.arange(lo, min(lo + step, n)))) for lo in range(0, n, step))
    assert am == f32_bits(amax_all)
    rng = np.random.default_rng(7)
    pos = np.unique(np.concatenate([rng.choice(n, 1 << 18, replace=False), np.arange(4096),
                                    np.arange(n - 40000, n),
                                    np.flatnonzero(x == 1000.0)]))
    codes, _ = ofp8.cast(get(pos), np.float32(scale), dsg.E4M3)
    assert np.array_equal(q[pos], codes)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("n", [(1 << 22) + 12345, (1 << 23) + 7])
def test_large_ragged_tensor_every_byte(fmt, bf16, n):
    """Tensors of 2^22 and 2^23 elements (many workgroups of 8192 elements): every
    byte, the amax and the saturation count of a ragged length (partial last
    workgroup, partial groups, a tail below one 16-byte piece) against the oracle."""
    rng = np.random.default_rng(n + 2 * fmt + int(bf16))
    x32 = (rng.standard_normal(n) * 3.0).astype(np.float32)
    x32[rng.choice(n, 101, replace=False)] = 7.0e4  # saturate both formats
    if bf16:
        bits = (x32.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16, any pattern
        x_dev, xw = dev_bf16(bits), obf16.widen(bits)
    else:
        x_dev, xw = dev_f32(x32), x32
    s = np.float32(448.0) / np.float32(3.7)
    q, _, su, am, sat = run_cast(x_dev, fmt, s)
    codes, oa, osat = oracle_cast(xw, fmt, s)
    assert np.array_equal(q, codes)
    assert am == oa and sat == osat and su == np.float32(s)

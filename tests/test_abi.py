"""The C-ABI library loads and exports every symbol include/fp8ds.h declares, and its
host-side validation rejects bad arguments before touching the GPU (CPU only:
no compute call is made)."""

import ctypes
import os
import re

import pytest

import delayed_scaling_gemm_amd as dsg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8ds.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsg.LIB_PATH),
                                reason="libfp8ds.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8ds_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8ds_amax", "fp8ds_cast", "fp8ds_cast_batched", "fp8ds_scale_update",
              "fp8ds_gemm", "fp8ds_gemm_batched", "fp8ds_status_string", "fp8ds_last_error",
              "fp8ds_abi_version", "fp8ds_adamw", "fp8ds_cast_health", "fp8ds_cast_rowwise",
              "fp8ds_cast_current", "fp8ds_gemm_rowcol", "fp8ds_cast_mx", "fp8ds_gemm_mx",
              "fp8ds_cast_acc", "fp8ds_gemm_acc", "fp8ds_scale_update_clear",
              "fp8ds_linear_batched"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dsg.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert dsg.abi_version() == 8


def test_status_strings():
    L = dsg.lib()
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.fp8ds_status_string(s)
    assert L.fp8ds_status_string(-99) == b"unknown status"


def _status(call):
    return call, dsg.lib().fp8ds_last_error().decode()


def test_validation_errors_without_gpu():
    L = dsg.lib()
    p = 0x1000  # aligned, never dereferenced: validation fails first
    st, msg = _status(L.fp8ds_amax(p, 1, 16, None, None))
    assert st == -1 and "amax" in msg
    assert L.fp8ds_amax(p, 7, 16, p, None) == -3
    assert L.fp8ds_amax(p, 1, -1, p, None) == -2
    assert L.fp8ds_amax(p + 2, 1, 16, p, None) == -4
    # cast
    assert L.fp8ds_cast(p, 1, 4, 4, 0, None, p, None, None, None, None, None) == -1
    assert L.fp8ds_cast(p, 1, 4, 4, 5, p, p, None, None, None, None, None) == -3
    assert L.fp8ds_cast(p, 1, -4, 4, 0, p, p, None, None, None, None, None) == -2
    assert L.fp8ds_cast(p, 1, 4, 4, 0, p, p + 8, None, None, None, None, None) == -4
    assert L.fp8ds_cast(None, 1, 4, 4, 0, p, p, None, None, None, None, None) == -1
    # scale update
    fm = (ctypes.c_int * 2)(0, 1)
    fmp = ctypes.cast(fm, ctypes.c_void_p)
    assert L.fp8ds_scale_update(0, 16, p, p, p, fmp, 0, 0, p, None, None) == -2
    assert L.fp8ds_scale_update(2, 0, p, p, p, fmp, 0, 0, p, None, None) == -2
    assert L.fp8ds_scale_update(2, 16, p, p, p, fmp, 3, 0, p, None, None) == -3
    assert L.fp8ds_scale_update(2, 16, p, p, p, fmp, 0, 200, p, None, None) == -2
    assert L.fp8ds_scale_update(2, 16, None, p, p, fmp, 0, 0, p, None, None) == -1
    bad = (ctypes.c_int * 2)(0, 9)
    assert L.fp8ds_scale_update(2, 16, p, p, p, ctypes.cast(bad, ctypes.c_void_p), 0, 0, p, None,
                                None) == -3
    # gemm: TT unsupported, bad op, small ld, misaligned ld, null C
    args = dict(M=64, N=64, K=64)
    g = lambda opa, opb, lda, ldb, ldc, C=p, mma=0: L.fp8ds_gemm(opa, opb, 64, 64, 64, p, 0, lda, p,
                                                                p, 0, ldb, p, C, 1, ldc, None, mma,
                                                                None)
    assert g(1, 1, 64, 64, 64) == -6
    assert g(2, 0, 64, 64, 64) == -3
    assert g(0, 0, 32, 64, 64) == -2
    assert g(0, 0, 72, 64, 64) == -4
    assert g(0, 0, 64, 64, 64, C=None) == -1
    assert g(0, 0, 64, 64, 64, mma=2) == -3
    assert g(0, 0, 64, 64, 66) == -4
    # M x N whose 128 x 128 tile count does not fit the launch grid: shape error
    # before any pointer is looked at
    big = (1 << 31) - 1
    assert L.fp8ds_gemm(0, 1, big, big, 16, p, 0, 16, p, p, 0, 16, p, p, 1, big, None, 0,
                        None) == -2
    assert args


def test_adamw_validation_errors_without_gpu():
    L = dsg.lib()
    p = 0x1000
    hp = dict(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, gs=1.0, step=1)

    def call(w=p, g=p, gt=1, m=p, v=p, rows=4, cols=16, grad_amax=None, fmt=0, scale=p, q=p,
             q_t=None, scale_used=None, amax=None, sat=None, **kw):
        h = dict(hp, **kw)
        st = L.fp8ds_adamw(w, g, gt, m, v, rows, cols, h["lr"], h["b1"], h["b2"], h["eps"],
                           h["wd"], h["gs"], h["step"], grad_amax, fmt, scale, q, q_t, scale_used,
                           amax, sat, None)
        return st, L.fp8ds_last_error().decode()

    assert call(gt=5)[0] == -3
    assert call(fmt=7)[0] == -3
    assert call(rows=-1)[0] == -2
    for bad in (dict(b1=1.0), dict(b2=-0.1), dict(eps=0.0), dict(gs=0.0), dict(step=0),
                dict(lr=float("inf")), dict(wd=float("nan")), dict(eps=float("inf"))):
        st, msg = call(**bad)
        assert st == -7 and "fp8ds_adamw" in msg, bad
    assert call(q=None, q_t=p)[0] == -1        # a scale asks for q
    assert call(scale=None)[0] == -1           # q without a scale
    assert call(scale=None, q=None, amax=p)[0] == -1
    assert call(m=None)[0] == -1
    assert call(g=p + 4)[0] == -4
    assert call(q_t=p + 8)[0] == -4
    assert call(rows=65535 * 128 + 1, cols=1, q_t=p)[0] == -2


def test_finer_scaling_validation_errors_without_gpu():
    L = dsg.lib()
    p = 0x1000
    # fp8ds_cast_rowwise(x, xt, rows, cols, fmt, margin, q, scale, scale_inv, amax, stream)
    assert L.fp8ds_cast_rowwise(p, 5, 4, 16, 0, 0, p, p, None, None, None) == -3
    assert L.fp8ds_cast_rowwise(p, 1, 4, 16, 9, 0, p, p, None, None, None) == -3
    assert L.fp8ds_cast_rowwise(p, 1, -4, 16, 0, 0, p, p, None, None, None) == -2
    assert L.fp8ds_cast_rowwise(p, 1, 1 << 31, 1, 0, 0, p, p, None, None, None) == -2
    assert L.fp8ds_cast_rowwise(p, 1, 4, 16, 0, 200, p, p, None, None, None) == -2
    assert L.fp8ds_cast_rowwise(p, 1, 4, 16, 0, 0, p, None, None, None, None) == -1
    assert L.fp8ds_cast_rowwise(p, 1, 4, 16, 0, 0, p + 4, p, None, None, None) == -4
    # fp8ds_cast_current(x, xt, rows, cols, fmt, margin, q, q_t, scale, scale_inv, amax, sat, s)
    assert L.fp8ds_cast_current(p, 1, 4, 16, 0, 0, p, None, None, None, p, None, None) == -1
    assert L.fp8ds_cast_current(p, 1, 4, 16, 0, 0, p, None, p, None, None, None, None) == -1
    assert L.fp8ds_cast_current(p, 1, 4, 16, 0, -127, p, None, p, None, p, None, None) == -2
    assert L.fp8ds_cast_current(p, 1, 4, 16, 0, 0, p, p + 2, p, None, p, None, None) == -4
    # fp8ds_gemm_rowcol: TT, misaligned scale_inv_b, null scales
    g = lambda opa, opb, sa=p, sb=p: L.fp8ds_gemm_rowcol(opa, opb, 64, 64, 64, p, 0, 64, sa, p, 0,
                                                        64, sb, p, 1, 64, None, None)
    assert g(1, 1) == -6
    assert g(0, 1, sb=p + 4) == -4
    assert g(0, 1, sa=None) == -1


def test_mx_validation_errors_without_gpu():
    L = dsg.lib()
    p = 0x1000
    # fp8ds_cast_mx(x, xt, rows, cols, fmt, q, scales, q_t, scales_t, stream)
    c = lambda *a: L.fp8ds_cast_mx(*a)
    assert c(p, 1, 4, 48, 0, p, p, None, None, None) == -2     # cols not a multiple of 32
    assert c(p, 1, 4, 64, 5, p, p, None, None, None) == -3     # bad format
    assert c(p, 9, 4, 64, 0, p, p, None, None, None) == -3     # bad dtype
    assert c(p, 1, 4, 64, 0, p, None, None, None, None) == -1  # scales missing
    assert c(p + 8, 1, 4, 64, 0, p, p, None, None, None) == -4
    assert c(p, 1, 0, 64, 0, None, None, None, None, None) == 0  # empty: no-op
    assert c(p, 1, 128, 128, 0, p, p, p, None, None) == -1       # q_t without scales_t
    assert c(p, 1, 96, 128, 0, p, p, p, p, None) == -2           # transposed copy: rows % 128
    assert c(p, 1, 128, 128, 0, p, p, p + 4, p, None) == -4      # q_t misaligned
    # fp8ds_gemm_mx(M, N, K, A, fa, lda, sa, ldsa, B, fb, ldb, sb, ldsb, C, ct, ldc, amax, mma, s)
    g = lambda K=256, lda=256, sa=p, ldsa=8, sb=p, C=p, mma=0: L.fp8ds_gemm_mx(
        64, 64, K, p, 0, lda, sa, ldsa, p, 1, 256, sb, 8, C, 1, 64, None, mma, None)
    assert g(K=192, lda=192) == -2   # K not a multiple of 128
    assert g(lda=128) == -2          # lda < K
    assert g(ldsa=4) == -2           # scale leading dimension < K / 32
    assert g(sa=None) == -1
    assert g(C=None) == -1
    assert g(sb=p + 2) == -4         # scale array not 4-byte aligned
    assert g(ldsa=10) == -4          # scale leading dimension not a multiple of 4
    assert L.fp8ds_gemm_mx(64, 64, 256, p, 7, 256, p, 8, p, 0, 256, p, 8, p, 1, 64, None, 0,
                           None) == -3
    assert g(mma=5) == -3


def test_accumulating_variants_validate_like_the_plain_calls():
    """fp8ds_cast_acc and fp8ds_gemm_acc reject what fp8ds_cast and fp8ds_gemm
    reject; fp8ds_scale_update_clear checks its clear range (CPU only)."""
    L = dsg.lib()
    p = 0x1000
    assert L.fp8ds_cast_acc(p, 1, 4, 4, 0, None, p, None, None, None, None, None) == -1
    assert L.fp8ds_cast_acc(p, 1, 4, 4, 5, p, p, None, None, None, None, None) == -3
    assert L.fp8ds_cast_acc(p, 1, 4, 4, 0, p, p + 8, None, None, None, None, None) == -4
    assert L.fp8ds_gemm_acc(1, 1, 64, 64, 64, p, 0, 64, p, p, 0, 64, p, p, 1, 64, None, 0,
                            None) == -6
    assert L.fp8ds_gemm_acc(0, 1, 64, 64, 64, p, 0, 32, p, p, 0, 64, p, p, 1, 64, None, 0,
                            None) == -2
    fm = (ctypes.c_int * 2)(0, 1)
    fmp = ctypes.cast(fm, ctypes.c_void_p)
    clr = L.fp8ds_scale_update_clear
    assert clr(2, 16, p, p, p, fmp, 0, 0, p, None, p + 0x100, 6, None) == -2   # not a multiple of 4
    assert clr(2, 16, p, p, p, fmp, 0, 0, p, None, None, 8, None) == -1        # clear is null
    assert clr(2, 16, p, p, p, fmp, 0, 0, p, None, p + 0x102, 8, None) == -4   # misaligned
    assert clr(2, 16, p, p, p, fmp, 0, 0, p, None, p + 4, 8, None) == -7       # overlaps amax
    assert clr(0, 16, p, p, p, fmp, 0, 0, p, None, p + 0x100, 8, None) == -2   # as scale_update


def test_linear_batched_validation_errors_without_gpu():
    """fp8ds_linear_batched rejects bad sizes, enums, null pointers, short strides
    and misalignment before any launch (CPU only)."""
    L = dsg.lib()
    p = 0x1000

    def call(B=2, M=64, N=64, K=64, xt=1, x=p, sx=None, fx=0, w=p, sw=None, fw=0, L_=16,
             hist=p, cur=p, algo=0, margin=0, scale=p, su=None, amax=p, sat=None, xq=None,
             sxq=None, wq=None, swq=None, y=p, sy=None, amy=None):
        sx = M * K if sx is None else sx
        sw = K * N if sw is None else sw
        sy = M * N if sy is None else sy
        sxq = M * K if sxq is None else sxq
        swq = K * N if swq is None else swq
        st = L.fp8ds_linear_batched(B, M, N, K, xt, x, sx, fx, w, sw, fw, L_, hist, cur, algo,
                                    margin, scale, su, amax, sat, xq, sxq, wq, swq, y, sy, amy,
                                    None)
        return st, L.fp8ds_last_error().decode()

    assert call(xt=0)[0] == -6                      # FP32 inputs: not supported
    assert call(xt=3)[0] == -3
    assert call(fx=2)[0] == -3 and call(fw=-1)[0] == -3
    assert call(algo=2)[0] == -3
    for bad in (dict(B=0), dict(B=65536), dict(M=8), dict(N=272), dict(K=40), dict(L_=0),
                dict(margin=127), dict(sx=64 * 64 - 16), dict(sy=16), dict(xq=p, sxq=16)):
        st, msg = call(**bad)
        assert st == -2 and "fp8ds_linear_batched" in msg, bad
    for bad in (dict(x=None), dict(w=None), dict(hist=None), dict(cur=None), dict(scale=None),
                dict(amax=None), dict(y=None)):
        assert call(**bad)[0] == -1, bad
    for bad in (dict(x=p + 8), dict(y=p + 2), dict(xq=p + 4), dict(sx=64 * 64 + 4),
                dict(wq=p, swq=64 * 64 + 8)):
        assert call(**bad)[0] == -4, bad

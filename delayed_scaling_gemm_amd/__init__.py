"""FP8 delayed-scaling Linear for AMD MI355X (gfx950): Python binding.

This module only marshals arguments: it turns torch tensors (used for device
memory and streams) into the pointers and sizes of the C ABI declared in
``include/fp8ds.h`` and calls ``libfp8ds.so``.  Every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is not
built or cannot be loaded, every call raises.

Functions keep the C names: ``fp8ds_amax``, ``fp8ds_cast``, ``fp8ds_cast_batched``,
``fp8ds_scale_update``, ``fp8ds_gemm``, ``fp8ds_gemm_batched``.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8ds.so")

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
ALGO_MAX, ALGO_MOST_RECENT = 0, 1
OP_N, OP_T = 0, 1
MMA_EXACT, MMA_FP8 = 0, 1

FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

_lock = threading.Lock()
_lib = None


class Fp8dsError(RuntimeError):
    """A C-ABI call returned a negative status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"fp8ds status {status}: {message}")
        self.status = status


def _declare(lib):
    c = ctypes
    i64, vp, i32 = c.c_int64, c.c_void_p, c.c_int
    lib.fp8ds_abi_version.restype = i32
    lib.fp8ds_abi_version.argtypes = []
    lib.fp8ds_status_string.restype = c.c_char_p
    lib.fp8ds_status_string.argtypes = [i32]
    lib.fp8ds_last_error.restype = c.c_char_p
    lib.fp8ds_last_error.argtypes = []
    lib.fp8ds_amax.restype = i32
    lib.fp8ds_amax.argtypes = [vp, i32, i64, vp, vp]
    lib.fp8ds_cast.restype = i32
    lib.fp8ds_cast.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8ds_cast_batched.restype = i32
    lib.fp8ds_cast_batched.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i64, vp, vp, vp, vp]
    lib.fp8ds_scale_update.restype = i32
    lib.fp8ds_scale_update.argtypes = [i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.fp8ds_gemm.restype = i32
    lib.fp8ds_gemm.argtypes = [i32, i32, i64, i64, i64, vp, i32, i64, vp, vp, i32, i64, vp, vp, i32,
                               i64, vp, i32, vp]
    lib.fp8ds_gemm_batched.restype = i32
    lib.fp8ds_gemm_batched.argtypes = [i32, i32, i64, i64, i64, i64, vp, i32, i64, i64, vp, vp, i32,
                                       i64, i64, vp, vp, i32, i64, i64, vp, i32, vp]
    return lib


def lib():
    """The loaded ``libfp8ds.so`` (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built; run `python -m delayed_scaling_gemm_amd.build` "
                        "(the FP8 path has no CPU fallback)")
                _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().fp8ds_last_error().decode(errors="replace")
        raise Fp8dsError(status, msg)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def fp8ds_amax(x, amax, stream=None):
    """amax[0] = max |x| (fp32 device tensor of 1 element)."""
    _check(lib().fp8ds_amax(_ptr(x), _dtype_code(x), x.numel(), _ptr(amax), _stream(stream)))


def fp8ds_cast(x, fmt, scale, q, q_t=None, scale_used=None, amax=None, sat_count=None,
               stream=None):
    """Fused amax + scaled saturating cast of ``x`` ([rows, cols] or 1-D) into ``q`` (uint8)."""
    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    _check(lib().fp8ds_cast(_ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(scale), _ptr(q),
                            _ptr(q_t), _ptr(scale_used), _ptr(amax), _ptr(sat_count),
                            _stream(stream)))


def fp8ds_cast_batched(x, fmt, scale, q, scale_used=None, amax=None, sat_count=None, stream=None):
    """Casts of ``x[b]`` (a [batch, ...] tensor) with per-tensor ``scale[b]`` into ``q[b]``."""
    batch = x.shape[0]
    n = x[0].numel() if batch else 0
    _check(lib().fp8ds_cast_batched(_ptr(x), _dtype_code(x), batch, n,
                                    x.stride(0) if batch else n, fmt, _ptr(scale), _ptr(q),
                                    q.stride(0) if batch else n, _ptr(scale_used), _ptr(amax),
                                    _ptr(sat_count), _stream(stream)))


def fp8ds_scale_update(history, cursor, amax, fmts, algo, margin, scale, scale_inv=None,
                       stream=None):
    """Push ``amax[t]`` into ``history[t]`` and write the next ``scale[t]``.

    ``history`` is [n, L] fp32, ``cursor`` [n] int32, ``amax`` and ``scale`` [n] fp32,
    ``fmts`` a host sequence of n formats."""
    n, L = history.shape
    arr = (ctypes.c_int * n)(*[int(f) for f in fmts])
    _check(lib().fp8ds_scale_update(n, L, _ptr(history), _ptr(cursor), _ptr(amax),
                                    ctypes.cast(arr, ctypes.c_void_p), algo, margin, _ptr(scale),
                                    _ptr(scale_inv), _stream(stream)))


def fp8ds_gemm(opa, opb, M, N, K, a, fa, lda, scale_a, b, fb, ldb, scale_b, c, ldc, amax_c=None,
               stream=None, mma=MMA_EXACT):
    """``c = dequant(op(a) @ op(b))`` with FP32 accumulation; ``c`` is bf16 or fp32."""
    _check(lib().fp8ds_gemm(opa, opb, M, N, K, _ptr(a), fa, lda, _ptr(scale_a), _ptr(b), fb, ldb,
                            _ptr(scale_b), _ptr(c), _dtype_code(c), ldc, _ptr(amax_c), mma,
                            _stream(stream)))


def fp8ds_gemm_batched(opa, opb, M, N, K, batch, a, fa, lda, stride_a, scale_a, b, fb, ldb,
                       stride_b, scale_b, c, ldc, stride_c, amax_c=None, stream=None,
                       mma=MMA_EXACT):
    """``batch`` GEMMs of one shape with per-problem scales and output amax."""
    _check(lib().fp8ds_gemm_batched(opa, opb, M, N, K, batch, _ptr(a), fa, lda, stride_a,
                                    _ptr(scale_a), _ptr(b), fb, ldb, stride_b, _ptr(scale_b),
                                    _ptr(c), _dtype_code(c), ldc, stride_c, _ptr(amax_c), mma,
                                    _stream(stream)))


def abi_version() -> int:
    return lib().fp8ds_abi_version()

"""FP8 delayed-scaling Linear for AMD MI355X (gfx950): Python binding.

This module only marshals arguments: it turns torch tensors (used for device
memory and streams) into the pointers and sizes of the C ABI declared in
``include/fp8ds.h`` and calls ``libfp8ds.so``.  Every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is not
built or cannot be loaded, every call raises.

Functions keep the C names: ``fp8ds_amax``, ``fp8ds_cast``, ``fp8ds_cast_health``,
``fp8ds_cast_batched``, ``fp8ds_scale_update``, ``fp8ds_gemm``, ``fp8ds_gemm_batched``,
``fp8ds_linear_batched``, ``fp8ds_adamw``.
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
    lib.fp8ds_cast_acc.restype = i32
    lib.fp8ds_cast_acc.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8ds_scale_update_clear.restype = i32
    lib.fp8ds_scale_update_clear.argtypes = [i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, i64,
                                             vp]
    lib.fp8ds_gemm_acc.restype = i32
    lib.fp8ds_gemm_acc.argtypes = [i32, i32, i64, i64, i64, vp, i32, i64, vp, vp, i32, i64, vp, vp,
                                   i32, i64, vp, i32, vp]
    lib.fp8ds_cast_health.restype = i32
    lib.fp8ds_cast_health.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8ds_cast_batched.restype = i32
    lib.fp8ds_cast_batched.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i64, vp, vp, vp, vp]
    lib.fp8ds_scale_update.restype = i32
    lib.fp8ds_scale_update.argtypes = [i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.fp8ds_gemm.restype = i32
    lib.fp8ds_gemm.argtypes = [i32, i32, i64, i64, i64, vp, i32, i64, vp, vp, i32, i64, vp, vp, i32,
                               i64, vp, i32, vp]
    f = c.c_float
    lib.fp8ds_adamw.restype = i32
    lib.fp8ds_adamw.argtypes = [vp, vp, i32, vp, vp, i64, i64, f, f, f, f, f, f, i64, vp, i32, vp,
                                vp, vp, vp, vp, vp, vp]
    lib.fp8ds_cast_rowwise.restype = i32
    lib.fp8ds_cast_rowwise.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.fp8ds_cast_current.restype = i32
    lib.fp8ds_cast_current.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fp8ds_gemm_rowcol.restype = i32
    lib.fp8ds_gemm_rowcol.argtypes = [i32, i32, i64, i64, i64, vp, i32, i64, vp, vp, i32, i64, vp,
                                      vp, i32, i64, vp, vp]
    lib.fp8ds_cast_mx.restype = i32
    lib.fp8ds_cast_mx.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.fp8ds_gemm_mx.restype = i32
    lib.fp8ds_gemm_mx.argtypes = [i64, i64, i64, vp, i32, i64, vp, i64, vp, i32, i64, vp, i64, vp,
                                  i32, i64, vp, i32, vp]
    lib.fp8ds_gemm_batched.restype = i32
    lib.fp8ds_gemm_batched.argtypes = [i32, i32, i64, i64, i64, i64, vp, i32, i64, i64, vp, vp, i32,
                                       i64, i64, vp, vp, i32, i64, i64, vp, i32, vp]
    lib.fp8ds_linear_batched.restype = i32
    lib.fp8ds_linear_batched.argtypes = [i64, i64, i64, i64, i32, vp, i64, i32, vp, i64, i32, i32,
                                         vp, vp, i32, i32, vp, vp, vp, vp, vp, i64, vp, i64, vp,
                                         i64, vp, vp]
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


# While a launch sequence is being prepared (see `prepare`), the C calls are
# validated by their wrappers and recorded here instead of made.
_recording = threading.local()


def _call(name: str, *args):
    rec = getattr(_recording, "calls", None)
    if rec is not None:
        rec.append((getattr(lib(), name), args))
        return
    _check(getattr(lib(), name)(*args))


def prepare(fn):
    """Run ``fn()`` once with every library call it makes validated and recorded
    instead of launched; return a function that launches the recorded calls, in
    order, with the same arguments (the same tensors and stream) each time it is
    called.  For tight loops whose Python-side checks would otherwise cost more
    than the kernels: the step must not change Python-side state between calls
    (``BatchedDelayedScalingLinear.step`` does not; ``DelayedScalingLinear.step``
    alternates accumulator sets and must be called itself)."""
    if getattr(_recording, "calls", None) is not None:
        raise RuntimeError("prepare() does not nest")
    _recording.calls = []
    try:
        fn()
        calls = tuple(_recording.calls)
    finally:
        _recording.calls = None

    def launch():
        for f, args in calls:
            _check(f(*args))

    return launch


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


def _need(t, name, dtypes, n, contiguous=True):
    """Raise unless ``t`` (a torch tensor; raw integer pointers and None are not
    checked) is a CUDA tensor of one of ``dtypes`` with at least ``n`` elements
    addressable from its data pointer: a contiguous tensor of ``n`` elements
    when the C call reads it as a dense array, else enough storage past the
    pointer for the matrices that the leading dimensions describe.  The C ABI
    sees only pointers; this keeps a mis-sized or strided tensor from being read
    or written past its end."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if contiguous:
        if not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous tensor")
        avail = t.numel()
    else:  # addressed through leading dimensions: what the storage holds past data_ptr
        avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if avail < n:
        raise ValueError(f"{name}: {avail} elements reachable, at least {n} needed")


def _span(rows, cols, ld, batch=1, stride=0):
    """Elements addressed by ``batch`` row-major [rows x cols] matrices with
    leading dimension ``ld``, ``stride`` elements apart (0 when empty)."""
    if rows <= 0 or cols <= 0 or batch <= 0:
        return 0
    return (batch - 1) * stride + (rows - 1) * ld + cols


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def fp8ds_amax(x, amax, stream=None):
    """amax[0] = max |x| (fp32 device tensor of 1 element)."""
    import torch

    _need(x, "x", (torch.bfloat16, torch.float32), 0)
    _need(amax, "amax", (torch.float32,), 1)
    _call("fp8ds_amax", _ptr(x), _dtype_code(x), x.numel(), _ptr(amax), _stream(stream))


def fp8ds_cast(x, fmt, scale, q, q_t=None, scale_used=None, amax=None, sat_count=None,
               stream=None):
    """Fused amax + scaled saturating cast of ``x`` ([rows, cols] or 1-D) into ``q`` (uint8)."""
    import torch

    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), 0)
    _need(q, "q", (torch.uint8,), rows * cols)
    _need(q_t, "q_t", (torch.uint8,), rows * cols)
    _need(scale, "scale", f32, 1)
    _need(scale_used, "scale_used", f32, 1)
    _need(amax, "amax", f32, 1)
    _need(sat_count, "sat_count", (torch.int64,), 1)
    _call("fp8ds_cast", _ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(scale), _ptr(q),
          _ptr(q_t), _ptr(scale_used), _ptr(amax), _ptr(sat_count),
          _stream(stream))


def fp8ds_cast_acc(x, fmt, scale, q, q_t=None, scale_used=None, amax=None, sat_count=None,
                   stream=None):
    """:func:`fp8ds_cast` that max-/add-accumulates into ``amax`` / ``sat_count``."""
    import torch

    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), 0)
    _need(q, "q", (torch.uint8,), rows * cols)
    _need(q_t, "q_t", (torch.uint8,), rows * cols)
    _need(scale, "scale", f32, 1)
    _need(scale_used, "scale_used", f32, 1)
    _need(amax, "amax", f32, 1)
    _need(sat_count, "sat_count", (torch.int64,), 1)
    _call("fp8ds_cast_acc", _ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(scale), _ptr(q),
          _ptr(q_t), _ptr(scale_used), _ptr(amax), _ptr(sat_count),
          _stream(stream))


HEALTH_COUNTS = 5
HEALTH_NAMES = ("saturated", "nan", "inf", "zero", "near_max")


def fp8ds_cast_health(x, fmt, scale, q, counts, q_t=None, scale_used=None, amax=None,
                      stream=None):
    """``fp8ds_cast`` plus the health counts of the same pass into ``counts``
    (int64 device tensor of ``HEALTH_COUNTS``: saturated, NaN inputs, infinite
    inputs, zero codes, top-binade codes)."""
    import torch

    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), 0)
    _need(q, "q", (torch.uint8,), rows * cols)
    _need(q_t, "q_t", (torch.uint8,), rows * cols)
    _need(scale, "scale", f32, 1)
    _need(scale_used, "scale_used", f32, 1)
    _need(amax, "amax", f32, 1)
    if counts is None:
        raise ValueError("counts is required")
    _need(counts, "counts", (torch.int64,), HEALTH_COUNTS)
    _call("fp8ds_cast_health", _ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(scale), _ptr(q),
          _ptr(q_t), _ptr(scale_used), _ptr(amax), _ptr(counts),
          _stream(stream))


def fp8ds_cast_batched(x, fmt, scale, q, scale_used=None, amax=None, sat_count=None, stream=None):
    """Casts of ``x[b]`` (a [batch, ...] tensor) with per-tensor ``scale[b]`` into ``q[b]``."""
    import torch

    batch = x.shape[0]
    n = x[0].numel() if batch else 0
    if batch and not (x[0].is_contiguous() and q[0].is_contiguous()):
        raise ValueError("x[b] and q[b] must be contiguous")
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), _span(batch, n, x.stride(0) if batch else n),
          contiguous=False)
    _need(q, "q", (torch.uint8,), _span(batch, n, q.stride(0) if batch else n), contiguous=False)
    _need(scale, "scale", f32, batch)
    _need(scale_used, "scale_used", f32, batch)
    _need(amax, "amax", f32, batch)
    _need(sat_count, "sat_count", (torch.int64,), batch)
    _call("fp8ds_cast_batched", _ptr(x), _dtype_code(x), batch, n,
          x.stride(0) if batch else n, fmt, _ptr(scale), _ptr(q),
          q.stride(0) if batch else n, _ptr(scale_used), _ptr(amax),
          _ptr(sat_count), _stream(stream))


def fp8ds_scale_update(history, cursor, amax, fmts, algo, margin, scale, scale_inv=None,
                       stream=None):
    """Push ``amax[t]`` into ``history[t]`` and write the next ``scale[t]``.

    ``history`` is [n, L] fp32, ``cursor`` [n] int32, ``amax`` and ``scale`` [n] fp32,
    ``fmts`` a host sequence of n formats."""
    import torch

    n, L = history.shape
    if len(fmts) < n:
        raise ValueError(f"fmts: {len(fmts)} formats for {n} tensors")
    f32 = (torch.float32,)
    _need(history, "history", f32, n * L)
    _need(cursor, "cursor", (torch.int32,), n)
    _need(amax, "amax", f32, n)
    _need(scale, "scale", f32, n)
    _need(scale_inv, "scale_inv", f32, n)
    arr = (ctypes.c_int * n)(*[int(f) for f in fmts[:n]])
    _call("fp8ds_scale_update", n, L, _ptr(history), _ptr(cursor), _ptr(amax),
          ctypes.cast(arr, ctypes.c_void_p), algo, margin, _ptr(scale),
          _ptr(scale_inv), _stream(stream))


def fp8ds_scale_update_clear(history, cursor, amax, fmts, algo, margin, scale, clear,
                             scale_inv=None, stream=None):
    """:func:`fp8ds_scale_update` that also zeroes the device tensor ``clear`` (the
    next step's accumulators; contiguous, 4-byte elements or wider)."""
    import torch

    n, L = history.shape
    if len(fmts) < n:
        raise ValueError(f"fmts: {len(fmts)} formats for {n} tensors")
    f32 = (torch.float32,)
    _need(history, "history", f32, n * L)
    _need(cursor, "cursor", (torch.int32,), n)
    _need(amax, "amax", f32, n)
    _need(scale, "scale", f32, n)
    _need(scale_inv, "scale_inv", f32, n)
    if not clear.is_cuda or not clear.is_contiguous():
        raise ValueError("clear: expected a contiguous CUDA tensor")
    arr = (ctypes.c_int * n)(*[int(f) for f in fmts[:n]])
    _call("fp8ds_scale_update_clear", n, L, _ptr(history), _ptr(cursor), _ptr(amax),
          ctypes.cast(arr, ctypes.c_void_p), algo, margin,
          _ptr(scale), _ptr(scale_inv), _ptr(clear),
          clear.numel() * clear.element_size(), _stream(stream))


def _check_gemm(opa, opb, M, N, K, batch, a, lda, stride_a, scale_a, b, ldb, stride_b, scale_b, c,
                ldc, stride_c, amax_c):
    """Tensor arguments cover the matrices the C call will address (the C ABI
    itself validates the sizes, leading dimensions and alignment)."""
    import torch

    if min(M, N, K, batch) < 0:
        return  # the C call reports the bad size
    ra, ca = (M, K) if opa == OP_N else (K, M)
    rb, cb = (K, N) if opb == OP_N else (N, K)
    f32 = (torch.float32,)
    _need(amax_c, "amax_c", f32, batch)
    if M == 0 or N == 0 or batch == 0:
        return  # nothing but the output amax is touched
    if K > 0:
        _need(a, "a", (torch.uint8,), _span(ra, ca, lda, batch, stride_a), contiguous=False)
        _need(b, "b", (torch.uint8,), _span(rb, cb, ldb, batch, stride_b), contiguous=False)
    _need(c, "c", (torch.bfloat16, torch.float32), _span(M, N, ldc, batch, stride_c),
          contiguous=False)
    _need(scale_a, "scale_a", f32, batch)
    _need(scale_b, "scale_b", f32, batch)


def fp8ds_gemm(opa, opb, M, N, K, a, fa, lda, scale_a, b, fb, ldb, scale_b, c, ldc, amax_c=None,
               stream=None, mma=MMA_EXACT):
    """``c = dequant(op(a) @ op(b))`` with FP32 accumulation; ``c`` is bf16 or fp32."""
    _check_gemm(opa, opb, M, N, K, 1, a, lda, 0, scale_a, b, ldb, 0, scale_b, c, ldc, 0, amax_c)
    _call("fp8ds_gemm", opa, opb, M, N, K, _ptr(a), fa, lda, _ptr(scale_a), _ptr(b), fb, ldb,
          _ptr(scale_b), _ptr(c), _dtype_code(c), ldc, _ptr(amax_c), mma,
          _stream(stream))


def fp8ds_gemm_acc(opa, opb, M, N, K, a, fa, lda, scale_a, b, fb, ldb, scale_b, c, ldc,
                   amax_c=None, stream=None, mma=MMA_EXACT):
    """:func:`fp8ds_gemm` that max-accumulates the output amax into ``amax_c``."""
    _check_gemm(opa, opb, M, N, K, 1, a, lda, 0, scale_a, b, ldb, 0, scale_b, c, ldc, 0, amax_c)
    _call("fp8ds_gemm_acc", opa, opb, M, N, K, _ptr(a), fa, lda, _ptr(scale_a), _ptr(b), fb,
          ldb, _ptr(scale_b), _ptr(c), _dtype_code(c), ldc, _ptr(amax_c),
          mma, _stream(stream))


def fp8ds_gemm_batched(opa, opb, M, N, K, batch, a, fa, lda, stride_a, scale_a, b, fb, ldb,
                       stride_b, scale_b, c, ldc, stride_c, amax_c=None, stream=None,
                       mma=MMA_EXACT):
    """``batch`` GEMMs of one shape with per-problem scales and output amax."""
    _check_gemm(opa, opb, M, N, K, batch, a, lda, stride_a, scale_a, b, ldb, stride_b, scale_b, c,
                ldc, stride_c, amax_c)
    _call("fp8ds_gemm_batched", opa, opb, M, N, K, batch, _ptr(a), fa, lda, stride_a,
          _ptr(scale_a), _ptr(b), fb, ldb, stride_b, _ptr(scale_b),
          _ptr(c), _dtype_code(c), ldc, stride_c, _ptr(amax_c), mma,
          _stream(stream))


def fp8ds_linear_batched(x, w, fx, fw, history, cursor, algo, margin, scale, amax, y,
                         scale_used=None, sat_count=None, xq=None, wq=None, amax_y=None,
                         stream=None):
    """Forward step of ``batch`` small Linears in one launch: ``x`` [B, M, K] and
    ``w`` [B, K, N] (bf16, contiguous) are cast with their delayed scales
    (``scale[i]`` for X_i, ``scale[B + i]`` for W_i; codes into ``xq``, ``wq``),
    ``y`` [B, M, N] bf16 = the exact-datapath products, and the 2B tensors'
    ``history`` [2B, L], ``cursor``, ``scale`` are updated with this step's
    ``amax`` [2B]."""
    import torch

    B, M, K = x.shape
    B2, K2, N = w.shape
    if B2 != B or K2 != K:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} do not match")
    n, L = history.shape
    if n != 2 * B:
        raise ValueError(f"history: {n} tensors for a batch of {B}")
    bf, f32 = (torch.bfloat16,), (torch.float32,)
    _need(x, "x", bf, B * M * K)
    _need(w, "w", bf, B * K * N)
    _need(y, "y", bf, B * M * N)
    _need(xq, "xq", (torch.uint8,), B * M * K)
    _need(wq, "wq", (torch.uint8,), B * K * N)
    _need(history, "history", f32, n * L)
    _need(cursor, "cursor", (torch.int32,), n)
    for t, name in ((scale, "scale"), (amax, "amax"), (scale_used, "scale_used")):
        _need(t, name, f32, n)
    _need(sat_count, "sat_count", (torch.int64,), n)
    _need(amax_y, "amax_y", f32, B)
    _call("fp8ds_linear_batched", B, M, N, K, BF16, _ptr(x), M * K, fx, _ptr(w), K * N, fw, L,
          _ptr(history), _ptr(cursor), algo, margin, _ptr(scale),
          _ptr(scale_used), _ptr(amax), _ptr(sat_count), _ptr(xq),
          M * K, _ptr(wq), K * N, _ptr(y), M * N, _ptr(amax_y),
          _stream(stream))


def fp8ds_adamw(w, g, m, v, lr, beta1, beta2, eps, weight_decay, step, grad_scale=1.0,
                grad_amax=None, fmt=E4M3, scale=None, q=None, q_t=None, scale_used=None,
                amax=None, sat_count=None, stream=None):
    """Fused AdamW step on the fp32 master weights ``w`` ([rows, cols] or 1-D),
    moments ``m``, ``v`` (fp32, in place) with gradient ``g`` (bf16 or fp32), step
    count ``step`` >= 1; with ``scale`` also the FP8 copy of the new weights into
    ``q`` (uint8; ``q_t`` transposed, ``scale_used``, ``amax``, ``sat_count`` as
    ``fp8ds_cast``).
    ``grad_amax`` (fp32 device scalar): a non-finite value skips the update."""
    import torch

    rows, cols = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, w.numel())
    n = rows * cols
    f32 = (torch.float32,)
    for t, name in ((w, "w"), (m, "m"), (v, "v")):
        if t is None:
            raise ValueError(f"{name} is required")
        _need(t, name, f32, n)
    if g is None:
        raise ValueError("g is required")
    _need(g, "g", (torch.bfloat16, torch.float32), n)
    _need(grad_amax, "grad_amax", f32, 1)
    _need(q, "q", (torch.uint8,), n)
    _need(q_t, "q_t", (torch.uint8,), n)
    _need(scale, "scale", f32, 1)
    _need(scale_used, "scale_used", f32, 1)
    _need(amax, "amax", f32, 1)
    _need(sat_count, "sat_count", (torch.int64,), 1)
    _call("fp8ds_adamw", _ptr(w), _ptr(g), _dtype_code(g), _ptr(m), _ptr(v), rows, cols,
          float(lr), float(beta1), float(beta2), float(eps),
          float(weight_decay), float(grad_scale), int(step), _ptr(grad_amax),
          fmt, _ptr(scale), _ptr(q), _ptr(q_t), _ptr(scale_used), _ptr(amax),
          _ptr(sat_count), _stream(stream))



def fp8ds_cast_rowwise(x, fmt, margin, q, scale, scale_inv=None, amax=None, stream=None):
    """Per-row current scaling of the 2-D ``x`` into ``q`` (uint8) with
    ``scale`` / ``scale_inv`` / ``amax`` per row (fp32 device tensors of rows)."""
    import torch

    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), rows * cols)
    _need(q, "q", (torch.uint8,), rows * cols)
    if scale is None:
        raise ValueError("scale is required")
    _need(scale, "scale", f32, rows)
    _need(scale_inv, "scale_inv", f32, rows)
    _need(amax, "amax", f32, rows)
    _call("fp8ds_cast_rowwise", _ptr(x), _dtype_code(x), rows, cols, fmt, int(margin), _ptr(q),
          _ptr(scale), _ptr(scale_inv), _ptr(amax), _stream(stream))


def fp8ds_cast_current(x, fmt, margin, q, scale, amax, q_t=None, scale_inv=None, sat_count=None,
                       stream=None):
    """Per-tensor current scaling: amax of ``x``, its scale, then the cast."""
    import torch

    rows, cols = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.numel())
    f32 = (torch.float32,)
    _need(x, "x", (torch.bfloat16, torch.float32), rows * cols)
    _need(q, "q", (torch.uint8,), rows * cols)
    _need(q_t, "q_t", (torch.uint8,), rows * cols)
    if scale is None or amax is None:
        raise ValueError("scale and amax are required")
    _need(scale, "scale", f32, 1)
    _need(amax, "amax", f32, 1)
    _need(scale_inv, "scale_inv", f32, 1)
    _need(sat_count, "sat_count", (torch.int64,), 1)
    _call("fp8ds_cast_current", _ptr(x), _dtype_code(x), rows, cols, fmt, int(margin), _ptr(q),
          _ptr(q_t), _ptr(scale), _ptr(scale_inv), _ptr(amax),
          _ptr(sat_count), _stream(stream))


def fp8ds_gemm_rowcol(opa, opb, M, N, K, a, fa, lda, scale_inv_a, b, fb, ldb, scale_inv_b, c, ldc,
                      amax_c=None, stream=None):
    """GEMM with an inverse scale per row of op(A) (``scale_inv_a`` [M]) and per
    column of op(B) (``scale_inv_b`` [N]); exact datapath."""
    import torch

    _check_gemm(opa, opb, M, N, K, 1, a, lda, 0, None, b, ldb, 0, None, c, ldc, 0, amax_c)
    _need(scale_inv_a, "scale_inv_a", (torch.float32,), M)
    _need(scale_inv_b, "scale_inv_b", (torch.float32,), N)
    _call("fp8ds_gemm_rowcol", opa, opb, M, N, K, _ptr(a), fa, lda, _ptr(scale_inv_a), _ptr(b),
          fb, ldb, _ptr(scale_inv_b), _ptr(c), _dtype_code(c), ldc,
          _ptr(amax_c), _stream(stream))


def fp8ds_cast_mx(x, fmt, q, scales, q_t=None, scales_t=None, stream=None):
    """MXFP8 cast of the 2-D ``x`` [rows, cols] (cols a multiple of 32) along its
    rows: element codes into ``q`` (uint8 [rows, cols]) and one E8M0 code per
    block of 32 into ``scales`` (uint8 [rows, cols / 32]); optionally the
    transpose blocked along its own rows into ``q_t`` [cols, rows] and
    ``scales_t`` [cols, rows / 32] (rows and cols multiples of 128)."""
    import torch

    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    _need(x, "x", (torch.bfloat16, torch.float32), rows * cols)
    _need(q, "q", (torch.uint8,), rows * cols)
    _need(scales, "scales", (torch.uint8,), rows * cols // 32)
    _need(q_t, "q_t", (torch.uint8,), rows * cols)
    _need(scales_t, "scales_t", (torch.uint8,), rows * cols // 32)
    _call("fp8ds_cast_mx", _ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(q), _ptr(scales),
          _ptr(q_t), _ptr(scales_t), _stream(stream))


def fp8ds_gemm_mx(M, N, K, a, fa, lda, scales_a, ld_scales_a, b, fb, ldb, scales_b, ld_scales_b,
                  c, ldc, amax_c=None, stream=None, mma=MMA_EXACT):
    """MXFP8 GEMM ``C = A B^T``: A [M, K] and B [N, K] element codes with E8M0
    block scales [M, ld_scales_a] / [N, ld_scales_b] along K; K a multiple of 128."""
    import torch

    for t, name, n in ((a, "a", _span(M, K, lda)), (b, "b", _span(N, K, ldb)),
                       (scales_a, "scales_a", _span(M, K // 32, ld_scales_a)),
                       (scales_b, "scales_b", _span(N, K // 32, ld_scales_b))):
        _need(t, name, (torch.uint8,), n, contiguous=False)
    _need(c, "c", (torch.bfloat16, torch.float32), _span(M, N, ldc), contiguous=False)
    _need(amax_c, "amax_c", (torch.float32,), 1)
    _call("fp8ds_gemm_mx", M, N, K, _ptr(a), fa, lda, _ptr(scales_a), ld_scales_a, _ptr(b), fb,
          ldb, _ptr(scales_b), ld_scales_b, _ptr(c), _dtype_code(c), ldc,
          _ptr(amax_c), mma, _stream(stream))


def abi_version() -> int:
    return lib().fp8ds_abi_version()

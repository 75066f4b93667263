// C ABI of the FP8 delayed-scaling Linear: host-side validation, error
// reporting and dispatch to the HIP launchers.  See include/fp8ds.h for the
// contract of each entry point.

#include "fp8ds.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return FP8DS_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FP8DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;

// Compute units of the current device, cached per device id.
int num_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool valid_fmt(int f) { return f == FP8DS_E4M3 || f == FP8DS_E5M2; }
bool valid_dtype(int t) { return t == FP8DS_F32 || t == FP8DS_BF16; }

}  // namespace

extern "C" {

int fp8ds_abi_version(void) { return FP8DS_ABI_VERSION; }

const char* fp8ds_status_string(int status) {
  switch (status) {
    case FP8DS_OK: return "ok";
    case FP8DS_ERR_NULL: return "required pointer is null";
    case FP8DS_ERR_SHAPE: return "invalid size or leading dimension";
    case FP8DS_ERR_ENUM: return "enum value out of range";
    case FP8DS_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case FP8DS_ERR_HIP: return "HIP runtime error";
    case FP8DS_ERR_UNSUPPORTED: return "unsupported combination";
    case FP8DS_ERR_VALUE: return "scalar argument out of range";
    default: return "unknown status";
  }
}

const char* fp8ds_last_error(void) { return g_err; }

int fp8ds_amax(const void* x, fp8ds_dtype xt, int64_t n, float* amax, hipStream_t stream) {
  if (!amax) return fail(FP8DS_ERR_NULL, "fp8ds_amax: amax is null");
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "fp8ds_amax: bad dtype %d", (int)xt);
  if (n < 0 || n > kMaxElems) return fail(FP8DS_ERR_SHAPE, "fp8ds_amax: bad n %lld", (long long)n);
  if (n > 0 && !x) return fail(FP8DS_ERR_NULL, "fp8ds_amax: x is null");
  if (n > 0 && !aligned16(x)) return fail(FP8DS_ERR_ALIGN, "fp8ds_amax: x not 16-byte aligned");
  hipError_t e = fp8ds::launch_prologue(1, nullptr, nullptr, amax, nullptr, stream);
  if (e == hipSuccess && n > 0)
    e = fp8ds::launch_cast(x, xt == FP8DS_BF16, 1, n, n, 0, nullptr, nullptr, 0, amax, nullptr,
                           nullptr, num_cus(), stream);
  return hip_status(e, "fp8ds_amax");
}

// acc: amax / sat_count are combined into (max / add) instead of reset, and the
// cast kernel writes scale_used itself: no reset kernel before the cast.
static int cast_common(const char* who, const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols,
                       fp8ds_format fmt, const float* scale, uint8_t* q, uint8_t* q_t,
                       float* scale_used, float* amax, uint64_t* sat_count, uint64_t* health,
                       hipStream_t stream, bool acc = false) {
  if (!scale) return fail(FP8DS_ERR_NULL, "%s: scale is null", who);
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "%s: bad dtype %d", who, (int)xt);
  if (!valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "%s: bad format %d", who, (int)fmt);
  if (rows < 0 || cols < 0 || (cols > 0 && rows > kMaxElems / cols))
    return fail(FP8DS_ERR_SHAPE, "%s: bad shape %lld x %lld", who, (long long)rows,
                (long long)cols);
  const int64_t n = rows * cols;
  if (n > 0) {
    if (!x || !q) return fail(FP8DS_ERR_NULL, "%s: x or q is null", who);
    if (!aligned16(x) || !aligned16(q) || (q_t && !aligned16(q_t)))
      return fail(FP8DS_ERR_ALIGN, "%s: x, q and q_t must be 16-byte aligned", who);
  }
  if (q_t && (rows + 127) / 128 > 65535)
    return fail(FP8DS_ERR_SHAPE, "%s: a transposed copy supports at most %d rows", who,
                65535 * 128);
  hipError_t e = hipSuccess;
  if (!acc)  // with health counts, sat_count is counts[0] and the four others follow it
    e = fp8ds::launch_prologue(1, scale, scale_used, amax, sat_count, stream,
                               health ? FP8DS_HEALTH_COUNTS : 1);
  else if (n == 0)  // nothing to combine; the snapshot is still written
    e = fp8ds::launch_prologue(1, scale, scale_used, nullptr, nullptr, stream);
  float* snap = acc ? scale_used : nullptr;
  if (e == hipSuccess && n > 0) {
    if (q_t)
      e = fp8ds::launch_cast_transpose(x, xt == FP8DS_BF16, rows, cols, (int)fmt, scale, q, q_t,
                                       amax, sat_count, health, stream, snap);
    else
      e = fp8ds::launch_cast(x, xt == FP8DS_BF16, 1, n, n, (int)fmt, scale, q, n, amax, sat_count,
                             health, num_cus(), stream, snap);
  }
  return hip_status(e, who);
}

int fp8ds_cast(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
               const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
               uint64_t* sat_count, hipStream_t stream) {
  return cast_common("fp8ds_cast", x, xt, rows, cols, fmt, scale, q, q_t, scale_used, amax,
                     sat_count, nullptr, stream);
}

int fp8ds_cast_acc(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                   const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                   uint64_t* sat_count, hipStream_t stream) {
  return cast_common("fp8ds_cast_acc", x, xt, rows, cols, fmt, scale, q, q_t, scale_used, amax,
                     sat_count, nullptr, stream, true);
}

int fp8ds_cast_health(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                      const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                      uint64_t* counts, hipStream_t stream) {
  if (!counts) return fail(FP8DS_ERR_NULL, "fp8ds_cast_health: counts is null");
  return cast_common("fp8ds_cast_health", x, xt, rows, cols, fmt, scale, q, q_t, scale_used, amax,
                     counts, counts + 1, stream);
}

int fp8ds_cast_batched(const void* x, fp8ds_dtype xt, int64_t batch, int64_t n, int64_t stride_x,
                       fp8ds_format fmt, const float* scale, uint8_t* q, int64_t stride_q,
                       float* scale_used, float* amax, uint64_t* sat_count, hipStream_t stream) {
  if (!scale) return fail(FP8DS_ERR_NULL, "fp8ds_cast_batched: scale is null");
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "fp8ds_cast_batched: bad dtype %d", (int)xt);
  if (!valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "fp8ds_cast_batched: bad format %d", (int)fmt);
  if (batch < 0 || batch > 65535 || n < 0 || n > kMaxElems)
    return fail(FP8DS_ERR_SHAPE, "fp8ds_cast_batched: bad batch %lld or n %lld", (long long)batch,
                (long long)n);
  if (batch == 0) return ok();
  const int esz = xt == FP8DS_BF16 ? 2 : 4;
  if (n > 0) {
    if (!x || !q) return fail(FP8DS_ERR_NULL, "fp8ds_cast_batched: x or q is null");
    if (stride_x < n || stride_q < n || stride_x > kMaxElems || stride_q > kMaxElems)
      return fail(FP8DS_ERR_SHAPE, "fp8ds_cast_batched: strides must be >= n");
    if (!aligned16(x) || !aligned16(q) || (stride_x * esz) % 16 || stride_q % 16)
      return fail(FP8DS_ERR_ALIGN, "fp8ds_cast_batched: operands and strides must keep 16-byte "
                                   "alignment");
  }
  return hip_status(fp8ds::launch_cast_batched(x, xt == FP8DS_BF16, batch, n, stride_x, (int)fmt,
                                               scale, q, stride_q, scale_used, amax, sat_count,
                                               stream),
                    "fp8ds_cast_batched");
}

static int scale_update_common(const char* who, int n_tensors, int hist_len, float* history,
                               int32_t* cursor, const float* amax, const fp8ds_format* fmt,
                               fp8ds_algo algo, int margin, float* scale, float* scale_inv,
                               void* clear, int64_t clear_bytes, hipStream_t stream);

int fp8ds_scale_update(int n_tensors, int hist_len, float* history, int32_t* cursor,
                       const float* amax, const fp8ds_format* fmt, fp8ds_algo algo, int margin,
                       float* scale, float* scale_inv, hipStream_t stream) {
  return scale_update_common("fp8ds_scale_update", n_tensors, hist_len, history, cursor, amax,
                             fmt, algo, margin, scale, scale_inv, nullptr, 0, stream);
}

int fp8ds_scale_update_clear(int n_tensors, int hist_len, float* history, int32_t* cursor,
                             const float* amax, const fp8ds_format* fmt, fp8ds_algo algo,
                             int margin, float* scale, float* scale_inv, void* clear,
                             int64_t clear_bytes, hipStream_t stream) {
  const char* who = "fp8ds_scale_update_clear";
  if (clear_bytes < 0 || clear_bytes % 4 || clear_bytes > (int64_t(1) << 30))
    return fail(FP8DS_ERR_SHAPE, "%s: clear_bytes %lld must be a multiple of 4 in [0, 2^30]", who,
                (long long)clear_bytes);
  if (clear_bytes > 0 && !clear) return fail(FP8DS_ERR_NULL, "%s: clear is null", who);
  if (clear && (reinterpret_cast<uintptr_t>(clear) & 3u))
    return fail(FP8DS_ERR_ALIGN, "%s: clear must be 4-byte aligned", who);
  if (clear && amax && n_tensors > 0) {
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(clear), c1 = c0 + (uintptr_t)clear_bytes;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(amax), a1 = a0 + 4u * (uintptr_t)n_tensors;
    if (c0 < a1 && a0 < c1)
      return fail(FP8DS_ERR_VALUE, "%s: the cleared bytes overlap the amax being consumed", who);
  }
  return scale_update_common(who, n_tensors, hist_len, history, cursor, amax, fmt, algo, margin,
                             scale, scale_inv, clear, clear_bytes, stream);
}

static int scale_update_common(const char* who, int n_tensors, int hist_len, float* history,
                               int32_t* cursor, const float* amax, const fp8ds_format* fmt,
                               fp8ds_algo algo, int margin, float* scale, float* scale_inv,
                               void* clear, int64_t clear_bytes, hipStream_t stream) {
  if (n_tensors < 1 || n_tensors > 4096)
    return fail(FP8DS_ERR_SHAPE, "%s: n_tensors %d not in [1, 4096]", who, n_tensors);
  if (hist_len < 1 || hist_len > 65536)
    return fail(FP8DS_ERR_SHAPE, "%s: hist_len %d not in [1, 65536]", who, hist_len);
  if (!history || !cursor || !amax || !fmt || !scale)
    return fail(FP8DS_ERR_NULL, "%s: history, cursor, amax, fmt and scale are "
                                "required", who);
  if (algo != FP8DS_ALGO_MAX && algo != FP8DS_ALGO_MOST_RECENT)
    return fail(FP8DS_ERR_ENUM, "%s: bad algo %d", who, (int)algo);
  if (margin < -126 || margin > 126)
    return fail(FP8DS_ERR_SHAPE, "%s: margin %d not in [-126, 126]", who, margin);
  fp8ds::FmtBits bits;
  std::memset(&bits, 0, sizeof(bits));
  for (int t = 0; t < n_tensors; ++t) {
    if (!valid_fmt(fmt[t]))
      return fail(FP8DS_ERR_ENUM, "%s: bad format %d for tensor %d", who, (int)fmt[t], t);
    if (fmt[t] == FP8DS_E5M2) bits.w[t >> 5] |= 1u << (t & 31);
  }
  return hip_status(fp8ds::launch_scale_update(n_tensors, hist_len, history, cursor, amax, bits,
                                               (int)algo, margin, scale, scale_inv, stream,
                                               static_cast<uint32_t*>(clear), clear_bytes / 4),
                    who);
}

static int gemm_common(const char* who, fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N,
                       int64_t K, int64_t batch, const uint8_t* A, fp8ds_format fa, int64_t lda,
                       int64_t stride_a, const float* scale_a, const uint8_t* B, fp8ds_format fb,
                       int64_t ldb, int64_t stride_b, const float* scale_b, void* C,
                       fp8ds_dtype ct, int64_t ldc, int64_t stride_c, float* amax_c,
                       fp8ds_mma mma, hipStream_t stream, bool rowcol = false,
                       bool reset = true) {
  // rowcol: scale_a / scale_b are inverse-scale vectors [M] / [N] (exact datapath)
  if (mma != FP8DS_MMA_EXACT && mma != FP8DS_MMA_FP8)
    return fail(FP8DS_ERR_ENUM, "%s: bad mma %d", who, (int)mma);
  if ((opa != FP8DS_OP_N && opa != FP8DS_OP_T) || (opb != FP8DS_OP_N && opb != FP8DS_OP_T))
    return fail(FP8DS_ERR_ENUM, "%s: bad op", who);
  if (opa == FP8DS_OP_T && opb == FP8DS_OP_T)
    return fail(FP8DS_ERR_UNSUPPORTED, "%s: (T, T) is not supported", who);
  if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8DS_ERR_ENUM, "%s: bad format", who);
  if (!valid_dtype(ct)) return fail(FP8DS_ERR_ENUM, "%s: bad output dtype", who);
  const int64_t lim = int64_t(1) << 31;
  if (M < 0 || N < 0 || K < 0 || M >= lim || N >= lim || K >= lim)
    return fail(FP8DS_ERR_SHAPE, "%s: bad M/N/K %lld/%lld/%lld", who, (long long)M, (long long)N,
                (long long)K);
  if (batch < 0 || batch > 65535) return fail(FP8DS_ERR_SHAPE, "%s: bad batch", who);
  // the launch grid counts 128 x 128 output tiles in one dimension
  if (((M + 127) / 128) * ((N + 127) / 128) >= lim)
    return fail(FP8DS_ERR_SHAPE, "%s: M x N %lld x %lld has too many tiles", who, (long long)M,
                (long long)N);
  if (M == 0 || N == 0 || batch == 0) {
    if (amax_c && batch > 0 && reset)
      return hip_status(fp8ds::launch_prologue(batch, nullptr, nullptr, amax_c, nullptr, stream),
                        who);
    return ok();
  }
  // Stored shapes: A is [M x K] (N) or [K x M] (T); B is [K x N] (N) or [N x K] (T).
  const int64_t a_cols = opa == FP8DS_OP_N ? K : M;
  const int64_t b_cols = opb == FP8DS_OP_N ? N : K;
  if (lda < a_cols || ldb < b_cols || ldc < N || lda < 1 || ldb < 1)
    return fail(FP8DS_ERR_SHAPE, "%s: leading dimension too small (lda %lld >= %lld, ldb %lld >= "
                "%lld, ldc %lld >= %lld)", who, (long long)lda, (long long)a_cols, (long long)ldb,
                (long long)b_cols, (long long)ldc, (long long)N);
  if (!C || !scale_a || !scale_b || (K > 0 && (!A || !B)))
    return fail(FP8DS_ERR_NULL, "%s: A, B, C and the two scales are required", who);
  if (rowcol && !aligned16(scale_b))
    return fail(FP8DS_ERR_ALIGN, "%s: scale_inv_b must be 16-byte aligned", who);
  const int esz = ct == FP8DS_BF16 ? 2 : 4;
  if ((K > 0 && (!aligned16(A) || !aligned16(B) || lda % 16 || ldb % 16)) || !aligned16(C) ||
      (ldc * esz) % 16)
    return fail(FP8DS_ERR_ALIGN, "%s: A, B, C and lda, ldb, ldc*elem_size must be 16-byte aligned",
                who);
  if (batch > 1 && (stride_a % 16 || stride_b % 16 || (stride_c * esz) % 16 || stride_a < 0 ||
                    stride_b < 0 || stride_c < 0))
    return fail(FP8DS_ERR_ALIGN, "%s: batch strides must keep 16-byte alignment", who);
  hipError_t e = hipSuccess;
  if (amax_c && reset) e = fp8ds::launch_prologue(batch, nullptr, nullptr, amax_c, nullptr, stream);
  if (e == hipSuccess) {
    fp8ds::GemmProblem p;
    p.opa = (int)opa; p.opb = (int)opb;
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.fa = (int)fa; p.lda = lda; p.scale_a = scale_a;
    p.B = B; p.fb = (int)fb; p.ldb = ldb; p.scale_b = scale_b;
    p.C = C; p.out_bf16 = ct == FP8DS_BF16; p.ldc = ldc; p.amax_c = amax_c;
    p.batch = batch; p.stride_a = stride_a; p.stride_b = stride_b; p.stride_c = stride_c;
    if (rowcol) {
      p.inv_a = scale_a;
      p.inv_b = scale_b;
      e = fp8ds::launch_gemm_rowcol(p, num_cus(), stream);
    } else {
      e = mma == FP8DS_MMA_EXACT ? fp8ds::launch_gemm_exact(p, num_cus(), stream)
                                 : fp8ds::launch_gemm_fp8(p, num_cus(), stream);
    }
  }
  return hip_status(e, who);
}

int fp8ds_gemm(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K, const uint8_t* A,
               fp8ds_format fa, int64_t lda, const float* scale_a, const uint8_t* B,
               fp8ds_format fb, int64_t ldb, const float* scale_b, void* C, fp8ds_dtype ct,
               int64_t ldc, float* amax_c, fp8ds_mma mma, hipStream_t stream) {
  return gemm_common("fp8ds_gemm", opa, opb, M, N, K, 1, A, fa, lda, 0, scale_a, B, fb, ldb, 0,
                     scale_b, C, ct, ldc, 0, amax_c, mma, stream);
}

int fp8ds_gemm_acc(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                   fp8ds_format fa, int64_t lda, const float* scale_a, const uint8_t* B,
                   fp8ds_format fb, int64_t ldb, const float* scale_b, void* C, fp8ds_dtype ct,
                   int64_t ldc, float* amax_c, fp8ds_mma mma, hipStream_t stream) {
  return gemm_common("fp8ds_gemm_acc", opa, opb, M, N, K, 1, A, fa, lda, 0, scale_a, B, fb, ldb, 0,
                     scale_b, C, ct, ldc, 0, amax_c, mma, stream, false, false);
}

int fp8ds_gemm_batched(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K, int64_t batch,
                       const uint8_t* A, fp8ds_format fa, int64_t lda, int64_t stride_a,
                       const float* scale_a, const uint8_t* B, fp8ds_format fb, int64_t ldb,
                       int64_t stride_b, const float* scale_b, void* C, fp8ds_dtype ct,
                       int64_t ldc, int64_t stride_c, float* amax_c, fp8ds_mma mma,
                       hipStream_t stream) {
  return gemm_common("fp8ds_gemm_batched", opa, opb, M, N, K, batch, A, fa, lda, stride_a, scale_a,
                     B, fb, ldb, stride_b, scale_b, C, ct, ldc, stride_c, amax_c, mma, stream);
}

int fp8ds_linear_batched(int64_t batch, int64_t M, int64_t N, int64_t K, fp8ds_dtype xt,
                         const void* x, int64_t stride_x, fp8ds_format fx, const void* w,
                         int64_t stride_w, fp8ds_format fw, int hist_len, float* history,
                         int32_t* cursor, fp8ds_algo algo, int margin, float* scale,
                         float* scale_used, float* amax, uint64_t* sat_count, uint8_t* xq,
                         int64_t stride_xq, uint8_t* wq, int64_t stride_wq, void* y,
                         int64_t stride_y, float* amax_y, hipStream_t stream) {
  const char* who = "fp8ds_linear_batched";
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "%s: bad dtype %d", who, (int)xt);
  if (xt != FP8DS_BF16) return fail(FP8DS_ERR_UNSUPPORTED, "%s: only BF16 inputs", who);
  if (!valid_fmt(fx) || !valid_fmt(fw)) return fail(FP8DS_ERR_ENUM, "%s: bad format", who);
  if (algo != FP8DS_ALGO_MAX && algo != FP8DS_ALGO_MOST_RECENT)
    return fail(FP8DS_ERR_ENUM, "%s: bad algo %d", who, (int)algo);
  if (batch < 1 || batch > 65535)
    return fail(FP8DS_ERR_SHAPE, "%s: batch %lld not in [1, 65535]", who, (long long)batch);
  auto dim_ok = [](int64_t v) { return v >= 16 && v <= 256 && v % 16 == 0; };
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K))
    return fail(FP8DS_ERR_SHAPE, "%s: M, N, K (%lld, %lld, %lld) must be multiples of 16 in "
                "[16, 256]", who, (long long)M, (long long)N, (long long)K);
  if (hist_len < 1 || hist_len > 65536)
    return fail(FP8DS_ERR_SHAPE, "%s: hist_len %d not in [1, 65536]", who, hist_len);
  if (margin < -126 || margin > 126)
    return fail(FP8DS_ERR_SHAPE, "%s: margin %d not in [-126, 126]", who, margin);
  if (!x || !w || !history || !cursor || !scale || !amax || !y)
    return fail(FP8DS_ERR_NULL, "%s: x, w, history, cursor, scale, amax and y are required", who);
  if (stride_x < M * K || stride_w < K * N || stride_y < M * N || (xq && stride_xq < M * K) ||
      (wq && stride_wq < K * N) || stride_x > kMaxElems || stride_w > kMaxElems ||
      stride_y > kMaxElems || stride_xq > kMaxElems || stride_wq > kMaxElems)
    return fail(FP8DS_ERR_SHAPE, "%s: every stride must be at least its problem's size", who);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (xq && !aligned16(xq)) ||
      (wq && !aligned16(wq)) || (stride_x * 2) % 16 || (stride_w * 2) % 16 ||
      (stride_y * 2) % 16 || (xq && stride_xq % 16) || (wq && stride_wq % 16))
    return fail(FP8DS_ERR_ALIGN, "%s: pointers and strides must keep 16-byte alignment", who);
  fp8ds::LinearBatchedArgs a;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.batch = (int)batch;
  a.x = static_cast<const uint16_t*>(x);
  a.stride_x = stride_x;
  a.w = static_cast<const uint16_t*>(w);
  a.stride_w = stride_w;
  a.xq = xq;
  a.stride_xq = xq ? stride_xq : 0;
  a.wq = wq;
  a.stride_wq = wq ? stride_wq : 0;
  a.y = static_cast<uint16_t*>(y);
  a.stride_y = stride_y;
  a.amax_y = amax_y;
  a.history = history;
  a.cursor = cursor;
  a.hist_len = hist_len;
  a.algo = (int)algo;
  a.margin = margin;
  a.scale = scale;
  a.scale_used = scale_used;
  a.amax = amax;
  a.sat = reinterpret_cast<unsigned long long*>(sat_count);
  return hip_status(fp8ds::launch_linear_batched(a, (int)fx, (int)fw, stream), who);
}

int fp8ds_adamw(float* w, const void* g, fp8ds_dtype gt, float* m, float* v, int64_t rows,
                int64_t cols, float lr, float beta1, float beta2, float eps, float weight_decay,
                float grad_scale, int64_t step, const float* grad_amax, fp8ds_format fmt,
                const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                uint64_t* sat_count, hipStream_t stream) {
#pragma clang fp contract(off)
  const char* who = "fp8ds_adamw";
  if (!valid_dtype(gt)) return fail(FP8DS_ERR_ENUM, "%s: bad gradient dtype %d", who, (int)gt);
  if (rows < 0 || cols < 0 || (cols > 0 && rows > kMaxElems / cols))
    return fail(FP8DS_ERR_SHAPE, "%s: bad shape %lld x %lld", who, (long long)rows,
                (long long)cols);
  if (!(std::isfinite(lr) && std::isfinite(weight_decay) && beta1 >= 0.0f && beta1 < 1.0f &&
        beta2 >= 0.0f && beta2 < 1.0f && std::isfinite(eps) && eps > 0.0f &&
        std::isfinite(grad_scale) && grad_scale > 0.0f && step >= 1))
    return fail(FP8DS_ERR_VALUE,
                "%s: need finite lr and weight_decay, 0 <= beta1, beta2 < 1, finite eps > 0, "
                "finite grad_scale > 0 and step >= 1",
                who);
  // the FP8 copy is requested by a scale
  const bool cast = scale != nullptr;
  if (cast && !valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "%s: bad format %d", who, (int)fmt);
  if (!cast && (q || q_t || scale_used || amax || sat_count))
    return fail(FP8DS_ERR_NULL, "%s: q, q_t, scale_used, amax and sat_count need scale", who);
  const int64_t n = rows * cols;
  if (n > 0) {
    if (!w || !g || !m || !v) return fail(FP8DS_ERR_NULL, "%s: w, g, m and v are required", who);
    if (cast && !q) return fail(FP8DS_ERR_NULL, "%s: q is null", who);
    if (!aligned16(w) || !aligned16(g) || !aligned16(m) || !aligned16(v) || (q && !aligned16(q)) ||
        (q_t && !aligned16(q_t)))
      return fail(FP8DS_ERR_ALIGN, "%s: w, g, m, v, q and q_t must be 16-byte aligned", who);
  }
  if (q_t && (rows + 127) / 128 > 65535)
    return fail(FP8DS_ERR_SHAPE, "%s: a transposed copy supports at most %d rows", who,
                65535 * 128);
  // Per-step constants: float64 from the fp32 hyperparameters, one rounding to fp32.
  const double lr_d = lr, wd_d = weight_decay, b1 = beta1, b2 = beta2;
  fp8ds::AdamWConsts c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.omb1 = (float)(1.0 - b1);
  c.omb2 = (float)(1.0 - b2);
  c.eps = eps;
  c.decay = (float)(1.0 - lr_d * wd_d);
  c.step_size = (float)(lr_d / (1.0 - std::pow(b1, (double)step)));
  c.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)step)));
  c.grad_scale = grad_scale;
  fp8ds::AdamWLaunch a{w, g, gt == FP8DS_BF16, m, v, rows, cols, c, grad_amax, (int)fmt, scale,
                       cast ? q : nullptr, cast ? q_t : nullptr, amax, sat_count};
  hipError_t e = hipSuccess;
  if (cast) e = fp8ds::launch_prologue(1, scale, scale_used, amax, sat_count, stream);
  if (e == hipSuccess && n > 0) e = fp8ds::launch_adamw(a, stream);
  return hip_status(e, who);
}

int fp8ds_gemm_rowcol(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K,
                      const uint8_t* A, fp8ds_format fa, int64_t lda, const float* scale_inv_a,
                      const uint8_t* B, fp8ds_format fb, int64_t ldb, const float* scale_inv_b,
                      void* C, fp8ds_dtype ct, int64_t ldc, float* amax_c, hipStream_t stream) {
  return gemm_common("fp8ds_gemm_rowcol", opa, opb, M, N, K, 1, A, fa, lda, 0, scale_inv_a, B, fb,
                     ldb, 0, scale_inv_b, C, ct, ldc, 0, amax_c, FP8DS_MMA_EXACT, stream, true);
}

int fp8ds_cast_rowwise(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                       int margin, uint8_t* q, float* scale, float* scale_inv, float* amax,
                       hipStream_t stream) {
  const char* who = "fp8ds_cast_rowwise";
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "%s: bad dtype %d", who, (int)xt);
  if (!valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "%s: bad format %d", who, (int)fmt);
  if (rows < 0 || cols < 0 || rows >= (int64_t(1) << 31) || (cols > 0 && rows > kMaxElems / cols))
    return fail(FP8DS_ERR_SHAPE, "%s: bad shape %lld x %lld", who, (long long)rows,
                (long long)cols);
  if (margin < -126 || margin > 126)
    return fail(FP8DS_ERR_SHAPE, "%s: margin %d not in [-126, 126]", who, margin);
  if (rows > 0 && !scale) return fail(FP8DS_ERR_NULL, "%s: scale is null", who);
  if (rows * cols > 0) {
    if (!x || !q) return fail(FP8DS_ERR_NULL, "%s: x or q is null", who);
    if (!aligned16(x) || !aligned16(q))
      return fail(FP8DS_ERR_ALIGN, "%s: x and q must be 16-byte aligned", who);
  }
  return hip_status(fp8ds::launch_rowwise_cast(x, xt == FP8DS_BF16, rows, cols, (int)fmt, margin,
                                               q, scale, scale_inv, amax, stream),
                    who);
}

int fp8ds_cast_current(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols,
                       fp8ds_format fmt, int margin, uint8_t* q, uint8_t* q_t, float* scale,
                       float* scale_inv, float* amax, uint64_t* sat_count, hipStream_t stream) {
  const char* who = "fp8ds_cast_current";
  if (!scale || !amax) return fail(FP8DS_ERR_NULL, "%s: scale and amax are required", who);
  if (margin < -126 || margin > 126)
    return fail(FP8DS_ERR_SHAPE, "%s: margin %d not in [-126, 126]", who, margin);
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "%s: bad dtype %d", who, (int)xt);
  if (!valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "%s: bad format %d", who, (int)fmt);
  if (rows < 0 || cols < 0 || (cols > 0 && rows > kMaxElems / cols))
    return fail(FP8DS_ERR_SHAPE, "%s: bad shape %lld x %lld", who, (long long)rows,
                (long long)cols);
  const int64_t n = rows * cols;
  if (n > 0) {
    if (!x || !q) return fail(FP8DS_ERR_NULL, "%s: x or q is null", who);
    if (!aligned16(x) || !aligned16(q) || (q_t && !aligned16(q_t)))
      return fail(FP8DS_ERR_ALIGN, "%s: x, q and q_t must be 16-byte aligned", who);
  }
  if (q_t && (rows + 127) / 128 > 65535)
    return fail(FP8DS_ERR_SHAPE, "%s: a transposed copy supports at most %d rows", who,
                65535 * 128);
  // amax pass, scale from it, then the cast with that scale
  hipError_t e = fp8ds::launch_prologue(1, nullptr, nullptr, amax, sat_count, stream);
  if (e == hipSuccess && n > 0)
    e = fp8ds::launch_cast(x, xt == FP8DS_BF16, 1, n, n, 0, nullptr, nullptr, n, amax, nullptr,
                           nullptr, num_cus(), stream);
  if (e == hipSuccess) e = fp8ds::launch_current_scale(amax, (int)fmt, margin, scale, scale_inv,
                                                       stream);
  if (e == hipSuccess && n > 0) {
    if (q_t)
      e = fp8ds::launch_cast_transpose(x, xt == FP8DS_BF16, rows, cols, (int)fmt, scale, q, q_t,
                                       nullptr, sat_count, nullptr, stream);
    else
      e = fp8ds::launch_cast(x, xt == FP8DS_BF16, 1, n, n, (int)fmt, scale, q, n, nullptr,
                             sat_count, nullptr, num_cus(), stream);
  }
  return hip_status(e, who);
}

}  // extern "C"

extern "C" {

int fp8ds_cast_mx(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                  uint8_t* q, uint8_t* scales, uint8_t* q_t, uint8_t* scales_t,
                  hipStream_t stream) {
  const char* who = "fp8ds_cast_mx";
  if (!valid_dtype(xt)) return fail(FP8DS_ERR_ENUM, "%s: bad dtype %d", who, (int)xt);
  if (!valid_fmt(fmt)) return fail(FP8DS_ERR_ENUM, "%s: bad format %d", who, (int)fmt);
  if (rows < 0 || cols < 0 || (cols > 0 && rows > kMaxElems / cols))
    return fail(FP8DS_ERR_SHAPE, "%s: bad shape %lld x %lld", who, (long long)rows,
                (long long)cols);
  if (cols % 32 != 0)
    return fail(FP8DS_ERR_SHAPE, "%s: the row length %lld is not a multiple of the block (32)",
                who, (long long)cols);
  const int64_t n = rows * cols;
  if (n == 0) return ok();
  if (!x || !q || !scales) return fail(FP8DS_ERR_NULL, "%s: x, q and scales are required", who);
  if (!aligned16(x) || !aligned16(q))
    return fail(FP8DS_ERR_ALIGN, "%s: x and q must be 16-byte aligned", who);
  if (!q_t != !scales_t)
    return fail(FP8DS_ERR_NULL, "%s: q_t and scales_t go together", who);
  if (q_t) {
    if (rows % 128 || cols % 128)
      return fail(FP8DS_ERR_SHAPE, "%s: a transposed copy needs rows and cols in multiples of "
                  "128 (got %lld x %lld)", who, (long long)rows, (long long)cols);
    if (rows / 128 > 65535 || cols / 128 > (int64_t(1) << 31) - 1)
      return fail(FP8DS_ERR_SHAPE, "%s: too many 128-row tiles for a transposed copy", who);
    if (!aligned16(q_t)) return fail(FP8DS_ERR_ALIGN, "%s: q_t must be 16-byte aligned", who);
    return hip_status(fp8ds::launch_mx_cast_transpose(x, xt == FP8DS_BF16, rows, cols, (int)fmt,
                                                      q, scales, q_t, scales_t, stream),
                      who);
  }
  return hip_status(fp8ds::launch_mx_cast(x, xt == FP8DS_BF16, n, (int)fmt, q, scales, stream),
                    who);
}

int fp8ds_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* A, fp8ds_format fa, int64_t lda,
                  const uint8_t* scales_a, int64_t ld_scales_a, const uint8_t* B, fp8ds_format fb,
                  int64_t ldb, const uint8_t* scales_b, int64_t ld_scales_b, void* C,
                  fp8ds_dtype ct, int64_t ldc, float* amax_c, fp8ds_mma mma, hipStream_t stream) {
  const char* who = "fp8ds_gemm_mx";
  if (mma != FP8DS_MMA_EXACT && mma != FP8DS_MMA_FP8)
    return fail(FP8DS_ERR_ENUM, "%s: bad mma %d", who, (int)mma);
  if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8DS_ERR_ENUM, "%s: bad format", who);
  if (!valid_dtype(ct)) return fail(FP8DS_ERR_ENUM, "%s: bad output dtype", who);
  const int64_t lim = int64_t(1) << 31;
  if (M < 0 || N < 0 || K < 0 || M >= lim || N >= lim || K >= lim)
    return fail(FP8DS_ERR_SHAPE, "%s: bad M/N/K %lld/%lld/%lld", who, (long long)M, (long long)N,
                (long long)K);
  if (K % 128 != 0)
    return fail(FP8DS_ERR_SHAPE, "%s: K = %lld is not a multiple of 128", who, (long long)K);
  if (((M + 127) / 128) * ((N + 127) / 128) >= lim)
    return fail(FP8DS_ERR_SHAPE, "%s: M x N %lld x %lld has too many tiles", who, (long long)M,
                (long long)N);
  if (M == 0 || N == 0) {
    if (amax_c)
      return hip_status(fp8ds::launch_prologue(1, nullptr, nullptr, amax_c, nullptr, stream), who);
    return ok();
  }
  if (lda < K || ldb < K || ldc < N || ld_scales_a < K / 32 || ld_scales_b < K / 32)
    return fail(FP8DS_ERR_SHAPE, "%s: leading dimension too small", who);
  if (!C || (K > 0 && (!A || !B || !scales_a || !scales_b)))
    return fail(FP8DS_ERR_NULL, "%s: A, B, their scales and C are required", who);
  const int esz = ct == FP8DS_BF16 ? 2 : 4;
  if ((K > 0 && (!aligned16(A) || !aligned16(B) || lda % 16 || ldb % 16)) || !aligned16(C) ||
      (ldc * esz) % 16)
    return fail(FP8DS_ERR_ALIGN, "%s: A, B, C and lda, ldb, ldc*elem_size must be 16-byte aligned",
                who);
  if (K > 0 && ((reinterpret_cast<uintptr_t>(scales_a) & 3u) ||
                (reinterpret_cast<uintptr_t>(scales_b) & 3u) || ld_scales_a % 4 || ld_scales_b % 4))
    return fail(FP8DS_ERR_ALIGN, "%s: the scale arrays and their leading dimensions must be "
                "4-byte aligned", who);
  hipError_t e = hipSuccess;
  if (amax_c) e = fp8ds::launch_prologue(1, nullptr, nullptr, amax_c, nullptr, stream);
  if (e == hipSuccess) {
    fp8ds::GemmProblem p;
    p.opa = 0; p.opb = 1;
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.fa = (int)fa; p.lda = lda; p.scale_a = nullptr;
    p.B = B; p.fb = (int)fb; p.ldb = ldb; p.scale_b = nullptr;
    p.C = C; p.out_bf16 = ct == FP8DS_BF16; p.ldc = ldc; p.amax_c = amax_c;
    p.batch = 1; p.stride_a = 0; p.stride_b = 0; p.stride_c = 0;
    p.sc_a = scales_a; p.sc_b = scales_b; p.ldsa = ld_scales_a; p.ldsb = ld_scales_b;
    e = fp8ds::launch_gemm_mx(p, mma == FP8DS_MMA_EXACT, num_cus(), stream);
  }
  return hip_status(e, who);
}

}  // extern "C"

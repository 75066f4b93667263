/*
 * fp8ds.h -- C ABI of the FP8 delayed-scaling Linear for AMD MI355X (gfx950).
 *
 * The library computes the hot path of an FP8 training Linear with delayed
 * per-tensor scaling:
 *
 *   amax of a BF16/FP32 tensor  ->  scale from an amax-history window
 *   ->  saturating round-to-nearest-even cast to OCP E4M3 / E5M2
 *   ->  FP8 x FP8 GEMM with FP32 accumulation (NN, NT, TN)
 *   ->  dequant by 1/(s_a * s_b) into BF16, with the output amax fused.
 *
 * Sources (cited by page title and section):
 *   [P1] "算子与编译器：FP8 训练与优化器 Kernel" (charles2530.github.io)
 *   [P2] "FP8 混合精度训练工程实践：从 H100 到大模型训练的范式跃迁" (ybb.press)
 *   [P3] "LLM FP8 微调上线生产实战：用 Amax Scaling、层级白名单与 BF16 回退守住收敛"
 *        (oh-bug.com)
 *   [OCP] the OCP 8-bit floating point formats (Micikevicius et al., "FP8 Formats
 *        for Deep Learning", in [P3]'s reference list) for special values.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *     owns every buffer; the library keeps no pointer after the call returns and
 *     allocates no device memory.
 *   - Every call is asynchronous on `stream` (0 = the null stream): it validates
 *     its arguments on the host, enqueues kernels and returns.  Device-side
 *     results are ready after the stream is synchronised.
 *   - Return value: FP8DS_OK (0) or a negative fp8ds_status.  On failure nothing
 *     has been enqueued (validation) or a launch failed (FP8DS_ERR_HIP), and
 *     fp8ds_last_error() returns a thread-local message.  No C++ exception,
 *     abort or exit crosses the ABI.  A device fault (e.g. a pointer that does
 *     not span the stated size) surfaces at the caller's next synchronisation.
 *   - Zero-size inputs are legal no-ops that still write their scalar outputs
 *     (amax = 0, saturation count = 0, scale_used = *scale).
 *   - Row-major layouts; `ld*` are leading dimensions in elements.
 *   - Calls that write the same output buffers must not overlap (the fused
 *     amax / counters are reset by the call that writes them).  The `_acc`
 *     variants (fp8ds_cast_acc, fp8ds_gemm_acc) combine into their amax and
 *     counters instead; fp8ds_scale_update_clear zeroes such accumulators for
 *     the next step, so a training step needs no reset launches.
 */
#ifndef FP8DS_H
#define FP8DS_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8DS_ABI_VERSION 8

typedef enum {
  FP8DS_OK = 0,
  FP8DS_ERR_NULL = -1,        /* a required pointer is NULL */
  FP8DS_ERR_SHAPE = -2,       /* negative / overflowing size, or ld too small */
  FP8DS_ERR_ENUM = -3,        /* a format, dtype, op or algo value out of range */
  FP8DS_ERR_ALIGN = -4,       /* pointer or leading dimension not 16-byte aligned */
  FP8DS_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  FP8DS_ERR_UNSUPPORTED = -6, /* valid but unsupported combination (e.g. TT) */
  FP8DS_ERR_VALUE = -7        /* a scalar argument out of its range (fp8ds_adamw) */
} fp8ds_status;

/* FP8 formats ([P2] §一 "FP8 格式设计"; [P3] §核心原理 "E4M3 与 E5M2 承担不同职责"):
 * E4M3: bias 7, largest finite 448, no infinity (OCP "fn" variant, [OCP]).
 * E5M2: bias 15, largest finite 57344, with +-inf ([OCP]). */
typedef enum { FP8DS_E4M3 = 0, FP8DS_E5M2 = 1 } fp8ds_format;

/* High-precision element types of inputs and GEMM outputs. */
typedef enum { FP8DS_F32 = 0, FP8DS_BF16 = 1 } fp8ds_dtype;

/* Window reductions of the amax history ([P3] §核心原理 "Delayed Scaling
 * 用历史换取稳定性", the table of strategies: max over the window, or the most
 * recent value). */
typedef enum { FP8DS_ALGO_MAX = 0, FP8DS_ALGO_MOST_RECENT = 1 } fp8ds_algo;

/* GEMM operand layout: N = used as stored, T = the stored array is transposed. */
typedef enum { FP8DS_OP_N = 0, FP8DS_OP_T = 1 } fp8ds_op;

/* GEMM datapath.
 * FP8DS_MMA_EXACT: the FP8 operands are widened exactly to F16 inside the kernel
 *   and multiplied on the F16 matrix cores; products are exact and every sum is an
 *   FP32 addition, so |acc - exact| stays at FP32 rounding level.  Default.
 * FP8DS_MMA_FP8: the FP8 matrix instructions of gfx950 on the FP8 bytes, at twice
 *   the F16 rate.  These instructions add each group of 8 products at a fixed
 *   point about 13 bits below the group's largest product, so a product 2^14 or
 *   more smaller than its largest neighbour is lost.  Measured worst case about
 *   2^-11 of the largest product per instruction; on Gaussian-like operands the
 *   error is FP32-like, on heavy-tailed gradients (outliers next to small values)
 *   it exceeds 1e-5 * sum|a*b| for most elements.  Opt-in only. */
typedef enum { FP8DS_MMA_EXACT = 0, FP8DS_MMA_FP8 = 1 } fp8ds_mma;

/* ABI version (FP8DS_ABI_VERSION of the built library). */
int fp8ds_abi_version(void);

/* Static description of a status code (never NULL). */
const char* fp8ds_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* fp8ds_last_error(void);

/*
 * fp8ds_amax -- amax = max_i |x_i| of the unscaled tensor.
 * [P2] §四 "动态缩放" (the quantize step takes the maximum absolute value of the
 * high-precision tensor); [P3] §核心原理 "Scale 决定数值是否进入可表示区间".
 *
 *   x      device, n elements of `xt` (BF16 or FP32), 16-byte aligned.
 *   n      element count, n >= 0.
 *   amax   device, 1 float: overwritten with the result.  Exact (the maximum is
 *          one of the inputs).  NaN anywhere gives the canonical qNaN 0x7FC00000;
 *          otherwise +inf if any element is infinite; 0 for n == 0; |-0| = +0.
 */
int fp8ds_amax(const void* x, fp8ds_dtype xt, int64_t n, float* amax, hipStream_t stream);

/*
 * fp8ds_cast -- scaled saturating cast of a [rows x cols] tensor to FP8, with the
 * input amax fused into the same pass.
 * [P2] §四 "动态缩放" (quantize: multiply by the scale, clamp to the format's
 * range, convert); [P2] §五 (the fp8 linear op casts input and weight with their
 * scales before the product).
 *
 *   q[i] = encode_fmt( fl32(x[i] * (*scale)) )
 * where fl32 is one IEEE fp32 multiply (round to nearest even) and encode is the
 * saturating round-to-nearest-even conversion: |v| > max (infinities included)
 * gives the largest finite code of v's sign, NaN gives 0x7F | sign << 7, and the
 * sign is kept on underflow to zero.
 *
 *   x          device, rows*cols elements of `xt`, row-major, contiguous, 16-byte aligned.
 *   rows,cols  >= 0.
 *   fmt        target format.
 *   scale      device, 1 float: the delayed scale of this step (read once).
 *   q          device, rows*cols bytes, row-major, 16-byte aligned.
 *   q_t        device or NULL: if non-NULL also receives the transposed copy,
 *              [cols x rows] row-major (q_t[c*rows + r] == q[r*cols + c]), for GEMM
 *              operands the caller wants K-contiguous.  16-byte aligned; rows at
 *              most 65535 * 128 (else FP8DS_ERR_SHAPE).
 *   scale_used device or NULL: receives a copy of *scale -- the snapshot the FP8
 *              bytes were made with.  GEMMs must be given this snapshot, because
 *              fp8ds_scale_update overwrites *scale for the next step.
 *   amax       device or NULL: receives max|x| of the UNSCALED input (as fp8ds_amax).
 *   sat_count  device or NULL: receives #{i : |fl32(x[i]*scale)| > max}
 *              (infinities counted, NaN not).
 */
int fp8ds_cast(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
               const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
               uint64_t* sat_count, hipStream_t stream);

/*
 * fp8ds_cast_acc -- fp8ds_cast that accumulates its reductions instead of
 * resetting them (same arguments, same bytes q / q_t):
 *   amax       device or NULL: on return max(previous amax, max|x|) (fp32 bits of
 *              non-negative values compared as integers; NaN as fp8ds_amax).
 *   sat_count  device or NULL: the saturation count of this call added to it.
 *   scale_used device or NULL: written by the cast kernel itself.
 * With amax and sat_count zeroed before a step (fp8ds_scale_update_clear of the
 * previous step does it), the results equal fp8ds_cast's, with no reset kernel
 * launched before the cast.
 */
int fp8ds_cast_acc(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                   const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                   uint64_t* sat_count, hipStream_t stream);

/*
 * fp8ds_cast_health -- fp8ds_cast plus quantization-health counts of the same pass.
 * [P3] "第四步：建立 Amax 与低精度异常画像" (per-module metrics: the share of values
 * near the FP8 upper limit, the share of zeros after quantization, NaN / Inf /
 * overflow counts); [P2] §七 "陷阱 1：NaN/Inf 难以定位" (NaN and Inf checks).
 *
 * Arguments as fp8ds_cast, with sat_count replaced by
 *   counts     device, FP8DS_HEALTH_COUNTS uint64 (required), reset by the call:
 *              [0] saturated: #{|fl32(x*scale)| > max} (infinities counted, NaN not)
 *              [1] NaN inputs
 *              [2] infinite inputs
 *              [3] zero codes: q[i] is +-0 (underflow to zero and exact zeros)
 *              [4] near-max codes: q[i] finite with magnitude in the format's top
 *                  binade [2^emax, max] ([256, 448] E4M3, [32768, 57344] E5M2).
 */
#define FP8DS_HEALTH_COUNTS 5
int fp8ds_cast_health(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                      const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                      uint64_t* counts, hipStream_t stream);

/*
 * fp8ds_cast_batched -- `batch` independent casts of equal size n, each with its
 * own scale (the per-problem scales of a batch of small Linears).
 * [P3] §适用场景 (among the cases to treat with care: many small matrices) and
 * §常见误区 误区一 (small matrices, frequent casts and scale kernels can eat the FP8
 * gain): one launch casts every tensor of the batch, so a small matrix's cast
 * costs no launch of its own.  Each tensor's cast is the scaled saturating cast
 * of fp8ds_cast ([P2] §四 "动态缩放", the quantize step).
 *
 *   x          device, batch tensors of n elements, tensor b at x + b*stride_x elements
 *              (stride_x >= n, stride_x*elem_size a multiple of 16).
 *   scale      device [batch].
 *   q          device, tensor b at q + b*stride_q bytes (stride_q >= n, multiple of 16).
 *   scale_used, amax: device [batch] or NULL.   sat_count: device [batch] or NULL.
 * Semantics per tensor as fp8ds_cast without the transposed copy.
 */
int fp8ds_cast_batched(const void* x, fp8ds_dtype xt, int64_t batch, int64_t n, int64_t stride_x,
                       fp8ds_format fmt, const float* scale, uint8_t* q, int64_t stride_q,
                       float* scale_used, float* amax, uint64_t* sat_count, hipStream_t stream);

/*
 * fp8ds_scale_update -- push this step's amax into each tensor's history ring and
 * compute the scale of the next step.
 * [P3] §核心原理 "Scale 决定数值是否进入可表示区间" (scale = (FP8_MAX/amax)/2^margin);
 * [P3] §核心原理 "Delayed Scaling 用历史换取稳定性" (history window, max or
 * most_recent); [P2] §四 "Delayed Scaling 的工程细节" (ring buffer with a cursor
 * advanced modulo the history length; scale 1.0 when the history maximum is not
 * positive).
 *
 * For each tensor t in [0, n_tensors):
 *   history[t*hist_len + cursor[t]] = amax[t];  cursor[t] = (cursor[t] + 1) % hist_len;
 *   w = max over history[t*hist_len .. +hist_len)  (ALGO_MAX; NaN propagates)
 *     | amax[t]                                       (ALGO_MOST_RECENT);
 *   scale[t] = ldexp(fl32(FP8_MAX(fmt[t]) / w), -margin)   if w is finite and > 0 and
 *              the result is finite and > 0;   1.0 otherwise.
 * The quotient is one correctly rounded fp32 division.
 *
 *   n_tensors  1 .. 4096.          hist_len  1 .. 65536.
 *   history    device [n_tensors][hist_len] fp32, in/out (initially zeros).
 *   cursor     device [n_tensors] int32, in/out (initially 0; must be in [0, hist_len)).
 *   amax       device [n_tensors] fp32 (e.g. the amax outputs of fp8ds_cast).
 *   fmt        HOST [n_tensors] fp8ds_format, read during the call only.
 *   algo       window reduction.       margin  integer exponent, -126..126.
 *   scale      device [n_tensors] fp32, overwritten with the next step's scale.
 *   scale_inv  device [n_tensors] or NULL: receives fl32(1 / scale).
 */
int fp8ds_scale_update(int n_tensors, int hist_len, float* history, int32_t* cursor,
                       const float* amax, const fp8ds_format* fmt, fp8ds_algo algo, int margin,
                       float* scale, float* scale_inv, hipStream_t stream);

/*
 * fp8ds_scale_update_clear -- fp8ds_scale_update that also zeroes `clear_bytes`
 * bytes at `clear` (device, 4-byte aligned, a multiple of 4 bytes up to 2^30)
 * in the same launch: the accumulators that the next step's fp8ds_cast_acc and
 * fp8ds_gemm_acc calls combine into.  The cleared bytes must not overlap the
 * other arguments (an overlap with amax returns FP8DS_ERR_VALUE); clear may be
 * NULL when clear_bytes is 0.
 */
int fp8ds_scale_update_clear(int n_tensors, int hist_len, float* history, int32_t* cursor,
                             const float* amax, const fp8ds_format* fmt, fp8ds_algo algo,
                             int margin, float* scale, float* scale_inv, void* clear,
                             int64_t clear_bytes, hipStream_t stream);

/*
 * fp8ds_gemm -- C = dequant( op(A) . op(B) ), FP8 x FP8 with FP32 accumulation.
 * [P2] §五 (the fp8 linear op: FP8 product divided by the product of the two
 * scales; the per-tensor FP8 GEMM: FP8 inputs, FP32 accumulate, BF16 output);
 * [P2] §三 (the three products of a training step: Y = X W, dX = dY W^T,
 * dW = X^T dY; HYBRID formats per [P3] §核心原理: E4M3 forward, E5M2 gradients).
 *
 *   acc[i][j] = sum_k a(i,k) * b(k,j)   over decoded FP8 values, FP32 accumulation
 *   C[i][j]   = convert_ct( acc[i][j] * d ),  d = fl32(1 / fl32((*scale_a) * (*scale_b)))
 * with round-to-nearest-even to BF16 (ct = BF16) or no rounding (ct = F32).
 *
 *   opa, opb   (N,N), (N,T) or (T,N); (T,T) returns FP8DS_ERR_UNSUPPORTED.
 *   M, N, K    >= 0 and < 2^31, with ceil(M/128) * ceil(N/128) < 2^31 (else
 *              FP8DS_ERR_SHAPE).  op(A) is M x K, op(B) is K x N, C is M x N.
 *   A          device: opa == N: [M x K] with lda >= K;  opa == T: [K x M] with lda >= M.
 *   B          device: opb == N: [K x N] with ldb >= N;  opb == T: [N x K] with ldb >= K.
 *   fa, fb     formats of A and B, independently E4M3 or E5M2.
 *   lda, ldb   multiples of 16 bytes; A and B 16-byte aligned.
 *   scale_a/b  device, 1 float each: the scale snapshots the operands were cast with.
 *   C          device [M x N] of `ct` with ldc >= N; C and ldc*elem_size 16-byte aligned.
 *   amax_c     device or NULL: receives max |C[i][j]| of the stored output (NaN as
 *              fp8ds_amax).
 *   mma        datapath (FP8DS_MMA_EXACT unless the caller accepts the FP8 matrix
 *              instructions' summation precision, see fp8ds_mma).
 */
int fp8ds_gemm(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K,
               const uint8_t* A, fp8ds_format fa, int64_t lda, const float* scale_a,
               const uint8_t* B, fp8ds_format fb, int64_t ldb, const float* scale_b,
               void* C, fp8ds_dtype ct, int64_t ldc, float* amax_c, fp8ds_mma mma,
               hipStream_t stream);

/*
 * fp8ds_gemm_acc -- fp8ds_gemm whose output amax is combined into amax_c
 * (max(previous, max|C|)) instead of reset; otherwise identical.
 */
int fp8ds_gemm_acc(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K,
                   const uint8_t* A, fp8ds_format fa, int64_t lda, const float* scale_a,
                   const uint8_t* B, fp8ds_format fb, int64_t ldb, const float* scale_b,
                   void* C, fp8ds_dtype ct, int64_t ldc, float* amax_c, fp8ds_mma mma,
                   hipStream_t stream);

/*
 * fp8ds_gemm_batched -- `batch` independent GEMMs of one shape, each with its own
 * scales and output amax (many small Linears in one launch).
 * [P3] §适用场景 (many small matrices among the cases to treat with care) and
 * §常见误区 误区一 (small matrices can cancel the FP8 gain): the products of a
 * batch of small Linears share one launch, one workgroup per output tile of any
 * problem.  Each product is fp8ds_gemm's ([P2] §五).
 * Problem b uses A + b*stride_a, B + b*stride_b (bytes), C + b*stride_c (elements),
 * scale_a[b], scale_b[b], amax_c[b]; otherwise as fp8ds_gemm.  Strides must keep
 * every operand 16-byte aligned.
 */
int fp8ds_gemm_batched(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K, int64_t batch,
                       const uint8_t* A, fp8ds_format fa, int64_t lda, int64_t stride_a,
                       const float* scale_a, const uint8_t* B, fp8ds_format fb, int64_t ldb,
                       int64_t stride_b, const float* scale_b, void* C, fp8ds_dtype ct,
                       int64_t ldc, int64_t stride_c, float* amax_c, fp8ds_mma mma,
                       hipStream_t stream);

/*
 * fp8ds_linear_batched -- the whole forward step of `batch` independent small
 * Linears Y_i = X_i W_i, each with its own delayed scaling of X_i and W_i, in one
 * launch.  [P3] §适用场景 (many small matrices among the cases to treat with care)
 * and §常见误区 误区一 (with small matrices the conversion work can cancel the
 * FP8 gain): one workgroup per problem reads X_i and W_i once, casts them, keeps
 * the codes on chip for the product and updates both tensors' scaling state, so
 * the codes are never read back and no other launch is needed.
 *
 * Per problem i (tensor t = i is X_i, tensor t = batch + i is W_i):
 *   xq_i = cast(X_i, scale[i]), wq_i = cast(W_i, scale[batch + i])   (fp8ds_cast)
 *   y_i  = fp8ds_gemm(N, N) of xq_i and wq_i with those scales, BF16, amax_y[i]
 *   then for both tensors, with this step's amax: fp8ds_scale_update
 * The results equal those of fp8ds_cast_batched (X, then W), fp8ds_gemm_batched
 * (exact datapath) and fp8ds_scale_update over the 2 * batch tensors, in that
 * order; the outputs amax, sat_count, amax_y are stored, not combined into.
 *
 *   batch            1 .. 65535 problems
 *   M, N, K          multiples of 16 in [16, 256]
 *   x                [batch][M][K] BF16 (problem i at x + i*stride_x elements)
 *   w                [batch][K][N] BF16 (at w + i*stride_w elements)
 *   fx, fw           formats of the X and W codes
 *   hist_len, history, cursor, algo, margin: as fp8ds_scale_update, over the
 *                    2 * batch tensors ([2 batch][hist_len], [2 batch])
 *   scale            [2 batch] in: this step's scales; out: the next step's
 *   scale_used       [2 batch] (nullable): this step's scales
 *   amax             [2 batch] out: max |X_i|, then max |W_i| (NaN canonical)
 *   sat_count        [2 batch] (nullable) out: saturated values of each cast
 *   xq, wq           (nullable) codes: [batch][M][K] at stride_xq bytes,
 *                    [batch][K][N] at stride_wq bytes
 *   y                [batch][M][N] BF16 at stride_y elements
 *   amax_y           [batch] (nullable) out: max |y_i|
 * Every pointer 16-byte aligned, every stride a multiple of 16 bytes, strides at
 * least the problem's size.  Only the BF16 input dtype is supported
 * (FP8DS_ERR_UNSUPPORTED otherwise); the products run on the exact datapath.
 */
int fp8ds_linear_batched(int64_t batch, int64_t M, int64_t N, int64_t K, fp8ds_dtype xt,
                         const void* x, int64_t stride_x, fp8ds_format fx, const void* w,
                         int64_t stride_w, fp8ds_format fw, int hist_len, float* history,
                         int32_t* cursor, fp8ds_algo algo, int margin, float* scale,
                         float* scale_used, float* amax, uint64_t* sat_count, uint8_t* xq,
                         int64_t stride_xq, uint8_t* wq, int64_t stride_wq, void* y,
                         int64_t stride_y, float* amax_y, hipStream_t stream);

/*
 * fp8ds_adamw -- fused AdamW step on FP32 master weights that also writes the
 * FP8 copy of the updated weights for the next forward.
 * "算子与编译器：FP8 训练与优化器 Kernel" (charles2530.github.io): §"FP8 训练主路径图"
 * (unscale/clip -> fused optimizer -> master weight -> cast/scale to FP8) and
 * §"Fused Optimizer 的意义" (one kernel reads the gradient, updates both moments,
 * applies the bias corrections and the weight decay, updates the parameter);
 * [P2] §"自动混合精度与 FP8 的协同" (gradient un-scaling, FP32 AdamW, the updated
 * weights cast to FP8 with scaling for the next forward).
 *
 * The pages name AdamW without its formula; this is AdamW with decoupled weight
 * decay (Loshchilov & Hutter) and bias-corrected moments (Kingma & Ba).  Per
 * element, each operation one correctly rounded fp32 operation in this order,
 * no fused multiply-add:
 *   g' = g * grad_scale
 *   m  = beta1 * m + (1 - beta1) * g'
 *   v  = beta2 * v + ((1 - beta2) * g') * g'
 *   w  = decay * w - step_size * (m / (sqrt(v) * inv_sqrt_bc2 + eps))
 * with the fp32 constants decay = 1 - lr*weight_decay, 1 - beta1, 1 - beta2,
 * step_size = lr / (1 - beta1^step), inv_sqrt_bc2 = 1 / sqrt(1 - beta2^step),
 * each evaluated in float64 (C library pow and sqrt) and rounded once.
 * If scale != NULL, the updated weights are then cast exactly as fp8ds_cast
 * casts them (q, q_t, scale_used, amax, sat_count with fp8ds_cast's meaning, amax
 * and saturation of the NEW weights), so the next forward needs no weight cast.
 *
 *   w          device [rows x cols] fp32 master weights, row-major, updated in place.
 *   g          device [rows x cols] gradient of dtype gt (BF16 or FP32), read only.
 *   m, v       device [rows x cols] fp32 first and second moments, updated in
 *              place (zeros before the first step).  w, g, m, v must not overlap.
 *   rows,cols  >= 0.  All of w, g, m, v, q, q_t 16-byte aligned.
 *   lr, weight_decay  finite.   beta1, beta2  in [0, 1).   eps  finite, > 0.
 *   grad_scale finite, > 0: multiplies the gradient first (1/K for a loss
 *              scaled by K, times any clipping factor the caller computed).
 *   step       the step count t >= 1 of this update (bias corrections).
 *   grad_amax  device or NULL: if it holds an infinity or NaN (e.g. the amax_c of
 *              the fp8ds_gemm that produced g), the update is skipped -- w, m, v
 *              are left unchanged -- and the FP8 copy is made of the unchanged w.
 *   scale      device or NULL: the delayed scale of the weights.  NULL = no FP8
 *              copy (then q, q_t, scale_used, amax and sat_count must be NULL).
 *   fmt        FP8 format of the copy (checked when scale != NULL).
 *   q          device, rows*cols bytes (required with scale when rows*cols > 0): the
 *              FP8 copy of the new weights.
 *   q_t        device or NULL: the transposed copy [cols x rows]; rows at most
 *              65535 * 128.
 *   scale_used, amax, sat_count  device or NULL: as fp8ds_cast (written also when
 *              rows*cols == 0).
 * Out-of-range scalars return FP8DS_ERR_VALUE.
 */
int fp8ds_adamw(float* w, const void* g, fp8ds_dtype gt, float* m, float* v, int64_t rows,
                int64_t cols, float lr, float beta1, float beta2, float eps, float weight_decay,
                float grad_scale, int64_t step, const float* grad_amax, fp8ds_format fmt,
                const float* scale, uint8_t* q, uint8_t* q_t, float* scale_used, float* amax,
                uint64_t* sat_count, hipStream_t stream);

/*
 * Finer-grained scaling: current (just-in-time) scales and one scale per row.
 * [P2] §"FBGEMM_GPU 底层优化" (per-tensor, per-channel and per-token FP8 GEMM modes:
 * FP8 operands, FP32 accumulation, BF16 output); the scale formula of [P3]
 * §核心原理 "Scale 决定数值是否进入可表示区间" applied to the amax of what is being
 * cast, with no history ([P3]'s reference list names current scaling beside
 * delayed scaling).  In every case
 *   s = ldexp(fl32(FP8_MAX(fmt) / a), -margin)  if a and the result are finite and
 *       > 0, else 1.0;        scale_inv = fl32(1 / s)
 * with a the amax of the tensor (current) or of the row (per row).
 */

/*
 * fp8ds_cast_rowwise -- per-row current scaling of a [rows x cols] matrix:
 *   a_r = max_c |x[r][c]|,  s_r from a_r as above,  q[r][c] = encode(fl32(x[r][c] * s_r)).
 * Per-token scaling of activations X [M x K] is this call on X; per-channel
 * scaling of a weight W [K x N] (a scale per output channel) is this call on
 * W^T [N x K], the K-contiguous layout the forward GEMM reads with op T.
 *
 *   x          device, rows*cols elements of `xt`, row-major, 16-byte aligned.
 *   rows       0 .. 2^31 - 1.   cols >= 0.
 *   margin     integer exponent, -126..126.
 *   q          device, rows*cols bytes, 16-byte aligned.
 *   scale      device [rows] fp32 (required when rows > 0).
 *   scale_inv  device [rows] or NULL: fl32(1 / scale[r]) -- the GEMM's row/column factors.
 *   amax       device [rows] or NULL: a_r (NaN as fp8ds_amax).
 */
int fp8ds_cast_rowwise(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                       int margin, uint8_t* q, float* scale, float* scale_inv, float* amax,
                       hipStream_t stream);

/*
 * fp8ds_cast_current -- per-tensor current scaling: the amax of x, the scale from
 * it, then fp8ds_cast with that scale (three passes: amax, scale, cast).
 *
 *   x, xt, rows, cols, fmt, q, q_t  as fp8ds_cast.    margin  -126..126.
 *   scale      device, 1 float (required): receives s.
 *   scale_inv  device or NULL: receives fl32(1 / s).
 *   amax       device, 1 float (required): receives the amax of x.
 *   sat_count  device or NULL: as fp8ds_cast (non-zero only for margin < 0).
 */
int fp8ds_cast_current(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols,
                       fp8ds_format fmt, int margin, uint8_t* q, uint8_t* q_t, float* scale,
                       float* scale_inv, float* amax, uint64_t* sat_count, hipStream_t stream);

/*
 * fp8ds_gemm_rowcol -- fp8ds_gemm with one scale per row of op(A) and per column
 * of op(B) (per-token x per-channel), exact datapath:
 *   C[i][j] = convert_ct( fl32( fl32(acc[i][j] * scale_inv_a[i]) * scale_inv_b[j] ) )
 * with acc as fp8ds_gemm (FP32 accumulation of the decoded FP8 products).
 *
 *   scale_inv_a  device [M] fp32: inverse scale of each row of op(A) (e.g. the
 *                scale_inv of fp8ds_cast_rowwise on X).
 *   scale_inv_b  device [N] fp32, 16-byte aligned: inverse scale of each column of
 *                op(B) (e.g. fp8ds_cast_rowwise on W^T).  A per-tensor scale is
 *                passed as a vector of equal values.
 *   Other arguments as fp8ds_gemm (no batch, no datapath choice).
 * A scale that varies along K cannot be taken out of the sum: the products whose
 * contraction runs along the scaled dimension need operands cast in the other
 * orientation.
 */
int fp8ds_gemm_rowcol(fp8ds_op opa, fp8ds_op opb, int64_t M, int64_t N, int64_t K,
                      const uint8_t* A, fp8ds_format fa, int64_t lda, const float* scale_inv_a,
                      const uint8_t* B, fp8ds_format fb, int64_t ldb, const float* scale_inv_b,
                      void* C, fp8ds_dtype ct, int64_t ldc, float* amax_c, hipStream_t stream);

/*
 * MXFP8: FP8 elements in blocks of 32 consecutive elements along a row (the
 * contraction dimension of the GEMM below), each block with one E8M0 scale.
 * [P2] §九 "展望：Blackwell 的 Microscaling 与未来" (32 FP8 values share an 8-bit
 * E8M0 scale, scaled block by block); the block rule, which that figure leaves
 * garbled, is the OCP Microscaling Formats (MX) specification's:
 *   a = max |x_i| over the block;   E8M0 code = floor(log2 a) - emax + 127,
 *   clamped to [0, 254] (emax = 8 for E4M3, 15 for E5M2; a zero block has code 0);
 *   q_i = encode(x_i / 2^(code - 127)), saturating round-to-nearest-even.
 * A block holding a NaN or an infinity gets code 255 (NaN) and the element code
 * 0x7F (NaN) throughout.  The value of element i is 2^(code - 127) * decode(q_i).
 */

/*
 * fp8ds_cast_mx -- MXFP8 quantization of a [rows x cols] matrix along its rows,
 * optionally also of its transpose, from one read of x.
 *
 *   x          device, rows*cols elements of `xt`, row-major, 16-byte aligned.
 *   cols       a multiple of 32 (else FP8DS_ERR_SHAPE).
 *   q          device, rows*cols bytes, 16-byte aligned: the element codes.
 *   scales     device, rows*cols/32 bytes: the E8M0 code of block b of row r at
 *              [r * cols/32 + b].
 *   q_t        device or NULL: [cols x rows] codes of x^T quantized along its rows
 *              (blocks of 32 consecutive rows of a column of x), 16-byte aligned;
 *              requires rows and cols to be multiples of 128 (else FP8DS_ERR_SHAPE).
 *   scales_t   device [cols x rows/32] E8M0 codes of q_t; NULL exactly when q_t is.
 * The GEMMs of a training step all run as fp8ds_gemm_mx (A B^T, both blocked
 * along K): Y = X W takes (q of X, q_t of W); dX = dY W^T takes (q of dY, q of W);
 * dW = X^T dY takes (q_t of X, q_t of dY).  No amax, scale state or history is
 * involved.
 */
int fp8ds_cast_mx(const void* x, fp8ds_dtype xt, int64_t rows, int64_t cols, fp8ds_format fmt,
                  uint8_t* q, uint8_t* scales, uint8_t* q_t, uint8_t* scales_t,
                  hipStream_t stream);

/*
 * fp8ds_gemm_mx -- MXFP8 GEMM  C = A B^T  with FP32 accumulation:
 *   C[i][j] = convert_ct( sum_k X_a(i, k/32) a(i,k) X_b(j, k/32) b(j,k) )
 * with a, b the decoded element codes and X the block scales.  Exact datapath:
 * every element is widened to BF16 times its block scale (exact while the scaled
 * value is a normal BF16 number, i.e. |X * decode| >= 2^-126, or zero: blocks whose
 * scale code is above about 17) and multiplied on the BF16 matrix cores with
 * FP32 sums; a NaN block makes every output it touches NaN.
 *
 *   A          device [M x K] codes (K-contiguous, leading dimension lda), format fa.
 *   scales_a   device [M x ld_scales_a] E8M0 codes; block b of row i at
 *              [i * ld_scales_a + b] (fp8ds_cast_mx of A writes ld = K/32).
 *   B          device [N x K] codes (leading dimension ldb), format fb; for a
 *              Linear Y = X W with W [K x N], B is the MX cast of W^T.
 *   scales_b   device [N x ld_scales_b] E8M0 codes.
 *   C          device [M x ldc], BF16 or FP32 (ct).   amax_c  device or NULL: max |C|.
 *   K          a multiple of 128 (four blocks per pipeline stage), else FP8DS_ERR_SHAPE.
 *   A, B, C, lda, ldb, ldc * element size: 16-byte aligned; the scale arrays and
 *   ld_scales_a / ld_scales_b: 4-byte aligned (FP8DS_ERR_ALIGN otherwise).
 *   mma        FP8DS_MMA_EXACT (the BF16 widening above, default) or FP8DS_MMA_FP8:
 *              gfx950's block-scaled FP8 matrix instruction, each lane passing the
 *              E8M0 scale of its 32 K values, at twice the rate and with the FP8
 *              instructions' summation precision (see fp8ds_mma).
 */
int fp8ds_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* A, fp8ds_format fa, int64_t lda,
                  const uint8_t* scales_a, int64_t ld_scales_a, const uint8_t* B, fp8ds_format fb,
                  int64_t ldb, const uint8_t* scales_b, int64_t ld_scales_b, void* C,
                  fp8ds_dtype ct, int64_t ldc, float* amax_c, fp8ds_mma mma, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8DS_H */

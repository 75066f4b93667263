// Host-side launchers of the HIP kernels (internal to the library; the public
// interface is the C ABI in include/fp8ds.h).  All launchers enqueue work on
// `stream` and return the launch status; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ds {

// scale_used[i] = scale[i]; amax[i] = 0; sat[i * counters + k] = 0 for k < counters,
// i < count (null outputs skipped).
hipError_t launch_prologue(int64_t count, const float* scale, float* scale_used, float* amax,
                           uint64_t* sat, hipStream_t stream, int counters = 1);

// Fused amax + cast over `batch` tensors of n elements (q == nullptr: amax only).
// amax, sat and health are combined into (max / add): reset them first
// (launch_prologue) unless accumulating.  health (or null): [batch][4] counts of
// NaN inputs, infinite inputs, zero codes and top-binade codes.  scale_used (or
// null): [batch] scale snapshots, written by the cast kernel.
hipError_t launch_cast(const void* x, bool bf16, int64_t batch, int64_t n, int64_t stride_x,
                       int fmt, const float* scale, uint8_t* q, int64_t stride_q, float* amax,
                       uint64_t* sat, uint64_t* health, int num_cus, hipStream_t stream,
                       float* scale_used = nullptr);
// Batched cast with its output resets and scale snapshot (scale_used, amax, sat:
// [batch] or null), taken by the cast kernel itself where one workgroup covers a
// tensor, else by the prologue kernel.
hipError_t launch_cast_batched(const void* x, bool bf16, int64_t batch, int64_t n,
                               int64_t stride_x, int fmt, const float* scale, uint8_t* q,
                               int64_t stride_q, float* scale_used, float* amax, uint64_t* sat,
                               hipStream_t stream);

// Cast of a [rows x cols] tensor writing q and its transpose qt (health and
// scale_used as above).
hipError_t launch_cast_transpose(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                                 const float* scale, uint8_t* q, uint8_t* qt, float* amax,
                                 uint64_t* sat, uint64_t* health, hipStream_t stream,
                                 float* scale_used = nullptr);

// Fused AdamW step + FP8 cast of the updated weights.  The per-step fp32
// constants are derived on the host from the hyperparameters and the step count.
struct AdamWConsts {
  float b1, b2, omb1, omb2;  // beta1, beta2, 1 - beta1, 1 - beta2
  float eps;
  float decay;         // 1 - lr * weight_decay
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float grad_scale;
};
struct AdamWLaunch {
  float* w;          // [rows x cols] fp32 master weights, updated in place
  const void* g;     // gradient, BF16 (g_bf16) or fp32
  bool g_bf16;
  float* m;          // first moment, fp32, in place
  float* v;          // second moment, fp32, in place
  int64_t rows, cols;
  AdamWConsts c;
  const float* grad_amax;  // or null: a non-finite value skips the update
  int fmt;
  const float* scale;      // delayed scale of the weights (q != null)
  uint8_t* q;              // or null: no cast
  uint8_t* qt;             // or null: no transposed copy (requires q)
  float* amax;             // or null; reset by launch_prologue
  uint64_t* sat;           // or null; reset by launch_prologue
};
hipError_t launch_adamw(const AdamWLaunch& a, hipStream_t stream);

// Current scaling with one scale per row of a [rows x cols] matrix: q, scale[rows],
// scale_inv[rows] (or null), amax[rows] (or null).
hipError_t launch_rowwise_cast(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                               int margin, uint8_t* q, float* scale, float* scale_inv,
                               float* amax, hipStream_t stream);
// scale[0] (and scale_inv[0], or null) from amax[0] by the scale formula.
hipError_t launch_current_scale(const float* amax, int fmt, int margin, float* scale,
                                float* scale_inv, hipStream_t stream);

// History push + window reduction + next scale for n tensors.
// fmt_bits: bit t set = tensor t is E5M2.
struct FmtBits {
  uint32_t w[128];
};
// clear (or null): n_clear 32-bit words zeroed by the same kernel (the next
// step's accumulators; must not overlap the other arguments).
hipError_t launch_scale_update(int n, int hist_len, float* history, int32_t* cursor,
                               const float* amax, const FmtBits& fmt, int algo, int margin,
                               float* scale, float* scale_inv, hipStream_t stream,
                               uint32_t* clear = nullptr, int64_t n_clear = 0);

// Forward step of `batch` small Linears in one launch, one workgroup per problem:
// casts of X_i and W_i with their delayed scales, Y_i = X_i W_i on the exact
// datapath with the dequant epilogue, and the scaling-state update of both
// tensors.  BF16 inputs; M, N, K multiples of 16 in [16, 256]; every pointer
// 16-byte aligned and every stride a multiple of 16 bytes.  Tensor t of the
// per-tensor arrays ([2 batch]) is X_t for t < batch, W_{t - batch} after.
struct LinearBatchedArgs {
  int M, N, K, batch;
  const uint16_t* x;     // [batch][M][K]
  int64_t stride_x;      // elements
  const uint16_t* w;     // [batch][K][N]
  int64_t stride_w;
  uint8_t* xq;           // [batch][M][K] or null
  int64_t stride_xq;     // bytes
  uint8_t* wq;           // [batch][K][N] or null
  int64_t stride_wq;
  uint16_t* y;           // [batch][M][N] BF16
  int64_t stride_y;      // elements
  float* amax_y;         // [batch] or null
  float* history;        // [2 batch][hist_len]
  int32_t* cursor;       // [2 batch]
  int hist_len, algo, margin;
  float* scale;          // [2 batch] in: this step's scales; out: the next step's
  float* scale_used;     // [2 batch] or null: this step's scales
  float* amax;           // [2 batch]: this step's amax of each input
  unsigned long long* sat;  // [2 batch] or null: saturated values of each cast
};
hipError_t launch_linear_batched(const LinearBatchedArgs& a, int fx, int fw, hipStream_t stream);

// FP8 GEMM.  opa/opb: 0 = N, 1 = T.  out_bf16: BF16 output, else FP32.
struct GemmProblem {
  int opa, opb;
  int64_t M, N, K;
  const uint8_t* A;
  int fa;
  int64_t lda;
  const float* scale_a;
  const uint8_t* B;
  int fb;
  int64_t ldb;
  const float* scale_b;
  void* C;
  bool out_bf16;
  int64_t ldc;
  float* amax_c;  // reset by the caller
  int64_t batch;
  int64_t stride_a, stride_b, stride_c;  // bytes, bytes, elements
  const float* inv_a = nullptr;  // scale vectors (launch_gemm_rowcol): [M], [N]
  const float* inv_b = nullptr;
  const uint8_t* sc_a = nullptr;  // MX block scales (launch_gemm_mx): [M][ldsa], [N][ldsb]
  const uint8_t* sc_b = nullptr;
  int64_t ldsa = 0, ldsb = 0;
};
// EXACT datapath: FP8 widened to F16, F16 MFMA, FP32 sums.
hipError_t launch_gemm_exact(const GemmProblem& p, int num_cus, hipStream_t stream);
// FP8 datapath: native FP8 MFMA (hardware summation precision).
hipError_t launch_gemm_fp8(const GemmProblem& p, int num_cus, hipStream_t stream);
// EXACT datapath with one inverse scale per row of op(A) and per column of op(B)
// (p.inv_a, p.inv_b; batch 1).
hipError_t launch_gemm_rowcol(const GemmProblem& p, int num_cus, hipStream_t stream);
// MXFP8 GEMM C = A B^T (opa N, opb T), A and B blocked along K with E8M0 scales
// p.sc_a / p.sc_b; K a multiple of 128, operands 16-byte aligned, batch 1.
// exact: scales folded into the BF16 widening; else the block-scaled FP8 MFMA.
hipError_t launch_gemm_mx(const GemmProblem& p, bool exact, int num_cus, hipStream_t stream);

// MXFP8 cast of n elements (blocks of 32 consecutive elements): q [n], scales [n / 32].
hipError_t launch_mx_cast(const void* x, bool bf16, int64_t n, int fmt, uint8_t* q,
                          uint8_t* scales, hipStream_t stream);
// The same of a [rows x cols] matrix (both multiples of 128) plus its transpose q_t
// [cols x rows] blocked along its own rows, scales_t [cols][rows / 32].
hipError_t launch_mx_cast_transpose(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                                    uint8_t* q, uint8_t* scales, uint8_t* qt, uint8_t* scales_t,
                                    hipStream_t stream);

}  // namespace fp8ds

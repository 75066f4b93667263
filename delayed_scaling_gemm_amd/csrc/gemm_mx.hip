// The MXFP8 GEMM ("FP8 混合精度训练工程实践" §九: blocks of 32 FP8 values along the
// contraction, each with its own E8M0 scale; FP32 accumulation), instantiated in
// a translation unit of its own.  Exact datapath: the kernel of gemm_kernel.h
// with each FP8 byte widened to BF16 times its block's scale, so C = sum over
// blocks of X_a X_b sum_i Pa_i Pb_i needs no per-block rescaling of the
// accumulator.  FP8 datapath: gfx950's block-scaled FP8 MFMA, each lane handing
// the instruction the E8M0 scale of the 32 K values it supplies.
#include "gemm_kernel.h"

namespace fp8ds {

template <int BM, int BN, int FA, int FB, bool EXACT>
static hipError_t launch_mx_t(const GemmProblem& q, hipStream_t s) {
  return launch_cfg<BM, BN, true, true, FA, FB, EXACT, true, false, true>(q, s);
}

template <int BM, int BN, bool EXACT>
static hipError_t launch_mx_tile(const GemmProblem& q, hipStream_t s) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return launch_mx_t<BM, BN, kE4M3, kE4M3, EXACT>(q, s);
  if (q.fa == kE4M3 && q.fb == kE5M2) return launch_mx_t<BM, BN, kE4M3, kE5M2, EXACT>(q, s);
  if (q.fa == kE5M2 && q.fb == kE4M3) return launch_mx_t<BM, BN, kE5M2, kE4M3, EXACT>(q, s);
  if (q.fa == kE5M2 && q.fb == kE5M2) return launch_mx_t<BM, BN, kE5M2, kE5M2, EXACT>(q, s);
  return hipErrorInvalidValue;
}

// The FP8 datapath keeps 128 x 128 tiles: at 256 x 256 its raw operand registers
// leave no room for the per-lane scale dwords (the compiler spills 76 of them).
template <bool EXACT>
static hipError_t launch_mx_path(const GemmProblem& q, int num_cus, hipStream_t stream) {
  if constexpr (EXACT) {
    const int64_t big_tiles = ((q.M + 255) / 256) * ((q.N + 255) / 256);
    if (big_tiles >= num_cus && q.K >= kBigTileMinK) return launch_mx_tile<256, 256, EXACT>(q, stream);
  }
  return launch_mx_tile<128, 128, EXACT>(q, stream);
}

hipError_t launch_gemm_mx(const GemmProblem& q, bool exact, int num_cus, hipStream_t stream) {
  if (q.opa != 0 || q.opb != 1 || q.batch != 1 || q.K % 128 != 0 || (q.K > 0 && (!q.sc_a || !q.sc_b)))
    return hipErrorInvalidValue;
  if (q.M <= 0 || q.N <= 0) return hipSuccess;
  return exact ? launch_mx_path<true>(q, num_cus, stream) : launch_mx_path<false>(q, num_cus, stream);
}

}  // namespace fp8ds

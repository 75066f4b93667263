// The exact-datapath GEMM with per-row / per-column scales ("FP8 混合精度训练工程
// 实践" §FBGEMM_GPU 底层优化: per-token and per-channel FP8 GEMM, FP32 accumulation,
// BF16 output): the kernels of gemm_exact.hip with the scale-vector epilogue,
// instantiated in a translation unit of their own.
#include "gemm_kernel.h"

namespace fp8ds {

hipError_t launch_gemm_rowcol(const GemmProblem& q, int num_cus, hipStream_t stream) {
  if (!q.inv_a || !q.inv_b || q.batch != 1) return hipErrorInvalidValue;
  return launch_path<true, true>(q, num_cus, stream);
}

}  // namespace fp8ds

// Instantiations of the EXACT datapath of the FP8 GEMM (FP8 bytes widened to
// F16 in registers, F16 MFMA with FP32 accumulation); see gemm_kernel.h.
#include "gemm_kernel.h"

namespace fp8ds {

hipError_t launch_gemm_exact(const GemmProblem& q, int num_cus, hipStream_t stream) {
  return launch_path<true>(q, num_cus, stream);
}

}  // namespace fp8ds

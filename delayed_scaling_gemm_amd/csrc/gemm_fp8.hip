// Instantiations of the FP8 datapath of the FP8 GEMM (native FP8 MFMA, with the
// hardware's summation precision); see gemm_kernel.h.
#include "gemm_kernel.h"

namespace fp8ds {

hipError_t launch_gemm_fp8(const GemmProblem& q, int num_cus, hipStream_t stream) {
  return launch_path<false>(q, num_cus, stream);
}

}  // namespace fp8ds

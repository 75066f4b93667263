// Delayed-scaling state update of many tensors: one wave per tensor runs
// scale_update_wave (history push, window reduction, next scale; the passages
// it follows are cited there).  Optionally the same launch zeroes a caller
// buffer: the accumulators the next step's casts and GEMMs combine into, so that
// no reset kernel runs before them.

#include "launch.h"
#include "scale_update.h"

namespace fp8ds {

__global__ __launch_bounds__(64) void scale_update_kernel(int n, int hist_len,
                                                          float* __restrict__ history,
                                                          int32_t* __restrict__ cursor,
                                                          const float* __restrict__ amax, FmtBits fmt,
                                                          int algo, int margin,
                                                          float* __restrict__ scale,
                                                          float* __restrict__ scale_inv,
                                                          uint32_t* __restrict__ clear,
                                                          int64_t n_clear) {
  const int t = blockIdx.x;
  if (t >= n) return;
  const int lane = threadIdx.x;
  // the next step's accumulators, spread over the blocks
  for (int64_t i = (int64_t)t * 64 + lane; i < n_clear; i += (int64_t)n * 64) clear[i] = 0u;
  const bool e5m2 = (fmt.w[t >> 5] >> (t & 31)) & 1u;
  scale_update_wave(history + (int64_t)t * hist_len, hist_len, cursor + t, amax[t], e5m2, algo,
                    margin, scale + t, scale_inv ? scale_inv + t : nullptr, lane);
}

hipError_t launch_scale_update(int n, int hist_len, float* history, int32_t* cursor,
                               const float* amax, const FmtBits& fmt, int algo, int margin,
                               float* scale, float* scale_inv, hipStream_t stream,
                               uint32_t* clear, int64_t n_clear) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_update_kernel, dim3(n), dim3(64), 0, stream, n, hist_len, history,
                     cursor, amax, fmt, algo, margin, scale, scale_inv, clear,
                     clear ? n_clear : 0);
  return hipGetLastError();
}

}  // namespace fp8ds

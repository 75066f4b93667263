// Delayed-scaling state update: history ring push, window reduction, next scale.
//
// "LLM FP8 微调上线生产实战" §核心原理: scale = (FP8_MAX / amax) / 2^margin, with the
// amax taken from a history window (max) or the newest entry (most_recent).
// "FP8 混合精度训练工程实践" §四 (Delayed Scaling 的工程细节): the new amax is written at
// the cursor, the cursor advances modulo the history length, and the scale falls
// back to 1.0 when the window maximum is not positive.
//
// One wave per tensor.  Optionally the same launch zeroes a caller buffer: the
// accumulators the next step's casts and GEMMs combine into, so that no reset
// kernel runs before them.  The window (up to 65536 fp32) is read with a stride of 64
// lanes; the slot being overwritten takes the new amax in registers, so no lane
// depends on another lane's store.  The max tracks NaN separately so that the
// result is NaN whenever any entry is, whatever the entries' signs.

#include "device_common.h"
#include "launch.h"

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
  float* h = history + (int64_t)t * hist_len;
  // The cursor is caller state in device memory; reduce it modulo the history
  // length so that a corrupted value can never address outside this history.
  int c = cursor[t] % hist_len;
  if (c < 0) c += hist_len;
  const float a = amax[t];

  float m = -INFINITY;
  int any_nan = 0;
  for (int i = lane; i < hist_len; i += 64) {
    float v = (i == c) ? a : h[i];
    if (v != v) any_nan = 1;
    else m = fmaxf(m, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    m = fmaxf(m, __shfl_xor(m, off, 64));
    any_nan |= __shfl_xor(any_nan, off, 64);
  }
  if (lane != 0) return;

  h[c] = a;
  cursor[t] = (c + 1 == hist_len) ? 0 : c + 1;

  float w = (algo == 0) ? (any_nan ? __uint_as_float(0x7FC00000u) : m) : a;
  const bool e5m2 = (fmt.w[t >> 5] >> (t & 31)) & 1u;
  const float fmax = e5m2 ? FmtTraits<kE5M2>::kMax : FmtTraits<kE4M3>::kMax;
  const float s = scale_from_amax(w, fmax, margin);
  scale[t] = s;
  if (scale_inv) scale_inv[t] = __fdiv_rn(1.0f, s);
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

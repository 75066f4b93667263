// Delayed-scaling state update of one tensor by one wave: history ring push,
// window reduction, next scale.
//
// "LLM FP8 微调上线生产实战" §核心原理: scale = (FP8_MAX / amax) / 2^margin, with the
// amax taken from a history window (max) or the newest entry (most_recent).
// "FP8 混合精度训练工程实践" §四 (Delayed Scaling 的工程细节): the new amax is written at
// the cursor, the cursor advances modulo the history length, and the scale falls
// back to 1.0 when the window maximum is not positive.
//
// The window (up to 65536 fp32) is read with a stride of 64 lanes; the slot
// being overwritten takes the new amax in registers, so no lane depends on
// another lane's store.  The max tracks NaN separately so that the result is
// NaN whenever any entry is, whatever the entries' signs.
#pragma once

#include "device_common.h"

namespace fp8ds {

// h: the tensor's history [hist_len]; cursor, scale, scale_inv (or null): its
// entries; a: this step's amax; all 64 lanes of the wave call it.
__device__ __forceinline__ void scale_update_wave(float* __restrict__ h, int hist_len,
                                                  int32_t* __restrict__ cursor, float a, bool e5m2,
                                                  int algo, int margin, float* __restrict__ scale,
                                                  float* __restrict__ scale_inv, int lane) {
  // The cursor is caller state in device memory; reduce it modulo the history
  // length so that a corrupted value can never address outside this history.
  int c = *cursor % hist_len;
  if (c < 0) c += hist_len;

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
  if (lane == 0) {
    h[c] = a;
    *cursor = (c + 1 == hist_len) ? 0 : c + 1;
    const float w = (algo == 0) ? (any_nan ? __uint_as_float(0x7FC00000u) : m) : a;
    const float fmax = e5m2 ? FmtTraits<kE5M2>::kMax : FmtTraits<kE4M3>::kMax;
    const float s = scale_from_amax(w, fmax, margin);
    *scale = s;
    if (scale_inv) *scale_inv = __fdiv_rn(1.0f, s);
  }
}

}  // namespace fp8ds

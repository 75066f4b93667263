// Device-side helpers shared by the HIP kernels of the FP8 delayed-scaling Linear.
//
// FP8 encoding follows the OCP formats named on "FP8 混合精度训练工程实践" §一
// (E4M3: bias 7, max 448; E5M2: bias 15, max 57344) with saturation to the
// largest finite value, round to nearest even, canonical NaN 0x7F|sign.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8ds {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

// Largest finite value of each format and its fp32 bit pattern.
template <int FMT> struct FmtTraits;
template <> struct FmtTraits<kE4M3> {
  static constexpr float kMax = 448.0f;
  static constexpr uint32_t kMaxBits = 0x43E00000u;      // 448.0f
  static constexpr uint32_t kMinNormalBits = 0x3C800000u; // 2^-6
  static constexpr int kMantBits = 3;
  static constexpr uint32_t kRebias = (127u - 7u);        // fp32 bias - fp8 bias
  static constexpr uint32_t kSubMagicBits = 0x46800000u;  // 2^14: fp32 ulp there is 2^-9
};
template <> struct FmtTraits<kE5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr uint32_t kMaxBits = 0x47600000u;      // 57344.0f
  static constexpr uint32_t kMinNormalBits = 0x38800000u; // 2^-14
  static constexpr int kMantBits = 2;
  static constexpr uint32_t kRebias = (127u - 15u);
  static constexpr uint32_t kSubMagicBits = 0x43000000u;  // 2^7: fp32 ulp there is 2^-16
};

// Magnitude code (7 bits) of a non-NaN fp32 magnitude |v| given as bits `a`
// (a <= 0x7F800000).  Saturating round-to-nearest-even.
template <int FMT>
__device__ __forceinline__ uint32_t encode_magnitude(uint32_t a) {
  using T = FmtTraits<FMT>;
  constexpr int kDrop = 23 - T::kMantBits;
  a = min(a, T::kMaxBits);  // saturation: everything above max (inf included) -> max
  // Normal range: round the fp32 mantissa to kMantBits bits (ties to even), then
  // move the exponent from bias 127 to the format's bias.  A rounding carry
  // propagates into the exponent field, which is the correct next binade.
  uint32_t r = a + ((1u << (kDrop - 1)) - 1u) + ((a >> kDrop) & 1u);
  uint32_t cn = (r - (T::kRebias << 23)) >> kDrop;
  // Subnormal range: add a power of two whose fp32 ulp equals the format's
  // subnormal quantum; the IEEE add then rounds |v| to a multiple of the quantum
  // (ties to even), and the difference of the bit patterns counts the quanta,
  // which is the code (8 or 4 quanta is the smallest normal, also correct).
  float f = __uint_as_float(a) + __uint_as_float(T::kSubMagicBits);
  uint32_t cs = __float_as_uint(f) - T::kSubMagicBits;
  return a < T::kMinNormalBits ? cs : cn;
}

// Full FP8 code of an fp32 value (sign, NaN -> 0x7F|sign).
template <int FMT>
__device__ __forceinline__ uint32_t encode_fp8(float v) {
  uint32_t b = __float_as_uint(v);
  uint32_t a = b & 0x7FFFFFFFu;
  uint32_t c = encode_magnitude<FMT>(a);
  c = a > 0x7F800000u ? 0x7Fu : c;
  return c | ((b >> 24) & 0x80u);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
  return v;
}

// Turn the max of |x| bit patterns into the amax bits: any NaN pattern becomes the
// canonical quiet NaN, so that an atomic max over blocks stays canonical.
__device__ __forceinline__ uint32_t canonical_amax_bits(uint32_t m) {
  return m > 0x7F800000u ? 0x7FC00000u : m;
}

// Scale from an amax or window value w ("LLM FP8 微调上线生产实战" §核心原理: scale =
// (FP8_MAX / amax) / 2^margin): one correctly rounded fp32 division and an exact
// power-of-two rescale (rounded only if subnormal); 1.0 unless w and the result are
// finite and positive (NaN fails every comparison).
__device__ __forceinline__ float scale_from_amax(float w, float fmax, int margin) {
  float s = 1.0f;
  if (w > 0.0f && w <= __uint_as_float(0x7F7FFFFFu)) {
    const float sc = ldexpf(__fdiv_rn(fmax, w), -margin);
    if (sc > 0.0f && sc <= __uint_as_float(0x7F7FFFFFu)) s = sc;
  }
  return s;
}


}  // namespace fp8ds

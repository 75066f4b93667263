// MXFP8 quantization: FP8 elements in blocks of 32 consecutive elements of a row,
// each block sharing one E8M0 (power-of-two) scale.
//
// What is computed ("FP8 混合精度训练工程实践" §九: groups of 32 FP8 values share an
// 8-bit E8M0 scale, each block scaled locally; the block rule of the OCP
// Microscaling Formats specification the figure there refers to):
//   a = max |x_i| over the block,
//   code = floor(log2 a) - emax_elem + 127, clamped to [0, 254]   (emax_elem 8 / 15)
//        = 0 for a zero block, 255 (NaN) for a block holding NaN or Inf,
//   q_i  = encode(x_i * 2^(127 - code)), saturating round-to-nearest-even,
//        = 0x7F (NaN) for every element of a NaN block.
// For a normal fp32 amax with biased exponent f, floor(log2 a) = f - 127, so the
// code is f - emax_elem (0 when that is not positive: zero, subnormal and tiny
// amaxes all clamp to the smallest scale); the multiplier 2^(127 - code) is the
// normal fp32 number with biased exponent 254 - code, and the product with an
// fp32 input is exact wherever the FP8 code does not round to zero.
//
// Design for gfx950: the pass is HBM-bound (2 or 4 bytes read, 1 + 1/32 written
// per element).  Rows are a whole number of blocks, so the tensor is a flat
// sequence of blocks; lanes take consecutive 16-byte pieces (a wave's load is one
// contiguous 1 KiB run), 4 (BF16) or 8 (FP32) consecutive lanes hold one block and
// reduce its amax with lane shuffles, and every lane converts its own piece with
// the block's multiplier.  Each thread issues all its loads first.

#include "cast_common.h"
#include "launch.h"

namespace fp8ds {

constexpr int kMxPieces = 8;  // 16-byte pieces per thread

template <int FMT>
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t abits) {
  constexpr uint32_t kEmax = FMT == kE4M3 ? 8u : 15u;  // exponent of the largest normal value
  const uint32_t f = abits >> 23;                       // biased exponent of the amax
  if (f == 255u) return 255u;
  return f > kEmax ? f - kEmax : 0u;
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void mx_cast_kernel(const void* __restrict__ x, int64_t npieces,
                                                      uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ scales) {
  constexpr int PPB = BF16 ? 4 : 8;  // pieces (lanes) per block of 32 elements
  const int64_t base = (int64_t)blockIdx.x * 256 * kMxPieces + threadIdx.x;
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4 v[kMxPieces];
#pragma unroll
  for (int j = 0; j < kMxPieces; ++j) {
    const int64_t pc = base + 256 * j;
    v[j] = pc < npieces ? __builtin_nontemporal_load(xv + pc) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kMxPieces; ++j) {
    const int64_t pc = base + 256 * j;  // a block's lanes are all in range or all out
    uint32_t a = piece_amax<BF16>(v[j]);
    a = max(a, (uint32_t)__shfl_xor((int)a, 1));
    a = max(a, (uint32_t)__shfl_xor((int)a, 2));
    if constexpr (PPB == 8) a = max(a, (uint32_t)__shfl_xor((int)a, 4));
    if (pc < npieces) {
      const uint32_t code = mx_scale_code<FMT>(a);
      u32x2 c;
      if (code == 255u) {
        c = u32x2{0x7F7F7F7Fu, BF16 ? 0x7F7F7F7Fu : 0u};
      } else {
        c = piece_codes<BF16, FMT>(v[j], __uint_as_float((254u - code) << 23));
      }
      if constexpr (BF16)
        __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(q) + pc);
      else
        __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(q) + pc);
      if ((threadIdx.x & (PPB - 1)) == 0) scales[pc / PPB] = (uint8_t)code;
    }
  }
}

template <bool BF16>
static hipError_t launch_mx_b(const void* x, int64_t n, int fmt, uint8_t* q, uint8_t* scales,
                              hipStream_t stream) {
  const int64_t npieces = n / (BF16 ? 8 : 4);
  const int64_t per = 256 * kMxPieces;
  const int64_t blocks = (npieces + per - 1) / per;
  if (fmt == kE4M3)
    hipLaunchKernelGGL((mx_cast_kernel<BF16, kE4M3>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, npieces, q, scales);
  else
    hipLaunchKernelGGL((mx_cast_kernel<BF16, kE5M2>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, npieces, q, scales);
  return hipGetLastError();
}

hipError_t launch_mx_cast(const void* x, bool bf16, int64_t n, int fmt, uint8_t* q,
                          uint8_t* scales, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  return bf16 ? launch_mx_b<true>(x, n, fmt, q, scales, stream)
              : launch_mx_b<false>(x, n, fmt, q, scales, stream);
}

}  // namespace fp8ds

// Current (just-in-time) FP8 scaling, per tensor and per row.
//
// What is computed ("FP8 混合精度训练工程实践" §FBGEMM_GPU 底层优化: per-token and
// per-channel FP8 GEMM operands; the scale formula of "LLM FP8 微调上线生产实战"
// §核心原理 applied to the amax of what is being cast, with no history):
//   per row r of an [R x C] matrix:  a_r = max_c |x[r][c]|,
//     s_r = (FP8_MAX / a_r) / 2^margin (1.0 if a_r is 0, infinite or NaN),
//     q[r][c] = encode(fl32(x[r][c] * s_r)),  scale_inv[r] = fl32(1 / s_r).
// Per-token scaling of X [M x K] is this on X; per-channel scaling of a weight
// W [K x N] is this on its transpose [N x K], the layout the forward GEMM reads.
//
// Design for gfx950: one workgroup per row.  Pass 1 reads the row as
// lane-contiguous 16-byte pieces (8 BF16 or 4 FP32 elements), keeping the first
// 4 pieces of each thread in registers (rows up to 8192 BF16 / 4096 FP32
// elements are read from memory once), and reduces the amax over the
// workgroup; pass 2 converts with the row's scale, re-reading only the pieces
// not kept.  HBM-bound: 3 (BF16) or 5 (FP32) bytes per element.

#include "cast_common.h"
#include "launch.h"

namespace fp8ds {

template <bool BF16>
__device__ __forceinline__ float elem(const void* x, int64_t i, uint32_t& bits) {
  if constexpr (BF16) {
    bits = (uint32_t)static_cast<const uint16_t*>(x)[i] << 16;
  } else {
    bits = static_cast<const uint32_t*>(x)[i];
  }
  return __uint_as_float(bits);
}

constexpr int kRowCache = 4;  // pieces per thread kept in registers between the passes

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void rowwise_cast_kernel(const void* __restrict__ x, int64_t cols,
                                                           int margin, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale,
                                                           float* __restrict__ scale_inv,
                                                           float* __restrict__ amax_out) {
  constexpr int PER = BF16 ? 8 : 4;
  __shared__ uint32_t red[4];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const void* xr = static_cast<const char*>(x) + r * cols * (BF16 ? 2 : 4);
  uint8_t* qr = q + r * cols;
  // pieces: whole rows of 16-byte pieces whose codes land on 8- / 4-byte boundaries
  const bool vec = cols % PER == 0;
  const int64_t np = vec ? cols / PER : 0;
  const u32x4* xv = static_cast<const u32x4*>(xr);

  uint32_t am = 0;
  u32x4 cache[kRowCache];
#pragma unroll
  for (int j = 0; j < kRowCache; ++j) {
    const int64_t pc = tid + 256 * j;
    if (pc < np) {
      cache[j] = __builtin_nontemporal_load(xv + pc);
      am = max(am, piece_amax<BF16>(cache[j]));
    }
  }
  for (int64_t pc = tid + 256 * kRowCache; pc < np; pc += 256)
    am = max(am, piece_amax<BF16>(xv[pc]));
  if (!vec) {
    for (int64_t i = tid; i < cols; i += 256) {
      uint32_t b;
      elem<BF16>(xr, i, b);
      am = max(am, b & 0x7FFFFFFFu);
    }
  }
  am = wave_max_u32(am);
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = max(max(red[0], red[1]), max(red[2], red[3]));
  const float w = __uint_as_float(canonical_amax_bits(am));
  const float s = scale_from_amax(w, FmtTraits<FMT>::kMax, margin);
  if (tid == 0) {
    scale[r] = s;
    if (scale_inv) scale_inv[r] = __fdiv_rn(1.0f, s);
    if (amax_out) amax_out[r] = w;
  }

#pragma unroll
  for (int j = 0; j < kRowCache; ++j) {
    const int64_t pc = tid + 256 * j;
    if (pc < np) {
      const u32x2 c = piece_codes<BF16, FMT>(cache[j], s);
      if constexpr (BF16) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(qr) + pc);
      else __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(qr) + pc);
    }
  }
  for (int64_t pc = tid + 256 * kRowCache; pc < np; pc += 256) {
    const u32x2 c = piece_codes<BF16, FMT>(xv[pc], s);
    if constexpr (BF16) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(qr) + pc);
    else __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(qr) + pc);
  }
  if (!vec) {
    for (int64_t i = tid; i < cols; i += 256) {
      uint32_t b;
      qr[i] = (uint8_t)encode_fp8<FMT>(elem<BF16>(xr, i, b) * s);
    }
  }
}

// scale = scale_from_amax(*amax), scale_inv = fl32(1 / scale): one thread.
__global__ void current_scale_kernel(const float* __restrict__ amax, float fmax, int margin,
                                     float* __restrict__ scale, float* __restrict__ scale_inv) {
  const float s = scale_from_amax(*amax, fmax, margin);
  *scale = s;
  if (scale_inv) *scale_inv = __fdiv_rn(1.0f, s);
}

// ------------------------------------------------------------------ host launchers

hipError_t launch_rowwise_cast(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                               int margin, uint8_t* q, float* scale, float* scale_inv,
                               float* amax, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)rows);
  if (bf16) {
    if (fmt == kE4M3)
      hipLaunchKernelGGL((rowwise_cast_kernel<true, kE4M3>), grid, dim3(256), 0, stream, x, cols,
                         margin, q, scale, scale_inv, amax);
    else
      hipLaunchKernelGGL((rowwise_cast_kernel<true, kE5M2>), grid, dim3(256), 0, stream, x, cols,
                         margin, q, scale, scale_inv, amax);
  } else {
    if (fmt == kE4M3)
      hipLaunchKernelGGL((rowwise_cast_kernel<false, kE4M3>), grid, dim3(256), 0, stream, x, cols,
                         margin, q, scale, scale_inv, amax);
    else
      hipLaunchKernelGGL((rowwise_cast_kernel<false, kE5M2>), grid, dim3(256), 0, stream, x, cols,
                         margin, q, scale, scale_inv, amax);
  }
  return hipGetLastError();
}

hipError_t launch_current_scale(const float* amax, int fmt, int margin, float* scale,
                                float* scale_inv, hipStream_t stream) {
  const float fmax = fmt == kE4M3 ? FmtTraits<kE4M3>::kMax : FmtTraits<kE5M2>::kMax;
  hipLaunchKernelGGL(current_scale_kernel, dim3(1), dim3(1), 0, stream, amax, fmax, margin, scale,
                     scale_inv);
  return hipGetLastError();
}

}  // namespace fp8ds

// amax and the fused amax + scaled saturating cast (BF16/FP32 -> FP8).
//
// What is computed ("FP8 混合精度训练工程实践" §四 动态缩放, the quantize step):
//   amax = max |x|           of the unscaled input
//   q    = encode(fl32(x*s)) with s the delayed scale of this step
// Both in one pass over x: the scale is known before the pass (delayed scaling,
// "LLM FP8 微调上线生产实战" §核心原理), so the input is read once.
//
// Design for gfx950: the pass is HBM-bound (2 or 4 bytes read, 1 written per
// element).  Each thread moves 16 elements per step with 16-byte vector loads and
// one 16-byte store; a grid-stride loop over ~8 workgroups per CU keeps enough
// bytes in flight.  amax is an integer max over |x| bit patterns (exact and order
// independent), reduced by wave shuffles, then LDS, then one global atomic per
// workgroup.  The saturation count is reduced the same way with integer adds.

#include "device_common.h"
#include "launch.h"

namespace fp8ds {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ prologue
// Resets the reduction outputs and snapshots the scale, so the main kernels only
// ever combine into them.  A kernel (not a memset) so the sequence can be
// captured into a graph.
__global__ void prologue_kernel(int64_t count, const float* __restrict__ scale,
                                float* __restrict__ scale_used, uint32_t* __restrict__ amax_bits,
                                unsigned long long* __restrict__ sat) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  if (scale_used) scale_used[i] = scale[i];
  if (amax_bits) amax_bits[i] = 0u;
  if (sat) sat[i] = 0ull;
}

// ------------------------------------------------------------------ element access

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  return encode_fp8<FMT>(a) | (encode_fp8<FMT>(b) << 8) | (encode_fp8<FMT>(c) << 16) |
         (encode_fp8<FMT>(d) << 24);
}

template <int FMT>
__device__ __forceinline__ uint32_t sat4(float a, float b, float c, float d) {
  constexpr float M = FmtTraits<FMT>::kMax;
  return (uint32_t)(fabsf(a) > M) + (uint32_t)(fabsf(b) > M) + (uint32_t)(fabsf(c) > M) +
         (uint32_t)(fabsf(d) > M);
}

// Process 16 consecutive elements already loaded as 4 dwords of bf16 pairs (x2)
// or 4 x 4 floats.  Returns the 16 codes; accumulates amax bits and saturations.
template <int FMT>
__device__ __forceinline__ u32x4 cast16_bf16(const uint32_t (&d)[8], float s, u16x2& amax2,
                                              uint32_t& sat, bool want_sat) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t d0 = d[2 * j], d1 = d[2 * j + 1];
    u16x2 m0 = __builtin_bit_cast(u16x2, d0 & 0x7FFF7FFFu);
    u16x2 m1 = __builtin_bit_cast(u16x2, d1 & 0x7FFF7FFFu);
    amax2 = __builtin_elementwise_max(amax2, __builtin_elementwise_max(m0, m1));
    float a = bf16_lo(d0) * s, b = bf16_hi(d0) * s, c = bf16_lo(d1) * s, e = bf16_hi(d1) * s;
    out[j] = encode4<FMT>(a, b, c, e);
    if (want_sat) sat += sat4<FMT>(a, b, c, e);
  }
  return out;
}

template <int FMT>
__device__ __forceinline__ u32x4 cast16_f32(const uint32_t (&d)[16], float s, uint32_t& amax,
                                             uint32_t& sat, bool want_sat) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t b = d[4 * j + i];
      amax = max(amax, b & 0x7FFFFFFFu);
      v[i] = __uint_as_float(b) * s;
    }
    out[j] = encode4<FMT>(v[0], v[1], v[2], v[3]);
    if (want_sat) sat += sat4<FMT>(v[0], v[1], v[2], v[3]);
  }
  return out;
}

// ------------------------------------------------------------------ cast kernel
// One tensor per blockIdx.y (batched casts use gridDim.y > 1).  WRITE_Q = false
// gives the standalone amax.

struct CastArgs {
  const void* x;
  int64_t n;          // elements per tensor
  int64_t stride_x;   // elements between tensors
  const float* scale; // [batch]
  uint8_t* q;         // may be null (amax only)
  int64_t stride_q;   // bytes between tensors
  uint32_t* amax;     // [batch] or null
  unsigned long long* sat;  // [batch] or null
};

template <bool BF16, int FMT, bool WRITE_Q>
__global__ __launch_bounds__(256) void cast_kernel(CastArgs p) {
  __shared__ uint32_t red[8];
  const int b = blockIdx.y;
  const float s = WRITE_Q ? p.scale[b] : 1.0f;
  const bool want_sat = WRITE_Q && p.sat != nullptr;
  const int64_t n = p.n;
  const int64_t ngroups = n >> 4;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  uint32_t amax = 0, sat = 0;
  u16x2 amax2 = {0, 0};

  if constexpr (BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(p.x) + b * p.stride_x;
    uint8_t* q = WRITE_Q ? p.q + b * p.stride_q : nullptr;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t g = tid; g < ngroups; g += nthreads) {
      u32x4 v0 = xv[2 * g];
      u32x4 v1 = xv[2 * g + 1];
      uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if constexpr (WRITE_Q) {
        u32x4 c = cast16_bf16<FMT>(d, s, amax2, sat, want_sat);
        reinterpret_cast<u32x4*>(q)[g] = c;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu));
      }
    }
    // ragged tail: fewer than 16 elements, one per thread
    const int64_t t0 = ngroups << 4;
    if (tid < n - t0) {
      uint32_t bits = x[t0 + tid];
      amax = max(amax, (bits & 0x7FFFu) << 16);
      if constexpr (WRITE_Q) {
        float v = __uint_as_float(bits << 16) * s;
        q[t0 + tid] = (uint8_t)encode_fp8<FMT>(v);
        if (want_sat) sat += (uint32_t)(fabsf(v) > FmtTraits<FMT>::kMax);
      }
    }
    amax = max(amax, ((uint32_t)max(amax2.x, amax2.y)) << 16);
  } else {
    const uint32_t* x = static_cast<const uint32_t*>(p.x) + b * p.stride_x;
    uint8_t* q = WRITE_Q ? p.q + b * p.stride_q : nullptr;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t g = tid; g < ngroups; g += nthreads) {
      uint32_t d[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 v = xv[4 * g + i];
        d[4 * i] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
      }
      if constexpr (WRITE_Q) {
        u32x4 c = cast16_f32<FMT>(d, s, amax, sat, want_sat);
        reinterpret_cast<u32x4*>(q)[g] = c;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = max(amax, d[i] & 0x7FFFFFFFu);
      }
    }
    const int64_t t0 = ngroups << 4;
    if (tid < n - t0) {
      uint32_t bits = x[t0 + tid];
      amax = max(amax, bits & 0x7FFFFFFFu);
      if constexpr (WRITE_Q) {
        float v = __uint_as_float(bits) * s;
        q[t0 + tid] = (uint8_t)encode_fp8<FMT>(v);
        if (want_sat) sat += (uint32_t)(fabsf(v) > FmtTraits<FMT>::kMax);
      }
    }
  }
  block_commit_amax_sat(amax, sat, p.amax ? p.amax + b : nullptr, want_sat ? p.sat + b : nullptr,
                        red);
}

// ------------------------------------------------------------------ cast + transposed copy
// Tiles of 64 x 64 elements: each thread converts 16 consecutive elements of one
// row (coalesced read, 16-byte store to q), parks the codes in LDS, and after a
// barrier writes 16 consecutive rows of one column to q_t.  Partial tiles take
// element-wise guarded paths.

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void cast_transpose_kernel(const void* __restrict__ xp,
                                                             int64_t rows, int64_t cols,
                                                             const float* __restrict__ scale,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ qt,
                                                             uint32_t* __restrict__ g_amax,
                                                             unsigned long long* __restrict__ g_sat) {
  __shared__ uint8_t tile[64][64 + 4];
  __shared__ uint32_t red[8];
  const float s = scale[0];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int tr = threadIdx.x >> 2;         // row within tile
  const int tc = (threadIdx.x & 3) * 16;   // first column within tile
  const int64_t r = r0 + tr;
  uint32_t amax = 0, sat = 0;
  uint8_t codes[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t c = c0 + tc + i;
    uint32_t code = 0;
    if (r < rows && c < cols) {
      float v;
      if constexpr (BF16) {
        uint32_t bits = static_cast<const uint16_t*>(xp)[r * cols + c];
        amax = max(amax, (bits & 0x7FFFu) << 16);
        v = __uint_as_float(bits << 16) * s;
      } else {
        uint32_t bits = static_cast<const uint32_t*>(xp)[r * cols + c];
        amax = max(amax, bits & 0x7FFFFFFFu);
        v = __uint_as_float(bits) * s;
      }
      code = encode_fp8<FMT>(v);
      if (g_sat) sat += (uint32_t)(fabsf(v) > FmtTraits<FMT>::kMax);
    }
    codes[i] = (uint8_t)code;
    tile[tr][tc + i] = (uint8_t)code;
  }
  if (r < rows) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t c = c0 + tc + i;
      if (c < cols) q[r * cols + c] = codes[i];
    }
  }
  __syncthreads();
  // transposed: thread writes column (c0 + tr), rows r0 + tc .. +15
  const int64_t oc = c0 + tr;
  if (oc < cols) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t orow = r0 + tc + i;
      if (orow < rows) qt[oc * rows + orow] = tile[tc + i][tr];
    }
  }
  block_commit_amax_sat(amax, sat, g_amax, g_sat, red);
}

// ------------------------------------------------------------------ host launchers

static int grid_for(int64_t groups, int num_cus) {
  int64_t want = (groups + 255) / 256;
  int64_t cap = (int64_t)num_cus * 8;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

hipError_t launch_prologue(int64_t count, const float* scale, float* scale_used, float* amax,
                           uint64_t* sat, hipStream_t stream) {
  if (count <= 0 || (!scale_used && !amax && !sat)) return hipSuccess;
  int blocks = (int)((count + 255) / 256);
  hipLaunchKernelGGL(prologue_kernel, dim3(blocks), dim3(256), 0, stream, count, scale, scale_used,
                     reinterpret_cast<uint32_t*>(amax), reinterpret_cast<unsigned long long*>(sat));
  return hipGetLastError();
}

template <bool BF16, int FMT, bool WRITE_Q>
static hipError_t launch_cast_t(const CastArgs& a, int64_t batch, int num_cus, hipStream_t stream) {
  int64_t groups = (a.n >> 4) + 1;
  int gx = grid_for(groups, num_cus);
  if (batch > 1) {
    // spread ~8 blocks per CU over all tensors
    int64_t per = ((int64_t)num_cus * 8 + batch - 1) / batch;
    if (per < 1) per = 1;
    int64_t want = (groups + 255) / 256;
    gx = (int)(want < per ? (want < 1 ? 1 : want) : per);
  }
  hipLaunchKernelGGL((cast_kernel<BF16, FMT, WRITE_Q>), dim3(gx, (unsigned)batch), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_cast(const void* x, bool bf16, int64_t batch, int64_t n, int64_t stride_x,
                       int fmt, const float* scale, uint8_t* q, int64_t stride_q, float* amax,
                       uint64_t* sat, int num_cus, hipStream_t stream) {
  CastArgs a{x, n, stride_x, scale, q, stride_q, reinterpret_cast<uint32_t*>(amax),
             reinterpret_cast<unsigned long long*>(sat)};
  if (q == nullptr) {
    return bf16 ? launch_cast_t<true, kE4M3, false>(a, batch, num_cus, stream)
                : launch_cast_t<false, kE4M3, false>(a, batch, num_cus, stream);
  }
  if (bf16) {
    return fmt == kE4M3 ? launch_cast_t<true, kE4M3, true>(a, batch, num_cus, stream)
                        : launch_cast_t<true, kE5M2, true>(a, batch, num_cus, stream);
  }
  return fmt == kE4M3 ? launch_cast_t<false, kE4M3, true>(a, batch, num_cus, stream)
                      : launch_cast_t<false, kE5M2, true>(a, batch, num_cus, stream);
}

hipError_t launch_cast_transpose(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                                 const float* scale, uint8_t* q, uint8_t* qt, float* amax,
                                 uint64_t* sat, hipStream_t stream) {
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  uint32_t* am = reinterpret_cast<uint32_t*>(amax);
  unsigned long long* st = reinterpret_cast<unsigned long long*>(sat);
  if (bf16) {
    if (fmt == kE4M3)
      hipLaunchKernelGGL((cast_transpose_kernel<true, kE4M3>), grid, dim3(256), 0, stream, x, rows,
                         cols, scale, q, qt, am, st);
    else
      hipLaunchKernelGGL((cast_transpose_kernel<true, kE5M2>), grid, dim3(256), 0, stream, x, rows,
                         cols, scale, q, qt, am, st);
  } else {
    if (fmt == kE4M3)
      hipLaunchKernelGGL((cast_transpose_kernel<false, kE4M3>), grid, dim3(256), 0, stream, x, rows,
                         cols, scale, q, qt, am, st);
    else
      hipLaunchKernelGGL((cast_transpose_kernel<false, kE5M2>), grid, dim3(256), 0, stream, x, rows,
                         cols, scale, q, qt, am, st);
  }
  return hipGetLastError();
}

}  // namespace fp8ds

// Fused AdamW step on FP32 master weights that also writes the FP8 copy of the
// updated weights for the next forward.
//
// What is computed ("算子与编译器：FP8 训练与优化器 Kernel", §FP8 训练主路径图 and
// §Fused Optimizer 的意义: unscaled gradients feed one optimizer kernel that
// updates both moments and the master weights; "FP8 混合精度训练工程实践" §自动混合
// 精度与 FP8 的协同: gradient un-scaling, an FP32 AdamW step, then the updated
// weights cast to FP8 with scaling for the next forward).  Per element, every
// operation one rounded fp32 operation in this order, no fused multiply-add:
//   g = grad * grad_scale
//   m = beta1 * m + (1 - beta1) * g
//   v = beta2 * v + ((1 - beta2) * g) * g
//   w = (1 - lr * wd) * w - (lr / bc1) * (m / (sqrt(v) * (1 / sqrt(bc2)) + eps))
// (AdamW with decoupled weight decay, Loshchilov & Hutter; bias corrections
// bc_i = 1 - beta_i^t of Kingma & Ba), then q = encode(fl32(w * s)) with the
// delayed scale s of the weight tensor, q_t its transpose, amax = max |w|.
// A gradient whose amax (given) is not finite skips the update: w, m and v
// stay, and the FP8 copy is made of the unchanged weights.
//
// Design for gfx950: HBM-bound, 28 bytes per element with a BF16 gradient
// (read w, m, v 4 B each and g 2 B; write w, m, v and q, q_t 1 B each).  The
// FP8 copy costs 2 bytes per element here against 6 for a separate cast pass
// over the weights (read 4, write 2).  Each lane updates quads of 4 elements,
// placed so that every 16-byte non-temporal load and store instruction of a wave
// covers contiguous runs (lanes owning 64 contiguous bytes each, as the
// standalone casts' loads do, left every store writing 64 partial lines and
// measured 1.5 TB/s); the transposed copy goes through the same LDS tile and
// transposing reads as the standalone cast.

#include <math.h>

#include "cast_common.h"
#include "launch.h"

namespace fp8ds {

// One element of the update, in the order above.  The pragma keeps the
// compiler from contracting a multiply and an add into one rounding; the
// division and the square root are the correctly rounded fp32 operations.
__device__ __forceinline__ float adamw_elem(float w, float g, float& m, float& v,
                                            const AdamWConsts& c) {
#pragma clang fp contract(off)
  const float gs = g * c.grad_scale;
  m = c.b1 * m + c.omb1 * gs;
  v = c.b2 * v + (c.omb2 * gs) * gs;
  const float den = __builtin_sqrtf(v) * c.inv_sqrt_bc2 + c.eps;
  return c.decay * w - c.step_size * (m / den);
}

__device__ __forceinline__ bool adamw_skip(const AdamWLaunch& p) {
  if (p.grad_amax == nullptr) return false;
  const uint32_t b = __float_as_uint(*p.grad_amax) & 0x7FFFFFFFu;
  return b >= 0x7F800000u;  // infinity or NaN
}

// Updates four quads of 4 consecutive elements, quad k at element offset
// off[k] (16-byte aligned in the fp32 arrays, 8-byte in a BF16 gradient), and
// returns the new weights' bits in wb (quad k in wb[4k .. 4k+3]).  Callers
// place the quads of consecutive lanes next to each other, so every load and
// store instruction of a wave covers one contiguous run (1 KB of fp32).
// Skipped steps only read w.
template <bool GBF16>
__device__ __forceinline__ void adamw_quads(const AdamWLaunch& p, const int64_t (&off)[4],
                                            bool skip, uint32_t (&wb)[16]) {
  u32x4 wv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    wv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.w + off[k]));
  if (skip) {
#pragma unroll
    for (int i = 0; i < 16; ++i) wb[i] = wv[i >> 2][i & 3];
    return;
  }
  u32x4 mv[4], vv[4], gv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    mv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.m + off[k]));
    vv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v + off[k]));
    if constexpr (GBF16) {
      const u32x2 h = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.g) + off[k]));
      gv[k] = u32x4{h.x << 16, h.x & 0xFFFF0000u, h.y << 16, h.y & 0xFFFF0000u};
    } else {
      gv[k] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const float*>(p.g) + off[k]));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = __uint_as_float(mv[i >> 2][i & 3]);
    float v = __uint_as_float(vv[i >> 2][i & 3]);
    const float w = adamw_elem(__uint_as_float(wv[i >> 2][i & 3]),
                               __uint_as_float(gv[i >> 2][i & 3]), m, v, p.c);
    wb[i] = __float_as_uint(w);
    wv[i >> 2][i & 3] = wb[i];
    mv[i >> 2][i & 3] = __float_as_uint(m);
    vv[i >> 2][i & 3] = __float_as_uint(v);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    __builtin_nontemporal_store(wv[k], reinterpret_cast<u32x4*>(p.w + off[k]));
    __builtin_nontemporal_store(mv[k], reinterpret_cast<u32x4*>(p.m + off[k]));
    __builtin_nontemporal_store(vv[k], reinterpret_cast<u32x4*>(p.v + off[k]));
  }
}

// One element (ragged tails and unaligned tiles); returns the new weight.
template <bool GBF16>
__device__ __forceinline__ float adamw1(const AdamWLaunch& p, int64_t i, bool skip) {
  const float w = p.w[i];
  if (skip) return w;
  const float g = GBF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p.g)[i] << 16)
                        : static_cast<const float*>(p.g)[i];
  float m = p.m[i], v = p.v[i];
  const float wn = adamw_elem(w, g, m, v, p.c);
  p.w[i] = wn;
  p.m[i] = m;
  p.v[i] = v;
  return wn;
}

// The cast of one updated weight (as the standalone cast's element path).
template <int FMT>
__device__ __forceinline__ uint32_t cast1(float w, float s, uint32_t& amax, uint32_t& sat) {
  amax = max(amax, __float_as_uint(w) & 0x7FFFFFFFu);
  const float y = w * s;
  sat += (uint32_t)(fabsf(y) > FmtTraits<FMT>::kMax);
  return encode_fp8<FMT>(y);
}

// Flat kernel: the rows*cols elements as one array.  A workgroup of 256
// threads owns 4096 consecutive elements; thread t takes the quads at
// 4t + 1024k, k = 0..3.  The last, partial workgroup goes element by element.
// CAST = false is the plain fused AdamW step.
template <bool GBF16, int FMT, bool CAST>
__global__ __launch_bounds__(256) void adamw_kernel(AdamWLaunch p) {
  __shared__ uint32_t red[2 * 4];
  const int64_t n = p.rows * p.cols;
  const bool skip = adamw_skip(p);
  if (!CAST && skip) return;
  const float s = CAST ? p.scale[0] : 1.0f;
  const int64_t base = (int64_t)blockIdx.x * 4096 + 4 * threadIdx.x;
  uint32_t amax = 0, sat = 0;
  if ((int64_t)(blockIdx.x + 1) * 4096 <= n) {
    const int64_t off[4] = {base, base + 1024, base + 2048, base + 3072};
    uint32_t wb[16];
    adamw_quads<GBF16>(p, off, skip, wb);
    if constexpr (CAST) {
      const u32x4 codes = cast16_f32<FMT, false>(wb, s, amax, sat, p.sat != nullptr);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_nontemporal_store(codes[k], reinterpret_cast<uint32_t*>(p.q + off[k]));
    }
  } else {
    for (int k = 0; k < 4; ++k)
      for (int j = 0; j < 4; ++j) {
        const int64_t i = base + 1024 * k + j;
        if (i < n) {
          const float w = adamw1<GBF16>(p, i, skip);
          if constexpr (CAST) p.q[i] = (uint8_t)cast1<FMT>(w, s, amax, sat);
        }
      }
  }
  if constexpr (CAST) {
    Health h;
    block_commit<false>(amax, sat, h, reinterpret_cast<uint32_t*>(p.amax),
                        reinterpret_cast<unsigned long long*>(p.sat), nullptr, red);
  }
}

// Transposing kernel: a 128 x 128 tile of the [rows x cols] weights per
// workgroup; q and q_t as the standalone transposing cast writes them.
template <bool GBF16, int FMT>
__global__ __launch_bounds__(256) void adamw_transpose_kernel(AdamWLaunch p) {
  constexpr int T = 128;
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * T];
  __shared__ uint32_t red[2 * 4];
  const bool skip = adamw_skip(p);
  const float s = p.scale[0];
  const int64_t rows = p.rows, cols = p.cols;
  const int64_t r0 = (int64_t)blockIdx.y * T, c0 = (int64_t)blockIdx.x * T;
  const int tid = threadIdx.x;
  uint32_t amax = 0, sat = 0;
  const bool vec = (r0 + T <= rows) && (c0 + T <= cols) && (cols % 16 == 0) && (rows % 16 == 0);
  if (vec) {
    // pass i: quad u = 1024 i + 256 k + tid of the tile's 4096 (32 per row), so a
    // wave instruction covers two 512-byte row runs of fp32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t off[4];
      int rr[4], cc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int u = 1024 * i + 256 * k + tid;
        rr[k] = u >> 5;
        cc[k] = (u & 31) * 4;
        off[k] = (r0 + rr[k]) * cols + c0 + cc[k];
      }
      uint32_t wb[16];
      adamw_quads<GBF16>(p, off, skip, wb);
      const u32x4 codes = cast16_f32<FMT, false>(wb, s, amax, sat, p.sat != nullptr);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_nontemporal_store(codes[k], reinterpret_cast<uint32_t*>(p.q + off[k]));
        tile_park4(tile, rr[k], cc[k], codes[k]);
      }
    }
    __syncthreads();
    tile_store_qt<4>(tile, p.qt, rows, r0, c0, tid);
  } else {
    const int tr = tid >> 1;        // row within the tile
    const int tc = (tid & 1) * 64;  // first of this thread's 64 columns
    const int64_t r = r0 + tr;
#pragma unroll 1  // unrolled, this rarely used path would set the kernel's register count
    for (int i = 0; i < 64; ++i) {
      const int64_t c = c0 + tc + i;
      uint32_t code = 0;
      if (r < rows && c < cols) {
        const float w = adamw1<GBF16>(p, r * cols + c, skip);
        code = cast1<FMT>(w, s, amax, sat);
        p.q[r * cols + c] = (uint8_t)code;
      }
      tile[tr * T + tc + i] = (uint8_t)code;
    }
    __syncthreads();
    const int oc_l = tid >> 1;       // column within the tile
    const int orr = (tid & 1) * 64;  // first of this thread's 64 rows
    const int64_t oc = c0 + oc_l;
    if (oc < cols) {
#pragma unroll 1
      for (int i = 0; i < 64; ++i) {
        const int64_t orow = r0 + orr + i;
        if (orow < rows) p.qt[oc * rows + orow] = tile[(orr + i) * T + oc_l];
      }
    }
  }
  Health h;
  block_commit<false>(amax, sat, h, reinterpret_cast<uint32_t*>(p.amax),
                      reinterpret_cast<unsigned long long*>(p.sat), nullptr, red);
}

// ------------------------------------------------------------------ host launcher

template <bool GBF16, int FMT>
static hipError_t launch_adamw_t(const AdamWLaunch& a, hipStream_t stream) {
  if (a.qt) {
    const dim3 grid((unsigned)((a.cols + 127) / 128), (unsigned)((a.rows + 127) / 128));
    hipLaunchKernelGGL((adamw_transpose_kernel<GBF16, FMT>), grid, dim3(256), 0, stream, a);
  } else {
    const int64_t pieces = (a.rows * a.cols + 15) / 16;
    const dim3 grid((unsigned)((pieces + 255) / 256));
    if (a.q)
      hipLaunchKernelGGL((adamw_kernel<GBF16, FMT, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((adamw_kernel<GBF16, FMT, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamWLaunch& a, hipStream_t stream) {
  if (a.rows * a.cols == 0) return hipSuccess;
  if (a.g_bf16)
    return a.fmt == kE4M3 ? launch_adamw_t<true, kE4M3>(a, stream)
                          : launch_adamw_t<true, kE5M2>(a, stream);
  return a.fmt == kE4M3 ? launch_adamw_t<false, kE4M3>(a, stream)
                        : launch_adamw_t<false, kE5M2>(a, stream);
}

}  // namespace fp8ds

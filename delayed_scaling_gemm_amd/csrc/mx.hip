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
      } else {  // the block's amax is finite: so is every value in it
        c = piece_codes_finite<BF16, FMT>(v[j], __uint_as_float((254u - code) << 23));
      }
      if constexpr (BF16)
        __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(q) + pc);
      else
        __builtin_nontemporal_store(c.x, reinterpret_cast<uint32_t*>(q) + pc);
      if ((threadIdx.x & (PPB - 1)) == 0) scales[pc / PPB] = (uint8_t)code;
    }
  }
}

// ------------------------------------------------------------------ both orientations
// One read of x, two MX copies: q [rows x cols] with blocks along rows (as
// mx_cast_kernel) and q_t [cols x rows] = the transpose with blocks of 32
// consecutive rows of each column, i.e. blocks along the rows of q_t, with
// scales_t [cols][rows / 32].  A 128 x 128 tile per 256-thread workgroup (the
// layout of cast_transpose_kernel): pass i holds rows 32 i .. 32 i + 31 of the
// tile -- exactly one column block -- as lane-contiguous 16-byte pieces, every
// piece of a thread in the same 8 (BF16) or 4 (FP32) columns.  Row blocks are
// reduced by lane shuffles as in mx_cast_kernel; a column block's amax is the
// max over the thread's own pieces, then over the lanes of the same columns
// (shuffles), then over the four waves through LDS.  Column codes are parked in
// an LDS tile and written transposed by tile_store_qt.  Whole tiles only.

// Codes of one piece with one multiplier per element (column).  Columns whose
// block holds NaN or Inf (scale code 255) get the NaN code: `nan_bytes` has
// 0xFF in their bytes.  Every other column's block has a finite amax, so its
// values are finite and the packed converts alone encode them; whatever they
// give for a NaN column's bytes is replaced.
template <bool BF16, int FMT>
__device__ __forceinline__ u32x2 piece_codes_cols(const u32x4& d, const float (&m)[8],
                                                  const uint32_t (&nan_bytes)[2]) {
  u32x2 c;
  if constexpr (BF16) {
    c = u32x2{encode4_hw<FMT>(bf16_lo(d.x) * m[0], bf16_hi(d.x) * m[1], bf16_lo(d.y) * m[2],
                              bf16_hi(d.y) * m[3]),
              encode4_hw<FMT>(bf16_lo(d.z) * m[4], bf16_hi(d.z) * m[5], bf16_lo(d.w) * m[6],
                              bf16_hi(d.w) * m[7])};
  } else {
    c = u32x2{encode4_hw<FMT>(__uint_as_float(d.x) * m[0], __uint_as_float(d.y) * m[1],
                              __uint_as_float(d.z) * m[2], __uint_as_float(d.w) * m[3]), 0u};
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) c[k] = (c[k] & ~nan_bytes[k]) | (0x7F7F7F7Fu & nan_bytes[k]);
  return c;
}

// |x| bit patterns of the elements of a piece, as fp32 bits (element e of 8 / 4).
template <bool BF16>
__device__ __forceinline__ void piece_abs(const u32x4& d, uint32_t (&a)[8]) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[2 * k] = (d[k] & 0x7FFFu) << 16;
      a[2 * k + 1] = d[k] & 0x7FFF0000u;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = d[k] & 0x7FFFFFFFu;
  }
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void mx_cast_transpose_kernel(
    const void* __restrict__ xp, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ qt, uint8_t* __restrict__ scales_t) {
  constexpr int T = 128;
  constexpr int PER = BF16 ? 8 : 4;   // elements per piece
  constexpr int NP = 16 / PER;        // pieces per thread per pass
  constexpr int PPR = T / PER;        // pieces per tile row
  constexpr int PPB = 32 / PER;       // pieces per row block
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * T];
  // column amax exchange; rows padded to PER + 1 words so that the lanes' stores
  // and reads of one element fall in different LDS banks
  __shared__ uint32_t red[2][4][PPR][PER + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * T, r0 = (int64_t)blockIdx.y * T;
  const int cc = (tid % PPR) * PER;  // this thread's columns in the tile
  const int64_t nbr = cols / 32, nbc = rows / 32;  // blocks per row of q / of q_t
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    u32x4 v[NP];
    int rr[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int u = 256 * (NP * i + k) + tid;
      rr[k] = u / PPR;
      v[k] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(xp) +
                                             ((r0 + rr[k]) * cols + c0 + cc) * (BF16 ? 2 : 4));
    }
    // column amax of this pass (one column block), first over the thread's pieces
    uint32_t ca[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      uint32_t a[8];
      piece_abs<BF16>(v[k], a);
#pragma unroll
      for (int e = 0; e < PER; ++e) ca[e] = max(ca[e], a[e]);
    }
    // ... then over the lanes holding the same columns (lane % PPR), then the waves
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      for (int o = PPR; o < 64; o <<= 1) ca[e] = max(ca[e], (uint32_t)__shfl_xor((int)ca[e], o));
    }
    if (lane < PPR) {
#pragma unroll
      for (int e = 0; e < PER; ++e) red[i & 1][wave][lane][e] = ca[e];
    }
    // rows: each piece is in one row block shared with PPB - 1 neighbouring lanes
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      uint32_t a = piece_amax<BF16>(v[k]);
      a = max(a, (uint32_t)__shfl_xor((int)a, 1));
      a = max(a, (uint32_t)__shfl_xor((int)a, 2));
      if constexpr (PPB == 8) a = max(a, (uint32_t)__shfl_xor((int)a, 4));
      const uint32_t code = mx_scale_code<FMT>(a);
      u32x2 c;
      if (code == 255u)
        c = u32x2{0x7F7F7F7Fu, BF16 ? 0x7F7F7F7Fu : 0u};
      else
        c = piece_codes_finite<BF16, FMT>(v[k], __uint_as_float((254u - code) << 23));
      const int64_t off = (r0 + rr[k]) * cols + c0 + cc;
      if constexpr (BF16)
        *reinterpret_cast<u32x2*>(q + off) = c;
      else
        *reinterpret_cast<uint32_t*>(q + off) = c.x;
      if ((tid & (PPB - 1)) == 0) scales[(r0 + rr[k]) * nbr + (c0 + cc) / 32] = (uint8_t)code;
    }
    __syncthreads();
    uint32_t ccode[8];
    float m[8];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int l = tid % PPR;
      const uint32_t a = max(max(red[i & 1][0][l][e], red[i & 1][1][l][e]),
                             max(red[i & 1][2][l][e], red[i & 1][3][l][e]));
      ccode[e] = mx_scale_code<FMT>(a);
      m[e] = __uint_as_float(ccode[e] == 255u ? 0x3F800000u : (254u - ccode[e]) << 23);
    }
    if constexpr (!BF16) {
#pragma unroll
      for (int e = 4; e < 8; ++e) { ccode[e] = 0u; m[e] = 1.0f; }
    }
    uint32_t nan_bytes[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (ccode[e] == 255u) nan_bytes[e >> 2] |= 0xFFu << (8 * (e & 3));
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const u32x2 c = piece_codes_cols<BF16, FMT>(v[k], m, nan_bytes);
      if constexpr (BF16)
        tile_park8(tile, rr[k], cc, c);
      else
        tile_park4(tile, rr[k], cc, c.x);
    }
    if (tid < PPR) {
#pragma unroll
      for (int e = 0; e < PER; ++e)
        scales_t[(c0 + cc + e) * nbc + r0 / 32 + i] = (uint8_t)ccode[e];
    }
  }
  __syncthreads();
  tile_store_qt<4>(tile, qt, rows, r0, c0, tid);
}

template <bool BF16, int FMT>
static hipError_t launch_mx_t(const void* x, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* scales, uint8_t* qt, uint8_t* scales_t,
                              hipStream_t stream) {
  dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
  hipLaunchKernelGGL((mx_cast_transpose_kernel<BF16, FMT>), grid, dim3(256), 0, stream, x, rows,
                     cols, q, scales, qt, scales_t);
  return hipGetLastError();
}

hipError_t launch_mx_cast_transpose(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                                    uint8_t* q, uint8_t* scales, uint8_t* qt, uint8_t* scales_t,
                                    hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (bf16)
    return fmt == kE4M3 ? launch_mx_t<true, kE4M3>(x, rows, cols, q, scales, qt, scales_t, stream)
                        : launch_mx_t<true, kE5M2>(x, rows, cols, q, scales, qt, scales_t, stream);
  return fmt == kE4M3 ? launch_mx_t<false, kE4M3>(x, rows, cols, q, scales, qt, scales_t, stream)
                      : launch_mx_t<false, kE5M2>(x, rows, cols, q, scales, qt, scales_t, stream);
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

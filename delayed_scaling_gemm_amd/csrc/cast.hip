// amax and the fused amax + scaled saturating cast (BF16/FP32 -> FP8).
//
// What is computed ("FP8 混合精度训练工程实践" §四 动态缩放, the quantize step):
//   amax = max |x|           of the unscaled input
//   q    = encode(fl32(x*s)) with s the delayed scale of this step
// Both in one pass over x: the scale is known before the pass (delayed scaling,
// "LLM FP8 微调上线生产实战" §核心原理), so the input is read once.
//
// Design for gfx950: the pass is HBM-bound (2 or 4 bytes read, 1 written per
// element).  Threads move lane-contiguous 16-byte pieces of input, issuing all
// their loads before converting, in a one-shot grid (each workgroup covers a
// fixed contiguous range once).  amax is an integer max over |x| bit patterns
// (exact and order independent), reduced by wave shuffles, then LDS, then at
// most one global atomic per workgroup.  The saturation count is reduced the
// same way with integer adds.

#include "cast_common.h"
#include "launch.h"

namespace fp8ds {


// ------------------------------------------------------------------ prologue
// Resets the reduction outputs and snapshots the scale, so the main kernels only
// ever combine into them.  A kernel (not a memset) so the sequence can be
// captured into a graph.
__global__ void prologue_kernel(int64_t count, const float* __restrict__ scale,
                                float* __restrict__ scale_used, uint32_t* __restrict__ amax_bits,
                                unsigned long long* __restrict__ sat, int nc) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  if (scale_used) scale_used[i] = scale[i];
  if (amax_bits) amax_bits[i] = 0u;
  if (sat)
    for (int k = 0; k < nc; ++k) sat[i * nc + k] = 0ull;
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
  unsigned long long* health;  // [batch][4] NaN, Inf, zero, near-max counts (STATS)
  float* scale_used;  // [batch] or null: the scale snapshot, written by the first
                      // workgroup of each tensor (no prologue kernel)
  int direct;         // one workgroup per tensor: it stores amax and saturation count
                      // itself instead of combining them atomically
};

// Each workgroup of T threads owns the contiguous range of T * kGroups * 16
// elements starting at blockIdx.x * T * kGroups * 16, cut into pieces of 16
// bytes of input: 8 elements of BF16, 4 of FP32.  Thread t takes pieces
// base + t + T j, so every load of a wave covers one contiguous 1 KB run and
// every code store a contiguous run (lanes owning 32 or 64 contiguous bytes each
// measured 6-9% slower in BF16 and ~30% slower in FP32 on a bandwidth probe).
// The pieces j = 2i, 2i+1 (BF16) or 4i .. 4i+3 (FP32) form the 16-element
// groups of cast16_*; a thread issues all its loads before converting and
// streams with non-temporal loads and stores (the input is read once; keeping
// it out of the caches measured faster).  A launch covers the whole tensor once
// (no grid-stride loop), so workgroups retire in address order and new ones
// start at once.  Atomics on one address serialise (about 11 ns each), so
// workgroups skip the amax atomic when the global value already covers theirs
// (see block_commit).  Pieces whose group partners lie past the end, and the last
// fewer-than-one-piece elements, go element by element.
//
// Workgroup shape (threads T, groups per thread G), measured on MI355X over
// BF16 casts to E4M3 (a sweep of 12 shapes): up to 2^28 elements small
// workgroups win, 256 x 2 (8 Ki elements) best: 2^22 elements 8.1 -> 4.5 us,
// 2^24 11.7 -> 11.4 us, 2^26 38 -> 34 us (5.3 -> 5.9 TB/s), 2^27 71 -> 65 us
// (5.6 -> 6.2 TB/s) against the 1024 x 4 (64 Ki) shape the casts used before;
// many workgroups leave only a short tail.  From 2^28 on 256 x 8 (32 Ki) and
// 256 x 2 are equal (5.9-6.2 TB/s) and 256 x 8 is kept.  Tensors of at most
// 64 Ki elements take one 1024 x 4 workgroup (the batched casts of small
// tensors rely on it).  The counting cast (STATS) and the amax alone stay at
// 1024 x 4 at every size: with their extra registers 256 x 8 measured 13% and
// 3% slower there.
constexpr int64_t kCastLargeElems = int64_t(1) << 28;  // from here on: 256 x 8
constexpr int64_t kCastMidElems = int64_t(1) << 16;    // above this: 256 x 2

template <bool BF16, int T, int G>
struct CastGroups {
  static constexpr int kGroups = G;             // 16-element groups per thread
  static constexpr int kThreads = T;            // threads per workgroup
  static constexpr int kPer = BF16 ? 8 : 4;     // elements per 16-byte piece
  static constexpr int kPieces = 16 / kPer;     // pieces per group
};

// One element of the cast (ragged pieces and tails): amax bits, saturation and
// health counts as the group casts take them.
template <bool BF16, int FMT, bool WRITE_Q, bool STATS>
__device__ __forceinline__ void cast1(const void* x, uint8_t* q, int64_t i, float s,
                                      uint32_t& amax, uint32_t& sat, bool want_sat, Health& h) {
  float v;
  uint32_t bits;
  if constexpr (BF16) {
    bits = static_cast<const uint16_t*>(x)[i];
    amax = max(amax, (bits & 0x7FFFu) << 16);
    v = __uint_as_float(bits << 16);
  } else {
    bits = static_cast<const uint32_t*>(x)[i];
    amax = max(amax, bits & 0x7FFFFFFFu);
    v = __uint_as_float(bits);
  }
  if constexpr (WRITE_Q) {
    v *= s;
    const uint32_t code = encode_fp8<FMT>(v);
    q[i] = (uint8_t)code;
    if (want_sat) sat += (uint32_t)(fabsf(v) > FmtTraits<FMT>::kMax);
    if constexpr (STATS) {
      health_code1<FMT>(code, h);
      if constexpr (BF16) health_bf16_pair(bits, h);
      else health_f32(bits, h);
    }
  }
}

template <bool BF16, int FMT, bool WRITE_Q, bool STATS, int TH, int GR>
__global__ __launch_bounds__(TH) void cast_kernel(CastArgs p) {
  using CG = CastGroups<BF16, TH, GR>;
  constexpr int G = CG::kGroups, T = CG::kThreads, PER = CG::kPer, NP = CG::kPieces;
  __shared__ uint32_t red[(STATS ? 6 : 2) * (T / 64)];
  Health h;
  const int b = blockIdx.y;
  const float s = WRITE_Q ? p.scale[b] : 1.0f;
  if (WRITE_Q && p.scale_used && blockIdx.x == 0 && threadIdx.x == 0) p.scale_used[b] = s;
  const bool want_sat = WRITE_Q && p.sat != nullptr;
  const int64_t n = p.n;
  const int64_t npieces = n / PER;
  const int64_t base = (int64_t)blockIdx.x * T * G * NP + threadIdx.x;
  const void* x = static_cast<const char*>(p.x) + b * p.stride_x * (BF16 ? 2 : 4);
  uint8_t* q = WRITE_Q ? p.q + b * p.stride_q : nullptr;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  uint32_t amax = 0, sat = 0;
  u16x2 amax2 = {0, 0};

  u32x4 v[G * NP];
#pragma unroll
  for (int j = 0; j < G * NP; ++j) {
    const int64_t pc = base + (int64_t)T * j;
    if (pc < npieces) v[j] = __builtin_nontemporal_load(&xv[pc]);
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int64_t p0 = base + (int64_t)T * NP * i;  // first piece of the group
    if (p0 + (int64_t)T * (NP - 1) < npieces) {
      uint32_t d[4 * NP];
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const u32x4 w = v[NP * i + k];
        d[4 * k] = w.x; d[4 * k + 1] = w.y; d[4 * k + 2] = w.z; d[4 * k + 3] = w.w;
      }
      if constexpr (WRITE_Q) {
        if constexpr (BF16) {
          const u32x4 c = cast16_bf16<FMT, STATS>(d, s, amax2, sat, want_sat, &h);
          __builtin_nontemporal_store(u32x2{c.x, c.y}, reinterpret_cast<u32x2*>(q) + p0);
          __builtin_nontemporal_store(u32x2{c.z, c.w}, reinterpret_cast<u32x2*>(q) + p0 + T);
        } else {
          const u32x4 c = cast16_f32<FMT, STATS>(d, s, amax, sat, want_sat, &h);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            __builtin_nontemporal_store(c[k], reinterpret_cast<uint32_t*>(q) + p0 + (int64_t)T * k);
        }
      } else if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu));
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = max(amax, d[j] & 0x7FFFFFFFu);
      }
    } else {
      // partners past the end: the pieces that exist, element by element
      for (int k = 0; k < NP; ++k) {
        const int64_t pc = p0 + (int64_t)T * k;
        if (pc >= npieces) break;
        for (int e = 0; e < PER; ++e)
          cast1<BF16, FMT, WRITE_Q, STATS>(x, q, pc * PER + e, s, amax, sat, want_sat, h);
      }
    }
  }
  // the last n % PER elements, taken by the first threads of block 0
  const int64_t t0 = npieces * PER;
  if (blockIdx.x == 0 && threadIdx.x < n - t0)
    cast1<BF16, FMT, WRITE_Q, STATS>(x, q, t0 + threadIdx.x, s, amax, sat, want_sat, h);
  if constexpr (BF16) amax = max(amax, ((uint32_t)max(amax2.x, amax2.y)) << 16);
  block_commit<STATS>(amax, sat, h, p.amax ? p.amax + b : nullptr, want_sat ? p.sat + b : nullptr,
                      STATS ? p.health + 4 * b : nullptr, red, p.direct != 0);
}

// ------------------------------------------------------------------ cast + transposed copy
// A 128 x 128 tile per workgroup of 256 threads.  Full tiles of suitably aligned
// tensors take the vector path: in each of four passes a thread converts one
// 16-element group made of lane-contiguous 16-byte input pieces, stores the codes
// of each piece to q and parks them in an LDS tile; after a barrier
// tile_store_qt writes the tile's columns as rows of q_t.  Other tiles (ragged edges, unaligned shapes) convert
// element by element.

// Row tiles per workgroup (walked in sequence, one amax/saturation commit).
#ifndef FP8DS_TRANSPOSE_TILES
#define FP8DS_TRANSPOSE_TILES 1
#endif
constexpr int kTransposeTiles = FP8DS_TRANSPOSE_TILES;

template <bool BF16, int FMT, bool STATS>
__global__ __launch_bounds__(256) void cast_transpose_kernel(
    const void* __restrict__ xp, int64_t rows, int64_t cols, const float* __restrict__ scale,
    uint8_t* __restrict__ q, uint8_t* __restrict__ qt, uint32_t* __restrict__ g_amax,
    unsigned long long* __restrict__ g_sat, unsigned long long* __restrict__ g_health,
    float* __restrict__ scale_used) {
  constexpr int T = 128;
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * T];
  __shared__ uint32_t red[(STATS ? 6 : 2) * 4];
  Health h;
  const float s = scale[0];
  const int64_t c0 = (int64_t)blockIdx.x * T;
  const int tid = threadIdx.x;
  if (scale_used && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) scale_used[0] = s;
  uint32_t amax = 0, sat = 0;
  for (int ti = 0; ti < kTransposeTiles; ++ti) {
    const int64_t r0 = ((int64_t)blockIdx.y * kTransposeTiles + ti) * T;
    if (r0 >= rows) break;
    if (ti > 0) __syncthreads();  // the previous tile's transposed reads are done
    // vector path: whole tile inside, 16-element pieces aligned for 16-byte
    // accesses in x, q and q_t
    const bool vec = (r0 + T <= rows) && (c0 + T <= cols) && (cols % 16 == 0) && (rows % 16 == 0);
    if (vec) {
      // pieces of 16 input bytes (8 BF16 or 4 FP32 elements); pass i takes pieces
      // u = 256 (NP i + k) + tid of the tile, so a wave's loads cover whole row runs
      constexpr int PER = BF16 ? 8 : 4, NP = 16 / PER, PPR = T / PER;
      // all of the tile's loads are issued before the first conversion (loaded
      // pass by pass, each pass waited for its own loads, and the tile paid the
      // load latency once per pass)
      u32x4 vin[4][NP];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int u = 256 * (NP * i + k) + tid;
          vin[i][k] = *reinterpret_cast<const u32x4*>(
              static_cast<const char*>(xp) +
              ((r0 + u / PPR) * cols + c0 + (u % PPR) * PER) * (BF16 ? 2 : 4));
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int rr[NP], cc[NP];
        int64_t off[NP];
        uint32_t d[4 * NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int u = 256 * (NP * i + k) + tid;
          rr[k] = u / PPR;
          cc[k] = (u % PPR) * PER;
          off[k] = (r0 + rr[k]) * cols + c0 + cc[k];
          const u32x4 w = vin[i][k];
          d[4 * k] = w.x; d[4 * k + 1] = w.y; d[4 * k + 2] = w.z; d[4 * k + 3] = w.w;
        }
        if constexpr (BF16) {
          u16x2 amax2 = {0, 0};
          const u32x4 codes = cast16_bf16<FMT, STATS>(d, s, amax2, sat, g_sat != nullptr, &h);
          amax = max(amax, ((uint32_t)max(amax2.x, amax2.y)) << 16);
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const u32x2 c2 = {codes[2 * k], codes[2 * k + 1]};
            *reinterpret_cast<u32x2*>(q + off[k]) = c2;
            tile_park8(tile, rr[k], cc[k], c2);
          }
        } else {
          const u32x4 codes = cast16_f32<FMT, STATS>(d, s, amax, sat, g_sat != nullptr, &h);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            *reinterpret_cast<uint32_t*>(q + off[k]) = codes[k];
            tile_park4(tile, rr[k], cc[k], codes[k]);
          }
        }
      }
      __syncthreads();
      tile_store_qt<4>(tile, qt, rows, r0, c0, tid);
    } else {
      const int tr = tid >> 1;         // row within the tile
      const int tc = (tid & 1) * 64;   // first of this thread's 64 columns
      const int64_t r = r0 + tr;
#pragma unroll 1  // unrolled, this rarely used path set the kernel's register count (157)
      for (int i = 0; i < 64; ++i) {
        const int64_t c = c0 + tc + i;
        uint32_t code = 0;
        if (r < rows && c < cols) {
          float v;
          if constexpr (BF16) {
            const uint32_t bits = static_cast<const uint16_t*>(xp)[r * cols + c];
            amax = max(amax, (bits & 0x7FFFu) << 16);
            v = __uint_as_float(bits << 16) * s;
            if constexpr (STATS) health_bf16_pair(bits, h);
          } else {
            const uint32_t bits = static_cast<const uint32_t*>(xp)[r * cols + c];
            amax = max(amax, bits & 0x7FFFFFFFu);
            v = __uint_as_float(bits) * s;
            if constexpr (STATS) health_f32(bits, h);
          }
          code = encode_fp8<FMT>(v);
          if (g_sat) sat += (uint32_t)(fabsf(v) > FmtTraits<FMT>::kMax);
          if constexpr (STATS) health_code1<FMT>(code, h);
          q[r * cols + c] = (uint8_t)code;
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
          if (orow < rows) qt[oc * rows + orow] = tile[(orr + i) * T + oc_l];
        }
      }
    }
  }
  block_commit<STATS>(amax, sat, h, g_amax, g_sat, g_health, red);
}

// ------------------------------------------------------------------ host launchers

hipError_t launch_prologue(int64_t count, const float* scale, float* scale_used, float* amax,
                           uint64_t* sat, hipStream_t stream, int counters) {
  if (count <= 0 || (!scale_used && !amax && !sat)) return hipSuccess;
  int blocks = (int)((count + 255) / 256);
  hipLaunchKernelGGL(prologue_kernel, dim3(blocks), dim3(256), 0, stream, count, scale, scale_used,
                     reinterpret_cast<uint32_t*>(amax), reinterpret_cast<unsigned long long*>(sat),
                     counters);
  return hipGetLastError();
}

template <bool BF16, int FMT, bool WRITE_Q, bool STATS, int TH, int GR>
static hipError_t launch_cast_shape(const CastArgs& a, int64_t batch, hipStream_t stream) {
  using CG = CastGroups<BF16, TH, GR>;
  constexpr int64_t per_block = (int64_t)CG::kThreads * CG::kGroups * CG::kPieces;  // pieces
  const int64_t pieces = a.n / CG::kPer;
  int64_t gx = (pieces + per_block - 1) / per_block;
  if (gx < 1) gx = 1;  // block 0 also takes the ragged tail (fewer than one piece)
  if (a.direct && gx != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((cast_kernel<BF16, FMT, WRITE_Q, STATS, TH, GR>),
                     dim3((unsigned)gx, (unsigned)batch), dim3((unsigned)CG::kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <bool BF16, int FMT, bool WRITE_Q, bool STATS>
static hipError_t launch_cast_t(const CastArgs& a, int64_t batch, hipStream_t stream) {
  if constexpr (WRITE_Q && !STATS) {
    if (a.n >= kCastLargeElems)
      return launch_cast_shape<BF16, FMT, WRITE_Q, STATS, 256, 8>(a, batch, stream);
    if (a.n > kCastMidElems)
      return launch_cast_shape<BF16, FMT, WRITE_Q, STATS, 256, 2>(a, batch, stream);
  }
  return launch_cast_shape<BF16, FMT, WRITE_Q, STATS, 1024, 4>(a, batch, stream);
}

template <bool BF16, bool STATS>
static hipError_t launch_cast_f(const CastArgs& a, int fmt, int64_t batch, hipStream_t stream) {
  return fmt == kE4M3 ? launch_cast_t<BF16, kE4M3, true, STATS>(a, batch, stream)
                      : launch_cast_t<BF16, kE5M2, true, STATS>(a, batch, stream);
}

hipError_t launch_cast(const void* x, bool bf16, int64_t batch, int64_t n, int64_t stride_x,
                       int fmt, const float* scale, uint8_t* q, int64_t stride_q, float* amax,
                       uint64_t* sat, uint64_t* health, int num_cus, hipStream_t stream,
                       float* scale_used) {
  (void)num_cus;
  CastArgs a{x, n, stride_x, scale, q, stride_q, reinterpret_cast<uint32_t*>(amax),
             reinterpret_cast<unsigned long long*>(sat),
             reinterpret_cast<unsigned long long*>(health), q ? scale_used : nullptr, 0};
  if (q == nullptr) {
    return bf16 ? launch_cast_t<true, kE4M3, false, false>(a, batch, stream)
                : launch_cast_t<false, kE4M3, false, false>(a, batch, stream);
  }
  if (health)
    return bf16 ? launch_cast_f<true, true>(a, fmt, batch, stream)
                : launch_cast_f<false, true>(a, fmt, batch, stream);
  return bf16 ? launch_cast_f<true, false>(a, fmt, batch, stream)
              : launch_cast_f<false, false>(a, fmt, batch, stream);
}

// Batched casts of tensors that one workgroup of the 1024 x 4 shape covers
// (64 Ki elements, e.g. 256 x 256) need no cross-workgroup reduction: that
// workgroup stores the tensor's amax and saturation count and snapshots its
// scale, and the prologue kernel (with its launch gap) is not needed.  Larger
// tensors take the prologue and the atomic reductions.
constexpr int64_t kOneBlockElems = 1024 * 4 * 16;
static_assert(kOneBlockElems <= kCastMidElems, "such tensors take the 1024 x 4 shape");

hipError_t launch_cast_batched(const void* x, bool bf16, int64_t batch, int64_t n,
                               int64_t stride_x, int fmt, const float* scale, uint8_t* q,
                               int64_t stride_q, float* scale_used, float* amax, uint64_t* sat,
                               hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  if (n > 0 && n <= kOneBlockElems) {
    CastArgs a{x, n, stride_x, scale, q, stride_q, reinterpret_cast<uint32_t*>(amax),
               reinterpret_cast<unsigned long long*>(sat), nullptr, scale_used, 1};
    return bf16 ? launch_cast_f<true, false>(a, fmt, batch, stream)
                : launch_cast_f<false, false>(a, fmt, batch, stream);
  }
  hipError_t e = launch_prologue(batch, scale, scale_used, amax, sat, stream);
  if (e == hipSuccess && n > 0)
    e = launch_cast(x, bf16, batch, n, stride_x, fmt, scale, q, stride_q, amax, sat, nullptr, 0,
                    stream);
  return e;
}

template <bool BF16, int FMT, bool STATS>
static hipError_t launch_transpose_t(dim3 grid, const void* x, int64_t rows, int64_t cols,
                                     const float* scale, uint8_t* q, uint8_t* qt, float* amax,
                                     uint64_t* sat, uint64_t* health, float* scale_used,
                                     hipStream_t stream) {
  hipLaunchKernelGGL((cast_transpose_kernel<BF16, FMT, STATS>), grid, dim3(256), 0, stream, x,
                     rows, cols, scale, q, qt, reinterpret_cast<uint32_t*>(amax),
                     reinterpret_cast<unsigned long long*>(sat),
                     reinterpret_cast<unsigned long long*>(health), scale_used);
  return hipGetLastError();
}

template <bool STATS>
static hipError_t launch_transpose_s(dim3 grid, const void* x, bool bf16, int64_t rows,
                                     int64_t cols, int fmt, const float* scale, uint8_t* q,
                                     uint8_t* qt, float* amax, uint64_t* sat, uint64_t* health,
                                     float* scale_used, hipStream_t stream) {
  if (bf16)
    return fmt == kE4M3
               ? launch_transpose_t<true, kE4M3, STATS>(grid, x, rows, cols, scale, q, qt, amax,
                                                        sat, health, scale_used, stream)
               : launch_transpose_t<true, kE5M2, STATS>(grid, x, rows, cols, scale, q, qt, amax,
                                                        sat, health, scale_used, stream);
  return fmt == kE4M3
             ? launch_transpose_t<false, kE4M3, STATS>(grid, x, rows, cols, scale, q, qt, amax, sat,
                                                       health, scale_used, stream)
             : launch_transpose_t<false, kE5M2, STATS>(grid, x, rows, cols, scale, q, qt, amax, sat,
                                                       health, scale_used, stream);
}

hipError_t launch_cast_transpose(const void* x, bool bf16, int64_t rows, int64_t cols, int fmt,
                                 const float* scale, uint8_t* q, uint8_t* qt, float* amax,
                                 uint64_t* sat, uint64_t* health, hipStream_t stream,
                                 float* scale_used) {
  dim3 grid((unsigned)((cols + 127) / 128),
            (unsigned)(((rows + 127) / 128 + kTransposeTiles - 1) / kTransposeTiles));
  if (health)
    return launch_transpose_s<true>(grid, x, bf16, rows, cols, fmt, scale, q, qt, amax, sat,
                                    health, scale_used, stream);
  return launch_transpose_s<false>(grid, x, bf16, rows, cols, fmt, scale, q, qt, amax, sat,
                                   nullptr, scale_used, stream);
}

}  // namespace fp8ds

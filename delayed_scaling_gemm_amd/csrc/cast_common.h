// Element-level pieces shared by the FP8 cast kernels and the fused optimizer
// step that casts its updated weights: the saturating RNE encoders, the
// saturation and health counts, the 16-element group casts, the workgroup
// commit of amax / counts, and the transposed store of a 128 x 128 code tile.
#pragma once

#include "device_common.h"

namespace fp8ds {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element access

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Four codes in one dword (first value in the low byte) with the software
// encoder: any input, NaN included.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_sw(float a, float b, float c, float d) {
  return encode_fp8<FMT>(a) | (encode_fp8<FMT>(b) << 8) | (encode_fp8<FMT>(c) << 16) |
         (encode_fp8<FMT>(d) << 24);
}

// Four codes with gfx950's packed converts, for inputs that are not NaN.  The
// converts round to nearest even exactly as the definition does for every value
// within the format's range (subnormals and ties included) but turn larger
// magnitudes into NaN (E4M3) or infinity (E5M2); clamping to +-max first gives
// the saturating result, since max is itself a code.  Over all 2^32 fp32 inputs
// that are not NaN this equals the software encoder bit for bit.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_hw(float a, float b, float c, float d) {
  constexpr float MX = FmtTraits<FMT>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -MX, MX);
  b = __builtin_amdgcn_fmed3f(b, -MX, MX);
  c = __builtin_amdgcn_fmed3f(c, -MX, MX);
  d = __builtin_amdgcn_fmed3f(d, -MX, MX);
  int w;
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// ------------------------------------------------------------------ 16-byte pieces
// A piece is 16 bytes of input: 8 BF16 or 4 FP32 elements.

// The largest |x| bit pattern of one 16-byte piece.
template <bool BF16>
__device__ __forceinline__ uint32_t piece_amax(const u32x4& d) {
  if constexpr (BF16) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max((d[k] & 0x7FFFu) << 16, d[k] & 0x7FFF0000u));
    return m;
  } else {
    return max(max(d.x & 0x7FFFFFFFu, d.y & 0x7FFFFFFFu), max(d.z & 0x7FFFFFFFu, d.w & 0x7FFFFFFFu));
  }
}

// Four codes of four scaled values (software encoder if any is NaN).
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  const bool nan = a != a || b != b || c != c || d != d;
  return nan ? encode4_sw<FMT>(a, b, c, d) : encode4_hw<FMT>(a, b, c, d);
}

// Codes of one piece whose scaled values are not NaN (finite inputs and a
// finite scale): the packed converts alone, no NaN test.
template <bool BF16, int FMT>
__device__ __forceinline__ u32x2 piece_codes_finite(const u32x4& d, float s) {
  if constexpr (BF16) {
    return u32x2{encode4_hw<FMT>(bf16_lo(d.x) * s, bf16_hi(d.x) * s, bf16_lo(d.y) * s, bf16_hi(d.y) * s),
                 encode4_hw<FMT>(bf16_lo(d.z) * s, bf16_hi(d.z) * s, bf16_lo(d.w) * s, bf16_hi(d.w) * s)};
  } else {
    return u32x2{encode4_hw<FMT>(__uint_as_float(d.x) * s, __uint_as_float(d.y) * s,
                                 __uint_as_float(d.z) * s, __uint_as_float(d.w) * s), 0u};
  }
}

// Codes of one piece: 8 bytes (BF16, returned in .x/.y) or 4 bytes (FP32, in .x).
template <bool BF16, int FMT>
__device__ __forceinline__ u32x2 piece_codes(const u32x4& d, float s) {
  if constexpr (BF16) {
    return u32x2{encode4<FMT>(bf16_lo(d.x) * s, bf16_hi(d.x) * s, bf16_lo(d.y) * s, bf16_hi(d.y) * s),
                 encode4<FMT>(bf16_lo(d.z) * s, bf16_hi(d.z) * s, bf16_lo(d.w) * s, bf16_hi(d.w) * s)};
  } else {
    return u32x2{encode4<FMT>(__uint_as_float(d.x) * s, __uint_as_float(d.y) * s,
                              __uint_as_float(d.z) * s, __uint_as_float(d.w) * s), 0u};
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t sat4(float a, float b, float c, float d) {
  constexpr float M = FmtTraits<FMT>::kMax;
  return (uint32_t)(fabsf(a) > M) + (uint32_t)(fabsf(b) > M) + (uint32_t)(fabsf(c) > M) +
         (uint32_t)(fabsf(d) > M);
}

// Quantization-health counts of one thread: NaN and infinite inputs, zero
// codes (+-0) and codes in the format's top binade [2^emax, max] (magnitude
// byte 0x78 up to the largest finite code in both formats).
struct Health {
  uint32_t nan = 0, inf = 0, zero = 0, near = 0;
};
// largest finite code magnitude: 0x7E (448) in E4M3, 0x7B (57344) in E5M2
template <int FMT>
constexpr uint32_t max_code() { return FMT == kE4M3 ? 0x7Eu : 0x7Bu; }

// Four codes in a dword: the byte tests are carry-free because every masked
// byte is at most 0x7F.
__device__ __forceinline__ void health_zero4(uint32_t c, Health& h) {
  const uint32_t t = c & 0x7F7F7F7Fu;
  const uint32_t nonzero = ((t + 0x7F7F7F7Fu) | t) & 0x80808080u;  // byte >= 1
  h.zero += 4u - (uint32_t)__builtin_popcount(nonzero);
}
template <int FMT>
__device__ __forceinline__ void health_near4(uint32_t c, Health& h) {
  constexpr uint32_t kMaxCode = max_code<FMT>();
  const uint32_t t = c & 0x7F7F7F7Fu;
  const uint32_t ge = (t + 0x08080808u) & 0x80808080u;                              // >= 0x78
  const uint32_t le = ((0x80808080u + kMaxCode * 0x01010101u) - t) & 0x80808080u;  // <= max
  h.near += (uint32_t)__builtin_popcount(ge & le);
}
// A group can hold a zero code only if its smallest scaled magnitude is below
// the smallest subnormal, and a top-binade code only if its largest reaches the
// binade below (both tests are monotonic in |x|, so groups that fail them are
// skipped exactly); groups with a NaN are always counted.
template <int FMT>
__device__ __forceinline__ void health_group(const u32x4& out, float lo, float hi, bool nan,
                                             Health& h) {
  constexpr float kMinSub = FMT == kE4M3 ? 0x1.0p-9f : 0x1.0p-16f;
  constexpr float kBelowTop = FMT == kE4M3 ? 128.0f : 16384.0f;
  if (nan || lo < kMinSub) {
#pragma unroll
    for (int j = 0; j < 4; ++j) health_zero4(out[j], h);
  }
  if (nan || hi >= kBelowTop) {
#pragma unroll
    for (int j = 0; j < 4; ++j) health_near4<FMT>(out[j], h);
  }
}
template <int FMT>
__device__ __forceinline__ void health_code1(uint32_t code, Health& h) {
  const uint32_t m = code & 0x7Fu;
  h.zero += (uint32_t)(m == 0u);
  h.near += (uint32_t)(m >= 0x78u && m <= max_code<FMT>());
}
__device__ __forceinline__ void health_bf16_pair(uint32_t d, Health& h) {
  const uint32_t lo = d & 0x7FFFu, hi = (d >> 16) & 0x7FFFu;
  h.nan += (uint32_t)(lo > 0x7F80u) + (uint32_t)(hi > 0x7F80u);
  h.inf += (uint32_t)(lo == 0x7F80u) + (uint32_t)(hi == 0x7F80u);
}
__device__ __forceinline__ void health_f32(uint32_t d, Health& h) {
  const uint32_t m = d & 0x7FFFFFFFu;
  h.nan += (uint32_t)(m > 0x7F800000u);
  h.inf += (uint32_t)(m == 0x7F800000u);
}

// Process 16 consecutive elements already loaded as 8 dwords of bf16 pairs or 16
// floats.  Returns the 16 codes; accumulates amax bits and saturations.  The
// group's largest magnitude (needed for amax anyway) tells whether any element
// is NaN; only such groups take the software encoder.
template <int FMT, bool STATS = false>
__device__ __forceinline__ u32x4 cast16_bf16(const uint32_t (&d)[8], float s, u16x2& amax2,
                                              uint32_t& sat, bool want_sat, Health* h = nullptr) {
  u16x2 gm = {0, 0}, gn = {0x7FFF, 0x7FFF};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u16x2 m = __builtin_bit_cast(u16x2, d[j] & 0x7FFF7FFFu);
    gm = __builtin_elementwise_max(gm, m);
    if constexpr (STATS) gn = __builtin_elementwise_min(gn, m);
  }
  amax2 = __builtin_elementwise_max(amax2, gm);
  const bool nan = gm.x > 0x7F80u || gm.y > 0x7F80u;
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d0 = d[2 * j], d1 = d[2 * j + 1];
    const float a = bf16_lo(d0) * s, b = bf16_hi(d0) * s, c = bf16_lo(d1) * s,
                e = bf16_hi(d1) * s;
    out[j] = nan ? encode4_sw<FMT>(a, b, c, e) : encode4_hw<FMT>(a, b, c, e);
    if (want_sat) sat += sat4<FMT>(a, b, c, e);
  }
  if constexpr (STATS) {
    const float lo = fabsf(__uint_as_float((uint32_t)min(gn.x, gn.y) << 16) * s);
    const float hi = fabsf(__uint_as_float((uint32_t)max(gm.x, gm.y) << 16) * s);
    health_group<FMT>(out, lo, hi, nan, *h);
    if (gm.x >= 0x7F80u || gm.y >= 0x7F80u) {  // some NaN or infinity in the group
#pragma unroll
      for (int j = 0; j < 8; ++j) health_bf16_pair(d[j], *h);
    }
  }
  return out;
}

template <int FMT, bool STATS = false>
__device__ __forceinline__ u32x4 cast16_f32(const uint32_t (&d)[16], float s, uint32_t& amax,
                                             uint32_t& sat, bool want_sat, Health* h = nullptr) {
  uint32_t gm = 0, gn = 0x7FFFFFFFu;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    gm = max(gm, d[i] & 0x7FFFFFFFu);
    if constexpr (STATS) gn = min(gn, d[i] & 0x7FFFFFFFu);
  }
  amax = max(amax, gm);
  const bool nan = gm > 0x7F800000u;
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(d[4 * j + i]) * s;
    out[j] = nan ? encode4_sw<FMT>(v[0], v[1], v[2], v[3]) : encode4_hw<FMT>(v[0], v[1], v[2], v[3]);
    if (want_sat) sat += sat4<FMT>(v[0], v[1], v[2], v[3]);
  }
  if constexpr (STATS) {
    health_group<FMT>(out, fabsf(__uint_as_float(gn) * s), fabsf(__uint_as_float(gm) * s), nan, *h);
    if (gm >= 0x7F800000u) {
#pragma unroll
      for (int i = 0; i < 16; ++i) health_f32(d[i], *h);
    }
  }
  return out;
}

// Commits a workgroup's amax bits, saturation count and (STATS) health counts
// (NaN, Inf, zero, near-max into g_health[0..3]): wave reductions, one LDS word
// per wave and quantity, then wave 0 reduces across the waves in parallel (lane
// w takes wave w's words) and issues at most one atomic per quantity.  The amax
// atomic is skipped when the global value already covers the workgroup's: it
// only grows, and a stale read only costs an extra atomic.  `direct`: the
// workgroup is the only one of its tensor, and stores the results instead (the
// outputs need no zeroing beforehand).
template <bool STATS>
__device__ __forceinline__ void block_commit(uint32_t amax_bits, uint32_t sat, const Health& h,
                                             uint32_t* g_amax, unsigned long long* g_sat,
                                             unsigned long long* g_health, uint32_t* smem,
                                             bool direct = false) {
  constexpr int NQ = STATS ? 6 : 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t v[NQ];
  v[0] = g_amax ? wave_max_u32(amax_bits) : 0u;
  v[1] = (g_sat && __any(sat != 0)) ? wave_sum_u32(sat) : 0u;  // most waves saturate nothing
  if constexpr (STATS) {
    const uint32_t c[4] = {h.nan, h.inf, h.zero, h.near};
#pragma unroll
    for (int k = 0; k < 4; ++k) v[2 + k] = __any(c[k] != 0) ? wave_sum_u32(c[k]) : 0u;
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < NQ; ++k) smem[k * nw + wave] = v[k];
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t t[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) t[k] = lane < nw ? smem[k * nw + lane] : 0u;
    t[0] = wave_max_u32(t[0]);
#pragma unroll
    for (int k = 1; k < NQ; ++k) t[k] = wave_sum_u32(t[k]);
    if (lane == 0 && direct) {
      if (g_amax) *g_amax = canonical_amax_bits(t[0]);
      if (g_sat) *g_sat = (unsigned long long)t[1];
      if constexpr (STATS) {
#pragma unroll
        for (int k = 0; k < 4; ++k) g_health[k] = (unsigned long long)t[2 + k];
      }
    } else if (lane == 0) {
      if (g_amax) {
        const uint32_t mb = canonical_amax_bits(t[0]);
        if (mb > __hip_atomic_load(g_amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
          atomicMax(g_amax, mb);
      }
      if (g_sat && t[1]) atomicAdd(g_sat, (unsigned long long)t[1]);
      if constexpr (STATS) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (t[2 + k]) atomicAdd(g_health + k, (unsigned long long)t[2 + k]);
      }
    }
  }
}

// gfx950 transposing LDS read of 8 bytes (ds_read_b64_tr_b8).
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  const v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i_t*)(p));
  return u32x2{(uint32_t)v[0], (uint32_t)v[1]};
}

// Transposed store of a 128 x 128 tile of codes parked in LDS (128-byte rows,
// 8-byte column groups XOR-swizzled by row % 8) into q_t [cols x rows].
// gfx950's transposing LDS read (ds_read_b64_tr_b8: within 16 lanes, lane i
// receives byte i % 8 of the 8-byte pieces addressed by lanes 2j + i / 8,
// j = 0..7) hands each lane 8 rows of one input column; two such reads give 16
// rows, one 16-byte piece of q_t.  The tile has 8 x 8 units of 16 columns x 16
// rows; a wave takes four units per step (its four 16-lane groups take
// consecutive 16-row blocks of the same 16 columns, so each store instruction
// writes 64-byte runs of 16 q_t rows), and the NW waves of the workgroup share
// the 16 steps.  The swizzle puts the 16 pieces of a group's read in distinct
// banks.  Requires the whole tile inside the tensor and rows % 16 == 0.
template <int NW>
__device__ __forceinline__ void tile_store_qt(const uint8_t* tile, uint8_t* __restrict__ qt,
                                              int64_t rows, int64_t r0, int64_t c0, int tid) {
  static_assert(16 % NW == 0, "16 wave steps shared by NW waves");
  constexpr int T = 128;
  const int lane = tid & 63, wv = tid >> 6;
  const int grp = lane >> 4, li = lane & 15;
  const int j = li >> 1, hh = li & 1;  // as addresser: row + j, column group + hh
#pragma unroll
  for (int it = 0; it < 16 / NW; ++it) {
    const int k = wv * (16 / NW) + it;
    const int cg = k >> 1;               // 16-column group of the tile
    const int rb = 4 * (k & 1) + grp;    // 16-row block
    u32x2 part[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int r = rb * 16 + 8 * half + j;
      const int c8 = 2 * cg + hh;
      part[half] = lds_read_tr8(tile + r * T + ((c8 ^ (r & 7)) << 3));
    }
    // lane li holds column 16 cg + li, rows 16 rb .. 16 rb + 15
    const int64_t oc = c0 + cg * 16 + li;
    *reinterpret_cast<u32x4*>(qt + oc * rows + r0 + rb * 16) =
        u32x4{part[0][0], part[0][1], part[1][0], part[1][1]};
  }
}

// Parks the 8 codes of row r, columns c .. c + 7 (c % 8 == 0): one 8-byte group.
__device__ __forceinline__ void tile_park8(uint8_t* tile, int r, int c, const u32x2& codes) {
  constexpr int T = 128;
  *reinterpret_cast<u32x2*>(tile + r * T + (((c >> 3) ^ (r & 7)) << 3)) = codes;
}

// Parks the 4 codes of row r, columns c .. c + 3 (c % 4 == 0) in the same layout.
__device__ __forceinline__ void tile_park4(uint8_t* tile, int r, int c, uint32_t codes) {
  constexpr int T = 128;
  *reinterpret_cast<uint32_t*>(tile + r * T + ((((c >> 3) ^ (r & 7))) << 3) + (c & 4)) = codes;
}

}  // namespace fp8ds

// FP8 x FP8 GEMM with FP32 accumulation and the dequant epilogue, for gfx950.
//
// What is computed ("FP8 混合精度训练工程实践" §五: the fp8 linear op multiplies the
// two quantised operands and divides by the product of their scales; the
// per-tensor FP8 GEMM row there: FP8 in, FP32 accumulate, BF16 out; §三: the
// three products of a step, Y = X W (NN), dX = dY W^T (NT), dW = X^T dY (TN)):
//
//   acc[m][n] = sum_k a(m,k) b(k,n)                 (FP32 accumulation)
//   C[m][n]   = out( acc[m][n] * fl32(1 / fl32(s_a s_b)) ),  amax_C = max |C|
//
// Two datapaths:
//
//  * EXACT (default).  gfx950's FP8 matrix instructions add the products of each
//    group of 8 at a fixed point aligned to the group's largest product, about 13
//    bits wide: a product 2^14 or more below the largest of its group is dropped
//    entirely.  With heavy-tailed E5M2 gradients that loses far more than the
//    FP32 accumulation the method states.  The EXACT path keeps FP8 bytes in LDS
//    (one byte per element in HBM and LDS); each wave reads its fragments and
//    widens them exactly to F16 in registers (every E4M3 and E5M2 value is an F16
//    value), one step ahead of the MFMAs that use them, and runs
//    V_MFMA_F32_32X32X16_F16: exact products, FP32 sums.
//  * FP8.  V_MFMA_F32_32X32X64_F8F6F4 on FP8 tiles in LDS (format of each operand
//    as an immediate), twice the F16 rate, with the hardware's summation
//    precision described above.
//
// Common structure: block tile BM x BN, four waves in a 2 x 2 grid, each wave
// owning a (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA blocks in accumulator
// registers.  K-major LDS rows are 128 bytes (128 FP8 values of K) split in
// eight 16-byte chunks XOR-swizzled by ((r ^ (r >> 4)) & 7), so that fragment
// reads (consecutive rows, same chunk) and the loaders' stores are free of bank
// conflicts.  Two LDS stages: the loads of the next stage are in flight while a
// stage's MFMAs run (direct loads two stages ahead; register-staged loads are
// written to the other buffer half way through), and the only barrier of a stage
// sits before its last MFMA group, after which the next stage's first fragments
// are read while those MFMAs run.
// K-contiguous sources (A in NN/NT, B in NT) are copied 16 bytes per lane;
// MN-contiguous sources (B in NN, A and B in TN) are either loaded straight into
// LDS in their own orientation and read with gfx950's transposing LDS read, or
// (ragged or unaligned shapes) read 16 bytes along M/N for consecutive k and
// byte-transposed in registers on the way into LDS, so no layout needs an extra
// HBM pass.
//
// The MFMA is issued with the B block as its first operand, so each lane ends
// with runs of 4 consecutive output columns of one row: 8-byte BF16 stores.
// Workgroups are remapped so that each XCD (workgroup id mod 8) gets a contiguous
// range of tiles, walked in groups of 8 tile-rows, to keep shared operand panels
// in that XCD's L2.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8ds {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRowBytes = 128;  // bytes per LDS tile row (both datapaths)

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* A;
  int64_t lda;
  const float* scale_a;
  const uint8_t* B;
  int64_t ldb;
  const float* scale_b;
  void* C;
  int64_t ldc;
  uint32_t* amax_c;
  int64_t stride_a, stride_b, stride_c;
  int tiles_m, tiles_n;
  int out_f32;
  const float* inv_a;  // VS: inverse scale per row of op(A) [M]
  const float* inv_b;  // VS: inverse scale per column of op(B) [N]
  const uint8_t* sc_a;  // MX: E8M0 scale of each 32-element block of a row of A [M][ldsa]
  const uint8_t* sc_b;  // MX: the same for B [N][ldsb]
  int64_t ldsa, ldsb;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 4)) & 7; }

// Byte offset in an LDS operand tile of (row r, 16-byte chunk c).
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowBytes + ((c ^ swz(r)) << 4);
}

// 4x4 byte transpose: out[b] holds byte b of in0..in3 (in0 in the low byte).
__device__ __forceinline__ void transpose4x4(uint32_t i0, uint32_t i1, uint32_t i2, uint32_t i3,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2,
                                             uint32_t& o3) {
  // __builtin_amdgcn_perm(hi, lo, sel): byte i of the result is byte sel.byte_i of
  // the 8-byte value hi:lo (selector 0..3 = lo bytes, 4..7 = hi bytes).
  uint32_t t0 = __builtin_amdgcn_perm(i1, i0, 0x05010400u);  // i0.b0 i1.b0 i0.b1 i1.b1
  uint32_t t1 = __builtin_amdgcn_perm(i1, i0, 0x07030602u);  // i0.b2 i1.b2 i0.b3 i1.b3
  uint32_t t2 = __builtin_amdgcn_perm(i3, i2, 0x05010400u);  // i2.b0 i3.b0 i2.b1 i3.b1
  uint32_t t3 = __builtin_amdgcn_perm(i3, i2, 0x07030602u);  // i2.b2 i3.b2 i2.b3 i3.b3
  o0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);           // i0.b0 i1.b0 i2.b0 i3.b0
  o1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);           // i0.b1 i1.b1 i2.b1 i3.b1
  o2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);           // i0.b2 ...
  o3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);           // i0.b3 ...
}

// ------------------------------------------------------------------ FP8 -> F16 widening
// Exact: every finite E4M3 value is a normal F16 value and every E5M2 value is
// an F16 value (E5M2 is the upper byte of F16).  NaN stays NaN.
//
// E4M3: V_CVT_SCALEF32_PK_F16_FP8 at scale 1.0 converts two bytes (the low or the
// high 16 bits of a dword) to two F16.  Its result is only ever used as a whole
// dword: the compiler builtin was seen to fold the second half into the first
// when the halves are extracted one by one.
// E5M2: a byte permute makes each byte the high byte of its 16-bit half.
template <int FMT>
__device__ __forceinline__ uint32_t widen_pair(uint32_t d, bool hi) {
  if constexpr (FMT == kE4M3) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true))
              : __builtin_bit_cast(uint32_t,
                                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false));
  } else {
    // selector bytes: 0x0C = constant 0x00; 0x00..0x03 = bytes of d
    return __builtin_amdgcn_perm(0u, d, hi ? 0x030C020Cu : 0x010C000Cu);
  }
}

// MX: two FP8 bytes -> two BF16 values times the block's power-of-two scale s
// (V_CVT_SCALEF32_PK_BF16_FP8 / _BF8).  BF16 has the exponent range of fp32 and
// 8 significant bits, so decode(byte) * s is exact while it stays a normal BF16
// number; a NaN byte stays NaN.
template <int FMT>
__device__ __forceinline__ uint32_t widen_pair_mx(uint32_t d, bool hi, float s) {
  if constexpr (FMT == kE4M3) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, s, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, s, false));
  } else {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d, s, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d, s, false));
  }
}

// The value 2^(code - 127) of an E8M0 scale code (2^128 = inf for the NaN code
// 255, whose blocks hold NaN bytes only).
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  return __builtin_amdgcn_ldexpf(1.0f, (int)code - 127);
}

// ------------------------------------------------------------------ global -> LDS loaders
//
// KC: K-contiguous source, rows [row0, row0 + ROWS) of a [rows x K] byte matrix
// (leading dimension ld); one stage covers KB bytes of K starting at k0.  Each
// lane moves 16-byte chunks; bytes past K read as zero.
template <int ROWS, int NT, int KB>
struct LoaderKC {
  static constexpr int kPerRow = KB / 16;  // source chunks per row per stage
  static constexpr int kChunks = ROWS * kPerRow / NT;
  static_assert(kChunks * NT == ROWS * kPerRow, "tile and thread count must divide");
  u32x4 v[kChunks];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ src, int64_t ld, int64_t row0,
                                       int64_t rows, int64_t k0, int64_t K, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int q = tid + NT * i;
      const int r = q / kPerRow, c = q % kPerRow;
      const int64_t gr = row0 + r;
      const int64_t gk = k0 + c * 16;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (gr < rows && gk < K) {
        val = *reinterpret_cast<const u32x4*>(src + gr * ld + gk);
        const int64_t valid = K - gk;
        if (valid < 16) {  // ragged K: zero the bytes past K
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int64_t vb = valid - 4 * w;
            const uint32_t keep = vb >= 4 ? 0xFFFFFFFFu : (vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u));
            val[w] &= keep;
          }
        }
      }
      v[i] = val;
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int q = tid + NT * i;
      const int r = q / kPerRow, c = q % kPerRow;
      *reinterpret_cast<u32x4*>(lds + lds_off(r, c)) = v[i];
    }
  }
};

// MN: MN-contiguous source, element (k, r) at src[(k0 + k) * ld + row0 + r].  A
// unit is KU = 8 consecutive k x 16 rows: 8 loads of 16 bytes along the rows,
// byte-transposed into 16 rows of 8 K-bytes; unit (mc, kg) fills bytes
// [8 kg, 8 kg + 8) of its 16 LDS rows.  A stage (KB = 128) holds ROWS/16 x 16 units.
template <int ROWS, int NT, int KB>
struct LoaderMN {
  static constexpr int KU = 8;
  static constexpr int kGroups = KB / KU;  // k groups per stage
  static constexpr int kUnitsTotal = (ROWS / 16) * kGroups;
  static constexpr int kUnits = (kUnitsTotal + NT - 1) / NT;
  static_assert(kGroups == 16, "unit numbering assumes 16 k groups per stage");
  static_assert(kUnitsTotal % NT == 0 || NT % kUnitsTotal == 0, "units and threads must nest");
  u32x4 v[kUnits][KU];

  // unit u -> 16-row chunk mc and k group kg; 8 consecutive lanes read 128
  // contiguous bytes of one k row.
  __device__ __forceinline__ static void unit_coords(int u, int& mc, int& kg) {
    mc = (u & 7) + ((u >> 7) << 3);
    kg = (u >> 3) & 15;
  }

  __device__ __forceinline__ void load(const uint8_t* __restrict__ src, int64_t ld, int64_t row0,
                                       int64_t rows, int64_t k0, int64_t K, int tid) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      if (tid + NT * i >= kUnitsTotal) break;
      int mc, kg;
      unit_coords(tid + NT * i, mc, kg);
      const int64_t gr = row0 + mc * 16;
#pragma unroll
      for (int kk = 0; kk < KU; ++kk) {
        const int64_t gk = k0 + kg * KU + kk;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (gk < K && gr < rows) {
          const int64_t valid = rows - gr;
          if (valid >= 16) {
            val = *reinterpret_cast<const u32x4*>(src + gk * ld + gr);
          } else {  // ragged M/N edge: byte loads of the valid part
            const uint8_t* p = src + gk * ld + gr;
#pragma unroll
            for (int b = 0; b < 16; ++b) {
              const uint32_t byte = b < valid ? (uint32_t)p[b] : 0u;
              val[b >> 2] |= byte << (8 * (b & 3));
            }
          }
        }
        v[i][kk] = val;
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      if (tid + NT * i >= kUnitsTotal) break;
      int mc, kg;
      unit_coords(tid + NT * i, mc, kg);
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // dword column j: rows 4j .. 4j+3 of the unit
        uint32_t lo[4], hi[4];
        transpose4x4(v[i][0][j], v[i][1][j], v[i][2][j], v[i][3][j], lo[0], lo[1], lo[2], lo[3]);
        transpose4x4(v[i][4][j], v[i][5][j], v[i][6][j], v[i][7][j], hi[0], hi[1], hi[2], hi[3]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = mc * 16 + 4 * j + b;
          *reinterpret_cast<u32x2*>(lds + lds_off(r, kg >> 1) + (kg & 1) * 8) = u32x2{lo[b], hi[b]};
        }
      }
    }
  }
};

template <bool KC, int ROWS, int NT, int KB>
struct LoaderSel;
template <int ROWS, int NT, int KB>
struct LoaderSel<true, ROWS, NT, KB> {
  using type = LoaderKC<ROWS, NT, KB>;
};
template <int ROWS, int NT, int KB>
struct LoaderSel<false, ROWS, NT, KB> {
  using type = LoaderMN<ROWS, NT, KB>;
};

// KC source loaded straight into LDS (gfx950 global_load_lds_dwordx4: each
// lane's 16 bytes land at LDS base + 16 * lane, no registers involved; issued
// as buffer loads, see LoaderKCDirect).  A wave instruction fills one 1 KiB
// segment = 8 LDS rows of 128 bytes; lane l takes physical chunk l % 8 of row
// l / 8 and therefore loads the logical chunk (l % 8) ^ swz(row), which keeps
// the swizzled layout of lds_off.  Requires the stage to lie inside K (K a
// multiple of 128).
// Wait until every vector-memory operation of this wave has completed.  Direct
// LDS loads write no registers, so the compiler does not wait for them on its
// own, and a workgroup barrier's fence only waits for LDS operations.
// (s_waitcnt immediate: vmcnt = 0, expcnt and lgkmcnt unconstrained.)
__device__ __forceinline__ void vmem_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until at most N vector memory instructions of this wave are outstanding
// (they complete in issue order): vmcnt in bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void vmem_wait_n() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Buffer resource of the bytes [base, base + nbytes): a load at an offset past
// nbytes returns zeros (dword 3 = 0x00020000: 32-bit data format, the gfx9
// setting for raw byte-addressed buffers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const uint8_t* base, int64_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)nbytes, 0x00020000);
}

// The loads go through a buffer resource whose base is the tile's first row, so
// a load's address is a per-lane offset (row within the 8-row segment and
// swizzled chunk, fixed for the kernel) plus a scalar offset (segment row and
// stage K): no per-load address arithmetic beyond one XOR and one add, and rows
// past the matrix read as zeros (they only feed outputs that are never stored).
// Requires every offset of the operand below 2^31 (checked by the caller).
template <int ROWS, int NT>
struct LoaderKCDirect {
  static constexpr int kSegs = ROWS / 8;
  static constexpr int kWaves = NT / 64;
  static constexpr int kPerWave = kSegs / kWaves;
  static_assert(kPerWave * kWaves == kSegs, "segments must divide among the waves");
  __amdgpu_buffer_rsrc_t rsrc;
  int ld;
  int w;         // wave index (scalar)
  int lane_row;  // (lane / 8) * ld
  int colx;      // ((lane % 8) ^ (lane / 8)) * 16

  // rows [row0, rows) of a [rows x K] byte matrix with leading dimension ld
  __device__ __forceinline__ LoaderKCDirect(const uint8_t* src, int64_t ld_, int64_t row0,
                                            int64_t rows, int64_t K, int tid) {
    ld = (int)ld_;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, rr = lane >> 3, pc = lane & 7;
    lane_row = rr * ld;
    colx = (pc ^ rr) << 4;
    rsrc = byte_rsrc(src + row0 * ld_, (rows - row0 - 1) * ld_ + K);
  }

  // issues this wave's load instructions i in [lo, hi) of the stage at k0.
  // Instruction i fills LDS segment seg = w kPerWave + i (rows 8 seg .. +8);
  // lane l takes physical chunk l % 8 of row r = 8 seg + l / 8, i.e. the
  // logical chunk (l % 8) ^ swz(r) = (l % 8) ^ (l / 8) ^ ((seg / 2) % 8).
  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds, int lo = 0,
                                        int hi = kPerWave) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      if (i < lo || i >= hi) continue;
      const int seg = w * kPerWave + i;
      const int voff = lane_row + (colx ^ (((seg >> 1) & 7) << 4));
      const int soff = seg * 8 * ld + (int)k0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (void __attribute__((address_space(3)))*)(lds + seg * 1024), 16, voff, soff, 0, 0);
    }
  }
};

// MN source (element (k, r) at src[k * ld + r]) loaded straight into LDS in its
// own orientation: LDS row k holds the tile's ROWS bytes of that k, split into
// 16-byte chunks XOR-swizzled by (k % 8) (times 2 for 256-byte rows, so that the
// 16 pieces of a 32-lane transposing read, two chunks over eight k rows, fall in
// 16 distinct chunk columns).  A wave instruction fills 1 KiB = 1024 / ROWS
// rows; lane l takes physical chunk l % (ROWS / 16) of its row and loads the
// logical chunk that lands there.  Requires whole 16-byte chunks (rows a
// multiple of 16) and the stage inside K.  Chunks past the matrix's last
// column read the next k row, or zeros past the end of the matrix; either
// feeds only outputs that are never stored.
template <int ROWS>
__device__ __forceinline__ int mn_swz(int k) {
  return ROWS >= 256 ? (k & 7) << 1 : (k & 7);
}
template <int ROWS>
__device__ __forceinline__ int mn_off(int k, int r) {
  return k * ROWS + (((r >> 4) ^ mn_swz<ROWS>(k)) << 4) + (r & 15);
}

template <int ROWS, int NT>
struct LoaderMNDirect {
  static constexpr int kCpr = ROWS / 16;      // chunks per LDS row
  static constexpr int kRps = 64 / kCpr;      // LDS rows per wave instruction
  static constexpr int kSegs = 128 / kRps;    // wave instructions per stage (128 k rows)
  static constexpr int kWaves = NT / 64;
  static constexpr int kPerWave = kSegs / kWaves;
  static_assert((ROWS == 128 || ROWS == 256) && kPerWave * kWaves == kSegs,
                "tile shape not supported");
  __amdgpu_buffer_rsrc_t rsrc;
  int ld;
  int w;         // wave index (scalar)
  int lane_row;  // (lane / kCpr) * ld
  int colx;      // swizzled chunk offset of even segments
  int seg_flip;  // XOR of the chunk offset for odd segments (256-row tiles)

  // columns [row0, rows) of a [K x rows] byte matrix with leading dimension ld
  __device__ __forceinline__ LoaderMNDirect(const uint8_t* src, int64_t ld_, int64_t row0,
                                            int64_t rows, int64_t K, int tid) {
    ld = (int)ld_;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, rr = lane / kCpr, pc = lane % kCpr;
    // k = kRps seg + rr: for 128-row tiles k % 8 = rr, for 256-row tiles
    // k % 8 = 4 (seg % 2) + rr, so the swizzled chunk is fixed per lane up to a
    // flip of bit 3 on odd segments
    const int c = ROWS >= 256 ? pc ^ (rr << 1) : pc ^ rr;
    lane_row = rr * ld;
    colx = c << 4;
    seg_flip = ROWS >= 256 ? (8 << 4) : 0;
    rsrc = byte_rsrc(src + row0, (K - 1) * ld_ + (rows - row0));
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds, int lo = 0,
                                        int hi = kPerWave) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      if (i < lo || i >= hi) continue;
      const int seg = w * kPerWave + i;
      const int voff = lane_row + (colx ^ ((seg & 1) ? seg_flip : 0));
      const int soff = ((int)k0 + seg * kRps) * ld;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (void __attribute__((address_space(3)))*)(lds + seg * 1024), 16, voff, soff, 0, 0);
    }
  }
};

template <bool KC, int ROWS, int NT>
struct DirectSel;
template <int ROWS, int NT>
struct DirectSel<true, ROWS, NT> {
  using type = LoaderKCDirect<ROWS, NT>;
};
template <int ROWS, int NT>
struct DirectSel<false, ROWS, NT> {
  using type = LoaderMNDirect<ROWS, NT>;
};

// Direct-load instructions one wave issues for one operand's stage.
template <bool KC, int ROWS, int NT>
constexpr int direct_issues() {
  if constexpr (KC) return LoaderKCDirect<ROWS, NT>::kPerWave;
  else return LoaderMNDirect<ROWS, NT>::kPerWave;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b8).  Within each group of 16
// lanes, lane i receives byte (i % 8) of the 8-byte pieces addressed by lanes
// 2j + i / 8 (j = 0..7), in order.  With even lanes addressing rows
// [r0, r0 + 8) and odd lanes rows [r0 + 8, r0 + 16) of the k rows kb + j, lane i
// obtains row r0 + i % 8 + 8 (i / 8) at k = kb .. kb + 7: a K-contiguous MFMA
// operand read from an MN-major tile.
__device__ __forceinline__ u32x2 ds_read_tr8(const uint8_t* p) {
  typedef int v2i_t __attribute__((ext_vector_type(2)));
  const v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i_t*)(p));
  return u32x2{(uint32_t)v[0], (uint32_t)v[1]};
}

// ------------------------------------------------------------------ tile order

__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  int logical = wg;
  if (T >= 8) {
    // XCD x = wg % 8 takes the contiguous logical range [start_x, start_x + cnt_x).
    const int q = T >> 3, rem = T & 7;
    const int x = wg & 7, idx = wg >> 3;
    logical = x * q + min(x, rem) + idx;
  }
  constexpr int GM = 8;  // tile-rows per group
  const int per_group = GM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// ------------------------------------------------------------------ epilogue

// Two FP32 values to packed BF16, round to nearest even (gfx950 v_cvt_pk_bf16_f32;
// equal to the rounding of the definition for every non-NaN input, subnormals
// included; a NaN stays a quiet NaN of its sign).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ u16x2_t abs_bf16x2(uint32_t v) {
  return __builtin_bit_cast(u16x2_t, v & 0x7FFF7FFFu);
}

// Dequant, convert, store and reduce the output amax.  Lane l holds, for each
// 32 x 32 block (i, j), row (l % 32) and the columns 8g + 4 (l / 32) + {0..3}
// for g = 0..3 (accumulator elements 4g .. 4g+3).  Tiles inside the matrix take
// a branch-free path (row pointers per block row, immediate column offsets);
// edge tiles check every row and group of four columns.
// VS (scale vectors): y = fl32(fl32(acc * inv_a[row]) * inv_b[col]) instead of
// fl32(acc * d); a lane loads its rows' factors once and four columns' factors
// with one 16-byte load per group.
template <bool VS>
__device__ __forceinline__ float dq(float a, float r, float c) {
  if constexpr (VS) return (a * r) * c;
  else return a * r;
}
// `stage0`, `stage1`: the two halves of the operand tiles' LDS (at least NW/2 WTM
// WTN 2 bytes each), free once every wave has passed the epilogue's first
// barrier; the first NW/2 waves stage their blocks in `stage0`, the others in
// `stage1`.  `red` holds NW words.  AMAX_STORE: the workgroup is the only one of
// its output, and stores the output amax instead of combining it atomically.
template <int BM, int BN, int FM, int FN, int WTM, int WTN, bool VS = false, int NW = 4,
          bool AMAX_STORE = false>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const v16f (&acc)[FM][FN], int64_t m0,
                                         int64_t n0, int wm, int wn, int tid, int64_t bz, float d,
                                         uint32_t* red, uint8_t* stage0, uint8_t* stage1) {
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t M = p.M, N = p.N;
  const int64_t mb = m0 + wm * WTM + (lane & 31);
  const int64_t nb = n0 + wn * WTN + (lane >> 5) * 4;
  const bool full = m0 + BM <= M && n0 + BN <= N;
  uint32_t amax = 0;
  if (!p.out_f32) {
    uint16_t* C = static_cast<uint16_t*>(p.C) + bz * p.stride_c;
    if (full) {
      // The wave's WTM x WTN block goes through LDS and leaves in whole row runs
      // (CH lanes per row, 16 bytes each).  Stored straight from the accumulator
      // layout, one instruction wrote 16 bytes into each of 32 rows; those stores
      // cost ~12 us per round of 256 tiles of 256 x 256, about twice the time the
      // output's HBM writes take.  Chunk c of staged row r sits at c ^ (r % CH).
      // The stores are non-temporal: this kernel never reads its output back, and
      // left in the caches as dirty lines it evicted the next kernels' operands
      // and was written back under them (the 4096-hidden training step measured
      // 1127 -> 1079 us, the weight-gradient GEMM after the dX one 382 -> 361 us).
      constexpr int RB = WTN * 2;   // bytes per staged row
      constexpr int CH = RB / 16;   // 16-byte chunks per row
      constexpr int RPI = 64 / CH;  // rows per read-back instruction
      static_assert((NW / 2) * WTM * RB <= BM * 2 * kRowBytes &&
                        (NW / 2) * WTM * RB <= BN * 2 * kRowBytes,
                    "half of the waves' blocks fit in each half of the operand tiles' LDS");
      uint8_t* st = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * WTM * RB;
      __syncthreads();  // every wave has finished reading the operand tiles
      u16x2_t am2 = {0, 0};
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float r = VS ? p.inv_a[mb + i * 32] : d;
        const int sr = i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4_t c = {1.f, 1.f, 1.f, 1.f};
            if constexpr (VS) c = *reinterpret_cast<const f32x4_t*>(p.inv_b + nb + j * 32 + 8 * g);
            const uint32_t lo = pack_bf16x2(dq<VS>(acc[i][j][4 * g], r, c[0]),
                                            dq<VS>(acc[i][j][4 * g + 1], r, c[1]));
            const uint32_t hi = pack_bf16x2(dq<VS>(acc[i][j][4 * g + 2], r, c[2]),
                                            dq<VS>(acc[i][j][4 * g + 3], r, c[3]));
            const int ch = 4 * j + g;  // columns 32 j + 8 g + [0, 8) of the block
            *reinterpret_cast<u32x2*>(st + sr * RB + ((ch ^ (sr % CH)) * 16) + 8 * (lane >> 5)) =
                u32x2{lo, hi};
            am2 = __builtin_elementwise_max(am2, __builtin_elementwise_max(abs_bf16x2(lo), abs_bf16x2(hi)));
          }
      }
      amax = (uint32_t)max(am2[0], am2[1]) << 16;
      __syncthreads();  // the block is staged
      const int ch = lane % CH;
      uint16_t* out = C + (m0 + wm * WTM) * p.ldc + n0 + wn * WTN + ch * 8;
#pragma unroll
      for (int it = 0; it < WTM / RPI; ++it) {
        const int sr = it * RPI + lane / CH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + sr * RB + ((ch ^ (sr % CH)) * 16));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + sr * p.ldc));
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = mb + i * 32;
        if (m >= M) continue;
        uint16_t* row = C + m * p.ldc;
        const float r = VS ? p.inv_a[m] : d;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int64_t n = nb + j * 32 + 8 * g;
            if (n >= N) continue;
            const int64_t left = N - n;  // >= 1
            f32x4_t c = {1.f, 1.f, 1.f, 1.f};
            if constexpr (VS) {
#pragma unroll
              for (int v = 0; v < 4; ++v) c[v] = v < left ? p.inv_b[n + v] : 0.f;
            }
            const uint32_t lo = pack_bf16x2(dq<VS>(acc[i][j][4 * g], r, c[0]),
                                            dq<VS>(acc[i][j][4 * g + 1], r, c[1]));
            const uint32_t hi = pack_bf16x2(dq<VS>(acc[i][j][4 * g + 2], r, c[2]),
                                            dq<VS>(acc[i][j][4 * g + 3], r, c[3]));
            const uint32_t mlo = left >= 2 ? 0x7FFF7FFFu : 0x7FFFu;
            const uint32_t mhi = left >= 4 ? 0x7FFF7FFFu : left == 3 ? 0x7FFFu : 0u;
            const u16x2_t m2 = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, lo & mlo),
                                                         __builtin_bit_cast(u16x2_t, hi & mhi));
            amax = max(amax, (uint32_t)max(m2[0], m2[1]) << 16);
            if (left >= 4) {
              *reinterpret_cast<u32x2*>(row + n) = u32x2{lo, hi};
            } else {
              row[n] = (uint16_t)lo;
              if (left >= 2) row[n + 1] = (uint16_t)(lo >> 16);
              if (left >= 3) row[n + 2] = (uint16_t)hi;
            }
          }
      }
    }
  } else {
    float* C = static_cast<float*>(p.C) + bz * p.stride_c;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = mb + i * 32;
      if (!full && m >= M) continue;
      float* row = C + m * p.ldc;
      const float r = VS ? p.inv_a[m] : d;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = nb + j * 32 + 8 * g;
          if (!full && n >= N) continue;
          float y[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float c = 1.f;
            if constexpr (VS) c = (full || n + v < N) ? p.inv_b[n + v] : 0.f;
            y[v] = dq<VS>(acc[i][j][4 * g + v], r, c);
            if (full || n + v < N) amax = max(amax, __float_as_uint(y[v]) & 0x7FFFFFFFu);
          }
          if (full || n + 3 < N) {
            *reinterpret_cast<u32x4*>(row + n) = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]),
                                                       __float_as_uint(y[2]), __float_as_uint(y[3])};
          } else {
            row[n] = y[0];
            if (n + 1 < N) row[n + 1] = y[1];
            if (n + 2 < N) row[n + 2] = y[2];
          }
        }
    }
  }
  if (p.amax_c) {
    amax = wave_max_u32(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = red[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = max(m, red[w]);
      if constexpr (AMAX_STORE) p.amax_c[bz] = canonical_amax_bits(m);
      else atomicMax(p.amax_c + bz, canonical_amax_bits(m));
    }
  }
}

// The number of workgroup barriers `epilogue` executes (for waves that do not
// run it but must meet its barriers): two around the staging of full BF16 tiles,
// one for the output amax.
template <int BM, int BN>
__device__ __forceinline__ int epilogue_barriers(const GemmArgs& p, int64_t m0, int64_t n0) {
  const bool full = m0 + BM <= p.M && n0 + BN <= p.N;
  return (!p.out_f32 && full ? 2 : 0) + (p.amax_c ? 1 : 0);
}

// ------------------------------------------------------------------ the kernel
//
// Both datapaths stage FP8 tiles of 128 K values per LDS row.  Lane l works on
// row (l % 32) of each 32-row block and on the four 16-byte chunks
// 4 (l / 32) .. 4 (l / 32) + 3 of that row; the MFMA's K index is mapped onto
// those bytes identically for A and B, so each output sums all of the stage's
// products.
//
// EXACT: a stage is 8 MFMA steps of K = 16 (32x32x16 F16); step t uses bytes
// [8 (t % 2), 8 (t % 2) + 8) of chunk t / 2.  Software pipeline per wave:
//   * raw chunks of unit u + 1 are read from LDS during the first step of unit u;
//   * the F16 operands of step t + 1 are widened while the MFMAs of step t run
//     (two F16 fragment sets alternate), about two converts per MFMA;
//   * the global loads of the next stage are issued at step 0 and written to the
//     other LDS buffer at step 4; the stage's barrier sits at step 6, after which
//     the next stage's first raw chunks are read, so its first step is widened
//     under step 7.
// FP8: a stage is 2 MFMA steps of K = 64 (32x32x64 F8F6F4), each on two chunks.

// KS = 2: two groups of four waves share each output tile, group g taking the
// g-th half of the K stages with LDS buffers of its own; at the end group 1
// hands its partial sums to group 0 through LDS, which adds them to its own
// (first half + second half, always in that order) and runs the epilogue.  For
// grids of 128 x 128 tiles that give each CU one tile or less: twice the waves
// per CU, without partial results in memory.
template <int BM, int BN, bool A_KC, bool B_KC, int FA, int FB, bool EXACT, bool DIRECT,
          bool VS = false, bool MX = false, int KS = 1>
__global__ __launch_bounds__(256 * KS, 1) void gemm_kernel(GemmArgs p) {
  static_assert(!MX || (DIRECT && A_KC && B_KC && !VS),
                "MX blocks run along K: both operands K-contiguous, direct loads");
  static_assert(KS == 1 || (KS == 2 && DIRECT && !MX && BM == 128 && BN == 128),
                "the K split runs on direct loads of 128 x 128 tiles");
  constexpr int NT = 256;  // threads per group
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KB = 128;  // K values per stage
  __shared__ __attribute__((aligned(16))) uint8_t lds_a_g[KS][2][BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b_g[KS][2][BN * kRowBytes];
  __shared__ uint32_t red[4];

  const int grp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);
  uint8_t (*lds_a)[BM * kRowBytes] = lds_a_g[grp];
  uint8_t (*lds_b)[BN * kRowBytes] = lds_b_g[grp];
  const int tid = threadIdx.x & (NT - 1);  // thread within the group
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bz = blockIdx.y;

  int tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const uint8_t* A = p.A + bz * p.stride_a;
  const uint8_t* B = p.B + bz * p.stride_b;

  typename LoaderSel<A_KC, BM, NT, KB>::type la;
  typename LoaderSel<B_KC, BN, NT, KB>::type lb;

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // stages of this group: [kbase, kbase + nk) (KS = 2 requires an even stage count)
  const int nk = (int)((K + KB - 1) / KB) / KS;
  const int kbase = grp * nk;
  // dequant factor (VS: the per-row / per-column factors are applied in the epilogue)
  const float d = (VS || MX) ? 1.0f : __fdiv_rn(1.0f, p.scale_a[bz] * p.scale_b[bz]);
  const int fr = lane & 31;
  const int fc = (lane >> 5) * 4;  // first of this lane's four chunks

  // Raw operand bytes of one unit (16 K values per lane per 32-row block: the
  // two MFMA steps 2u and 2u + 1).  K-major LDS tiles give them as one 16-byte
  // chunk; MN-major tiles (direct loads of MN-contiguous operands) as two
  // transposing reads of 8 bytes whose K values follow the same order.
  constexpr bool A_MN_LDS = DIRECT && !A_KC;
  constexpr bool B_MN_LDS = DIRECT && !B_KC;
  const int tr_i = lane & 15;
  const int tr_row = 16 * ((lane >> 4) & 1) + 8 * (tr_i & 1);  // row offset in a 32-row block
  const int tr_k = 64 * (lane >> 5) + (tr_i >> 1);              // + 16 u + 8 h
  // Byte offsets, within a stage buffer, of this lane's reads of unit u of each
  // 32-row block: the 16-byte chunk fc + u of its row (K-major tiles, h = 0) or
  // the two 8-byte transposing reads h (MN-major tiles).  They do not change
  // from stage to stage, so a read adds only its buffer's base (recomputed per
  // read, the address arithmetic cost ~1% of the exact GEMMs' time).
  int offa[4][FM][2], offb[4][FN][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        offa[u][i][h] = A_MN_LDS ? mn_off<BM>(tr_k + 16 * u + 8 * h, wm * WTM + i * 32 + tr_row)
                                 : lds_off(wm * WTM + i * 32 + fr, fc + u);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        offb[u][j][h] = B_MN_LDS ? mn_off<BN>(tr_k + 16 * u + 8 * h, wn * WTN + j * 32 + tr_row)
                                 : lds_off(wn * WTN + j * 32 + fr, fc + u);
    }
  }
  // unit u of a block: one 16-byte read, or two transposing 8-byte reads
  auto read_frag = [&](const uint8_t* tile, const int (&off)[2], auto mn_tag) {
    if constexpr (decltype(mn_tag)::value) {
      const u32x2 lo = ds_read_tr8(tile + off[0]);
      const u32x2 hi = ds_read_tr8(tile + off[1]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      return *reinterpret_cast<const u32x4*>(tile + off[0]);
    }
  };
  auto read_unit = [&](int buf, int u, u32x4 (&xa)[FM], u32x4 (&xb)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
      xb[j] = read_frag(lds_b[buf], offb[u][j], std::integral_constant<bool, B_MN_LDS>{});
#pragma unroll
    for (int i = 0; i < FM; ++i)
      xa[i] = read_frag(lds_a[buf], offa[u][i], std::integral_constant<bool, A_MN_LDS>{});
  };

  // DIRECT: stages are loaded straight into LDS two stages ahead: stage k + 2
  // goes into the buffer of stage k right after stage k's barrier (all waves
  // have read it by then), and that barrier's wait on outstanding loads makes
  // stage k + 1 complete before it is read.
  // The wave's load instructions of a stage, A's then B's, numbered 0 ..
  // kIssuesA + kIssuesB; issue_direct issues those in [lo, hi).
  constexpr int kIssuesA = direct_issues<A_KC, BM, NT>();
  constexpr int kIssuesB = direct_issues<B_KC, BN, NT>();
  using DLA = typename DirectSel<A_KC, BM, NT>::type;
  using DLB = typename DirectSel<B_KC, BN, NT>::type;
  const DLA dla(DIRECT ? A : nullptr, p.lda, m0, M, K, tid);
  const DLB dlb(DIRECT ? B : nullptr, p.ldb, n0, N, K, tid);
  auto issue_direct = [&](int kt, int buf, int lo = 0, int hi = 1 << 20) {
    if constexpr (DIRECT) {
      const int la = lo, ha = hi < kIssuesA ? hi : kIssuesA;
      const int lb = lo > kIssuesA ? lo - kIssuesA : 0;
      const int hb = hi < kIssuesA + kIssuesB ? hi - kIssuesA : kIssuesB;
      dla.issue((int64_t)(kt + kbase) * KB, lds_a[buf], la, ha);
      dlb.issue((int64_t)(kt + kbase) * KB, lds_b[buf], lb, hb);
    }
  };
  if constexpr (EXACT) {
    u32x4 ra[2][FM], rb[2][FN];      // raw chunks, by unit parity
    u32x2 ha[2][FM][2], hb[2][FN][2]; // F16 operands of a step (8 values = 2 x u32x2), by step parity

    // MX: the E8M0 scales of this lane's rows, 4 blocks (one stage of 128 K) per
    // dword.  A unit u of a stage covers K bytes [64 (lane / 32) + 16 u, + 16),
    // i.e. block 2 (lane / 32) + u / 2 of the stage.  `sc*_nxt` holds the running
    // stage's dwords until its second half has taken them (step 3), then the next
    // stage's, loaded there; `sf*` the scale values of the running half stage.
    uint32_t sca_nxt[FM], scb_nxt[FN];
    float sfa[FM], sfb[FN];
    const int sc_shift = 16 * (lane >> 5);
    auto load_scales = [&](int kt) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int64_t r = min(m0 + wm * WTM + i * 32 + fr, M - 1);
          sca_nxt[i] = *reinterpret_cast<const uint32_t*>(p.sc_a + r * p.ldsa + 4 * (int64_t)kt);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t r = min(n0 + wn * WTN + j * 32 + fr, N - 1);
          scb_nxt[j] = *reinterpret_cast<const uint32_t*>(p.sc_b + r * p.ldsb + 4 * (int64_t)kt);
        }
      }
    };
    auto scale_f = [&](uint32_t dw, int hb2) {
      return e8m0_to_f32(__builtin_amdgcn_ubfe(dw, sc_shift + 8 * hb2, 8));
    };
    auto take_scales = [&](int hb2) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sfa[i] = scale_f(sca_nxt[i], hb2);
#pragma unroll
        for (int j = 0; j < FN; ++j) sfb[j] = scale_f(scb_nxt[j], hb2);
      }
    };

    // widen one half (8 bytes) of every raw chunk of a unit into F16 (MX: scaled
    // BF16) set `dst`; `u` is the unit within its stage, `next`: the unit belongs
    // to the stage after the running one (MX scales not taken yet)
    auto widen_step = [&](const u32x4 (&xa)[FM], const u32x4 (&xb)[FN], int half,
                          u32x2 (&da)[FM][2], u32x2 (&db)[FN][2], int u, bool next) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t w0 = xb[j][2 * half], w1 = xb[j][2 * half + 1];
        if constexpr (MX) {
          const float s = next ? scale_f(scb_nxt[j], 0) : sfb[j];
          db[j][0] = u32x2{widen_pair_mx<FB>(w0, false, s), widen_pair_mx<FB>(w0, true, s)};
          db[j][1] = u32x2{widen_pair_mx<FB>(w1, false, s), widen_pair_mx<FB>(w1, true, s)};
        } else {
          db[j][0] = u32x2{widen_pair<FB>(w0, false), widen_pair<FB>(w0, true)};
          db[j][1] = u32x2{widen_pair<FB>(w1, false), widen_pair<FB>(w1, true)};
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t w0 = xa[i][2 * half], w1 = xa[i][2 * half + 1];
        if constexpr (MX) {
          const float s = next ? scale_f(sca_nxt[i], 0) : sfa[i];
          da[i][0] = u32x2{widen_pair_mx<FA>(w0, false, s), widen_pair_mx<FA>(w0, true, s)};
          da[i][1] = u32x2{widen_pair_mx<FA>(w1, false, s), widen_pair_mx<FA>(w1, true, s)};
        } else {
          da[i][0] = u32x2{widen_pair<FA>(w0, false), widen_pair<FA>(w0, true)};
          da[i][1] = u32x2{widen_pair<FA>(w1, false), widen_pair<FA>(w1, true)};
        }
      }
    };
    auto mma = [&](const u32x2 (&da)[FM][2], const u32x2 (&db)[FN][2]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v8h av = __builtin_bit_cast(v8h, u32x4{da[i][0][0], da[i][0][1], da[i][1][0], da[i][1][1]});
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v8h bv =
              __builtin_bit_cast(v8h, u32x4{db[j][0][0], db[j][0][1], db[j][1][0], db[j][1][1]});
          // first operand = B block, second = A block: the result is the C^T block
          if constexpr (MX)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(v8bf, bv), __builtin_bit_cast(v8bf, av), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, av, acc[i][j], 0, 0, 0);
        }
      }
    };

    if (nk > 0) {
      if constexpr (DIRECT) {
        load_scales(0);
        issue_direct(0, 0);
        if (nk > 1) {
          // stage 0 (and everything before it) complete, stage 1 still in flight
          issue_direct(1, 1);
          vmem_wait_n<direct_issues<A_KC, BM, NT>() + direct_issues<B_KC, BN, NT>()>();
        } else {
          vmem_wait_all();
        }
      } else {
        la.load(A, p.lda, m0, M, 0, K, tid);
        lb.load(B, p.ldb, n0, N, 0, K, tid);
        la.store(lds_a[0], tid);
        lb.store(lds_b[0], tid);
      }
      __syncthreads();
      read_unit(0, 0, ra[0], rb[0]);
      widen_step(ra[0], rb[0], 0, ha[0], hb[0], 0, true);
    }

    // Direct loads of stage kt + 2 go into stage kt's buffer once stage kt's
    // barrier (step 6) has passed: half of them in step 6, half in step 7, each
    // load instruction placed after one of the step's MFMAs.  Issued in one burst
    // after the barrier, the 16 load instructions of a wave held up its MFMAs
    // (~20% of the kernel's time, measured by leaving the loads out).  They are
    // not spread further into the next stage: an LDS read that follows a direct
    // load in the same iteration makes the compiler wait for the load.
    constexpr int kIss = kIssuesA + kIssuesB;
    constexpr int kPart0 = kIss / 2;
    // LOADS: this stage issues the direct loads of stage kt + 2 (every stage but
    // the last two; a separate instantiation, so that no branch separates the
    // loads from the MFMAs they are interleaved with)
    auto stage = [&](int kt, auto more_tag, auto loads_tag) {
      constexpr bool MORE = decltype(more_tag)::value;
      constexpr bool LOADS = DIRECT && decltype(loads_tag)::value;
      const int cur = kt & 1;
      if constexpr (MX) take_scales(0);  // units 0, 1 of this stage (loaded a stage ago)
      if constexpr (MORE && !DIRECT) {
        la.load(A, p.lda, m0, M, (int64_t)(kt + 1) * KB, K, tid);
        lb.load(B, p.ldb, n0, N, (int64_t)(kt + 1) * KB, K, tid);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int u = t >> 1;
        if ((t & 1) == 0 && u + 1 < 4) read_unit(cur, u + 1, ra[(u + 1) & 1], rb[(u + 1) & 1]);
        if constexpr (MORE) {
          if constexpr (!DIRECT) {
            if (t == 4) {
              la.store(lds_a[cur ^ 1], tid);
              lb.store(lds_b[cur ^ 1], tid);
            }
          }
          if (t == 6) {
            if constexpr (DIRECT) vmem_wait_all();
            __syncthreads();
            read_unit(cur ^ 1, 0, ra[0], rb[0]);
            if constexpr (LOADS) issue_direct(kt + 2, cur, 0, kPart0);
          }
          if constexpr (LOADS) {
            if (t == 7) issue_direct(kt + 2, cur, kPart0, kIss);
          }
        }
        if constexpr (MX) {
          if (t == 3) {
            take_scales(1);  // units 2, 3: widened from step 3 on
            if constexpr (MORE) load_scales(kt + 1);
          }
        }
        // widen the operands of step t + 1 (the next stage's step 0 after t = 7)
        if (t < 7) {
          const int un = (t + 1) >> 1;
          widen_step(ra[un & 1], rb[un & 1], (t + 1) & 1, ha[(t + 1) & 1], hb[(t + 1) & 1], un,
                     false);
        } else if constexpr (MORE) {
          widen_step(ra[0], rb[0], 0, ha[0], hb[0], 0, true);
        }
        mma(ha[t & 1], hb[t & 1]);
        if constexpr (LOADS) {
          if (t >= 6) {  // one direct load after each of the first MFMAs
#pragma unroll
            for (int k = 0; k < kIss / 2; ++k) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
            }
          }
        }
        // keep each step's reads, stores and widening inside the step they were
        // placed in: the scheduler otherwise pulls the widening next to the LDS
        // reads it depends on and waits for them
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int kt = 0;
    if constexpr (DIRECT)
      for (; kt + 2 < nk; ++kt) stage(kt, std::true_type{}, std::true_type{});
    for (; kt + 1 < nk; ++kt) stage(kt, std::true_type{}, std::false_type{});
    if (nk > 0) stage(nk - 1, std::false_type{}, std::false_type{});
  } else {
    u32x4 ra[2][FM][2], rb[2][FN][2];  // two chunks per step, by step parity
    // Step s of a stage takes, per lane, 32 consecutive K values of its row:
    // k = 64 (l / 32) + 32 s + [0, 32), i.e. units 2 s and 2 s + 1 of the exact
    // path's reads (MX: the chunks described at `mma`).
    auto read_step = [&](int buf, int s, u32x4 (&xa)[FM][2], u32x4 (&xb)[FN][2]) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if constexpr (MX)
            xb[j][t] = *reinterpret_cast<const u32x4*>(
                lds_b[buf] + lds_off(wn * WTN + j * 32 + fr, 4 * s + 2 * t + (lane >> 5)));
          else
            xb[j][t] = read_frag(lds_b[buf], offb[2 * s + t][j],
                                 std::integral_constant<bool, B_MN_LDS>{});
        }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if constexpr (MX)
            xa[i][t] = *reinterpret_cast<const u32x4*>(
                lds_a[buf] + lds_off(wm * WTM + i * 32 + fr, 4 * s + 2 * t + (lane >> 5)));
          else
            xa[i][t] = read_frag(lds_a[buf], offa[2 * s + t][i],
                                 std::integral_constant<bool, A_MN_LDS>{});
        }
    };
    // MX: this lane's E8M0 scale dwords (the 4 blocks of a stage per row), loaded
    // a stage ahead.  The block-scaled instruction (probed on gfx950) scales
    // bytes 0..15 of lanes r and r + 32 by lane r's scale and bytes 16..31 of both
    // by lane r + 32's: each of its two K blocks is the first or the second 16
    // bytes of the two lanes of a row.  Step s therefore gives lane (r, h) the
    // chunks 4 s + h (bytes 0..15) and 4 s + 2 + h (bytes 16..31): the halves of
    // stage blocks 2 s and 2 s + 1, whose scales lanes h = 0 and h = 1 hand over.
    uint32_t fsa_cur[FM], fsb_cur[FN], fsa_nxt[FM], fsb_nxt[FN];
    auto load_scales8 = [&](int kt) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int64_t r = min(m0 + wm * WTM + i * 32 + fr, M - 1);
          fsa_nxt[i] = *reinterpret_cast<const uint32_t*>(p.sc_a + r * p.ldsa + 4 * (int64_t)kt);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t r = min(n0 + wn * WTN + j * 32 + fr, N - 1);
          fsb_nxt[j] = *reinterpret_cast<const uint32_t*>(p.sc_b + r * p.ldsb + 4 * (int64_t)kt);
        }
      }
    };
    auto mma = [&](const u32x4 (&xa)[FM][2], const u32x4 (&xb)[FN][2], int s) {
      const int sh = 16 * s + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v8i af = v8i{(int)xa[i][0][0], (int)xa[i][0][1], (int)xa[i][0][2], (int)xa[i][0][3],
                           (int)xa[i][1][0], (int)xa[i][1][1], (int)xa[i][1][2], (int)xa[i][1][3]};
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v8i bf = v8i{(int)xb[j][0][0], (int)xb[j][0][1], (int)xb[j][0][2],
                             (int)xb[j][0][3], (int)xb[j][1][0], (int)xb[j][1][1],
                             (int)xb[j][1][2], (int)xb[j][1][3]};
          if constexpr (MX) {
            const int scb = (int)__builtin_amdgcn_ubfe(fsb_cur[j], sh, 8);
            const int sca = (int)__builtin_amdgcn_ubfe(fsa_cur[i], sh, 8);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[i][j], FB, FA,
                                                                         0, scb, 0, sca);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[i][j], FB, FA,
                                                                         0, 0, 0, 0);
          }
        }
      }
    };
    if (nk > 0) {
      if constexpr (DIRECT) {
        load_scales8(0);
        issue_direct(0, 0);
        if (nk > 1) {
          issue_direct(1, 1);
          vmem_wait_n<direct_issues<A_KC, BM, NT>() + direct_issues<B_KC, BN, NT>()>();
        } else {
          vmem_wait_all();
        }
      } else {
        la.load(A, p.lda, m0, M, 0, K, tid);
        lb.load(B, p.ldb, n0, N, 0, K, tid);
        la.store(lds_a[0], tid);
        lb.store(lds_b[0], tid);
      }
      __syncthreads();
      read_step(0, 0, ra[0], rb[0]);
    }
    // LOADS: the stage issues the direct loads of stage kt + 2, one after each
    // of its second step's MFMAs (a separate instantiation for the last two
    // stages, so that no branch separates the loads from those MFMAs).
    // 256 x 256 tiles with direct loads fix the issue order further: step 1's
    // LDS reads go between step 0's MFMAs, and the next stage's reads and this
    // stage's loads between step 1's.  Left to the scheduler, the reads of step 1
    // followed all of step 0's MFMAs; with 16 or more LDS reads in flight the
    // in-order LDS counter cannot wait for the older ones alone, so the first
    // MFMA of the next step waited for all of them (+4-10% on the three layouts).
    constexpr bool kFixOrder = DIRECT && BM == 256 && BN == 256;
    constexpr int kMf = FM * FN;  // MFMAs per step
    constexpr int kDs = (A_MN_LDS ? 4 : 2) * FM + (B_MN_LDS ? 4 : 2) * FN;  // LDS reads per step
    static_assert(!kFixOrder || (kDs >= kMf && kDs <= 2 * kMf && kDs % (kMf / 2) == 0 &&
                                 (kIssuesA + kIssuesB) % (kMf / 2) == 0),
                  "issue pattern for 256 x 256 tiles");
    // one MFMA followed by two or one LDS reads, kDs reads over kMf MFMAs
    auto order_reads = [&]() {
      if constexpr (kFixOrder) {
#pragma unroll
        for (int k = 0; k < kDs - kMf; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
#pragma unroll
        for (int k = 0; k < 2 * kMf - kDs; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    auto stage = [&](int kt, auto more_tag, auto loads_tag) {
      constexpr bool MORE = decltype(more_tag)::value;
      constexpr bool LOADS = DIRECT && decltype(loads_tag)::value;
      const int cur = kt & 1;
      if constexpr (MORE && !DIRECT) {
        la.load(A, p.lda, m0, M, (int64_t)(kt + 1) * KB, K, tid);
        lb.load(B, p.ldb, n0, N, (int64_t)(kt + 1) * KB, K, tid);
      }
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fsa_cur[i] = fsa_nxt[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) fsb_cur[j] = fsb_nxt[j];
        if constexpr (MORE) load_scales8(kt + 1);
      }
      read_step(cur, 1, ra[1], rb[1]);
      if constexpr (MORE && !DIRECT) {
        la.store(lds_a[cur ^ 1], tid);
        lb.store(lds_b[cur ^ 1], tid);
      }
      mma(ra[0], rb[0], 0);
      if constexpr (kFixOrder) {
        order_reads();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (MORE) {
        if constexpr (DIRECT) vmem_wait_all();
        __syncthreads();
        read_step(cur ^ 1, 0, ra[0], rb[0]);
        if constexpr (LOADS) issue_direct(kt + 2, cur);
      }
      mma(ra[1], rb[1], 1);
      if constexpr (LOADS && kFixOrder) {
        // the next stage's reads over the first half of the MFMAs, the loads
        // over the second half
#pragma unroll
        for (int k = 0; k < kMf / 2; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, kDs / (kMf / 2), 0);
        }
#pragma unroll
        for (int k = 0; k < kMf / 2; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, (kIssuesA + kIssuesB) / (kMf / 2), 0);  // VMEM read
        }
      } else if constexpr (LOADS) {
#pragma unroll
        for (int k = 0; k < kIssuesA + kIssuesB; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
      } else if constexpr (MORE) {
        order_reads();
      }
    };
    int kt = 0;
    if constexpr (DIRECT)
      for (; kt + 2 < nk; ++kt) stage(kt, std::true_type{}, std::true_type{});
    for (; kt + 1 < nk; ++kt) stage(kt, std::true_type{}, std::false_type{});
    if (nk > 0) stage(nk - 1, std::false_type{}, std::false_type{});
  }

  if constexpr (KS == 2) {
    // Group 1's partial sums through its own LDS (each wave's 16 KiB: float4 q
    // of block (i, j) of lane l at ((i FN + j) 4 + q) 64 + l), added by the wave
    // of group 0 with the same index.
    static_assert(FM * FN * 16 * 64 * 4 * 2 == 2 * BM * kRowBytes, "two waves' sums per buffer");
    f32x4_t* xch = reinterpret_cast<f32x4_t*>(wave < 2 ? &lds_a_g[1][0][0] : &lds_b_g[1][0][0]) +
                   (wave & 1) * (FM * FN * 4 * 64);
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            xch[((i * FN + j) * 4 + q) * 64 + lane] =
                f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
    __syncthreads();
    if (grp == 1) {
      // the epilogue's barriers, which group 0 reaches there
      const int nb = epilogue_barriers<BM, BN>(p, m0, n0);
      for (int b = 0; b < nb; ++b) __syncthreads();
      return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t o = xch[((i * FN + j) * 4 + q) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = acc[i][j][4 * q + e] + o[e];
        }
  }
  epilogue<BM, BN, FM, FN, WTM, WTN, VS>(p, acc, m0, n0, wm, wn, tid, bz, d, red,
                                        reinterpret_cast<uint8_t*>(lds_a),
                                        reinterpret_cast<uint8_t*>(lds_b));
}

// ------------------------------------------------------------------ dispatch

template <int BM, int BN, bool A_KC, bool B_KC, int FA, int FB, bool EXACT, bool DIRECT, bool VS,
          bool MX = false, int KS = 1>
static hipError_t launch_cfg(const GemmProblem& q, hipStream_t stream) {
  GemmArgs a;
  a.M = q.M; a.N = q.N; a.K = q.K;
  a.A = q.A; a.lda = q.lda; a.scale_a = q.scale_a;
  a.B = q.B; a.ldb = q.ldb; a.scale_b = q.scale_b;
  a.C = q.C; a.ldc = q.ldc; a.amax_c = reinterpret_cast<uint32_t*>(q.amax_c);
  a.stride_a = q.stride_a; a.stride_b = q.stride_b; a.stride_c = q.stride_c;
  a.tiles_m = (int)((q.M + BM - 1) / BM);
  a.tiles_n = (int)((q.N + BN - 1) / BN);
  a.out_f32 = q.out_bf16 ? 0 : 1;
  a.inv_a = q.inv_a;
  a.inv_b = q.inv_b;
  a.sc_a = q.sc_a; a.sc_b = q.sc_b;
  a.ldsa = q.ldsa; a.ldsb = q.ldsb;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)q.batch);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, A_KC, B_KC, FA, FB, EXACT, DIRECT, VS, MX, KS>), grid,
                     dim3(256 * KS), 0, stream, a);
  return hipGetLastError();
}

// K a multiple of the stage depth and operands in aligned 16-byte chunks: LDS is
// filled by direct loads; otherwise through registers.
// ks2: run 128 x 128 tiles as two K halves per workgroup (K a multiple of 256,
// direct loads only).
template <int BM, int BN, bool A_KC, bool B_KC, int FA, int FB, bool EXACT, bool VS>
static hipError_t launch_direct(const GemmProblem& q, hipStream_t stream, bool ks2 = false) {
  {
    // Direct loads move aligned 16-byte chunks; MN-contiguous operands are
    // loaded in whole chunks along M / N.
    auto aligned = [&](const uint8_t* ptr, int64_t ld, int64_t stride) {
      return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && ld % 16 == 0 &&
             (q.batch == 1 || stride % 16 == 0);
    };
    // the buffer loads address each operand with 32-bit offsets
    auto fits = [&](int64_t rows, int64_t cols, int64_t ld) {
      return (rows + 256) * ld + cols < (int64_t(1) << 31);  // a tile may run past `rows`
    };
    const bool a_ok = aligned(q.A, q.lda, q.stride_a) && (A_KC || q.M % 16 == 0) &&
                      (A_KC ? fits(q.M, q.K, q.lda) : fits(q.K, q.M, q.lda));
    const bool b_ok = aligned(q.B, q.ldb, q.stride_b) && (B_KC || q.N % 16 == 0) &&
                      (B_KC ? fits(q.N, q.K, q.ldb) : fits(q.K, q.N, q.ldb));
    if (q.K % 128 == 0 && a_ok && b_ok) {
      if constexpr (BM == 128 && BN == 128) {
        if (ks2 && q.K % 256 == 0)
          return launch_cfg<BM, BN, A_KC, B_KC, FA, FB, EXACT, true, VS, false, 2>(q, stream);
      }
      return launch_cfg<BM, BN, A_KC, B_KC, FA, FB, EXACT, true, VS>(q, stream);
    }
  }
  return launch_cfg<BM, BN, A_KC, B_KC, FA, FB, EXACT, false, VS>(q, stream);
}

template <int BM, int BN, bool A_KC, bool B_KC, bool EXACT, bool VS>
static hipError_t launch_layout(const GemmProblem& q, hipStream_t s, bool ks2) {
  if (q.fa == kE4M3 && q.fb == kE4M3) return launch_direct<BM, BN, A_KC, B_KC, kE4M3, kE4M3, EXACT, VS>(q, s, ks2);
  if (q.fa == kE4M3 && q.fb == kE5M2) return launch_direct<BM, BN, A_KC, B_KC, kE4M3, kE5M2, EXACT, VS>(q, s, ks2);
  if (q.fa == kE5M2 && q.fb == kE4M3) return launch_direct<BM, BN, A_KC, B_KC, kE5M2, kE4M3, EXACT, VS>(q, s, ks2);
  if (q.fa == kE5M2 && q.fb == kE5M2) return launch_direct<BM, BN, A_KC, B_KC, kE5M2, kE5M2, EXACT, VS>(q, s, ks2);
  return hipErrorInvalidValue;
}

template <int BM, int BN, bool EXACT, bool VS>
static hipError_t launch_tile(const GemmProblem& q, hipStream_t s, bool ks2 = false) {
  if (q.opa == 0 && q.opb == 0) return launch_layout<BM, BN, true, false, EXACT, VS>(q, s, ks2);  // NN
  if (q.opa == 0 && q.opb == 1) return launch_layout<BM, BN, true, true, EXACT, VS>(q, s, ks2);   // NT
  if (q.opa == 1 && q.opb == 0) return launch_layout<BM, BN, false, false, EXACT, VS>(q, s, ks2); // TN
  return hipErrorInvalidValue;
}

// Tile choice: 256 x 256 tiles when they alone give every CU at least one tile
// and K is long enough to amortise their longer prologue and epilogue, else
// 128 x 128 tiles (two resident per CU).  Measured on MI355X: from K = 2048 on
// the larger tiles are 10-17% faster (16384 x 4096 x 2048 NT: 226 -> 205 us;
// 8192 x 4096 x 2048 NN: 125 -> 106 us); at K = 1024 the two are within noise
// of each other, and below that the smaller ones are faster (512 x 256^3
// batched: 52 -> 46 us).
constexpr int64_t kBigTileMinK = 2048;
// 128 x 128 tiles with at most one per CU (e.g. a 4096 x 1024 weight gradient)
// run as two K halves per workgroup once K is this long.
constexpr int64_t kSplitMinK = 1024;

template <bool EXACT, bool VS = false>
static hipError_t launch_path(const GemmProblem& q, int num_cus, hipStream_t stream) {
  if (q.M <= 0 || q.N <= 0 || q.batch <= 0) return hipSuccess;
  const int64_t big_tiles = ((q.M + 255) / 256) * ((q.N + 255) / 256) * q.batch;
  if (big_tiles >= num_cus && q.K >= kBigTileMinK) return launch_tile<256, 256, EXACT, VS>(q, stream);
  const int64_t tiles = ((q.M + 127) / 128) * ((q.N + 127) / 128) * q.batch;
  const bool ks2 = tiles <= num_cus && q.K >= kSplitMinK;
  return launch_tile<128, 128, EXACT, VS>(q, stream, ks2);
}

}  // namespace fp8ds

// Forward step of a batch of small Linears in one launch.  For each problem i:
//
//   xq_i = cast(X_i, s[i]),   wq_i = cast(W_i, s[B + i])        (delayed scales)
//   Y_i  = bf16( (xq_i wq_i) * fl32(1 / fl32(s[i] s[B + i])) ),  amax_y[i] = max |Y_i|
//   amax[i] = max |X_i|, amax[B + i] = max |W_i|, then the delayed-scaling update of
//   both tensors' histories, cursors and scales
//
// "LLM FP8 微调上线生产实战" §适用场景 (应谨慎的场景) and §常见误区 (误区一): with many
// small matrices the conversion work and the launches outweigh the FP8 gain.  Here
// one workgroup owns a whole problem (M, N, K up to 256): it reads X_i and W_i
// once, keeps their codes in LDS for the product (and writes them to HBM for the
// backward pass), and updates the two tensors' scaling state itself, so the step
// is one launch and the FP8 operands are never read back from HBM.
//
// Each part is the arithmetic of its separate kernel: the cast is the batched
// cast's (saturating RNE codes of fl32(x s), amax of the unscaled input, count
// of saturated values), the product is the exact GEMM's (codes widened to F16,
// V_MFMA_F32_32X32X16_F16, FP32 sums over the same K order), the epilogue is the
// GEMM's, and the update is scale_update_wave over the tensors
// [X_0 .. X_{B-1}, W_0 .. W_{B-1}].
//
// Layout of the codes in LDS: X as K-major rows of 128 bytes per stage of 128 k
// (lds_off), W as k rows of 256 bytes (mn_off), both exactly as the GEMM's
// direct loads place them, so the GEMM's fragment reads apply unchanged.

#include "cast_common.h"
#include "gemm_kernel.h"
#include "launch.h"
#include "scale_update.h"

namespace fp8ds {

// The eight scaled values fl32(x s) of one piece (8 BF16 values).
__device__ __forceinline__ void piece_scaled(const u32x4& d, float s, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_lo(d[k]) * s;
    v[2 * k + 1] = bf16_hi(d[k]) * s;
  }
}
// Codes of one piece by the packed converts (saturating RNE for every value that
// is not NaN); folds the piece's |x| bit patterns into amax2.
template <int FMT>
__device__ __forceinline__ u32x2 cast_piece8_fast(const u32x4& d, float s, u16x2& amax2) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(u16x2, d[k] & 0x7FFF7FFFu));
  float v[8];
  piece_scaled(d, s, v);
  return u32x2{encode4_hw<FMT>(v[0], v[1], v[2], v[3]), encode4_hw<FMT>(v[4], v[5], v[6], v[7])};
}
// The same piece through the software encoder when it holds a NaN, with its
// count of saturated values (|fl32(x s)| > max).
template <int FMT>
__device__ __forceinline__ u32x2 cast_piece8_exact(const u32x4& d, float s, uint32_t& sat) {
  float v[8];
  piece_scaled(d, s, v);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) m = max(m, max(d[k] & 0x7FFFu, (d[k] >> 16) & 0x7FFFu));
  sat += sat4<FMT>(v[0], v[1], v[2], v[3]) + sat4<FMT>(v[4], v[5], v[6], v[7]);
  if (m > 0x7F80u)
    return u32x2{encode4_sw<FMT>(v[0], v[1], v[2], v[3]), encode4_sw<FMT>(v[4], v[5], v[6], v[7])};
  return u32x2{encode4_hw<FMT>(v[0], v[1], v[2], v[3]), encode4_hw<FMT>(v[4], v[5], v[6], v[7])};
}

// A thread's pieces all take the fast path; afterwards, a thread whose largest
// |x| is NaN or whose largest scaled magnitude exceeds the format's maximum
// (fl32(|x| |s|) is monotonic in |x|, so no other thread holds a saturated
// value) converts its pieces again on the exact path, rewriting their codes and
// counting the saturated values.
template <int FMT>
__device__ __forceinline__ bool needs_exact(u16x2 amax2, float s) {
  const uint32_t top = max((uint32_t)amax2.x, (uint32_t)amax2.y);
  return top > 0x7F80u || fabsf(__uint_as_float(top << 16) * s) > FmtTraits<FMT>::kMax;
}

// One workgroup of 512 threads per problem (one resident per CU: the
// accumulators of a 256 x 256 output fill half of the CU's registers and the
// codes 128 KiB of its LDS).  Eight waves in a 4 x 2 grid, each owning 64 x 128
// outputs (2 x 4 blocks of 32 x 32).  Every thread issues the loads of all its
// pieces of X_i and W_i (16 + 16 at 256^3) before converting any.
// (Measured on MI355X over 512 problems of 256^3: 62 us.  Workgroups that take
// two problems each and issue the second one's loads while the first one's
// output is stored took 75 us.)
// FULL: M = N = K = 256, the whole piece walk known at compile time (straight-line
// code, so that each conversion waits only for its own load; with a guard per
// piece the compiler waits for every outstanding load and store at each one).
template <int FX, int FW, bool FULL>
__global__ __launch_bounds__(512) void linear_batched_kernel(LinearBatchedArgs p) {
  constexpr int NT = 512, NW = NT / 64;
  constexpr int BM = 256, BN = 256, WTM = 64, WTN = 128;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int PMAX = 256 * 256 / 8 / NT;  // pieces per thread per operand, largest shape
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kRowBytes];  // X codes
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][128 * BN];        // W codes
  __shared__ uint32_t red[4 * NW];  // per wave: amax bits and saturations of X, then of W
  __shared__ uint32_t red_y[NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t b = blockIdx.x;
  const int B = p.batch;
  const int M = FULL ? 256 : p.M, N = FULL ? 256 : p.N, K = FULL ? 256 : p.K;
  const int kpx = K >> 3, npx = M * kpx;  // X: pieces per row, pieces
  const int kpw = N >> 3, npw = K * kpw;  // W
  const int nk = (K + 127) >> 7;          // stages of 128 k
  const float sx = p.scale[b], sw = p.scale[B + b];

  // ---- loads: every piece of X_b and W_b (contiguous [M][K] and [K][N])
  const u32x4* xv = reinterpret_cast<const u32x4*>(p.x + b * p.stride_x);
  const u32x4* wv = reinterpret_cast<const u32x4*>(p.w + b * p.stride_w);
  u32x4 vx[PMAX], vw[PMAX];
#pragma unroll
  for (int j = 0; j < PMAX; ++j) {
    const int pc = tid + NT * j;
    if (FULL || pc < npx) vx[j] = __builtin_nontemporal_load(xv + pc);
  }
#pragma unroll
  for (int j = 0; j < PMAX; ++j) {
    const int pc = tid + NT * j;
    if (FULL || pc < npw) vw[j] = __builtin_nontemporal_load(wv + pc);
  }

  // ---- K ending inside a stage: zero that stage's tiles first, so that the k
  // past K hold zero codes in both operands (no stale NaN code meets a zero)
  if (!FULL && (K & 127)) {
    u32x4* za = reinterpret_cast<u32x4*>(lds_a[nk - 1]);
    u32x4* zb = reinterpret_cast<u32x4*>(lds_b[nk - 1]);
    for (int i = tid; i < BM * kRowBytes / 16; i += NT) za[i] = u32x4{0u, 0u, 0u, 0u};
    for (int i = tid; i < 128 * BN / 16; i += NT) zb[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }

  // ---- cast: codes into LDS in the GEMM's layouts and into HBM.  X piece pc is
  // row pc / kpx, k = 8 (pc % kpx); W piece pc is row k = pc / kpw, n = 8 (pc % kpw);
  // both walked incrementally (a thread's pieces are NT apart).
  auto walk_x = [&](auto fn) {
    int r = tid / kpx, kp = tid - r * kpx;
    const int dr = NT / kpx, dk = NT - dr * kpx;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const int pc = tid + NT * j;
      if (FULL || pc < npx) {
        const int k = kp << 3;
        fn(j, pc, lds_a[k >> 7] + lds_off(r, (k & 127) >> 4) + (k & 8));
      }
      r += dr;
      kp += dk;
      if (kp >= kpx) {
        kp -= kpx;
        ++r;
      }
    }
  };
  auto walk_w = [&](auto fn) {
    int k = tid / kpw, np = tid - k * kpw;
    const int dk = NT / kpw, dn = NT - dk * kpw;
#pragma unroll
    for (int j = 0; j < PMAX; ++j) {
      const int pc = tid + NT * j;
      if (FULL || pc < npw) fn(j, pc, lds_b[k >> 7] + mn_off<BN>(k & 127, np << 3));
      k += dk;
      np += dn;
      if (np >= kpw) {
        np -= kpw;
        ++k;
      }
    }
  };
  uint8_t* xq = p.xq ? p.xq + b * p.stride_xq : nullptr;
  uint8_t* wq = p.wq ? p.wq + b * p.stride_wq : nullptr;
  u16x2 ax2 = {0, 0}, aw2 = {0, 0};
  uint32_t satx = 0, satw = 0;
  walk_x([&](int j, int pc, uint8_t* l) {
    const u32x2 c = cast_piece8_fast<FX>(vx[j], sx, ax2);
    *reinterpret_cast<u32x2*>(l) = c;
    if (xq) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(xq) + pc);
  });
  walk_w([&](int j, int pc, uint8_t* l) {
    const u32x2 c = cast_piece8_fast<FW>(vw[j], sw, aw2);
    *reinterpret_cast<u32x2*>(l) = c;
    if (wq) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(wq) + pc);
  });
  // (the exact path starts from opaque copies of the input registers: otherwise
  // the compiler keeps the fast path's unpacked and scaled values of every piece
  // live to reuse them there.  Reading the pieces again from memory instead
  // measured 13% slower over the whole kernel.)
  if (__builtin_amdgcn_ballot_w64(needs_exact<FX>(ax2, sx))) {
    if (needs_exact<FX>(ax2, sx)) {
#pragma unroll
      for (int j = 0; j < PMAX; ++j) asm volatile("" : "+v"(vx[j]));
      walk_x([&](int j, int pc, uint8_t* l) {
        const u32x2 c = cast_piece8_exact<FX>(vx[j], sx, satx);
        *reinterpret_cast<u32x2*>(l) = c;
        if (xq) reinterpret_cast<u32x2*>(xq)[pc] = c;
      });
    }
  }
  if (__builtin_amdgcn_ballot_w64(needs_exact<FW>(aw2, sw))) {
    if (needs_exact<FW>(aw2, sw)) {
#pragma unroll
      for (int j = 0; j < PMAX; ++j) asm volatile("" : "+v"(vw[j]));
      walk_w([&](int j, int pc, uint8_t* l) {
        const u32x2 c = cast_piece8_exact<FW>(vw[j], sw, satw);
        *reinterpret_cast<u32x2*>(l) = c;
        if (wq) reinterpret_cast<u32x2*>(wq)[pc] = c;
      });
    }
  }
  {
    const uint32_t ax = wave_max_u32((uint32_t)max(ax2.x, ax2.y) << 16);
    const uint32_t aw = wave_max_u32((uint32_t)max(aw2.x, aw2.y) << 16);
    const uint32_t sx_n = __any(satx != 0) ? wave_sum_u32(satx) : 0u;
    const uint32_t sw_n = __any(satw != 0) ? wave_sum_u32(satw) : 0u;
    if (lane == 0) {
      red[4 * wave] = ax;
      red[4 * wave + 1] = sx_n;
      red[4 * wave + 2] = aw;
      red[4 * wave + 3] = sw_n;
    }
  }
  __syncthreads();  // the codes are in LDS

  // ---- the product: the GEMM kernel's fragment reads, widening and MFMA order
  // (lane l works on row l % 32 of each block and on the four 16-byte chunks
  // 4 (l / 32) .. + 3 of each stage row), and its software pipeline: a stage is 8
  // MFMA steps of K = 16 (step t uses bytes [8 (t % 2), + 8) of unit t / 2); the
  // raw chunks of unit u + 1 are read during step 2u, the F16 operands of step
  // t + 1 are widened while the MFMAs of step t run, and the next stage's first
  // unit is read at step 6 (its buffer half is free from then on).
  const int fr = lane & 31, fc = (lane >> 5) * 4;
  const int tr_i = lane & 15;
  const int tr_row = 16 * ((lane >> 4) & 1) + 8 * (tr_i & 1);
  const int tr_k = 64 * (lane >> 5) + (tr_i >> 1);
  auto read_unit = [&](int st, int u, u32x4 (&xa)[FM], u32x4 (&xb)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r0 = wn * WTN + j * 32 + tr_row;
      const u32x2 lo = ds_read_tr8(lds_b[st] + mn_off<BN>(tr_k + 16 * u, r0));
      const u32x2 hi = ds_read_tr8(lds_b[st] + mn_off<BN>(tr_k + 16 * u + 8, r0));
      xb[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
      xa[i] = *reinterpret_cast<const u32x4*>(lds_a[st] + lds_off(wm * WTM + i * 32 + fr, fc + u));
  };
  auto widen = [&](const u32x4 (&xa)[FM], const u32x4 (&xb)[FN], int half, u32x2 (&da)[FM][2],
                   u32x2 (&db)[FN][2]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint32_t w0 = xb[j][2 * half], w1 = xb[j][2 * half + 1];
      db[j][0] = u32x2{widen_pair<FW>(w0, false), widen_pair<FW>(w0, true)};
      db[j][1] = u32x2{widen_pair<FW>(w1, false), widen_pair<FW>(w1, true)};
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t w0 = xa[i][2 * half], w1 = xa[i][2 * half + 1];
      da[i][0] = u32x2{widen_pair<FX>(w0, false), widen_pair<FX>(w0, true)};
      da[i][1] = u32x2{widen_pair<FX>(w1, false), widen_pair<FX>(w1, true)};
    }
  };
  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto mma = [&](const u32x2 (&da)[FM][2], const u32x2 (&db)[FN][2]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v8h av = __builtin_bit_cast(v8h, u32x4{da[i][0][0], da[i][0][1], da[i][1][0], da[i][1][1]});
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v8h bv =
            __builtin_bit_cast(v8h, u32x4{db[j][0][0], db[j][0][1], db[j][1][0], db[j][1][1]});
        // first operand = W block, second = X block: the result is the Y^T block
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, av, acc[i][j], 0, 0, 0);
      }
    }
  };
  {
    u32x4 ra[2][FM], rb[2][FN];
    u32x2 ha[2][FM][2], hb[2][FN][2];
    read_unit(0, 0, ra[0], rb[0]);
    widen(ra[0], rb[0], 0, ha[0], hb[0]);
    for (int st = 0; st < nk; ++st) {
      const bool more = st + 1 < nk;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int u = t >> 1;
        if ((t & 1) == 0 && u + 1 < 4) read_unit(st, u + 1, ra[(u + 1) & 1], rb[(u + 1) & 1]);
        if (t == 6 && more) read_unit(st + 1, 0, ra[0], rb[0]);
        if (t < 7) {
          const int un = (t + 1) >> 1;
          widen(ra[un & 1], rb[un & 1], (t + 1) & 1, ha[(t + 1) & 1], hb[(t + 1) & 1]);
        } else if (more) {
          widen(ra[0], rb[0], 0, ha[0], hb[0]);
        }
        mma(ha[t & 1], hb[t & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: y = bf16(acc * fl32(1 / fl32(s_x s_w))), each wave's 64 x 128
  // block staged in the codes' LDS as BF16 rows of 256 bytes (16-byte chunk c of
  // staged row r at c ^ (r % 16)) and stored in whole row runs, non-temporally
  // (8% faster over the step than cached stores), with the output amax (only
  // in-range elements count)
  constexpr int RB = WTN * 2, CH = RB / 16, RPI = 64 / CH;
  static_assert(NW * WTM * RB == sizeof(lds_a) + sizeof(lds_b) && sizeof(lds_a) == sizeof(lds_b),
                "the staged output fills the codes' LDS");
  uint8_t* stg = wave < NW / 2 ? &lds_a[0][0] + wave * WTM * RB
                               : &lds_b[0][0] + (wave - NW / 2) * WTM * RB;
  const float d = __fdiv_rn(1.0f, sx * sw);
  __syncthreads();  // every wave has finished reading the codes
  u16x2_t am2 = {0, 0};
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int sr = i * 32 + (lane & 31);
    const bool row_ok = FULL || wm * WTM + sr < M;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = pack_bf16x2(acc[i][j][4 * g] * d, acc[i][j][4 * g + 1] * d);
        const uint32_t hi = pack_bf16x2(acc[i][j][4 * g + 2] * d, acc[i][j][4 * g + 3] * d);
        const int ch = 4 * j + g;  // columns 32 j + 8 g + [0, 8) of the block
        *reinterpret_cast<u32x2*>(stg + sr * RB + ((ch ^ (sr % CH)) * 16) + 8 * (lane >> 5)) =
            u32x2{lo, hi};
        const bool ok = row_ok && (FULL || wn * WTN + 32 * j + 8 * g + 4 * (lane >> 5) < N);
        if (ok)
          am2 = __builtin_elementwise_max(
              am2, __builtin_elementwise_max(abs_bf16x2(lo), abs_bf16x2(hi)));
      }
  }
  {
    const uint32_t am = wave_max_u32((uint32_t)max(am2[0], am2[1]) << 16);
    if (lane == 0) red_y[wave] = am;
  }
  __syncthreads();  // the blocks are staged, the waves' output amax posted
  {
    uint16_t* y = p.y + b * p.stride_y;
    const int ch = lane % CH;
    const int n = wn * WTN + ch * 8;
#pragma unroll
    for (int r = 0; r < WTM / RPI; ++r) {
      const int sr = r * RPI + lane / CH;
      const int m = wm * WTM + sr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + sr * RB + ((ch ^ (sr % CH)) * 16));
      if (FULL || (m < M && n < N)) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y + (int64_t)m * N + n));
    }
  }

  // ---- output amax (wave 2); this step's amax, saturations and scale snapshot
  // of X_b (wave 0) and W_b (wave 1), then their scaling-state update
  if (wave == 2 && p.amax_y) {
    const uint32_t am = wave_max_u32(lane < NW ? red_y[lane] : 0u);
    if (lane == 0) p.amax_y[b] = __uint_as_float(canonical_amax_bits(am));
  }
  if (wave < 2) {
    const int t = wave == 0 ? (int)b : B + (int)b;
    uint32_t am = lane < NW ? red[4 * lane + 2 * wave] : 0u;
    uint32_t sc = lane < NW ? red[4 * lane + 2 * wave + 1] : 0u;
    am = canonical_amax_bits(wave_max_u32(am));
    sc = wave_sum_u32(sc);
    if (lane == 0) {
      p.amax[t] = __uint_as_float(am);
      if (p.sat) p.sat[t] = (unsigned long long)sc;
      if (p.scale_used) p.scale_used[t] = wave == 0 ? sx : sw;
    }
    const bool e5m2 = wave == 0 ? FX == kE5M2 : FW == kE5M2;
    scale_update_wave(p.history + (int64_t)t * p.hist_len, p.hist_len, p.cursor + t,
                      __uint_as_float(am), e5m2, p.algo, p.margin, p.scale + t, nullptr, lane);
  }
}

// One workgroup per problem.
template <int FX, int FW>
static hipError_t launch_fmt(const LinearBatchedArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.batch);
  if (a.M == 256 && a.N == 256 && a.K == 256)
    hipLaunchKernelGGL((linear_batched_kernel<FX, FW, true>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((linear_batched_kernel<FX, FW, false>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_linear_batched(const LinearBatchedArgs& a, int fx, int fw, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  if (fx == kE4M3 && fw == kE4M3) return launch_fmt<kE4M3, kE4M3>(a, stream);
  if (fx == kE4M3 && fw == kE5M2) return launch_fmt<kE4M3, kE5M2>(a, stream);
  if (fx == kE5M2 && fw == kE4M3) return launch_fmt<kE5M2, kE4M3>(a, stream);
  if (fx == kE5M2 && fw == kE5M2) return launch_fmt<kE5M2, kE5M2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fp8ds

// gemv.hip - batch-1 projections y = W x (a GEMV at M = 1) streamed from HBM.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
//
// [Qwen3-runtime] §4.1: at batch 1 every weight is read once and used for one multiply-add, so a
// projection is bound by the weight bytes it streams; §13.1 gives the W8A16 form (int8 weights,
// fp32 accumulation, the scale applied after the integer-weighted sum).  Plain VALU work: no
// MFMA, since M = 1 is not a dense contraction.
//
// k_gemv: a work-group of 4 waves handles 4/SPLIT row groups per round; a row group is R output
// rows (R gate + R up rows for SwiGLU, [Qwen3-runtime] §2.7) split along K over SPLIT waves.
//   1. Every wave first requests what does not depend on the weights: the input (its K-slice,
//      or, with the RMSNorm prologue of [Qwen3-runtime] §2.1 fused, the row and gamma -- per
//      wave when each wave has its own quarter of K, shared by the work-group otherwise) and
//      the epilogue operands of its rows (residual values, int8 row scales).  Then it issues the
//      loads of its rows' K-slice for the first round (lane l reads elements
//      kslice + c*64*VEC + l*VEC .. +VEC of each row: one wave-wide load is a contiguous 1 KiB of
//      a row; 8-byte loads, 512 B, for packed int4).  Row addresses are scalar: a load is a
//      scalar row base plus the lane's fixed 32-bit offset.  Group-wise int8 / int4 weights
//      ([Qwen3-runtime] §13.1: a scale per 128-value group) also load, per lane and load, the
//      scale of the group its VEC elements lie in; the lane multiplies its partial dot product
//      by that scale before the row reduction.  Loads complete in order, so the input is ready
//      -- and normalised, with one block reduction of the sum of squares -- while the weights
//      are still in flight.  Every weight load is unconditional (rows past the end are clamped
//      to the last row, chunks past the slice to its start, results discarded), so each
//      compiler-inserted wait covers exactly what its consumer needs.
//   2. Rounds: FMAs over the registers, a DPP + readlane reduction per row, a reduction over the
//      SPLIT waves through LDS, and the epilogue on lane r of row r: store (fp32 / bf16), the
//      residual add (from the prefetched residual value), or silu(gate) * up.  With several
//      rounds per work-group (the LM head), the next round's rows are requested before the
//      current one is reduced, and each lane keeps the running (max, lowest index) of its rows'
//      rounded outputs for the greedy argmax.
#include "common.h"
#include "launch.h"

#ifndef QD_GEMV_PART
#error "compile with -DQD_GEMV_PART=<weight type> or -1 (dispatcher)"
#endif

namespace qd {

template <int WT>
struct WTraits;
// VEC: elements per lane per load; BITS: bits per element; Vec: the loaded vector type; GROUPED:
// a scale per 128-value group; BIAS: what the unsigned reading of a code adds (dot16).
template <>
struct WTraits<W_F32> {
  static constexpr int VEC = 4, BITS = 32, BIAS = 0;
  static constexpr bool GROUPED = false;
  using Vec = uint4;
};
template <>
struct WTraits<W_BF16> {
  static constexpr int VEC = 8, BITS = 16, BIAS = 0;
  static constexpr bool GROUPED = false;
  using Vec = uint4;
};
template <>
struct WTraits<W_I8> {
  static constexpr int VEC = 16, BITS = 8, BIAS = 128;
  static constexpr bool GROUPED = false;
  using Vec = uint4;
};
template <>
struct WTraits<W_I8G> {
  static constexpr int VEC = 16, BITS = 8, BIAS = 128;
  static constexpr bool GROUPED = true;
  using Vec = uint4;
};
template <>
struct WTraits<W_I4G> {
  static constexpr int VEC = 16, BITS = 4, BIAS = 8;
  static constexpr bool GROUPED = true;
  using Vec = uint2;
};

// An int8 code q read as the unsigned byte u = q ^ 0x80 = q + 128: one conversion instruction per
// element (v_cvt_f32_ubyte0..3); the dot product then over-counts 128 * sum(x), which the caller
// subtracts once per row.
__device__ __forceinline__ float u8_at(uint32_t u, int b) { return (float)((u >> (8 * b)) & 0xFFu); }

// acc + sum over the VEC elements of one weight vector times VEC fp32 values (for int8: the
// codes plus 128, see u8_at; for int4: the stored nibbles, i.e. the codes plus 8, times 2^-24).
// int4: a nibble u masked into a 16-bit half, read as fp16, is the subnormal u * 2^-24, which
// v_fma_mix_f32 takes directly as one factor of an fp32 fma (exactly: it converts the half to
// fp32 first, and fp16 subnormals are kept).  A word holds elements e = 0..7 at bits 4e; the
// masks 0x000F000F and 0x00F000F0, on the word and on the word shifted right by 8, leave the
// element pairs (0,4), (1,5) times 16, (2,6) and (3,7) times 16 in the two halves -- the caller
// has divided the odd inputs by 16, which is exact -- so 5 bit operations and 8 fmas per 8
// elements remain, and the sum is the plain fp32 one scaled by 2^-24 (the caller undoes it).
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
template <int WT>
__device__ __forceinline__ float dot16(typename WTraits<WT>::Vec w, const float* __restrict__ x,
                                       float acc) {
  if constexpr (WT == W_F32) {
    acc = fmaf(__uint_as_float(w.x), x[0], acc);
    acc = fmaf(__uint_as_float(w.y), x[1], acc);
    acc = fmaf(__uint_as_float(w.z), x[2], acc);
    acc = fmaf(__uint_as_float(w.w), x[3], acc);
  } else if constexpr (WT == W_BF16) {
    acc = fmaf(bf16_lo(w.x), x[0], acc);
    acc = fmaf(bf16_hi(w.x), x[1], acc);
    acc = fmaf(bf16_lo(w.y), x[2], acc);
    acc = fmaf(bf16_hi(w.y), x[3], acc);
    acc = fmaf(bf16_lo(w.z), x[4], acc);
    acc = fmaf(bf16_hi(w.z), x[5], acc);
    acc = fmaf(bf16_lo(w.w), x[6], acc);
    acc = fmaf(bf16_hi(w.w), x[7], acc);
  } else if constexpr (WT == W_I4G) {
    const uint32_t wd[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t sh = wd[j] >> 8;
      const half2v p[4] = {__builtin_bit_cast(half2v, wd[j] & 0x000F000Fu),
                           __builtin_bit_cast(half2v, wd[j] & 0x00F000F0u),
                           __builtin_bit_cast(half2v, sh & 0x000F000Fu),
                           __builtin_bit_cast(half2v, sh & 0x00F000F0u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf((float)p[i].x, x[8 * j + i], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf((float)p[i].y, x[8 * j + 4 + i], acc);
    }
  } else {
    const uint32_t ws[4] = {w.x ^ 0x80808080u, w.y ^ 0x80808080u, w.z ^ 0x80808080u,
                            w.w ^ 0x80808080u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(u8_at(ws[j], 0), x[4 * j + 0], acc);
      acc = fmaf(u8_at(ws[j], 1), x[4 * j + 1], acc);
      acc = fmaf(u8_at(ws[j], 2), x[4 * j + 2], acc);
      acc = fmaf(u8_at(ws[j], 3), x[4 * j + 3], acc);
    }
  }
  return acc;
}

// Wave sums of NR = 1, 2, 4 or 8 per-lane values at once: lane l receives the sum over all 64
// lanes of v[l / (64 / NR)].  Each halving stage keeps half the rows per lane and adds the
// partner's copy: v_permlane32_swap(A, B) leaves A's lower and B's lower half in the first result
// and A's upper and B's upper half in the second, so their sum is A's pair sum in lanes 0-31 and
// B's in lanes 32-63 (v_permlane16_swap the same for 16-lane rows, a DPP rotate by 8 for the last
// stage); the rest is an ordinary sum over the 64 / NR lanes of a group.  NR rows cost about
// 1.25 NR + 4 operations instead of NR full reductions.
template <int NR>
__device__ __forceinline__ float reduce_rows(float (&v)[NR]) {
  static_assert(NR == 1 || NR == 2 || NR == 4 || NR == 8, "rows per reduction");
  if constexpr (NR == 1) {
    return wave_sum(v[0]);
  } else {
#pragma unroll
    for (int k = 0; k < NR / 2; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]),
                                                      __float_as_uint(v[k + NR / 2]), false, false);
      v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (NR >= 4) {
#pragma unroll
      for (int k = 0; k < NR / 4; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(
            __float_as_uint(v[k]), __float_as_uint(v[k + NR / 4]), false, false);
        v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
    }
    if constexpr (NR == 8) {  // lanes with bit 3 clear keep v[0], the others v[1]
      const bool hi8 = (__lane_id() & 8) != 0;
      const float recv = dpp<0x128>(hi8 ? v[0] : v[1]);
      v[0] = (hi8 ? v[1] : v[0]) + recv;
    }
    float t = v[0];
    if constexpr (NR == 2) {
      t = group_sum<16>(t);
      float lo, hi;
      lane_pair<16>(t, lo, hi);
      return lo + hi;
    } else if constexpr (NR == 4) {
      return group_sum<16>(t);
    } else {
      return group_sum<8>(t);
    }
  }
}

__device__ __forceinline__ bool argmax_better(float vb, int ib, float va, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return vb > va || (vb == va && ib < ia);
}

// VEC consecutive input values at element k (fp32, or bf16 when XB).
template <bool XB, int VEC>
__device__ __forceinline__ void load_vec(const void* x, int64_t k, float (&v)[VEC]) {
  if constexpr (XB) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + k;
    if constexpr (VEC == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    } else {
#pragma unroll
      for (int j = 0; j < VEC / 8; ++j) {
        const uint4 u = *reinterpret_cast<const uint4*>(p + 8 * j);
        v[8 * j + 0] = bf16_lo(u.x); v[8 * j + 1] = bf16_hi(u.x);
        v[8 * j + 2] = bf16_lo(u.y); v[8 * j + 3] = bf16_hi(u.y);
        v[8 * j + 4] = bf16_lo(u.z); v[8 * j + 5] = bf16_hi(u.z);
        v[8 * j + 6] = bf16_lo(u.w); v[8 * j + 7] = bf16_hi(u.w);
      }
    }
  } else {
    const float* p = static_cast<const float*>(x) + k;
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(p + 4 * j);
      v[4 * j + 0] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
    }
  }
}

// RMSNorm prologue: float4s of the input (and of gamma) each thread loads before the weights are
// requested (inputs up to 4096 values in one pass); x * gamma is staged in LDS, K floats, so
// norm inputs are limited to kGemvNormMaxK values.
constexpr int kNormThreads = 256;
constexpr int kNormSlots = 4;
// The NORM template argument: no RMSNorm prologue, the per-wave one (split 4: each wave loads
// its own quarter of the row) or the shared one (split 2 or 1, where waves would load the same
// slice).  The two prologues are separate instantiations: compiled into one kernel, the unused
// one's registers cost the other its occupancy (measured 1-7 % per step).
constexpr int kNormNone = 0, kNormWave = 1, kNormShared = 2;

template <int WT, int EPI, int NORM, bool XB, int R, int MAXCH, bool PIPE>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  constexpr int VEC = WTraits<WT>::VEC;
  constexpr int BITS = WTraits<WT>::BITS;
  constexpr bool GROUPED = WTraits<WT>::GROUPED;
  using Vec = typename WTraits<WT>::Vec;
  constexpr int CH = kWave * VEC;                  // elements per wave-wide load
  constexpr int SR = GROUPED ? 1 : 0;              // group-scale arrays are [1][1] otherwise
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  __shared__ float red_ss[4];
  __shared__ float red_acc[4][NR];
  __shared__ float red_bv[4];
  __shared__ int red_bi[4];

  // the wave index is uniform over the wave: readfirstlane lets the compiler keep it, and with
  // it every row index and row address, in scalar registers (a load is then a scalar base plus a
  // per-lane 32-bit offset, with no per-lane address arithmetic)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = a.split;
  const int gpw = 4 / split;                       // row groups per work-group round
  const int sub = wave % split;                    // K-slice of this wave
  const int grp = wave / split;                    // row group of this wave within the round
  const int K = (int)a.k;
  const int KW = K / split;                        // elements per slice
  const int kbase = sub * KW;
  const int64_t n = a.n;
  const int64_t ngroups = (n + R - 1) / R;
  const char* __restrict__ wbase = static_cast<const char*>(a.w);
  const int64_t row_bytes = (int64_t)K * BITS / 8;
  const int ng = K / kQGroup;                      // scale groups per row (grouped types)

  auto row_of = [&](int64_t gg, int r) -> int64_t {
    const int64_t row = gg * R + r;
    return row < n ? row : n - 1;  // clamp: loads stay in bounds, results are discarded
  };
  // per-lane byte offset of each chunk within a row, and its scale group (grouped types)
  uint32_t loff[MAXCH], lgrp[MAXCH];
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    const int kk = c * CH + lane * VEC;
    const int kc = kbase + (kk < KW ? kk : 0);
    loff[c] = (uint32_t)kc * BITS / 8;
    lgrp[c] = (uint32_t)kc / kQGroup;
  }
  // the weight vectors of group gg's rows, and for grouped types the scale of each vector's group
  auto load_rows = [&](int64_t gg, Vec (&dst)[NR][MAXCH],
                       float (&sdst)[SR ? NR : 1][SR ? MAXCH : 1]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row_of(gg, r);
      const char* __restrict__ rp = wbase + row * row_bytes;
      const char* __restrict__ up = rp + n * row_bytes;
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) {
        dst[r][c] = *reinterpret_cast<const Vec*>(rp + loff[c]);
        if constexpr (EPI == EPI_SWIGLU) dst[R + r][c] = *reinterpret_cast<const Vec*>(up + loff[c]);
      }
    }
    if constexpr (GROUPED) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row_of(gg, r);
        const float* __restrict__ sp = a.scale + row * ng;
        const float* __restrict__ su = sp + n * ng;
#pragma unroll
        for (int c = 0; c < MAXCH; ++c) {
          sdst[r][c] = sp[lgrp[c]];
          if constexpr (EPI == EPI_SWIGLU) sdst[R + r][c] = su[lgrp[c]];
        }
      }
    }
  };
  // after the row reduction lane l holds row l / GL of the round (reduce_rows); lane r GL takes
  // row r of the group, and lanes that hold no gate row read row 0
  constexpr int GL = kWave / NR;
  const int myrow = lane / GL;
  // epilogue operands of this lane's row in group gg
  auto load_epi = [&](int64_t gg, float& res, float& s1, float& s2) {
    const int64_t row = row_of(gg, myrow < R ? myrow : 0);
    if constexpr (EPI == EPI_RESID) res = a.resid[row];
    if constexpr (WT == W_I8) {
      s1 = a.scale[row];
      if constexpr (EPI == EPI_SWIGLU) s2 = a.scale[row + n];
    }
  };

  // 1. the input (and gamma), the epilogue operands, then the first round's weights.  RMSNorm
  //    prologue: with split 4 each wave loads its own quarter of the input and gamma; with a
  //    smaller split several waves would load the same slice, so the work-group's 256 threads
  //    instead load the input and gamma once between them (thread t the float4s t + 256 i, the
  //    first kNormSlots of them here), and each value crosses a CU's memory pipeline once per
  //    work-group instead of once per wave that uses it (kNormShared)
  constexpr bool shared = NORM == kNormShared;
  float xv[MAXCH][VEC];
  float gv[NORM == kNormWave ? MAXCH : 1][VEC];
  float4 xs[shared ? kNormSlots : 1], gs[shared ? kNormSlots : 1];
  const float4* __restrict__ x4 = static_cast<const float4*>(a.x);
  const float4* __restrict__ g4 = reinterpret_cast<const float4*>(a.gamma);
  if constexpr (shared) {
#pragma unroll
    for (int i = 0; i < kNormSlots; ++i) {
      const int j = tid + kNormThreads * i;
      xs[i] = gs[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * j < K) {
        xs[i] = x4[j];
        gs[i] = g4[j];
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      const int kk = c * CH + lane * VEC;
      const int64_t kc = kbase + (kk < KW ? kk : 0);
      load_vec<XB, VEC>(a.x, kc, xv[c]);
      if constexpr (NORM == kNormWave) load_vec<false, VEC>(a.gamma, kc, gv[c]);
    }
  }
  const int64_t round0 = blockIdx.x;
  const int64_t g = round0 * gpw + grp;
  float ep_res = 0.f, ep_s1 = 1.f, ep_s2 = 1.f;
  load_epi(g, ep_res, ep_s1, ep_s2);
  Vec wv[NR][MAXCH];
  float wsc[SR ? NR : 1][SR ? MAXCH : 1];
  load_rows(g, wv, wsc);

  // 2. the input while the weights arrive.  RMSNorm: the sum of squares over the whole row (one
  //    block reduction; work-group 0 also copies the raw input out) and x * gamma / rms.  Shared
  //    prologue: x * gamma goes through LDS, from which each wave reads its slice back; inputs
  //    longer than kNormSlots float4s per thread take further passes, after the weights were
  //    requested.
  if constexpr (NORM) {
    extern __shared__ float4 s_xg[];  // [K / 4], shared prologue only
    const bool copy_out = a.hidden_copy != nullptr && blockIdx.x == 0;
    const bool rh = a.round_h != 0;
    float ss = 0.f;
    if constexpr (shared) {
      auto stage = [&](int j, const float4 xx, const float4 gg) {
        ss = fmaf(xx.x, xx.x, ss);
        ss = fmaf(xx.y, xx.y, ss);
        ss = fmaf(xx.z, xx.z, ss);
        ss = fmaf(xx.w, xx.w, ss);
        s_xg[j] = make_float4(xx.x * gg.x, xx.y * gg.y, xx.z * gg.z, xx.w * gg.w);
        if (copy_out) reinterpret_cast<float4*>(a.hidden_copy)[j] = xx;
      };
#pragma unroll
      for (int i = 0; i < kNormSlots; ++i) {
        const int j = tid + kNormThreads * i;
        if (4 * j < K) stage(j, xs[i], gs[i]);
      }
      for (int j = tid + kNormThreads * kNormSlots; 4 * j < K; j += kNormThreads)
        stage(j, x4[j], g4[j]);
    } else {
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) {
        const int kk = c * CH + lane * VEC;
        if (kk < KW) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) ss = fmaf(xv[c][e], xv[c][e], ss);
          if (copy_out && grp == 0) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              *reinterpret_cast<float4*>(a.hidden_copy + kbase + kk + e) =
                  make_float4(xv[c][e], xv[c][e + 1], xv[c][e + 2], xv[c][e + 3]);
          }
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red_ss[wave] = ss;
    __syncthreads();
    // split 4: the four waves' slices make up the row; shared: the four waves' shares of the
    // work-group's loads do
    ss = (red_ss[0] + red_ss[1]) + (red_ss[2] + red_ss[3]);
    const float rinv = __builtin_amdgcn_rsqf(ss / (float)K + a.eps);  // v_rsq_f32, 1 ulp
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      const int kk = c * CH + lane * VEC;
      const int kc = kbase + (kk < KW ? kk : 0);
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        float4 t;
        if constexpr (shared) {
          t = s_xg[(kc + e) / 4];
        } else {
          t = make_float4(xv[c][e] * gv[c][e], xv[c][e + 1] * gv[c][e + 1],
                          xv[c][e + 2] * gv[c][e + 2], xv[c][e + 3] * gv[c][e + 3]);
        }
        const float v4[4] = {t.x * rinv, t.y * rinv, t.z * rinv, t.w * rinv};
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[c][e + q] = rh ? round_bf16(v4[q]) : v4[q];
      }
    }
  }
  // chunks past the slice contribute nothing
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    const int kk = c * CH + lane * VEC;
    if (kk >= KW) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) xv[c][e] = 0.f;
    }
  }

  // int8 / int4 read unsigned: each sum over the lane's elements exceeds the true one by
  // BIAS * sum(x), per row (per-row int8) or per vector (grouped types, whose scale is applied
  // per vector); the correction is the same for every row
  float x_corr = 0.f;
  float xc[SR ? MAXCH : 1];
  if constexpr (WT == W_I8) {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) x_corr += xv[c][e];
    x_corr *= -128.f;
  }
  if constexpr (GROUPED) {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) t += xv[c][e];
      xc[c] = t * -(float)WTraits<WT>::BIAS;
      if constexpr (WT == W_I4G) xc[c] *= 0x1p-24f;  // the units of dot16's int4 sums
    }
  }
  if constexpr (WT == W_I4G) {  // odd elements meet their nibble times 16 (dot16)
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
#pragma unroll
      for (int e = 1; e < VEC; e += 2) xv[c][e] *= 0.0625f;
  }

  float best_v = -INFINITY;
  int best_i = -1;
  const bool want_argmax = a.part_val != nullptr;

  // 3. rounds.  A round computes the rows of group g from the weights `cw` (with the epilogue
  //    operands c_*) and, when the launch has several rounds (PIPE), first requests the next
  //    round's rows into `nw` -- the last round requests its own rows again (cached), so that no
  //    load sits under a branch.  Two register sets alternate between rounds: copying registers
  //    of an in-flight load would make the compiler wait for it.
  using Scl = float[SR ? NR : 1][SR ? MAXCH : 1];
  auto do_round = [&](const Vec (&cw)[NR][MAXCH], const Scl& cs, float c_res, float c_s1,
                      float c_s2, Vec (&nw)[NR][MAXCH], Scl& ns, float& n_res, float& n_s1,
                      float& n_s2, int64_t rnd) {
    const int64_t gg = rnd * gpw + grp;
    if constexpr (PIPE) {
      const int64_t gn = (rnd + gridDim.x) * gpw + grp;
      const int64_t gl = gn < ngroups ? gn : gg;
      load_epi(gl, n_res, n_s1, n_s2);
      load_rows(gl, nw, ns);
    }
    const bool active = gg < ngroups;
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = x_corr;
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if constexpr (GROUPED)
          acc[r] = fmaf(cs[r][c], dot16<WT>(cw[r][c], xv[c], xc[c]), acc[r]);
        else  // a sum per vector, added to the row's: independent chains for the FMA pipeline
          acc[r] += dot16<WT>(cw[r][c], xv[c], 0.f);
      }
    if constexpr (WT == W_I4G) {  // dot16's int4 sums carry a factor 2^-24: exact to undo
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] *= 0x1p24f;
    }
    float mine = reduce_rows<NR>(acc);  // this lane: the total of row myrow of the round
    if (split > 1) {
      if (lane % GL == 0) red_acc[wave][myrow] = mine;
      __syncthreads();
      float t = 0.f;
      for (int s2 = 0; s2 < split; ++s2) t += red_acc[grp * split + s2][myrow];
      mine = t;
      // red_acc is reused by the work-group's next round, if it has one (uniform: every wave of
      // the work-group runs the same rounds)
      if ((rnd + gridDim.x) * gpw < ngroups) __syncthreads();
    }
    // lane r GL takes row r of the group; for SWIGLU the up row R + r is 32 lanes further on
    float vg = mine, vu = 0.f;
    if constexpr (EPI == EPI_SWIGLU) {
      float lo, hi;
      lane_pair<32>(mine, lo, hi);
      vg = lo;
      vu = hi;
    }
    const int64_t row = gg * R + myrow;
    if (active && sub == 0 && lane % GL == 0 && myrow < R && row < n) {
      float v = vg;
      if constexpr (WT == W_I8) v *= c_s1;
      if constexpr (EPI == EPI_SWIGLU) {
        const float u = (WT == W_I8) ? vu * c_s2 : vu;
        v = v / (1.0f + expf(-v)) * u;
      }
      if constexpr (EPI == EPI_RESID) {
        a.resid[row] = c_res + v;
      } else {
        if (a.y_bf16)
          static_cast<uint16_t*>(a.y)[row] = f32_to_bf16(v);
        else
          static_cast<float*>(a.y)[row] = v;
        if constexpr (EPI == EPI_STORE) {
          if (want_argmax) {
            const float rv = a.y_bf16 ? round_bf16(v) : v;
            if (rv == rv && (best_i < 0 || rv > best_v)) {  // rows rise with the rounds
              best_v = rv;
              best_i = (int)row;
            }
          }
        }
      }
    }
  };
  if constexpr (PIPE) {
    Vec wb[NR][MAXCH];
    Scl wscb;
    float rb = 0.f, s1b = 1.f, s2b = 1.f;
    for (int64_t rnd = round0;;) {
      do_round(wv, wsc, ep_res, ep_s1, ep_s2, wb, wscb, rb, s1b, s2b, rnd);
      rnd += gridDim.x;
      if (rnd * gpw >= ngroups) break;
      do_round(wb, wscb, rb, s1b, s2b, wv, wsc, ep_res, ep_s1, ep_s2, rnd);
      rnd += gridDim.x;
      if (rnd * gpw >= ngroups) break;
    }
  } else {
    // rounds without lookahead (usually one: the grid covers every group)
    float d0, d1, d2;
    do_round(wv, wsc, ep_res, ep_s1, ep_s2, wv, wsc, d0, d1, d2, round0);
    for (int64_t rnd = round0 + gridDim.x; rnd * gpw < ngroups; rnd += gridDim.x) {
      const int64_t gg = rnd * gpw + grp;
      load_epi(gg, ep_res, ep_s1, ep_s2);
      load_rows(gg, wv, wsc);
      do_round(wv, wsc, ep_res, ep_s1, ep_s2, wv, wsc, d0, d1, d2, rnd);
    }
  }

  if constexpr (EPI == EPI_STORE) {
    if (want_argmax) {  // a kernel argument: uniform over the work-group
      // (max, lowest index) over the lanes of the wave, then over the waves
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float ov = __shfl_xor(best_v, off);
        const int oi = __shfl_xor(best_i, off);
        if (argmax_better(ov, oi, best_v, best_i)) {
          best_v = ov;
          best_i = oi;
        }
      }
      if (lane == 0) {
        red_bv[wave] = best_v;
        red_bi[wave] = best_i;
      }
      __syncthreads();
      if (tid == 0) {
        float bv = red_bv[0];
        int bi = red_bi[0];
        for (int w = 1; w < 4; ++w)
          if (argmax_better(red_bv[w], red_bi[w], bv, bi)) {
            bv = red_bv[w];
            bi = red_bi[w];
          }
        a.part_val[blockIdx.x] = bv;
        a.part_idx[blockIdx.x] = bi;
      }
    }
  }
}

// ---- launch planning ------------------------------------------------------------------------------

// How a projection of n output rows and input length k is launched:
//   split: K is split over 4, 2 or 1 waves of a work-group: the largest split that leaves every
//          wave at least two wave-wide loads per row (and whole 16-byte vectors).  Each wave
//          reads its slice of x (and gamma) from L1/L2 into registers, so the input traffic per
//          weight byte is 1 / (R * rows per pair) whatever the split, and a larger split lets R
//          grow within the register budget;
//   R:     rows per wave, the largest of 4, 2, 1 that keeps at most 16 loads per lane in flight
//          (8 when the next round is prefetched) and at least 2048 waves in the grid (measured:
//          the small projections of a 0.6B-class step ran 4% faster per step than at 1024);
//          int4 lanes load 8 bytes, so their budgets double (larger int4 matrices: below);
//   wgs:   enough work-groups for one round, up to 4096; beyond that 1024 work-groups (4096
//          waves, all resident) each run several rounds with the next one requested ahead
//          (PIPE), R re-chosen for two sets of 8 loads; matrices above 64 MiB are streamed by
//          512 work-groups instead (below).
struct GemvPlan {
  int split, maxch, r;
  bool pipe;  // several rounds per work-group, the next round's rows requested ahead
  unsigned wgs;
  bool ok;    // every slice fits in 8 wave-wide chunks (the register-resident input)
};

// A single-round launch takes up to kMaxOneRoundWgs work-groups (the hardware schedules those
// beyond the resident ones as others finish); larger matrices (the LM head) run kPipeWgs
// work-groups of several rounds each, every round requesting the next one's rows ahead.
constexpr int64_t kMinWaves = 2048;  // R shrinks until the grid has this many waves
constexpr int64_t kMaxOneRoundWgs = 4096;
constexpr int64_t kPipeWgs = 1024;
// Matrices above kStreamBytes are streamed by kStreamWgs work-groups (two per CU) looping over
// row groups, each round requesting its rows and waiting for them: about 16 MiB in flight,
// which a read-bandwidth probe on MI355X found fastest (more outstanding requests lowered the
// rate); measured 6.2 TB/s on a 1.2 GB LM head against 5.7 with 1024 prefetching work-groups.
constexpr int64_t kStreamBytes = int64_t(64) << 20;
constexpr int64_t kStreamWgs = 512;
constexpr bool kStreamPipe = false;
constexpr int kStreamLoads = 8;
constexpr int64_t kStreamInFlight = int64_t(16) << 20;
constexpr int64_t kI4Bytes = int64_t(4) << 20;  // int4 matrices above this take their own plan

static GemvPlan plan_gemv(int wtype, int epi, int64_t n, int64_t k) {
  const int vec = wtype == W_F32 ? 4 : wtype == W_BF16 ? 8 : 16;
  const int bits = wtype == W_F32 ? 32 : wtype == W_BF16 ? 16 : wtype == W_I4G ? 4 : 8;
  const bool grouped = wtype == W_I8G || wtype == W_I4G;
  // load budgets below count 16-byte lane loads; int4 lanes load 8 bytes, so twice as many fit
  const int lmul = wtype == W_I4G ? 2 : 1;
  const int64_t ch = 64 * vec;
  const int pairs = epi == EPI_SWIGLU ? 2 : 1;
  auto chunks = [&](int s) { return (int)((k / s + ch - 1) / ch); };
  auto fits = [&](int s) { return k % ((int64_t)s * vec) == 0; };
  int split = 1;
  for (int s : {4, 2})
    if (fits(s) && k / s >= 2 * ch) {
      split = s;
      break;
    }
  // a slice longer than 8 chunks does not fit in registers: split further when possible
  while (chunks(split) > 8 && split < 4 && fits(split * 2)) split *= 2;
  GemvPlan p{};
  p.split = split;
  const int c = chunks(split);
  p.ok = c <= 8 && k % vec == 0 && (!grouped || k % kQGroup == 0);
  p.maxch = c <= 4 ? (c <= 1 ? 1 : c) : c <= 6 ? 6 : 8;
  const int gpw = 4 / split;
  // loads per lane in flight: 16, or 8 per set when the next round is requested ahead
  auto pick_r = [&](int budget) {
    budget *= lmul;
    for (int cand : {4, 2})
      if (cand * pairs * p.maxch <= budget && ((n + cand - 1) / cand) * split >= kMinWaves)
        return cand;
    return 1;
  };
  const int64_t wbytes = n * pairs * k * bits / 8;
  int64_t wgs;
  if (wbytes > kStreamBytes) {
    p.r = pick_r(kStreamLoads);
    // fewer than kStreamLoads loads per round (short int8 rows): request the next round ahead
    // so that a wave still keeps about that many in flight
    p.pipe = kStreamPipe || p.r * pairs * p.maxch < kStreamLoads * lmul;
    // a streamed bf16 gate-up pair: one row pair per wave with the next round requested ahead
    // (measured on the 8B-class gate-up, 24576 x 4096: 34.8 against 36.4 us for two pairs per
    // wave without lookahead; the single-row LM head is faster without it, 205 against 229 us)
    if (wtype == W_BF16 && pairs == 2) {
      p.r = 1;
      p.pipe = true;
    }
    wgs = ((n + p.r - 1) / p.r + gpw - 1) / gpw;
    int64_t cap = kStreamWgs;
    if (wtype == W_I8) {
      // per-row int8: enough work-groups for about kStreamInFlight bytes of rows in flight (a
      // work-group round reads gpw row groups of R rows, two rounds with lookahead).  Measured
      // on 130560 x 1536 (no lookahead): 512 work-groups (12 MiB) 37.3 us, 768 34.3 us, 1024
      // 35.5 us; 151936 x 1024 (lookahead, 16 MiB at 512) is fastest at 512
      const int64_t per_wg = (int64_t)gpw * p.r * pairs * (k * bits / 8) * (p.pipe ? 2 : 1);
      cap = (kStreamInFlight / per_wg + 128) / 256 * 256;
      cap = cap < kStreamWgs ? kStreamWgs : cap > 2 * kStreamWgs ? 2 * kStreamWgs : cap;
    }
    if (wgs > cap) wgs = cap;
  } else {
    p.r = pick_r(16);
    wgs = ((n + p.r - 1) / p.r + gpw - 1) / gpw;
    p.pipe = wgs > kMaxOneRoundWgs;
    if (p.pipe) {
      p.r = pick_r(8);
      wgs = ((n + p.r - 1) / p.r + gpw - 1) / gpw;
      if (wgs > kPipeWgs) wgs = kPipeWgs;
    }
  }
  if (wtype == W_I4G && wbytes > kI4Bytes) {
    // int4 spends about as long converting codes as the bytes take to arrive, so it needs more
    // waves per SIMD to overlap the two: 2 (4 above 64 MiB) rows per wave, up to 1024 (2048)
    // work-groups, the next round requested ahead when there are several (measured on MI355X
    // over R = 2/4/8, 512-4096 work-groups and both round modes for six matrix shapes)
    const bool big = wbytes > kStreamBytes;
    const int64_t cap = big ? 2048 : 1024;
    // four rows per wave when that covers every row in a single round of at most 2048
    // work-groups (no lookahead, no second round).  Measured on MI355X in the 8B-class w4a16 step
    // (fp32 inputs): QKV 6144 x 4096 7.5 -> 6.7 us, O 4096 x 4096 5.3 -> 4.8, down 4096 x 12288
    // 10.6 -> 9.3, the step 1.87 -> 1.77 ms; where four rows still take several rounds it measured
    // slower (24576 x 4096 STORE: 14.1 -> 16.0 us), so the rule below applies there
    const int64_t need4 = ((n + 3) / 4 + gpw - 1) / gpw;
    if (!big && need4 <= 2048 && 4 * pairs * p.maxch <= 16 * lmul) {
      p.r = 4;
      wgs = need4;
      p.pipe = false;
    } else {
      // wave slices of three or more 1024-value chunks (over 2048 values, e.g. K = 12288 split
      // four ways): one row per wave, the next round requested ahead (measured 8.8 against 9.5
      // us at 4096 x 12288)
      for (p.r = p.maxch >= 3 ? 1 : big ? 4 : 2;; p.r /= 2) {  // fewer when over the budget
        const int64_t need = ((n + p.r - 1) / p.r + gpw - 1) / gpw;
        wgs = need < cap ? need : cap;
        p.pipe = need > wgs;
        if (p.r == 1 || p.r * pairs * p.maxch <= (p.pipe ? 8 : 16) * lmul) break;
      }
    }
  }
  p.wgs = (unsigned)(wgs < 1 ? 1 : wgs);
  return p;
}

template <int WT, int EPI, int NORM, bool XB, int R, int MAXCH, bool PIPE>
static hipError_t go(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  constexpr int loads = (EPI == EPI_SWIGLU ? 2 : 1) * R * MAXCH;
  constexpr int lmul = WT == W_I4G ? 2 : 1;
  if constexpr (loads > (PIPE ? 8 : 16) * lmul) {
    return hipErrorInvalidConfiguration;  // never planned: over the register budget
  } else {
    const unsigned lds = NORM == kNormShared ? (unsigned)(a.k * 4) : 0u;  // x * gamma
    hipLaunchKernelGGL((k_gemv<WT, EPI, NORM, XB, R, MAXCH, PIPE>), dim3(p.wgs), dim3(256), lds, s,
                       a);
    return hipGetLastError();
  }
}

template <int WT, int EPI, int NORM, bool XB, int R, int MAXCH>
static hipError_t go_p(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  return p.pipe ? go<WT, EPI, NORM, XB, R, MAXCH, true>(a, p, s)
                : go<WT, EPI, NORM, XB, R, MAXCH, false>(a, p, s);
}

template <int WT, int EPI, int NORM, bool XB, int R>
static hipError_t go_ch(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (p.maxch) {
    case 1: return go_p<WT, EPI, NORM, XB, R, 1>(a, p, s);
    case 2: return go_p<WT, EPI, NORM, XB, R, 2>(a, p, s);
    case 3: return go_p<WT, EPI, NORM, XB, R, 3>(a, p, s);
    case 4: return go_p<WT, EPI, NORM, XB, R, 4>(a, p, s);
    case 6: return go_p<WT, EPI, NORM, XB, R, 6>(a, p, s);
    default: return go_p<WT, EPI, NORM, XB, R, 8>(a, p, s);
  }
}

template <int WT, int EPI, int NORM, bool XB>
static hipError_t go_r(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (p.r) {
    case 4: return go_ch<WT, EPI, NORM, XB, 4>(a, p, s);
    case 2: return go_ch<WT, EPI, NORM, XB, 2>(a, p, s);
    default: return go_ch<WT, EPI, NORM, XB, 1>(a, p, s);
  }
}

// k_gemv_i4mf: W4A16 GEMV (int4 codes in 128-value groups, bf16 input) with the dot products
// on v_mfma_f32_16x16x32_bf16, for plain STORE launches with k a multiple of 256, at most 2048
// (a wave keeps its rows' codes in registers).  The per-element VALU work of k_gemv
// (about 1.6 instructions: nibble masks and mixed-precision fmas) becomes about 1: a nibble u
// placed in the top four mantissa bits under the bf16 pattern of 1.0 is exactly 1 + u / 16, so a
// shift and an AND-OR turn two codes into a bf16 pair; the stored nibble is the code q plus 8, so
// the products sum to 1.5 sum(x) + sum(q x) / 16 and the group's result is 16 (C - 1.5 sum(x))
// (exact products, fp32 sums).  The offset is kept small on purpose: with the code in the low
// mantissa bits (128 + u) the fp32 sums carried 136 sum(x) and lost about 1e-6 of the result.
//   - A wave takes 16 consecutive rows: lane l loads 16 bytes of row l % 16 at byte 16 (l / 16)
//     + 64 s for group s, i.e. 32 codes k = 128 s + 32 (l / 16) .. +31, as four words.  Word i of
//     every lane forms the B operand of one MFMA (B[k][col] = code of row col at the lane's 8 k),
//     the A operand is x at the same k from LDS (every column of the product is then W x; lane l
//     keeps row l % 16's value), and the four MFMAs of group s cover exactly its 128 values.
//   - A word's nibbles come out of the masks in the order 0 4 1 5 2 6 3 7, so x is staged in LDS
//     permuted the same way within each 8 values; the group sums of x come from wave reductions.
//   - Codes and scales are requested before x is staged.
// Measured on MI355X: 130560 x 1536 (cold weights) 21.0-22.3 us, 0.64 of HBM peak, against
// 27.8 us on k_gemv.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// nibble word (elements e at bits 4e) -> bf16 1 + u / 16 in the order e0 e4 e1 e5 e2 e6 e3 e7
__device__ __forceinline__ u32x4_t nib_bf16x8(uint32_t w) {
  u32x4_t r;
  r[0] = ((w << 3) & 0x00780078u) | 0x3F803F80u;
  r[1] = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
  r[2] = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
  r[3] = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
  return r;
}

// Up to k = 1024 the kernel is built for 8 waves per SIMD (it fits in 64 registers without spilling;
// measured on MI355X, 151936 x 1024: 17.0 against 18.2 us without the occupancy target); longer
// rows keep the default, since capping them spills (130560 x 1536: 24.8 against 21.9 us)
template <int K>
constexpr int i4mf_waves_per_simd() { return K <= 1024 ? 8 : 1; }
template <int K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(i4mf_waves_per_simd<K>())))
void k_gemv_i4mf(GemvArgs a) {
  constexpr int NG = K / 128, XPT = K / 256;
  static_assert(K % 256 == 0 && K <= 2048, "k");
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint16_t sx[K];
  __shared__ float sbp[4][XPT];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t n = a.n;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  const int64_t row = min(r0 + c, n - 1);     // rows past the end read the last row (discarded)
  const uint8_t* rp = static_cast<const uint8_t*>(a.w) + row * (K / 2) + 16 * g;
  u32x4_t wv[NG];
#pragma unroll
  for (int s = 0; s < NG; ++s) wv[s] = *reinterpret_cast<const u32x4_t*>(rp + 64 * s);
  float sc[NG];   // the row's NG scales are contiguous (NG even): 8-byte loads
#pragma unroll
  for (int s = 0; s < NG; s += 2) {
    const float2 v = *reinterpret_cast<const float2*>(a.scale + row * NG + s);
    sc[s] = v.x;
    sc[s + 1] = v.y;
  }
  // x: thread t takes elements t + 256 j (group 2 j + t / 128)
  const uint16_t* xh = static_cast<const uint16_t*>(a.x);
  float xs[XPT];
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const int i = t + 256 * j;
    const uint16_t v = xh[i];
    xs[j] = bf16_to_f32(v);
    const int e = i & 7;
    sx[(i & ~7) + (e < 4 ? 2 * e : 2 * (e - 4) + 1)] = v;
  }
#pragma unroll
  for (int j = 0; j < XPT; ++j) {
    const float v = wave_sum(xs[j]);
    if (lane == 0) sbp[wave][j] = v;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < NG; ++s) {
    const int j = s >> 1, hf = s & 1;          // group s: elements of waves 2 hf, 2 hf + 1
    const float bias = 1.5f * (sbp[2 * hf][j] + sbp[2 * hf + 1][j]);
    f32x4_t cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8_t xa = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(&sx[128 * s + 32 * g + 8 * i]));
      const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, nib_bf16x8(wv[s][i]));
      cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, cs, 0, 0, 0);
    }
    acc = fmaf(16.f * sc[s], cs[0] - bias, acc);
  }
  if (g == 0 && r0 + c < n) {
    if (a.y_bf16)
      static_cast<uint16_t*>(a.y)[r0 + c] = f32_to_bf16(acc);
    else
      static_cast<float*>(a.y)[r0 + c] = acc;
  }
}

static hipError_t go_i4mf(const GemvArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.n + 63) / 64));
  switch (a.k) {
    case 256: hipLaunchKernelGGL((k_gemv_i4mf<256>), grid, dim3(256), 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_gemv_i4mf<512>), grid, dim3(256), 0, s, a); break;
    case 768: hipLaunchKernelGGL((k_gemv_i4mf<768>), grid, dim3(256), 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_gemv_i4mf<1024>), grid, dim3(256), 0, s, a); break;
    case 1280: hipLaunchKernelGGL((k_gemv_i4mf<1280>), grid, dim3(256), 0, s, a); break;
    case 1536: hipLaunchKernelGGL((k_gemv_i4mf<1536>), grid, dim3(256), 0, s, a); break;
    case 1792: hipLaunchKernelGGL((k_gemv_i4mf<1792>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemv_i4mf<2048>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

// Launches the matrix-core W4A16 kernel serves: STORE, bf16 input, no norm prologue, no argmax
// partials or input copy, k a multiple of 256 up to 2048, and enough rows to fill the chip.
static bool i4mf_serves(int epi, bool norm, const GemvArgs& a) {
  return epi == EPI_STORE && !norm && a.x_bf16 && a.part_val == nullptr &&
         a.hidden_copy == nullptr && a.k % 256 == 0 && a.k <= 2048 && a.n >= 4096;
}

// This file is compiled once per weight type (QD_GEMV_PART = W_F32 .. W_I4G: the kernels of
// that type) and once with QD_GEMV_PART = -1 (the dispatcher), so that the builds run in
// parallel.
template <int WT>
hipError_t launch_wt(int epi, bool norm, GemvArgs a, hipStream_t s);

#if QD_GEMV_PART >= 0
// The norm prologue reads the fp32 residual stream; other inputs are fp32 or bf16.
template <int WT>
hipError_t launch_wt(int epi, bool norm, GemvArgs a, hipStream_t s) {
  if constexpr (WT == W_I4G) {
    if (i4mf_serves(epi, norm, a)) return go_i4mf(a, s);
  }
  const GemvPlan p = plan_gemv(WT, epi, a.n, a.k);
  if (!p.ok || (norm && a.k > kGemvNormMaxK)) return hipErrorInvalidValue;
  // every work-group writes the argmax partial of its index: never past the buffer's end
  if (a.part_val && (int64_t)p.wgs > (int64_t)a.part_cap) return hipErrorInvalidValue;
  a.split = p.split;
  const bool xb = a.x_bf16 != 0;
  if (norm && xb) return hipErrorInvalidValue;
  const bool sh = p.split < 4;  // norm: waves would share input slices
  if (epi == EPI_STORE) {
    if (norm)
      return sh ? go_r<WT, EPI_STORE, kNormShared, false>(a, p, s)
                : go_r<WT, EPI_STORE, kNormWave, false>(a, p, s);
    return xb ? go_r<WT, EPI_STORE, kNormNone, true>(a, p, s)
              : go_r<WT, EPI_STORE, kNormNone, false>(a, p, s);
  }
  if (epi == EPI_RESID)
    return xb ? go_r<WT, EPI_RESID, kNormNone, true>(a, p, s)
              : go_r<WT, EPI_RESID, kNormNone, false>(a, p, s);
  if (!norm) return hipErrorInvalidValue;
  return sh ? go_r<WT, EPI_SWIGLU, kNormShared, false>(a, p, s)
            : go_r<WT, EPI_SWIGLU, kNormWave, false>(a, p, s);
}
template hipError_t launch_wt<QD_GEMV_PART>(int, bool, GemvArgs, hipStream_t);
#else
hipError_t launch_gemv(int wtype, int epi, bool norm, const GemvArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  switch (wtype) {
    case W_F32: return launch_wt<W_F32>(epi, norm, a, s);
    case W_BF16: return launch_wt<W_BF16>(epi, norm, a, s);
    case W_I8: return launch_wt<W_I8>(epi, norm, a, s);
    case W_I8G: return launch_wt<W_I8G>(epi, norm, a, s);
    case W_I4G: return launch_wt<W_I4G>(epi, norm, a, s);
    default: return hipErrorInvalidValue;
  }
}

int gemv_partials(int wtype, int epi, int64_t n, int64_t k) {
  return (int)plan_gemv(wtype, epi, n, k).wgs;
}

bool gemv_supported(int wtype, int epi, int64_t n, int64_t k) {
  return n >= 1 && k >= 1 && plan_gemv(wtype, epi, n, k).ok;
}
#endif

}  // namespace qd

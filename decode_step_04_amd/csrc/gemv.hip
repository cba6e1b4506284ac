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
//   1. Every wave first issues the 16-byte loads of its rows' K-slice for the first round (lane l
//      reads elements kslice + c*64*VEC + l*VEC .. +VEC of each row: one wave-wide load is a
//      contiguous 1 KiB of a row), so HBM latency overlaps everything below.
//   2. The work-group stages the input vector once in LDS (x * gamma when the RMSNorm prologue of
//      [Qwen3-runtime] §2.1 is fused, with the sum of squares reduced on the way).  The LDS layout
//      is interleaved per wave slice so that each lane's later 16-byte LDS reads are consecutive
//      across the wave.
//   3. Each wave copies its slice into registers (times rsqrt(mean + eps), rounded to bf16 when
//      activations are 16-bit).
//   4. Rounds: FMAs over the registers, a DPP + readlane reduction per row, a reduction over the
//      SPLIT waves through LDS, and the epilogue: store (fp32 / bf16), residual add into the fp32
//      stream, or silu(gate) * up.  With several rounds per work-group (the LM head), the next
//      round's rows are requested before the current one is reduced, and the work-group keeps
//      the running (max, lowest index) of its rounded outputs for the greedy argmax.
#include "common.h"
#include "launch.h"

namespace qd {

template <int WT>
struct WTraits;
template <>
struct WTraits<W_F32> {
  static constexpr int VEC = 4;
  static constexpr int ELEM = 4;
};
template <>
struct WTraits<W_BF16> {
  static constexpr int VEC = 8;
  static constexpr int ELEM = 2;
};
template <>
struct WTraits<W_I8> {
  static constexpr int VEC = 16;
  static constexpr int ELEM = 1;
};

__device__ __forceinline__ float i8_at(uint32_t w, int b) {
  return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * b));
}

// acc + sum over the VEC elements of one 16-byte weight vector times VEC fp32 values.
template <int WT>
__device__ __forceinline__ float dot16(uint4 w, const float* __restrict__ x, float acc) {
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
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(i8_at(ws[j], 0), x[4 * j + 0], acc);
      acc = fmaf(i8_at(ws[j], 1), x[4 * j + 1], acc);
      acc = fmaf(i8_at(ws[j], 2), x[4 * j + 2], acc);
      acc = fmaf(i8_at(ws[j], 3), x[4 * j + 3], acc);
    }
  }
  return acc;
}

// 4 consecutive input values starting at element k (fp32 or bf16 source), k % 4 == 0.
__device__ __forceinline__ float4 load4(const void* x, int x_bf16, int64_t k) {
  if (x_bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + k);
    return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + k);
}

__device__ __forceinline__ bool argmax_better(float vb, int ib, float va, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return vb > va || (vb == va && ib < ia);
}

template <int WT, int EPI, bool NORM, int R, int MAXCH, bool PIPE>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  constexpr int VEC = WTraits<WT>::VEC;
  constexpr int ELEM = WTraits<WT>::ELEM;
  constexpr int CH = kWave * VEC;                  // elements per wave-wide load
  constexpr int NP = VEC / 4;                      // float4 pieces per lane per chunk
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  extern __shared__ float4 xs4[];                  // interleaved input, see below
  __shared__ float red_ss[4];
  __shared__ float red_acc[4][NR];
  __shared__ float red_bv[4];
  __shared__ int red_bi[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = a.split;
  const int gpw = 4 / split;                       // row groups per work-group round
  const int sub = wave % split;                    // K-slice of this wave
  const int grp = wave / split;                    // row group of this wave within the round
  const int K = (int)a.k;
  const int KW = K / split;                        // elements per slice
  const int kbase = sub * KW;
  const int slice_f4 = ((KW + CH - 1) / CH) * CH / 4;  // LDS float4s per slice (whole chunks)
  const int64_t n = a.n;
  const int64_t ngroups = (n + R - 1) / R;
  const char* __restrict__ wbase = static_cast<const char*>(a.w);
  const int64_t row_bytes = (int64_t)K * ELEM;

  auto row_of = [&](int64_t gg, int r) -> int64_t {
    const int64_t row = gg * R + r;
    return row < n ? row : n - 1;  // clamp: loads stay in bounds, results are discarded
  };
  auto load_rows = [&](int64_t gg, uint4 (&dst)[NR][MAXCH]) {
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      const int kk = c * CH + lane * VEC;
      if (kk < KW) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t row = row_of(gg, r);
          dst[r][c] = *reinterpret_cast<const uint4*>(wbase + row * row_bytes +
                                                      (int64_t)(kbase + kk) * ELEM);
          if constexpr (EPI == EPI_SWIGLU)
            dst[R + r][c] = *reinterpret_cast<const uint4*>(wbase + (row + n) * row_bytes +
                                                            (int64_t)(kbase + kk) * ELEM);
        }
      }
    }
  };

  // 1. first round's weights
  const int64_t round0 = blockIdx.x;
  int64_t g = round0 * gpw + grp;
  uint4 wv[NR][MAXCH];
  if (g < ngroups) load_rows(g, wv);

  // 2. stage the input (x * gamma with the norm prologue) once per work-group.  Element k of
  //    slice s, chunk c, lane l, piece j (k = s*KW + c*CH + l*VEC + 4j + t) lives in float4
  //    s*slice_f4 + (c*NP + j)*64 + l, component t.
  float ss = 0.f;
  for (int q4 = tid; q4 < K / 4; q4 += 256) {
    const int k = q4 * 4;
    float4 v = load4(a.x, a.x_bf16, k);
    if constexpr (NORM) {
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
      if (a.hidden_copy != nullptr && blockIdx.x == 0)
        *reinterpret_cast<float4*>(a.hidden_copy + k) = v;
      const float4 gm = *reinterpret_cast<const float4*>(a.gamma + k);
      v.x *= gm.x; v.y *= gm.y; v.z *= gm.z; v.w *= gm.w;
    }
    const int s = k / KW, rem = k - s * KW;
    const int c = rem / CH, r2 = rem - c * CH;
    const int l = r2 / VEC, j = (r2 - l * VEC) / 4;
    xs4[s * slice_f4 + (c * NP + j) * kWave + l] = v;
  }
  float rinv = 1.f;
  if constexpr (NORM) {
    ss = wave_sum(ss);
    if (lane == 0) red_ss[wave] = ss;
  }
  __syncthreads();
  if constexpr (NORM) {
    const float tot = (red_ss[0] + red_ss[1]) + (red_ss[2] + red_ss[3]);
    rinv = 1.0f / sqrtf(tot / (float)K + a.eps);
  }

  // 3. this wave's slice into registers
  float xv[MAXCH][VEC];
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    const int kk = c * CH + lane * VEC;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (kk < KW) v = xs4[sub * slice_f4 + (c * NP + j) * kWave + lane];
      if constexpr (NORM) {
        v.x *= rinv; v.y *= rinv; v.z *= rinv; v.w *= rinv;
        if (a.round_h) {
          v.x = round_bf16(v.x); v.y = round_bf16(v.y);
          v.z = round_bf16(v.z); v.w = round_bf16(v.w);
        }
      }
      xv[c][4 * j + 0] = v.x; xv[c][4 * j + 1] = v.y;
      xv[c][4 * j + 2] = v.z; xv[c][4 * j + 3] = v.w;
    }
  }

  float best_v = -INFINITY;
  int best_i = -1;
  const bool want_argmax = a.part_val != nullptr;

  // 4. rounds
  for (int64_t rnd = round0; rnd * gpw < ngroups; rnd += gridDim.x) {
    g = rnd * gpw + grp;
    const bool active = g < ngroups;
    uint4 wn[NR][MAXCH];
    if constexpr (PIPE) {
      const int64_t gn = (rnd + gridDim.x) * gpw + grp;
      if (gn < ngroups) load_rows(gn, wn);
    }
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
    if (active) {
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) {
        const int kk = c * CH + lane * VEC;
        if (kk < KW) {
#pragma unroll
          for (int r = 0; r < NR; ++r) acc[r] = dot16<WT>(wv[r][c], xv[c], acc[r]);
        }
      }
    }
    float tot[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) tot[r] = wave_sum(acc[r]);
    if (split > 1) {
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < NR; ++r) red_acc[wave][r] = tot[r];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float t = 0.f;
        for (int s2 = 0; s2 < split; ++s2) t += red_acc[grp * split + s2][r];
        tot[r] = t;
      }
      __syncthreads();  // red_acc is reused next round
    }
    if (active && sub == 0) {
      if constexpr (WT == W_I8) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          tot[r] *= a.scale[row_of(g, r)];
          if constexpr (EPI == EPI_SWIGLU) tot[R + r] *= a.scale[row_of(g, r) + n];
        }
      }
      float outv = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float v = tot[r];
        if constexpr (EPI == EPI_SWIGLU) v = tot[r] / (1.0f + expf(-tot[r])) * tot[R + r];
        if (lane == r) outv = v;
        if constexpr (EPI == EPI_STORE) {
          if (want_argmax) {
            const int64_t row = g * R + r;
            const float rv = a.y_bf16 ? round_bf16(v) : v;
            if (row < n && rv == rv && (best_i < 0 || rv > best_v)) {
              best_v = rv;
              best_i = (int)row;
            }
          }
        }
      }
      const int64_t row = g * R + lane;
      if (lane < R && row < n) {
        if constexpr (EPI == EPI_RESID) {
          a.resid[row] += outv;
        } else {
          if (a.y_bf16)
            static_cast<uint16_t*>(a.y)[row] = f32_to_bf16(outv);
          else
            static_cast<float*>(a.y)[row] = outv;
        }
      }
    }
    if constexpr (PIPE) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < MAXCH; ++c) wv[r][c] = wn[r][c];
    }
  }

  if constexpr (EPI == EPI_STORE) {
    if (want_argmax) {  // a kernel argument: uniform over the work-group
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
//   split: K is split over 2 or 4 waves when one wave's slice would need more than 8 wave-wide
//          loads per row (register budget), or when even one row per wave leaves fewer than 1024
//          waves (4 per CU) -- slices stay whole multiples of the 16-byte vector;
//   R:     rows per wave, the largest of 4, 2, 1 that keeps at least 1024 waves and at most 16
//          loads per lane in flight (8 when the next round is prefetched);
//   wgs:   enough work-groups for one round, capped at 1024 for the store epilogue (the LM
//          head), which then runs several rounds with the next one prefetched.
struct GemvPlan {
  int split, maxch, r;
  unsigned wgs;
  size_t lds;
};

static GemvPlan plan_gemv(int wtype, int epi, int64_t n, int64_t k) {
  const int vec = wtype == W_F32 ? 4 : wtype == W_BF16 ? 8 : 16;
  const int64_t ch = 64 * vec;
  const int pairs = epi == EPI_SWIGLU ? 2 : 1;
  int split = 1;
  auto chunks = [&](int s) { return (int)((k / s + ch - 1) / ch); };
  auto can = [&](int s) { return s <= 4 && k % ((int64_t)s * vec) == 0; };
  while (can(split * 2) && chunks(split) > 8) split *= 2;
  while (can(split * 2) && n * split < 1024 && k / (split * 2) >= ch) split *= 2;
  GemvPlan p{};
  p.split = split;
  const int c = chunks(split);
  p.maxch = c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
  // loads per lane in flight: 16, or 8 when the next round is prefetched (two sets of registers)
  const int budget = epi == EPI_STORE ? 8 : 16;
  int r = 1;
  for (int cand : {4, 2}) {
    if (cand * pairs * p.maxch <= budget && ((n + cand - 1) / cand) * split >= 1024) {
      r = cand;
      break;
    }
  }
  p.r = r;
  const int64_t groups = (n + r - 1) / r;
  const int gpw = 4 / split;
  int64_t wgs = (groups + gpw - 1) / gpw;
  if (epi == EPI_STORE && wgs > 1024) wgs = 1024;
  p.wgs = (unsigned)(wgs < 1 ? 1 : wgs);
  const int64_t slice_f4 = ((k / split + ch - 1) / ch) * ch / 4;
  p.lds = (size_t)(split * slice_f4 * 16);
  return p;
}

template <int WT, int EPI, bool NORM, int R, int MAXCH>
static hipError_t go(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  constexpr bool PIPE = EPI == EPI_STORE;
  constexpr int loads = (EPI == EPI_SWIGLU ? 2 : 1) * R * MAXCH;
  if constexpr (loads > (PIPE ? 8 : 16)) {
    return hipErrorInvalidConfiguration;  // never planned: over the register budget
  } else {
    hipLaunchKernelGGL((k_gemv<WT, EPI, NORM, R, MAXCH, PIPE>), dim3(p.wgs), dim3(256), p.lds, s,
                       a);
    return hipGetLastError();
  }
}

template <int WT, int EPI, bool NORM, int R>
static hipError_t go_ch(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (p.maxch) {
    case 1: return go<WT, EPI, NORM, R, 1>(a, p, s);
    case 2: return go<WT, EPI, NORM, R, 2>(a, p, s);
    case 4: return go<WT, EPI, NORM, R, 4>(a, p, s);
    default: return go<WT, EPI, NORM, R, 8>(a, p, s);
  }
}

template <int WT, int EPI, bool NORM>
static hipError_t go_r(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (p.r) {
    case 4: return go_ch<WT, EPI, NORM, 4>(a, p, s);
    case 2: return go_ch<WT, EPI, NORM, 2>(a, p, s);
    default: return go_ch<WT, EPI, NORM, 1>(a, p, s);
  }
}

template <int WT>
static hipError_t launch_wt(int epi, bool norm, GemvArgs a, hipStream_t s) {
  const GemvPlan p = plan_gemv(WT, epi, a.n, a.k);
  a.split = p.split;
  if (epi == EPI_STORE)
    return norm ? go_r<WT, EPI_STORE, true>(a, p, s) : go_r<WT, EPI_STORE, false>(a, p, s);
  if (epi == EPI_RESID) return go_r<WT, EPI_RESID, false>(a, p, s);
  return go_r<WT, EPI_SWIGLU, true>(a, p, s);
}

hipError_t launch_gemv(int wtype, int epi, bool norm, const GemvArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  switch (wtype) {
    case W_F32: return launch_wt<W_F32>(epi, norm, a, s);
    case W_BF16: return launch_wt<W_BF16>(epi, norm, a, s);
    default: return launch_wt<W_I8>(epi, norm, a, s);
  }
}

int gemv_partials(int wtype, int epi, int64_t n, int64_t k) {
  return (int)plan_gemv(wtype, epi, n, k).wgs;
}

}  // namespace qd

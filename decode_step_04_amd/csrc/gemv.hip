// gemv.hip - batch-1 projections y = W x (a GEMV at M = 1) streamed from HBM.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
//
// [Qwen3-runtime] §4.1: at batch 1 every weight is read once and used for one multiply-add, so a
// projection is bound by the weight bytes it streams; §13.1 gives the W8A16 form (int8 weights,
// fp32 accumulation, the scale applied after the integer-weighted sum).  Plain VALU work: no
// MFMA, since M = 1 is not a dense contraction.
//
// k_gemv (the main kernel).  A work-group of 4 waves handles 4/SPLIT row groups per round; a row
// group is R = 2 output rows (2 gate + 2 up rows for SwiGLU, [Qwen3-runtime] §2.7), split along K
// over SPLIT waves.  Each wave:
//   1. issues the 16-byte loads of its rows' K-slice first (lane l reads elements
//      kslice + c*64*VEC + l*VEC .. +VEC of each row, so one wave-wide load is a contiguous 1 KiB
//      of a row), so HBM latency overlaps everything that follows;
//   2. loads its slice of the input vector into registers; with the RMSNorm prologue
//      ([Qwen3-runtime] §2.1) it sums x^2 over its slice, combines the SPLIT partial sums (LDS,
//      only when SPLIT > 1) and forms h = x * rsqrt(mean + eps) * gamma in registers (rounded to
//      bf16 when activations are 16-bit);
//   3. with several rounds per work-group (large N), prefetches the next round's rows while it
//      reduces the current one;
//   4. reduces each row over the wave with DPP + readlane, then over the SPLIT waves through LDS,
//      and applies the epilogue: store (fp32 / bf16), residual add into the fp32 stream, or
//      silu(gate) * up.  The LM head also keeps the running (max, lowest index) of its rounded
//      outputs and writes one partial argmax per work-group.
// k_gemv_lds: the same contraction with the input staged in LDS, for slices too long to hold in
// registers.
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

// VEC consecutive input values starting at element k (fp32 or bf16 source).
template <int VEC>
__device__ __forceinline__ void load_x(const void* x, int x_bf16, int k, float* out) {
  if (x_bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + k);
#pragma unroll
    for (int j = 0; j < VEC / 8; ++j) {
      const uint4 u = p[j];
      out[8 * j + 0] = bf16_lo(u.x); out[8 * j + 1] = bf16_hi(u.x);
      out[8 * j + 2] = bf16_lo(u.y); out[8 * j + 3] = bf16_hi(u.y);
      out[8 * j + 4] = bf16_lo(u.z); out[8 * j + 5] = bf16_hi(u.z);
      out[8 * j + 6] = bf16_lo(u.w); out[8 * j + 7] = bf16_hi(u.w);
    }
    if constexpr (VEC == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + k);
      out[0] = bf16_lo(u.x); out[1] = bf16_hi(u.x); out[2] = bf16_lo(u.y); out[3] = bf16_hi(u.y);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + k);
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      const float4 f = p[j];
      out[4 * j + 0] = f.x; out[4 * j + 1] = f.y; out[4 * j + 2] = f.z; out[4 * j + 3] = f.w;
    }
  }
}

__device__ __forceinline__ bool argmax_better(float vb, int ib, float va, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return vb > va || (vb == va && ib < ia);
}

template <int WT, int EPI, bool NORM, int MAXCH, bool PIPE>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  constexpr int R = 2;
  constexpr int VEC = WTraits<WT>::VEC;
  constexpr int ELEM = WTraits<WT>::ELEM;
  constexpr int CH = kWave * VEC;
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  __shared__ float red_ss[4];
  __shared__ float red_acc[4][NR];
  __shared__ float red_bv[4];
  __shared__ int red_bi[4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = a.split;
  const int gpw = 4 / split;              // row groups per work-group round
  const int sub = wave % split;           // K-slice of this wave
  const int grp = wave / split;           // row group of this wave within the round
  const int K = (int)a.k;
  const int KW = K / split;
  const int kbase = sub * KW;
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
  int64_t round0 = blockIdx.x;
  int64_t g = round0 * gpw + grp;
  uint4 wv[NR][MAXCH];
  if (g < ngroups) load_rows(g, wv);

  // 2. input slice in registers (normalised when the RMSNorm prologue is fused)
  float xv[MAXCH][VEC];
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    const int kk = c * CH + lane * VEC;
    if (kk < KW) {
      load_x<VEC>(a.x, a.x_bf16, kbase + kk, xv[c]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) xv[c][e] = 0.f;
    }
  }
  if constexpr (NORM) {
    if (a.hidden_copy != nullptr && blockIdx.x == 0 && grp == 0) {
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) {
        const int kk = c * CH + lane * VEC;
        if (kk < KW)
#pragma unroll
          for (int e = 0; e < VEC; ++e) a.hidden_copy[kbase + kk + e] = xv[c][e];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss = fmaf(xv[c][e], xv[c][e], ss);
    ss = wave_sum(ss);
    if (split > 1) {
      if (lane == 0) red_ss[wave] = ss;
      __syncthreads();
      ss = 0.f;
      for (int s2 = 0; s2 < split; ++s2) ss += red_ss[grp * split + s2];
    }
    const float rinv = 1.0f / sqrtf(ss / (float)K + a.eps);
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      const int kk = c * CH + lane * VEC;
      float gm[VEC];
      if (kk < KW) {
        load_x<VEC>(a.gamma, 0, kbase + kk, gm);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) gm[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float h = xv[c][e] * rinv * gm[e];
        xv[c][e] = a.round_h ? round_bf16(h) : h;
      }
    }
  }

  float best_v = -INFINITY;
  int best_i = -1;
  const bool want_argmax = a.part_val != nullptr;

  // 3. rounds
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
    if (want_argmax) {  // uniform: a kernel argument
      // best_v / best_i are wave-uniform (computed from wave-uniform totals)
      if (lane == 0) {
        red_bv[wave] = best_v;
        red_bi[wave] = best_i;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
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

// ---- input staged in LDS (long K slices) -----------------------------------------------------
template <int WT, int EPI, bool NORM>
__global__ __launch_bounds__(256) void k_gemv_lds(GemvArgs a) {
  extern __shared__ __align__(16) float xs[];
  __shared__ float red[4];
  constexpr int R = 2;
  constexpr int VEC = WTraits<WT>::VEC;
  constexpr int ELEM = WTraits<WT>::ELEM;
  constexpr int CH = kWave * VEC;
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = (int)a.k;
  if constexpr (NORM) {
    float ss = 0.f;
    for (int i = tid; i < K; i += 256) {
      const float v = a.x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[i])
                               : static_cast<const float*>(a.x)[i];
      xs[i] = v;
      ss = fmaf(v, v, ss);
      if (a.hidden_copy != nullptr && blockIdx.x == 0) a.hidden_copy[i] = v;
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rinv = 1.0f / sqrtf(tot / (float)K + a.eps);
    for (int i = tid; i < K; i += 256) {
      const float h = xs[i] * rinv * a.gamma[i];
      xs[i] = a.round_h ? round_bf16(h) : h;
    }
  } else {
    for (int i = tid; i < K; i += 256)
      xs[i] = a.x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.x)[i])
                       : static_cast<const float*>(a.x)[i];
  }
  __syncthreads();
  const int64_t n = a.n;
  const int64_t ngroups = (n + R - 1) / R;
  const char* __restrict__ wbase = static_cast<const char*>(a.w);
  const int64_t row_bytes = (int64_t)K * ELEM;
  float best_v = -INFINITY;
  int best_i = -1;
  for (int64_t g = (int64_t)blockIdx.x * 4 + wave; g < ngroups; g += (int64_t)gridDim.x * 4) {
    const char* rp[NR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = (g * R + r < n) ? g * R + r : n - 1;
      rp[r] = wbase + row * row_bytes;
      if constexpr (EPI == EPI_SWIGLU) rp[R + r] = wbase + (row + n) * row_bytes;
    }
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll 2
    for (int kk = lane * VEC; kk < K; kk += CH) {
      uint4 wv[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) wv[r] = *reinterpret_cast<const uint4*>(rp[r] + (int64_t)kk * ELEM);
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = dot16<WT>(wv[r], xs + kk, acc[r]);
    }
    float tot[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) tot[r] = wave_sum(acc[r]);
    if constexpr (WT == W_I8) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = (g * R + r < n) ? g * R + r : n - 1;
        tot[r] *= a.scale[row];
        if constexpr (EPI == EPI_SWIGLU) tot[R + r] *= a.scale[row + n];
      }
    }
    float outv = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v = tot[r];
      if constexpr (EPI == EPI_SWIGLU) v = tot[r] / (1.0f + expf(-tot[r])) * tot[R + r];
      if (lane == r) outv = v;
      if constexpr (EPI == EPI_STORE) {
        const int64_t row = g * R + r;
        const float rv = a.y_bf16 ? round_bf16(v) : v;
        if (a.part_val != nullptr && row < n && rv == rv && (best_i < 0 || rv > best_v)) {
          best_v = rv;
          best_i = (int)row;
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
  if constexpr (EPI == EPI_STORE) {
    if (a.part_val != nullptr) {
      __shared__ float bvs[4];
      __shared__ int bis[4];
      if (lane == 0) {
        bvs[wave] = best_v;
        bis[wave] = best_i;
      }
      __syncthreads();
      if (tid == 0) {
        float bv = bvs[0];
        int bi = bis[0];
        for (int w = 1; w < 4; ++w)
          if (argmax_better(bvs[w], bis[w], bv, bi)) {
            bv = bvs[w];
            bi = bis[w];
          }
        a.part_val[blockIdx.x] = bv;
        a.part_idx[blockIdx.x] = bi;
      }
    }
  }
}

// ---- launch selection ---------------------------------------------------------------------------

// How a projection of n output rows and input length k is launched.  K is split over waves when
// there are fewer than 2048 row groups (so a single round still puts enough loads in flight on
// 256 CUs) or when one wave's slice would exceed 8 wave-wide loads per row (register budget);
// slices stay multiples of the 16-byte vector.  Slices that still do not fit use the LDS kernel.
struct GemvPlan {
  bool lds;
  int split, maxch;
  unsigned wgs;
};

static GemvPlan plan_gemv(int wtype, int epi, int64_t n, int64_t k) {
  const int vec = wtype == W_F32 ? 4 : wtype == W_BF16 ? 8 : 16;
  const int64_t ch = 64 * vec;
  const int64_t groups = (n + 1) / 2;
  const bool pipe = epi == EPI_STORE;
  int split = 1;
  while (split < 4 && k % (2 * split * vec) == 0 &&
         (groups * split < 2048 || (k / split + ch - 1) / ch > 8))
    split *= 2;
  const int chunks = (int)((k / split + ch - 1) / ch);
  GemvPlan p{};
  if (chunks > 8 || k % (split * vec) != 0) {
    int64_t wgs = (groups + 3) / 4;
    p.lds = true;
    p.split = 1;
    p.maxch = 0;
    p.wgs = (unsigned)(wgs > 1024 ? 1024 : wgs < 1 ? 1 : wgs);
    return p;
  }
  p.lds = false;
  p.split = split;
  p.maxch = chunks <= 1 ? 1 : chunks <= 2 ? 2 : chunks <= 4 ? 4 : 8;
  const int gpw = 4 / split;
  int64_t wgs = (groups + gpw - 1) / gpw;
  if (pipe && wgs > 1024) wgs = 1024;  // several rounds per work-group, next round prefetched
  p.wgs = (unsigned)(wgs < 1 ? 1 : wgs);
  return p;
}

template <int WT, int EPI, bool NORM, int MAXCH, bool PIPE>
static hipError_t go(const GemvArgs& a, unsigned wgs, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv<WT, EPI, NORM, MAXCH, PIPE>), dim3(wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int WT, int EPI, bool NORM, bool PIPE>
static hipError_t go_ch(int maxch, const GemvArgs& a, unsigned wgs, hipStream_t s) {
  switch (maxch) {
    case 1: return go<WT, EPI, NORM, 1, PIPE>(a, wgs, s);
    case 2: return go<WT, EPI, NORM, 2, PIPE>(a, wgs, s);
    case 4: return go<WT, EPI, NORM, 4, PIPE>(a, wgs, s);
    default: return go<WT, EPI, NORM, 8, PIPE>(a, wgs, s);
  }
}

template <int WT>
static hipError_t launch_wt(int epi, bool norm, GemvArgs a, hipStream_t s) {
  const GemvPlan p = plan_gemv(WT, epi, a.n, a.k);
  if (p.lds) {
    const size_t lds = (size_t)a.k * sizeof(float);
    const dim3 grid(p.wgs), block(256);
    if (epi == EPI_STORE) {
      if (norm)
        hipLaunchKernelGGL((k_gemv_lds<WT, EPI_STORE, true>), grid, block, lds, s, a);
      else
        hipLaunchKernelGGL((k_gemv_lds<WT, EPI_STORE, false>), grid, block, lds, s, a);
    } else if (epi == EPI_RESID) {
      hipLaunchKernelGGL((k_gemv_lds<WT, EPI_RESID, false>), grid, block, lds, s, a);
    } else {
      hipLaunchKernelGGL((k_gemv_lds<WT, EPI_SWIGLU, true>), grid, block, lds, s, a);
    }
    return hipGetLastError();
  }
  a.split = p.split;
  if (epi == EPI_STORE)
    return norm ? go_ch<WT, EPI_STORE, true, true>(p.maxch, a, p.wgs, s)
                : go_ch<WT, EPI_STORE, false, true>(p.maxch, a, p.wgs, s);
  if (epi == EPI_RESID) return go_ch<WT, EPI_RESID, false, false>(p.maxch, a, p.wgs, s);
  return go_ch<WT, EPI_SWIGLU, true, false>(p.maxch, a, p.wgs, s);
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

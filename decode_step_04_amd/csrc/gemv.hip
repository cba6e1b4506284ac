// gemv.hip - batch-1 projections y = W x (a GEMV at M = 1) streamed from HBM.
//
// [Qwen3-runtime] §4.1: at batch 1 every weight is read once and used for one multiply-add,
// so a projection is bound by the weight bytes it streams, not by arithmetic; §13.1 gives the
// W8A16 form (int8 weights, 16-bit activations, fp32 accumulation, the scale applied after the
// integer-weighted sum).  This kernel is plain VALU work: no MFMA, since M = 1 is not a dense
// contraction.
//
// Layout of a launch (256 threads = 4 waves per work-group):
//   - the input vector (optionally RMS-normalised on the fly, [Qwen3-runtime] §2.1, and rounded
//     to bf16 on the bf16 path) is staged once per work-group in LDS as fp32;
//   - each wave owns R consecutive output rows (2R weight rows for SwiGLU: gate row i and up row
//     F + i, [Qwen3-runtime] §2.7) and streams them with one 16-byte load per lane per row per
//     step: lane l reads elements [c*64*VEC + l*VEC, +VEC) of every row, so a wave-wide load is
//     one contiguous 1 KiB span of each row;
//   - partial sums are reduced across the wave with DPP row operations + readlane;
//   - epilogues: store (fp32 or bf16), residual add into the fp32 stream, or SwiGLU.
// Row groups are distributed over waves grid-stride, so a launch never needs more work-groups
// than fill the GPU; out-of-range rows of the last group are clamped to the last row for loading
// and discarded.
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

// acc + sum over the VEC elements of one 16-byte weight vector times VEC x values from LDS.
template <int WT>
__device__ __forceinline__ float dot16(uint4 w, const float* __restrict__ xs, float acc) {
  if constexpr (WT == W_F32) {
    const float4 x = *reinterpret_cast<const float4*>(xs);
    acc = fmaf(__uint_as_float(w.x), x.x, acc);
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    acc = fmaf(__uint_as_float(w.w), x.w, acc);
  } else if constexpr (WT == W_BF16) {
    const float4 x0 = *reinterpret_cast<const float4*>(xs);
    const float4 x1 = *reinterpret_cast<const float4*>(xs + 4);
    acc = fmaf(bf16_lo(w.x), x0.x, acc);
    acc = fmaf(bf16_hi(w.x), x0.y, acc);
    acc = fmaf(bf16_lo(w.y), x0.z, acc);
    acc = fmaf(bf16_hi(w.y), x0.w, acc);
    acc = fmaf(bf16_lo(w.z), x1.x, acc);
    acc = fmaf(bf16_hi(w.z), x1.y, acc);
    acc = fmaf(bf16_lo(w.w), x1.z, acc);
    acc = fmaf(bf16_hi(w.w), x1.w, acc);
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(xs + 4 * j);
      acc = fmaf(i8_at(ws[j], 0), x.x, acc);
      acc = fmaf(i8_at(ws[j], 1), x.y, acc);
      acc = fmaf(i8_at(ws[j], 2), x.z, acc);
      acc = fmaf(i8_at(ws[j], 3), x.w, acc);
    }
  }
  return acc;
}

template <int WT, int EPI, bool NORM, int R>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  extern __shared__ __align__(16) float xs[];
  __shared__ float red[4];
  constexpr int VEC = WTraits<WT>::VEC;
  constexpr int ELEM = WTraits<WT>::ELEM;
  constexpr int CH = kWave * VEC;                         // elements per wave-wide load
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;      // weight rows per row group

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = (int)a.k;

  // ---- stage the input vector in LDS ----
  if constexpr (NORM) {
    float ss = 0.f;
    for (int i = tid; i < K; i += 256) {
      const float v = a.xn[i];
      xs[i] = v;
      ss = fmaf(v, v, ss);
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
    if (a.hidden_copy != nullptr && blockIdx.x == 0)
      for (int i = tid; i < K; i += 256) a.hidden_copy[i] = a.xn[i];
  } else {
    if (a.x_bf16) {
      const uint16_t* x = static_cast<const uint16_t*>(a.x);
      for (int i = tid; i < K; i += 256) xs[i] = bf16_to_f32(x[i]);
    } else {
      const float* x = static_cast<const float*>(a.x);
      for (int i = tid; i < K; i += 256) xs[i] = x[i];
    }
  }
  __syncthreads();

  // ---- stream the rows ----
  const int64_t n = a.n;
  const int nfull = K / CH;
  const int rem = K - nfull * CH;
  const int64_t ngroups = (n + R - 1) / R;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  const char* __restrict__ wbase = static_cast<const char*>(a.w);
  const int64_t row_bytes = (int64_t)K * ELEM;

  for (int64_t g = (int64_t)blockIdx.x * 4 + wave; g < ngroups; g += wstride) {
    const int64_t r0 = g * R;
    const char* rp[NR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = (r0 + r < n) ? r0 + r : n - 1;
      rp[r] = wbase + row * row_bytes;
      if constexpr (EPI == EPI_SWIGLU) rp[R + r] = wbase + (row + n) * row_bytes;
    }
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;

#pragma unroll 2
    for (int c = 0; c < nfull; ++c) {
      const int kk = c * CH + lane * VEC;
      uint4 wv[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r)
        wv[r] = *reinterpret_cast<const uint4*>(rp[r] + (int64_t)kk * ELEM);
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = dot16<WT>(wv[r], xs + kk, acc[r]);
    }
    if (rem > 0) {
      const int kk = nfull * CH + lane * VEC;
      if (kk < K) {
        uint4 wv[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r)
          wv[r] = *reinterpret_cast<const uint4*>(rp[r] + (int64_t)kk * ELEM);
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = dot16<WT>(wv[r], xs + kk, acc[r]);
      }
    }

    float tot[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) tot[r] = wave_sum(acc[r]);
    if constexpr (WT == W_I8) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = (r0 + r < n) ? r0 + r : n - 1;
        tot[r] *= a.scale[row];
        if constexpr (EPI == EPI_SWIGLU) tot[R + r] *= a.scale[row + n];
      }
    }

    float outv = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v = tot[r];
      if constexpr (EPI == EPI_SWIGLU) {
        const float gt = tot[r], up = tot[R + r];
        v = gt / (1.0f + expf(-gt)) * up;  // silu(gate) * up
      }
      if (lane == r) outv = v;
    }
    const int64_t row = r0 + lane;
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
}

template <int WT, int EPI, bool NORM>
static hipError_t launch_one(const GemvArgs& a, hipStream_t s) {
  constexpr int R = (EPI == EPI_SWIGLU) ? 2 : 4;
  const int64_t ngroups = (a.n + R - 1) / R;
  int64_t wgs = (ngroups + 3) / 4;
  if (wgs > kGemvMaxWgs) wgs = kGemvMaxWgs;
  if (wgs < 1) wgs = 1;
  const size_t lds = (size_t)a.k * sizeof(float);
  hipLaunchKernelGGL((k_gemv<WT, EPI, NORM, R>), dim3((unsigned)wgs), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int WT>
static hipError_t launch_wt(int epi, bool norm, const GemvArgs& a, hipStream_t s) {
  if (epi == EPI_STORE) return norm ? launch_one<WT, EPI_STORE, true>(a, s)
                                    : launch_one<WT, EPI_STORE, false>(a, s);
  if (epi == EPI_RESID) return norm ? launch_one<WT, EPI_RESID, true>(a, s)
                                    : launch_one<WT, EPI_RESID, false>(a, s);
  return norm ? launch_one<WT, EPI_SWIGLU, true>(a, s) : launch_one<WT, EPI_SWIGLU, false>(a, s);
}

hipError_t launch_gemv(int wtype, int epi, bool norm, const GemvArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  switch (wtype) {
    case W_F32: return launch_wt<W_F32>(epi, norm, a, s);
    case W_BF16: return launch_wt<W_BF16>(epi, norm, a, s);
    default: return launch_wt<W_I8>(epi, norm, a, s);
  }
}

}  // namespace qd

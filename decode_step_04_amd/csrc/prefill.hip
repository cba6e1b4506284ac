// prefill.hip - batched prefill of P prompt tokens: the first place MFMA belongs on this path.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
//
// [ETE] lists batched prefill as the step from a teaching engine to a usable one: the
// [1, hidden] GEMVs become [P, hidden] GEMMs, with a causal mask and FlashAttention-style
// prefill.  A prefill of P tokens computes what P decode steps would ([Qwen3-runtime] §2.1-2.7
// per token), with 16-bit activations at the GEMM inputs: the MFMA units take bf16 operands and
// accumulate in fp32.
//
// k_gemm: Y[M x N] = A[M x K] . W[N x K]^T, A and W bf16 row-major with K contiguous (the weight
// layout of the decode path), fp32 accumulation on v_mfma_f32_16x16x32_bf16.  A 256-thread
// work-group computes a 128 x 128 tile as 2 x 2 waves of 64 x 64; a wave holds 4 x 4 MFMA tiles
// of 16 x 16.  For one 16 x 16 x 32 step, lane l supplies A[row l % 16][k 8(l/16) .. +7] and
// W[row l % 16][k 8(l/16) .. +7] -- 16 contiguous bytes of each row -- and receives
// C[row 4(l/16) + i][col l % 16], i < 4 (layout checked on MI355X).  Each k step of 32 loads the
// next step's 8 fragments into a second register set before issuing the current 16 MFMAs.
// Epilogues: STORE (fp32), RESID (adds into an fp32 [M x N] residual), SWIGLU (the tile's 128
// weight rows are 64 gate rows and the matching 64 up rows; bf16 silu(g) * u).
#include "common.h"
#include "launch.h"

namespace qd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = a.m, N = a.n, K = a.k;
  const int m0 = blockIdx.y * 128 + (wave >> 1) * 64;
  // output columns of the tile: SWIGLU tiles cover 64 outputs (64 gate + 64 up weight rows)
  const int ncols = EPI == EPI_SWIGLU ? 64 : 128;
  const int n0 = blockIdx.x * ncols + (EPI == EPI_SWIGLU ? 0 : (wave & 1) * 64);
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  // row pointers of this lane's fragments (rows past the end are clamped; results discarded)
  const uint16_t* pa[4];
  const uint16_t* pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + 16 * i + r16, M - 1);
    pa[i] = A + (int64_t)m * K + kq;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int wr;
    if constexpr (EPI == EPI_SWIGLU) {
      // waves 0/1 x 2/3 split M; both column halves of a wave: j < 2 gate rows, j >= 2 up rows
      const int c = (wave & 1) * 32 + 16 * (j & 1);
      const int col = min(n0 + c + r16, N - 1);
      wr = (j < 2) ? col : N + col;
    } else {
      wr = min(n0 + 16 * j + r16, N - 1);
    }
    pw[j] = W + (int64_t)wr * K + kq;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa0[4], fw0[4], fa1[4], fw1[4];
  auto fetch = [&](bf16x8 (&fa)[4], bf16x8 (&fw)[4], int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = load_frag(pa[i] + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) fw[j] = load_frag(pw[j] + k);
  };
  auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fw)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fw[j], acc[i][j], 0, 0, 0);
  };
  // two register sets alternate; the last step re-fetches its own k (cached) so that no load
  // sits under a branch
  fetch(fa0, fw0, 0);
  for (int k = 0; k < K; k += 64) {
    fetch(fa1, fw1, k + 32 < K ? k + 32 : k);
    mma(fa0, fw0);
    if (k + 32 >= K) break;
    fetch(fa0, fw0, k + 64 < K ? k + 64 : k + 32);
    mma(fa1, fw1);
  }

  // epilogue: lane holds C[m0 + 16 i + 4 (l/16) + e][n of block j, col l % 16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * i + 4 * (lane >> 4) + e;
      if (m >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + (wave & 1) * 32 + 16 * j + r16;
          if (n >= N) continue;
          const float g = acc[i][j][e], u = acc[i][j + 2][e];
          const float v = g / (1.0f + expf(-g)) * u;
          static_cast<uint16_t*>(a.y)[(int64_t)m * N + n] = f32_to_bf16(v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + 16 * j + r16;
          if (n >= N) continue;
          const float v = acc[i][j][e];
          if constexpr (EPI == EPI_RESID)
            a.resid[(int64_t)m * N + n] += v;
          else if (a.y_bf16)
            static_cast<uint16_t*>(a.y)[(int64_t)m * N + n] = f32_to_bf16(v);
          else
            static_cast<float*>(a.y)[(int64_t)m * N + n] = v;
        }
      }
    }
  }
}

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.m <= 0 || a.n <= 0) return hipSuccess;
  if (a.k % 32 || a.k < 32) return hipErrorInvalidValue;
  const int ncols = epi == EPI_SWIGLU ? 64 : 128;
  const dim3 grid((unsigned)((a.n + ncols - 1) / ncols), (unsigned)((a.m + 127) / 128));
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<EPI_STORE>), grid, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<EPI_RESID>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm<EPI_SWIGLU>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace qd

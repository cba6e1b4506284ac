// attention.hip - split-KV causal GQA decode attention over a paged KV cache.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
//
// What is computed ([Qwen3-runtime] §2.5-2.6): for each query head h, with kv head
// g = h / (Hq / Hkv), scores s_j = q_h . k_j / sqrt(D) over positions j < ctx, and
// out_h = sum_j softmax(s)_j v_j.
//
// How ([Qwen3-runtime] §9.1, §10.1-10.2; [ETE] the (m, l, acc) passage):
//   k_attn_part: one work-group per (kv head g, partition).  A partition is a contiguous range of
//   whole 16-token pages.  The G = Hq / Hkv query heads of g are all handled by the same lanes, so
//   every K/V element is loaded from HBM once and used for all G heads (the GQA reuse of §2.5).
//   Each wave takes every 4th page of the partition; a page tile of one head (16 x D, contiguous
//   in the pool) is read with one 16-byte load per lane per 1 KiB, so lane l holds EPL
//   consecutive dims of one token per load: token row = l / LPT, dims (l % LPT) * EPL.  Scores
//   are reduced over the LPT lanes of a token with DPP, and every token row keeps its own fp32
//   online state (m, l, acc[dims]) per head.  Rows, then waves (through LDS), are combined with
//   the exact rescaling of §9.1.  With one partition the normalised output is written directly
//   (the short path of §10.1); otherwise the unnormalised state goes to scratch.
//   k_attn_merge: per query head, M = max m_p, out = sum acc_p 2^(m_p - M) / sum l_p 2^(m_p - M).
//
// Scores are kept in log2 units: q is pre-multiplied by log2(e)/sqrt(D), so exp(s - m) becomes
// exp2(s' - m') (one v_exp_f32).  The initial running max is -1e30 as in [ETE]; masked tokens
// get a score of -inf and weight 0.
#include "common.h"
#include "launch.h"

namespace qd {

template <int D, bool KVB>
struct Geo {
  static constexpr int ELEM = KVB ? 2 : 4;
  static constexpr int EPL = 16 / ELEM;       // elements per lane per 16-byte load
  static constexpr int LPT = D / EPL;         // lanes holding one token
  static constexpr int TPI = kWave / LPT;     // tokens per wave-wide load
  static constexpr int NI = kPage / TPI;      // loads per page tile
  static_assert(LPT >= 8 && LPT <= 32, "lane layout");
};

// Sum over aligned groups of N lanes, N in {8, 16, 32}.
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (N <= 16) {
    return group_sum<N>(v);
  } else {
    v = group_sum<16>(v);
    return v + __shfl_xor(v, 16);
  }
}

template <bool KVB, int EPL>
__device__ __forceinline__ void widen16(const uint4 w, float (&f)[EPL]) {
  if constexpr (KVB) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  } else {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, bool KVB, int G>
__global__ __launch_bounds__(256) void k_attn_part(AttnArgs a) {
  using Gm = Geo<D, KVB>;
  constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TPI = Gm::TPI, NI = Gm::NI, ELEM = Gm::ELEM;
  __shared__ float sm_acc[4][G][D];
  __shared__ float sm_m[4][G];
  __shared__ float sm_l[4][G];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ctx = a.desc ? a.desc->ctx : a.ctx_arg;
  const int part = part_tokens_for(ctx, a.part_fixed, a.n_kv_heads, a.target_wgs);
  const int np = n_parts_for(ctx, part);
  const int hkv = a.n_kv_heads;
  const int g = blockIdx.x % hkv;
  const int pi = blockIdx.x / hkv;
  if (pi >= np) return;
  const int tok0 = pi * part;
  const int tok1 = min(ctx, tok0 + part);
  const int pg0 = tok0 / kPage, pg1 = (tok1 + kPage - 1) / kPage;

  const int dsub = (lane % LPT) * EPL;
  const int trow = lane / LPT;

  // query slices of the G grouped heads, pre-scaled to log2 units
  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int hq = g * G + h;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int idx = hq * D + dsub + e;
      const float v = a.q_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[idx])
                               : static_cast<const float*>(a.q)[idx];
      q[h][e] = v * a.qscale;
    }
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -1e30f;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int64_t tile_bytes = (int64_t)kPage * D * ELEM;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);

  for (int pg = pg0 + wave; pg < pg1; pg += 4) {
    const int64_t phys = a.block_table[pg];
    const int64_t tile = (phys * hkv + g) * tile_bytes;
    uint4 kw[NI], vw[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kw[i] = *reinterpret_cast<const uint4*>(kbase + tile + (int64_t)(i * kWave + lane) * 16);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vw[i] = *reinterpret_cast<const uint4*>(vbase + tile + (int64_t)(i * kWave + lane) * 16);

    // scores of this lane's token row for every load slot i and head h
    float s[G][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      widen16<KVB, EPL>(kw[i], kf);
      const int tok = pg * kPage + i * TPI + trow;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], kf[e], p);
        p = lanes_sum<LPT>(p);
        s[h][i] = (tok < tok1) ? p : -INFINITY;
      }
    }
    // online update ([ETE]: new max, rescale the old state, add the new terms)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < NI; ++i) mx = fmaxf(mx, s[h][i]);
      const float c = fast_exp2(m[h] - mx);
      l[h] *= c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= c;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float p = fast_exp2(s[h][i] - mx);
        l[h] += p;
        float vf[EPL];
        widen16<KVB, EPL>(vw[i], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
      m[h] = mx;
    }
  }

  // combine the token rows of the wave (lanes with equal dims), exact rescaling
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mx = fmaxf(m[h], mo);
      const float ca = fast_exp2(m[h] - mx), cb = fast_exp2(mo - mx);
      l[h] = l[h] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * ca + ao * cb;
      }
      m[h] = mx;
    }
  }
  if (trow == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][h][dsub + e] = acc[h][e];
      if (lane == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // combine the 4 waves; threads cover (head, dim) pairs
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, r = idx % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c = fast_exp2(sm_m[w][h] - M);
      L = fmaf(sm_l[w][h], c, L);
      O = fmaf(sm_acc[w][h][r], c, O);
    }
    const int hq = g * G + h;
    if (np == 1) {
      const float o = O / L;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[hq * D + r] = f32_to_bf16(o);
      else
        static_cast<float*>(a.out)[hq * D + r] = o;
    } else {
      const int64_t slot = (int64_t)hq * a.max_parts + pi;
      a.part_acc[slot * D + r] = O;
      if (r == 0) {
        a.part_ml[slot * 2 + 0] = M;
        a.part_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// One work-group of D threads per query head.
template <int D>
__global__ __launch_bounds__(128) void k_attn_merge(AttnArgs a) {
  const int ctx = a.desc ? a.desc->ctx : a.ctx_arg;
  const int part = part_tokens_for(ctx, a.part_fixed, a.n_kv_heads, a.target_wgs);
  const int np = n_parts_for(ctx, part);
  if (np <= 1) return;  // the partition kernel already wrote the output
  const int hq = blockIdx.x, r = threadIdx.x;
  const int64_t base = (int64_t)hq * a.max_parts;
  float M = -1e30f;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_ml[(base + p) * 2]);
  float L = 0.f, O = 0.f;
  for (int p = 0; p < np; ++p) {
    const float c = fast_exp2(a.part_ml[(base + p) * 2] - M);
    L = fmaf(a.part_ml[(base + p) * 2 + 1], c, L);
    O = fmaf(a.part_acc[(base + p) * D + r], c, O);
  }
  const float o = O / L;
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[hq * D + r] = f32_to_bf16(o);
  else
    static_cast<float*>(a.out)[hq * D + r] = o;
}

template <int D, bool KVB>
static hipError_t launch_dk(int group, const AttnArgs& a, int grid_parts, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv_heads * grid_parts)), block(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((k_attn_part<D, KVB, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn_part<D, KVB, 2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn_part<D, KVB, 3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn_part<D, KVB, 4>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_attn_part<D, KVB, 5>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_attn_part<D, KVB, 6>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_attn_part<D, KVB, 7>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_attn_part<D, KVB, 8>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int head_dim, bool kv_bf16, int group, const AttnArgs& a,
                            int grid_parts, hipStream_t s) {
  if (head_dim == 64) return kv_bf16 ? launch_dk<64, true>(group, a, grid_parts, s)
                                     : launch_dk<64, false>(group, a, grid_parts, s);
  return kv_bf16 ? launch_dk<128, true>(group, a, grid_parts, s)
                 : launch_dk<128, false>(group, a, grid_parts, s);
}

hipError_t launch_attention_merge(int head_dim, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_q_heads);
  if (head_dim == 64)
    hipLaunchKernelGGL((k_attn_merge<64>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_merge<128>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace qd

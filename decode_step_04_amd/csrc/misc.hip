// misc.hip - the small kernels of the decode step and of the library's set-up paths.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
#include "common.h"
#include "launch.h"

namespace qd {

// ---- fused per-head Q/K RMSNorm + RoPE + paged K/V append ------------------------------------
// [Qwen3-runtime] §2.3 (per-head RMSNorm of Q and K over D, V untouched), §2.4 (half-rotation
// RoPE: pairs (r, r + D/2) rotated by pos * theta_r), §7.1 (one warp per head so the reduction
// and the rotation need no shared memory), §7.2 (the rotated K goes straight to its physical
// page).  On a 64-lane wave lane l owns the pair (l, l + D/2), so both halves of a rotation pair
// are in the same lane.  One wave per head: waves 0..Hq-1 take the Q heads, waves Hq..Hq+Hkv-1
// the K heads and the matching V heads.
template <int D>
__global__ __launch_bounds__(64) void k_rope_append(RopeAppendArgs a) {
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x;
  const int hh = blockIdx.x;
  const int pos = a.desc ? a.desc->pos : a.pos_arg;
  const bool act = lane < HALF;
  const bool is_q = hh < a.n_q_heads;
  const int g = hh - a.n_q_heads;
  const float* src = a.qkv + (int64_t)(is_q ? hh : a.n_q_heads + g) * D;
  float x0 = act ? src[lane] : 0.f;
  float x1 = act ? src[lane + HALF] : 0.f;
  const float* gam = is_q ? a.q_gamma : a.k_gamma;
  if (gam != nullptr) {
    const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
    const float rinv = 1.0f / sqrtf(ss / (float)D + a.eps);
    if (act) {
      x0 = x0 * rinv * gam[lane];
      x1 = x1 * rinv * gam[lane + HALF];
    }
  }
  if (!act) return;
  const float2 cs = reinterpret_cast<const float2*>(a.table)[(int64_t)pos * HALF + lane];
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x1 * cs.x + x0 * cs.y;
  if (is_q) {
    const int64_t o = (int64_t)hh * D + lane;
    if (a.q_bf16) {
      static_cast<uint16_t*>(a.q_out)[o] = f32_to_bf16(y0);
      static_cast<uint16_t*>(a.q_out)[o + HALF] = f32_to_bf16(y1);
    } else {
      static_cast<float*>(a.q_out)[o] = y0;
      static_cast<float*>(a.q_out)[o + HALF] = y1;
    }
    return;
  }
  const int64_t phys = a.block_table[pos / kPage];
  const int64_t off = ((phys * a.n_kv_heads + g) * kPage + pos % kPage) * D + lane;
  const float* vs = a.qkv + (int64_t)(a.n_q_heads + a.n_kv_heads + g) * D;
  const float v0 = vs[lane], v1 = vs[lane + HALF];
  if (a.kv_bf16) {
    uint16_t* kp = static_cast<uint16_t*>(a.k_pool);
    uint16_t* vp = static_cast<uint16_t*>(a.v_pool);
    kp[off] = f32_to_bf16(y0);
    kp[off + HALF] = f32_to_bf16(y1);
    vp[off] = f32_to_bf16(v0);
    vp[off + HALF] = f32_to_bf16(v1);
  } else {
    float* kp = static_cast<float*>(a.k_pool);
    float* vp = static_cast<float*>(a.v_pool);
    kp[off] = y0;
    kp[off + HALF] = y1;
    vp[off] = v0;
    vp[off + HALF] = v1;
  }
}

hipError_t launch_rope_append(int head_dim, const RopeAppendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_q_heads + a.n_kv_heads));
  if (head_dim == 64)
    hipLaunchKernelGGL((k_rope_append<64>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k_rope_append<128>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---- embedding row + step descriptor -----------------------------------------------------------
// x = E[token] widened to fp32, or the caller's embedding row ([ETE]: the block pipeline starts
// from the token's embedding row).  The token id is read on the device so it may come from the
// previous step's argmax.  An id outside [0, V) gives a zero row and sets the sticky error flag.
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  const int tid = threadIdx.x;
  int tok = 0;
  bool bad = false;
  if (a.emb == nullptr) {
    tok = *a.token;
    bad = tok < 0 || tok >= a.vocab;
  }
  if (tid == 0 && a.desc != nullptr) {
    a.desc->pos = a.pos;
    a.desc->ctx = a.pos + 1;
    if (bad) a.desc->error = 1;
  }
  if (a.rope_step != nullptr)
    for (int i = tid; i < a.rope_half; i += 256)
      reinterpret_cast<float2*>(a.rope_step)[i] =
          reinterpret_cast<const float2*>(a.rope_table)[(int64_t)a.pos * a.rope_half + i];
  const void* src = a.emb ? a.emb : a.table;
  const int64_t base = a.emb ? 0 : (int64_t)tok * a.d;
  for (int i = tid; i < a.d; i += 256) {
    float v = 0.f;
    if (!bad) v = a.table_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(src)[base + i])
                               : static_cast<const float*>(src)[base + i];
    a.x[i] = v;
  }
}

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

const void* embed_kernel_fn() { return reinterpret_cast<const void*>(&k_embed); }

// ---- argmax (greedy next token) ------------------------------------------------------------------
// Largest value, lowest index on ties, NaN never chosen; -1 when every value is NaN.
__device__ __forceinline__ bool better(float vb, int ib, float va, int ia) {
  if (ib < 0) return false;
  if (ia < 0) return true;
  return vb > va || (vb == va && ib < ia);
}

__global__ __launch_bounds__(1024) void k_argmax(const void* x, int x_bf16, int64_t n,
                                                 int32_t* out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  float best = -INFINITY;
  int bi = -1;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    const float v = x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i])
                           : static_cast<const float*>(x)[i];
    if (v == v && (bi < 0 || v > best)) {
      best = v;
      bi = (int)i;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = sv[0];
    int b = si[0];
    for (int w = 1; w < 16; ++w)
      if (better(sv[w], si[w], bv, b)) {
        bv = sv[w];
        b = si[w];
      }
    *out = b;
  }
}

hipError_t launch_argmax(const void* x, int x_bf16, int64_t n, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax, dim3(1), dim3(1024), 0, s, x, x_bf16, n, out);
  return hipGetLastError();
}

// Final step of the LM head's fused argmax: the best of n per-work-group (value, index) partials.
__global__ __launch_bounds__(1024) void k_argmax_partials(const float* val, const int32_t* idx,
                                                          int n, int32_t* out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  float best = -INFINITY;
  int bi = -1;
  for (int i = threadIdx.x; i < n; i += 1024)
    if (better(val[i], idx[i], best, bi)) {
      best = val[i];
      bi = idx[i];
    }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = sv[0];
    int b = si[0];
    for (int w = 1; w < 16; ++w)
      if (better(sv[w], si[w], bv, b)) {
        bv = sv[w];
        b = si[w];
      }
    *out = b;
  }
}

hipError_t launch_argmax_partials(const float* val, const int32_t* idx, int n, int32_t* out,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_partials, dim3(1), dim3(1024), 0, s, val, idx, n, out);
  return hipGetLastError();
}

// ---- per-row symmetric int8 quantisation (upload time) -----------------------------------------
// [ETE], the int8 passage: symmetric, one scale per row.  scale = max|row| / 127 in fp32, code =
// round-half-even(w / scale) clamped to [-127, 127] (IEEE fp32 division, v_rndne_f32); a zero
// row keeps scale 0 and zero codes.  One wave per row; k % 4 == 0.
template <bool SRC_BF16>
__global__ __launch_bounds__(256) void k_quantize(const void* w, int8_t* q, float* scale,
                                                  int64_t n, int64_t k) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < n; row += (int64_t)gridDim.x * 4) {
    float v[4];
    float mx = 0.f;
    for (int64_t c = (int64_t)lane * 4; c < k; c += 256) {
      if constexpr (SRC_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + row * k + c);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + row * k + c);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(v[j]));
    }
    mx = wave_max(mx);
    const float sc = mx / 127.0f;
    if (lane == 0) scale[row] = sc;
    for (int64_t c = (int64_t)lane * 4; c < k; c += 256) {
      if constexpr (SRC_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + row * k + c);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + row * k + c);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      }
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float r = 0.f;
        if (sc != 0.f) r = fminf(fmaxf(rintf(v[j] / sc), -127.f), 127.f);
        packed |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(q + row * k + c) = packed;
    }
  }
}

hipError_t launch_quantize(const void* w, int src_bf16, int8_t* q, float* scale, int64_t n,
                           int64_t k, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t wgs = (n + 3) / 4;
  if (wgs > 4096) wgs = 4096;
  if (src_bf16)
    hipLaunchKernelGGL((k_quantize<true>), dim3((unsigned)wgs), dim3(256), 0, s, w, q, scale, n, k);
  else
    hipLaunchKernelGGL((k_quantize<false>), dim3((unsigned)wgs), dim3(256), 0, s, w, q, scale, n, k);
  return hipGetLastError();
}

// ---- group-wise symmetric quantisation, 128-value groups (upload time) ---------------------------
// [Qwen3-runtime] §13.1 keeps a scale per 128-value group; 4-bit codes are the next step [ETE]
// names.  Per group: scale = max|w| / QMAX in fp32 (QMAX = 127 or 7), code = round-half-even(w /
// scale) clamped to [-QMAX, QMAX]; an all-zero group keeps scale 0 and zero codes.  One wave per
// group, lane l taking elements 2l and 2l + 1: int8 codes are written as two bytes, int4 codes as
// one byte (element 2l in the low nibble, each nibble code + 8).  k % 128 == 0.
template <bool SRC_BF16, int BITS>
__global__ __launch_bounds__(256) void k_quantize_groups(const void* w, uint8_t* q, float* scale,
                                                         int64_t n, int64_t k) {
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ng = k / kQGroup;
  for (int64_t grp = (int64_t)blockIdx.x * 4 + wave; grp < n * ng; grp += (int64_t)gridDim.x * 4) {
    const int64_t e = (grp / ng) * k + (grp % ng) * kQGroup + 2 * lane;  // element 2l of the group
    float v0, v1;
    if constexpr (SRC_BF16) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(w) + e);
      v0 = bf16_lo(u);
      v1 = bf16_hi(u);
    } else {
      const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(w) + e);
      v0 = f.x;
      v1 = f.y;
    }
    const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sc = mx / QMAX;
    if (lane == 0) scale[grp] = sc;
    float r0 = 0.f, r1 = 0.f;
    if (sc != 0.f) {
      r0 = fminf(fmaxf(rintf(v0 / sc), -QMAX), QMAX);
      r1 = fminf(fmaxf(rintf(v1 / sc), -QMAX), QMAX);
    }
    if constexpr (BITS == 8) {
      const uint32_t b0 = (uint8_t)(int8_t)(int)r0, b1 = (uint8_t)(int8_t)(int)r1;
      *reinterpret_cast<uint16_t*>(q + e) = (uint16_t)(b0 | (b1 << 8));
    } else {
      const uint32_t n0 = (uint32_t)((int)r0 + 8), n1 = (uint32_t)((int)r1 + 8);
      q[e / 2] = (uint8_t)(n0 | (n1 << 4));
    }
  }
}

hipError_t launch_quantize_groups(const void* w, int src_bf16, int bits, void* q, float* scale,
                                  int64_t n, int64_t k, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t wgs = (n * (k / kQGroup) + 3) / 4;
  if (wgs > 8192) wgs = 8192;
  uint8_t* qb = static_cast<uint8_t*>(q);
  const dim3 grid((unsigned)wgs), block(256);
  if (src_bf16) {
    if (bits == 8)
      hipLaunchKernelGGL((k_quantize_groups<true, 8>), grid, block, 0, s, w, qb, scale, n, k);
    else
      hipLaunchKernelGGL((k_quantize_groups<true, 4>), grid, block, 0, s, w, qb, scale, n, k);
  } else {
    if (bits == 8)
      hipLaunchKernelGGL((k_quantize_groups<false, 8>), grid, block, 0, s, w, qb, scale, n, k);
    else
      hipLaunchKernelGGL((k_quantize_groups<false, 4>), grid, block, 0, s, w, qb, scale, n, k);
  }
  return hipGetLastError();
}

// ---- KV pre-fill / read-back through the block table -------------------------------------------
// [Qwen3-runtime] §7.2: position p lives in slot p % 16 of physical page bt[p / 16].  One thread
// per 16-byte chunk of a (position, head) row.
__global__ __launch_bounds__(256) void k_kv_copy(char* pool, char* lin, const int32_t* bt,
                                                 int pos0, int n, int hkv, int row_bytes,
                                                 int to_pool) {
  const int cpr = row_bytes / 16;
  const int64_t total = (int64_t)n * hkv * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int c = (int)(idx % cpr);
    const int g = (int)((idx / cpr) % hkv);
    const int i = (int)(idx / ((int64_t)cpr * hkv));
    const int pos = pos0 + i;
    const int64_t phys = bt[pos / kPage];
    const int64_t poff = ((phys * hkv + g) * kPage + pos % kPage) * row_bytes + (int64_t)c * 16;
    const int64_t loff = ((int64_t)i * hkv + g) * row_bytes + (int64_t)c * 16;
    if (to_pool)
      *reinterpret_cast<uint4*>(pool + poff) = *reinterpret_cast<const uint4*>(lin + loff);
    else
      *reinterpret_cast<uint4*>(lin + loff) = *reinterpret_cast<const uint4*>(pool + poff);
  }
}

hipError_t launch_kv_copy(void* pool, void* linear, const int32_t* block_table, int pos0, int n,
                          int n_kv_heads, int head_dim, int elem, int to_pool, hipStream_t s) {
  const int row_bytes = head_dim * elem;
  const int64_t total = (int64_t)n * n_kv_heads * (row_bytes / 16);
  if (total <= 0) return hipSuccess;
  int64_t wgs = (total + 255) / 256;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(k_kv_copy, dim3((unsigned)wgs), dim3(256), 0, s, static_cast<char*>(pool),
                     static_cast<char*>(linear), block_table, pos0, n, n_kv_heads, row_bytes,
                     to_pool);
  return hipGetLastError();
}

// ---- RoPE cos/sin table ----------------------------------------------------------------------------
// table[p][i] = (cos(p * theta^(-2i/D)), sin(...)), angle and functions in fp64 (set-up time).
__global__ __launch_bounds__(256) void k_rope_table(float* t, int max_pos, int d, double theta) {
  const int half = d / 2;
  const int64_t total = (int64_t)max_pos * half;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t p = idx / half;
    const int i = (int)(idx % half);
    const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)d);
    t[2 * idx] = (float)cos(ang);
    t[2 * idx + 1] = (float)sin(ang);
  }
}

hipError_t launch_rope_table(float* table, int max_pos, int head_dim, float theta, hipStream_t s) {
  const int64_t total = (int64_t)max_pos * (head_dim / 2);
  int64_t wgs = (total + 255) / 256;
  if (wgs > 8192) wgs = 8192;
  if (wgs < 1) wgs = 1;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)wgs), dim3(256), 0, s, table, max_pos, head_dim,
                     (double)theta);
  return hipGetLastError();
}

// ---- plain streaming copy (bandwidth reference) -----------------------------------------------------
__global__ __launch_bounds__(256) void k_copy(uint4* __restrict__ dst,
                                              const uint4* __restrict__ src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s, int max_wgs) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  int64_t wgs = (n16 + 255) / 256;
  if (wgs > max_wgs) wgs = max_wgs;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)wgs), dim3(256), 0, s, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

// ---- storage conversions at upload --------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_convert(void* dst, int dst_type, const void* src,
                                                 int src_type, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = src_type == W_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(src)[i])
                                       : static_cast<const float*>(src)[i];
    if (dst_type == W_BF16)
      static_cast<uint16_t*>(dst)[i] = f32_to_bf16(v);
    else
      static_cast<float*>(dst)[i] = v;
  }
}

hipError_t launch_convert(void* dst, int dst_type, const void* src, int src_type, int64_t n,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t wgs = (n + 255) / 256;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(k_convert, dim3((unsigned)wgs), dim3(256), 0, s, dst, dst_type, src, src_type,
                     n);
  return hipGetLastError();
}

// ---- stand-alone RMSNorm ([Qwen3-runtime] §2.1), one work-group ------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const float* gamma, float eps,
                                                 void* y, int y_bf16, int n) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // one work-group per row
  x += (int64_t)blockIdx.x * n;
  y = static_cast<char*>(y) + (int64_t)blockIdx.x * n * (y_bf16 ? 2 : 4);
  float ss = 0.f;
  for (int i = tid; i < n; i += 256) ss = fmaf(x[i], x[i], ss);
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rinv = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = tid; i < n; i += 256) {
    const float h = x[i] * rinv * gamma[i];
    if (y_bf16)
      static_cast<uint16_t*>(y)[i] = f32_to_bf16(h);
    else
      static_cast<float*>(y)[i] = h;
  }
}

// The same row norm with the row held in registers: thread t loads the float4s t + 256 j of x
// and gamma (16-byte loads, x read once), and writes 4 outputs per store (8 bytes of bf16).  Each
// output is the same expression as k_rmsnorm's; only the sum of squares is added in another
// order.  Rows of n % 4 == 0 values up to 1024 V, with 16-byte aligned x rows and gamma and y rows
// aligned for the store.  (Measured on MI355X, 2048 rows of 1024: 5.4 us for k_rmsnorm, whose
// scalar loop reads each value twice.)
template <int V>
__global__ __launch_bounds__(256) void k_rmsnorm_v(const float* x, const float* gamma, float eps,
                                                   void* y, int y_bf16, int n) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = n / 4;
  const float4* x4 = reinterpret_cast<const float4*>(x + (int64_t)blockIdx.x * n);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  float4 v[V], g[V];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = tid + 256 * j;
    v[j] = g[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n4) {
      v[j] = x4[i];
      g[j] = g4[i];
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    ss = fmaf(v[j].x, v[j].x, ss);
    ss = fmaf(v[j].y, v[j].y, ss);
    ss = fmaf(v[j].z, v[j].z, ss);
    ss = fmaf(v[j].w, v[j].w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rinv = 1.0f / sqrtf(tot / (float)n + eps);
  char* yr = static_cast<char*>(y) + (int64_t)blockIdx.x * n * (y_bf16 ? 2 : 4);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = tid + 256 * j;
    if (i < n4) {
      const float h0 = v[j].x * rinv * g[j].x, h1 = v[j].y * rinv * g[j].y;
      const float h2 = v[j].z * rinv * g[j].z, h3 = v[j].w * rinv * g[j].w;
      if (y_bf16) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
        w.y = (uint32_t)f32_to_bf16(h2) | ((uint32_t)f32_to_bf16(h3) << 16);
        reinterpret_cast<uint2*>(yr)[i] = w;
      } else {
        reinterpret_cast<float4*>(yr)[i] = make_float4(h0, h1, h2, h3);
      }
    }
  }
}

hipError_t launch_rmsnorm(const float* x, const float* gamma, float eps, void* y, int y_bf16,
                          int n, hipStream_t s) {
  return launch_rmsnorm_rows(x, gamma, eps, y, y_bf16, n, 1, s);
}

hipError_t launch_rmsnorm_rows(const float* x, const float* gamma, float eps, void* y, int y_bf16,
                               int n, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const auto al = [](const void* p, uintptr_t b) { return reinterpret_cast<uintptr_t>(p) % b == 0; };
  const bool vec = n % 4 == 0 && n <= 8192 && al(x, 16) && al(gamma, 16) && al(y, y_bf16 ? 8 : 16);
  const dim3 grid((unsigned)rows), block(256);
  if (vec && n <= 1024)
    hipLaunchKernelGGL((k_rmsnorm_v<1>), grid, block, 0, s, x, gamma, eps, y, y_bf16, n);
  else if (vec && n <= 2048)
    hipLaunchKernelGGL((k_rmsnorm_v<2>), grid, block, 0, s, x, gamma, eps, y, y_bf16, n);
  else if (vec && n <= 4096)
    hipLaunchKernelGGL((k_rmsnorm_v<4>), grid, block, 0, s, x, gamma, eps, y, y_bf16, n);
  else if (vec)
    hipLaunchKernelGGL((k_rmsnorm_v<8>), grid, block, 0, s, x, gamma, eps, y, y_bf16, n);
  else
    hipLaunchKernelGGL(k_rmsnorm, grid, block, 0, s, x, gamma, eps, y, y_bf16, n);
  return hipGetLastError();
}

}  // namespace qd

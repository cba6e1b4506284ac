// sample.hip - temperature + top-p (nucleus) sampling of the next token on the device.
//
// [ETE] = the page "EdgeTransformerEngine", whose limitations passage names greedy-only decoding
// (no temperature, no top-p).  The method is the usual one, read plainly:
//   p_i = softmax(logits / T)_i;  the nucleus is the shortest prefix of the tokens ordered by p
//   descending (ties: lower index first) whose mass reaches top_p;  the draw is the nucleus token,
//   in index order, at which the cumulative nucleus mass first exceeds u times the nucleus mass,
//   u in [0, 1) from Philox4x32-10 (Salmon et al., SC 2011) keyed by the seed with the position
//   as counter (24 bits).
//
// k_sample: one 1024-thread work-group, thread t owning the contiguous index chunk
// [t C, (t + 1) C), so that block scans in thread order are scans in index order.  Each pass
// re-reads the logits (L2-resident after the first) and recomputes e_i = 2^((z_i / T - M) log2 e)
// the same way, so every pass sees the same values:
//   1. M = max z_i / T.
//   2. q_i = e_i * 2^40 as a 64-bit integer (e_i <= 1, so the sum over 2^18 tokens fits), and S =
//      sum q_i.  Integer sums are exact and independent of order: the nucleus decision does not
//      depend on how the threads' atomics interleave.
//   3-6. The nucleus threshold is found by radix selection on the bits of e_i (positive floats
//      order like their bit patterns), 8 bits per pass from the top: a 256-bin histogram of the
//      mass q_i among the tokens that match the prefix so far (LDS 64-bit atomics), then the
//      highest bin whose mass, added to the mass above it, reaches the target ceil(top_p S).
//      The result is the boundary value e* with the mass above it and the count of ties at it;
//      ceil((target - mass above) / q*) tied tokens, lowest indices first, complete the nucleus.
//   7. Index-order block scans of the tie counts and of the nucleus mass; the draw target
//      floor(u N) is located in the thread whose chunk holds it, which walks its chunk.
#include "common.h"
#include "launch.h"

namespace qd {

// Philox4x32-10 block (the published definition: multipliers 0xD2511F53 and 0xCD9E8D57, Weyl key
// increments 0x9E3779B9 and 0xBB67AE85, ten rounds).
__device__ inline void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

constexpr int kSampleThreads = 1024;

// Exclusive scan over the block in thread order; returns this thread's prefix, *total the sum.
__device__ inline uint64_t block_excl_scan(uint64_t v, uint64_t* lds, uint64_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  if (t == 0) {
    uint64_t acc = 0;
    for (int w = 0; w < kSampleThreads / 64; ++w) {
      const uint64_t s = lds[w];
      lds[w] = acc;
      acc += s;
    }
    lds[kSampleThreads / 64] = acc;
  }
  __syncthreads();
  const uint64_t r = lds[wave] + x - v;
  *total = lds[kSampleThreads / 64];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kSampleThreads) void k_sample(SampleArgs a) {
  __shared__ uint64_t hist[256];
  __shared__ uint64_t scan_lds[kSampleThreads / 64 + 1];
  __shared__ float red_f[kSampleThreads / 64];
  __shared__ uint64_t red_u[kSampleThreads / 64];
  __shared__ uint32_t sel_prefix;      // key bits decided so far
  __shared__ uint64_t sel_above;       // mass of the keys above the current prefix
  __shared__ float s_max;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t n = a.n;
  const int64_t chunk = (n + kSampleThreads - 1) / kSampleThreads;
  const int64_t i0 = min(n, (int64_t)t * chunk), i1 = min(n, i0 + chunk);
  const float inv_t = a.inv_temperature;
  auto logit = [&](int64_t i) -> float {
    return a.x_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.logits)[i])
                    : static_cast<const float*>(a.logits)[i];
  };

  // 1. the maximum of z / T
  float mx = -INFINITY;
  for (int64_t i = i0; i < i1; ++i) mx = fmaxf(mx, logit(i) * inv_t);
  mx = wave_max(mx);
  if (lane == 0) red_f[wave] = mx;
  __syncthreads();
  if (t == 0) {
    float m = red_f[0];
    for (int w = 1; w < kSampleThreads / 64; ++w) m = fmaxf(m, red_f[w]);
    s_max = m;
  }
  __syncthreads();
  const float M = s_max;
  constexpr float kLog2e = 1.4426950408889634f;
  // written with an explicit fma so that every pass computes e_i with the same instructions
  auto mass = [&](int64_t i, uint32_t& key) -> uint64_t {
    const float zt = fmaf(logit(i), inv_t, -M);
    const float e = __builtin_amdgcn_exp2f(zt * kLog2e);
    key = __float_as_uint(e);
    return (uint64_t)(e * 1099511627776.0f);  // e * 2^40
  };

  // 2. S = sum of q_i
  uint64_t loc = 0;
  for (int64_t i = i0; i < i1; ++i) {
    uint32_t key;
    loc += mass(i, key);
  }
  uint64_t S;
  (void)block_excl_scan(loc, scan_lds, &S);
  uint64_t target = (uint64_t)ceil((double)a.top_p * (double)S);
  if (target < 1) target = 1;
  if (target > S) target = S;

  // 3-6. radix selection of the boundary key, 8 bits per pass from the top
  if (t == 0) {
    sel_prefix = 0;
    sel_above = 0;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (t < 256) hist[t] = 0;
    __syncthreads();
    const uint32_t prefix = sel_prefix;
    for (int64_t i = i0; i < i1; ++i) {
      uint32_t key;
      const uint64_t q = mass(i, key);
      // tokens matching the bits decided so far (none decided before pass 0)
      if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&hist[(key >> shift) & 255u], q);
    }
    __syncthreads();
    if (t == 0) {
      uint64_t above = sel_above;
      int b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= target) break;
        above += hist[b];
      }
      sel_prefix = (prefix << 8) | (uint32_t)b;
      sel_above = above;
    }
    __syncthreads();
  }
  const uint32_t kstar = sel_prefix;
  const uint64_t above = sel_above;

  // 7. ties at the boundary (lowest indices first), nucleus mass, and the draw
  uint64_t qstar = 0;
  uint64_t ties = 0;
  for (int64_t i = i0; i < i1; ++i) {
    uint32_t key;
    const uint64_t q = mass(i, key);
    if (key == kstar) {
      ++ties;
      qstar = q;
    }
  }
  // every tied token has the same q; share it
  if (lane == 0) red_u[wave] = 0;
  __syncthreads();
  if (ties) red_u[wave] = qstar;  // benign: equal values
  __syncthreads();
  if (t == 0) {
    uint64_t qs = 0;
    for (int w = 0; w < kSampleThreads / 64; ++w) qs = red_u[w] ? red_u[w] : qs;
    scan_lds[kSampleThreads / 64] = qs;
  }
  __syncthreads();
  qstar = scan_lds[kSampleThreads / 64];
  __syncthreads();
  const uint64_t need = target > above ? target - above : 0;
  const uint64_t take = qstar ? (need + qstar - 1) / qstar : 0;
  uint64_t tie_total;
  const uint64_t tie_rank0 = block_excl_scan(ties, scan_lds, &tie_total);
  // nucleus mass of this chunk, walking the chunk in index order
  uint64_t nloc = 0, rank = tie_rank0;
  for (int64_t i = i0; i < i1; ++i) {
    uint32_t key;
    const uint64_t q = mass(i, key);
    if (key > kstar) {
      nloc += q;
    } else if (key == kstar) {
      if (rank < take) nloc += q;
      ++rank;
    }
  }
  uint64_t ntot;
  const uint64_t npre = block_excl_scan(nloc, scan_lds, &ntot);
  // u from Philox4x32-10: key (seed low, seed high), counter (position, 0, 0, 0)
  const int pos = a.desc ? a.desc->pos : a.pos_arg;
  uint32_t c[4] = {(uint32_t)pos, 0u, 0u, 0u};
  philox4x32_10(c, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
  const double u = (double)(c[0] >> 8) * (1.0 / 16777216.0);
  const uint64_t draw = (uint64_t)(u * (double)ntot);  // < ntot
  if (draw >= npre && draw < npre + nloc) {
    uint64_t cum = npre;
    rank = tie_rank0;
    int64_t pick = i1 - 1;
    for (int64_t i = i0; i < i1; ++i) {
      uint32_t key;
      const uint64_t q = mass(i, key);
      bool in = key > kstar;
      if (key == kstar) in = rank++ < take;
      if (!in) continue;
      cum += q;
      if (cum > draw) {
        pick = i;
        break;
      }
    }
    *a.out = (int32_t)pick;
  }
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_sample, dim3(1), dim3(kSampleThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qd

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
// Arithmetic, identical in every kernel below: M = max_i z_i / T (from maxima of parts of the
// stored logits: fp32 multiplication by 1/T is monotone), e_i = 2^((z_i / T - M) log2 e) with
// z_i / T - M one fma, key_i = the bits of e_i (positive floats order like their bit patterns,
// so key order is p order), and the mass q_i = e_i * 2^40 truncated to a 64-bit integer.  Every
// sum of masses is an exact integer sum, independent of order, so no decision depends on how
// work-groups or atomics interleave.  With S = sum q_i the nucleus is every token whose key is
// above a boundary key k*, plus the first `take` tokens (lowest indices) of the ties at k*,
// where k* and take are the least that bring the mass to target = ceil(top_p S).
//
// Batch-1 decode hands the sampler one row of up to 2^18 logits: too little work to fill the
// chip, and a pass over 152K logits costs one CU ~15 us of VALU time, so the row is split into
// kSB slices of at most 4096 tokens.  Each kernel is a few memory round trips: every thread
// issues all of its loads before it uses any, and scans across waves run on one wave's DPP
// steps.  Level-1 bins are 1/16 octave of e (the top 13 key bits, 16 bins per octave).
//   k_sample_max     (only when the caller gives no maxima) the maxima of the kSB slices;
//   k_sample_hist    per slice: M, then the mass per level-1 bin and per octave;
//   k_sample_gather  per slice: the kSB x 64 octave masses give S, target and the boundary
//                    octave; that octave's 16 bins over all slices give the boundary bin j1 and
//                    the mass above it; then the slice's mass above j1, and its keys in j1, in
//                    index order, into the slice's own candidate region;
//   k_sample_select  one work-group: the candidates (slice after slice, so in index order),
//                    two radix passes over their remaining 19 key bits give k* and take; then
//                    the nucleus mass N, the draw d = floor(u N), the slice that holds d, and an
//                    index-order scan of that slice alone finds the token.
// The workspace is rewritten in full by every call (no clearing, nothing carried over), so the
// pipeline can be captured into a graph.
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

constexpr int kSB = 64;                           // slices of the row
constexpr int kSBThreads = 256;                   // threads of the slice kernels
constexpr int kSliceMax = 4096;                   // 2^18 / kSB
constexpr int kRS = kSliceMax / kSBThreads;       // tokens per thread in the slice kernels
constexpr int kBins = 1024;                       // level-1 bins: 64 octaves x 16
constexpr int kOct = kBins / 16;
constexpr int kBinBase = 87 << 4;                 // key >> 19 of e = 2^-40 (biased exponent 87)
                                                  // opens bin 1; bin 0 holds the zero masses
constexpr int kFinal = 1024;                      // threads of k_sample_select
constexpr int kRW = kSliceMax / kFinal;           // tokens per thread of its slice scan
constexpr int kRC = 8;                            // candidates per thread per batch
constexpr int kSpec = 64;                         // candidates per slice loaded before the
                                                  // counts are known
constexpr int kTPS = kFinal / kSB;                // threads per slice for those loads
constexpr int kSPT = kSpec / kTPS;                // loads per thread
constexpr int kCandLds = 24576;                   // candidates kept in LDS (beyond: compacted
                                                  // into the workspace)
static_assert(kBins == 4 * kSBThreads, "k_sample_hist writes four bins per thread");
static_assert(kSB == 64 && kOct == 64, "one wave spans the slices and the octaves");
static_assert(kTPS * kSB == kFinal && kSPT * kTPS == kSpec, "speculative loads tile the slices");

struct SampleState {
  uint64_t S, target, A1;             // total mass, ceil(top_p S), mass of the bins above j1
  int32_t j1;                         // the boundary bin (-1: no positive mass)
  float M;                            // max z / T
};

struct SampleWs {
  float* pmax;        // [kSB] slice maxima (when the caller gives none)
  uint64_t* hist;     // [kSB][kBins] mass per slice and bin
  uint64_t* oct;      // [kSB][kOct] mass per slice and octave
  uint64_t* above;    // [kSB] mass of each slice above bin j1
  uint32_t* ccount;   // [kSB] candidates of each slice
  SampleState* st;
  uint32_t* cand;     // [kSB][kSliceMax] keys of bin j1, each slice's in index order
  uint32_t* cmp;      // [n] all candidates in index order (when they exceed kCandLds)
};

static inline int64_t ws_round(int64_t b) { return (b + 255) & ~int64_t(255); }

int64_t sample_workspace_bytes(int64_t n) {
  return ws_round(kSB * 4) + ws_round((int64_t)kSB * kBins * 8) + ws_round((int64_t)kSB * kOct * 8) +
         ws_round(kSB * 8) + ws_round(kSB * 4) + ws_round((int64_t)sizeof(SampleState)) +
         ws_round((int64_t)kSB * kSliceMax * 4) + ws_round(n * 4);
}

static SampleWs carve_ws(void* base, int64_t n) {
  char* p = static_cast<char*>(base);
  SampleWs w;
  auto take = [&](int64_t b) {
    char* r = p;
    p += ws_round(b);
    return r;
  };
  w.pmax = reinterpret_cast<float*>(take(kSB * 4));
  w.hist = reinterpret_cast<uint64_t*>(take((int64_t)kSB * kBins * 8));
  w.oct = reinterpret_cast<uint64_t*>(take((int64_t)kSB * kOct * 8));
  w.above = reinterpret_cast<uint64_t*>(take(kSB * 8));
  w.ccount = reinterpret_cast<uint32_t*>(take(kSB * 4));
  w.st = reinterpret_cast<SampleState*>(take((int64_t)sizeof(SampleState)));
  w.cand = reinterpret_cast<uint32_t*>(take((int64_t)kSB * kSliceMax * 4));
  w.cmp = reinterpret_cast<uint32_t*>(take(n * 4));
  return w;
}

// The slice [lo, hi) of work-group b.
__device__ inline void slice_of(int64_t n, int b, int64_t& lo, int64_t& hi) {
  const int64_t len = (n + kSB - 1) / kSB;
  lo = min(n, (int64_t)b * len);
  hi = min(n, lo + len);
}

// Token lo + r * NT + t of the slice into z[r], every load issued before any is used.
template <int R, int NT>
__device__ inline void load_slice(const SampleArgs& a, int64_t lo, int64_t hi, float (&z)[R]) {
  const int t = threadIdx.x;
  if (a.x_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(a.logits);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = lo + (int64_t)r * NT + t;
      z[r] = i < hi ? bf16_to_f32(p[i]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(a.logits);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = lo + (int64_t)r * NT + t;
      z[r] = i < hi ? p[i] : 0.0f;
    }
  }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwo40 = 1099511627776.0f;

// The key of a logit (bits of e); NaN logits get e = 0 (never drawn).
__device__ inline uint32_t tok_key(float z, float inv_t, float M) {
  float e = __builtin_amdgcn_exp2f(fmaf(z, inv_t, -M) * kLog2e);
  if (!(e <= 2.0f)) e = 0.0f;
  return __float_as_uint(e);
}

__device__ inline int key_bin(uint32_t key) {
  const int b = (int)(key >> 19) - kBinBase + 1;
  return b < 0 ? 0 : b;
}

__device__ inline uint64_t key_mass(uint32_t key) {
  return (uint64_t)(__uint_as_float(key) * kTwo40);
}

// 64-bit cross-lane steps as two 32-bit DPP moves (lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// DPP row_shr:1, 2, 4, 8 (shift up within each row of 16 lanes).
constexpr int kDppShr1 = 0x111;
constexpr int kDppShr2 = 0x112;
constexpr int kDppShr4 = 0x114;
constexpr int kDppShr8 = 0x118;

// Inclusive scan over the wave (all 64 lanes active): within rows by DPP shifts, then the
// totals of the rows below.
__device__ inline uint64_t wave_incl_u64(uint64_t x) {
  x += dpp64<kDppShr1>(x);
  x += dpp64<kDppShr2>(x);
  x += dpp64<kDppShr4>(x);
  x += dpp64<kDppShr8>(x);
  const uint64_t r0 = readlane64(x, 15), r1 = readlane64(x, 31), r2 = readlane64(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Sum over the wave (all 64 lanes active); the result is wave-uniform.
__device__ inline uint64_t wave_sum_u64(uint64_t v) {
  v += dpp64<kDppXor1>(v);
  v += dpp64<kDppXor2>(v);
  v += dpp64<kDppHalfMirror>(v);
  v += dpp64<kDppMirror>(v);
  return (readlane64(v, 0) + readlane64(v, 16)) + (readlane64(v, 32) + readlane64(v, 48));
}

__device__ inline uint64_t lanemask_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Adds v to h[bin] and 1 to c[bin] (either may be null) for the active lanes.  When the active
// lanes of the wave share one bin (a flat distribution), the wave sums first and one lane adds:
// 64 same-address LDS atomics in one instruction would serialise.  Call from wave-uniform
// control flow.
__device__ inline void hist_add(uint64_t* h, uint32_t* c, int bin, uint64_t v, bool act) {
  const uint64_t am = __ballot(act);
  if (am == 0) return;
  const int lane = threadIdx.x & 63;
  const int first = __ffsll((unsigned long long)am) - 1;
  const int b0 = __builtin_amdgcn_readlane(bin, first);
  if (__ballot(act && bin != b0) == 0) {
    const uint64_t s = wave_sum_u64(act ? v : 0);
    if (lane == first) {
      if (h) atomicAdd((unsigned long long*)&h[b0], (unsigned long long)s);
      if (c) atomicAdd(&c[b0], (uint32_t)__popcll(am));
    }
  } else if (act) {
    if (h) atomicAdd((unsigned long long*)&h[bin], (unsigned long long)v);
    if (c) atomicAdd(&c[bin], 1u);
  }
}

// Exclusive scan in place of tab[0 .. E) by the first wave, tab[E] = the total (E <= 128).
// Call from all threads between barriers.
template <int E>
__device__ inline void table_scan(uint64_t* tab) {
  static_assert(E <= 128, "two entries per lane");
  const int l = threadIdx.x;
  if (l < 64) {
    const uint64_t a = (2 * l < E) ? tab[2 * l] : 0, b = (2 * l + 1 < E) ? tab[2 * l + 1] : 0;
    const uint64_t inc = wave_incl_u64(a + b);
    const uint64_t ex = inc - (a + b);
    if (2 * l < E) tab[2 * l] = ex;
    if (2 * l + 1 < E) tab[2 * l + 1] = ex + a;
    if (l == 63) tab[E] = inc;
  }
}

// Exclusive index-order prefix of v[r] over a batch of R chunks (element r * NT + t) and the
// batch total.  tab: R * NT / 64 + 1 entries.  TAIL = false leaves out the closing barrier: the
// caller then must not write tab before its next barrier.
template <int NT, int R, bool TAIL = true>
__device__ inline void batch_excl(const uint64_t (&v)[R], uint64_t (&ex)[R], uint64_t* tab,
                                  uint64_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t inc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    inc[r] = wave_incl_u64(v[r]);
    if (lane == 63) tab[r * NW + wave] = inc[r];
  }
  __syncthreads();
  table_scan<R * NW>(tab);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) ex[r] = tab[r * NW + wave] + inc[r] - v[r];
  *total = tab[R * NW];
  if (TAIL) __syncthreads();
}

// Exclusive index-order ranks of set flags over a batch of R chunks, and their count.
template <int NT, int R, bool TAIL = true>
__device__ inline void batch_rank(const bool (&f)[R], uint32_t (&rank)[R], uint64_t* tab,
                                  uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t below[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint64_t m = __ballot(f[r]);
    below[r] = (uint32_t)__popcll(m & lanemask_lt());
    if (lane == 0) tab[r * NW + wave] = (uint64_t)__popcll(m);
  }
  __syncthreads();
  table_scan<R * NW>(tab);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) rank[r] = (uint32_t)tab[r * NW + wave] + below[r];
  *total = (uint32_t)tab[R * NW];
  if (TAIL) __syncthreads();
}

// batch_excl of v[r] and batch_rank of f[r] with one set of barriers (tv, tf: R * NT / 64 + 1
// entries each), no closing barrier.
template <int NT, int R>
__device__ inline void batch_excl_rank(const uint64_t (&v)[R], uint64_t (&ex)[R],
                                       const bool (&f)[R], uint32_t (&rank)[R], uint64_t* tv,
                                       uint64_t* tf) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t inc[R];
  uint32_t below[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    inc[r] = wave_incl_u64(v[r]);
    if (lane == 63) tv[r * NW + wave] = inc[r];
    const uint64_t m = __ballot(f[r]);
    below[r] = (uint32_t)__popcll(m & lanemask_lt());
    if (lane == 0) tf[r * NW + wave] = (uint64_t)__popcll(m);
  }
  __syncthreads();
  table_scan<R * NW>(tv);
  table_scan<R * NW>(tf);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ex[r] = tv[r * NW + wave] + inc[r] - v[r];
    rank[r] = (uint32_t)tf[r * NW + wave] + below[r];
  }
}

template <int NT>
__device__ inline float block_max(float v, float* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float m = lds[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, lds[w]);
  __syncthreads();
  return m;
}

template <int NT>
__device__ inline uint64_t block_sum_u64(uint64_t v, uint64_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_u64(v);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) s += lds[w];
  __syncthreads();
  return s;
}

// ---- k_sample_max: per-slice maxima of the stored logits ----
__global__ __launch_bounds__(kSBThreads) void k_sample_max(SampleArgs a, SampleWs w) {
  __shared__ float red[kSBThreads / 64];
  int64_t lo, hi;
  slice_of(a.n, blockIdx.x, lo, hi);
  float z[kRS];
  load_slice<kRS, kSBThreads>(a, lo, hi, z);
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < kRS; ++r)
    if (lo + r * kSBThreads + (int)threadIdx.x < hi) m = fmaxf(m, z[r]);
  m = block_max<kSBThreads>(m, red);
  if (threadIdx.x == 0) w.pmax[blockIdx.x] = m;
}

// ---- k_sample_hist: M, then the slice's mass per bin and per octave ----
__global__ __launch_bounds__(kSBThreads) void k_sample_hist(SampleArgs a, SampleWs w) {
  __shared__ uint64_t h[kBins];
  __shared__ float red[kSBThreads / 64];
  const int t = threadIdx.x, b = blockIdx.x;
  for (int j = t; j < kBins; j += kSBThreads) h[j] = 0;
  int64_t lo, hi;
  slice_of(a.n, b, lo, hi);
  float z[kRS];
  load_slice<kRS, kSBThreads>(a, lo, hi, z);
  const float* parts = a.part_val ? a.part_val : w.pmax;
  const int np = a.part_val ? a.n_parts : kSB;
  float m = -INFINITY;
  for (int j0 = 0; j0 < np; j0 += kRS * kSBThreads) {  // one round trip up to 4096 parts
    float pv[kRS];
#pragma unroll
    for (int k = 0; k < kRS; ++k) {
      const int j = j0 + k * kSBThreads + t;
      pv[k] = j < np ? parts[j] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < kRS; ++k) m = fmaxf(m, pv[k]);
  }
  m = block_max<kSBThreads>(m, red);  // its barriers also order the clearing above
  const float inv_t = a.inv_temperature;
  const float M = m * inv_t;
  if (b == 0 && t == 0) w.st->M = M;
#pragma unroll
  for (int r = 0; r < kRS; ++r) {
    const bool act = lo + r * kSBThreads + t < hi;
    const uint32_t key = act ? tok_key(z[r], inv_t, M) : 0u;
    const uint64_t q = key_mass(key);
    hist_add(h, nullptr, key_bin(key), q, act && q > 0);
  }
  __syncthreads();
  uint64_t s4 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = 4 * t + k;
    w.hist[(int64_t)b * kBins + j] = h[j];
    s4 += h[j];
  }
  // octave t / 4 = bins 16 (t / 4) .. + 15, held by the lanes of one quad
  s4 += dpp64<kDppXor1>(s4);
  s4 += dpp64<kDppXor2>(s4);
  if ((t & 3) == 0) w.oct[(int64_t)b * kOct + (t >> 2)] = s4;
}

// ---- k_sample_gather: S, target, j1; the slice's mass above j1 and its candidates of j1 ----
__global__ __launch_bounds__(kSBThreads) void k_sample_gather(SampleArgs a, SampleWs w) {
  __shared__ uint64_t red[4][kOct];
  __shared__ uint64_t tab[kRS * (kSBThreads / 64) + 1];
  __shared__ uint64_t tab2[kSBThreads / 64];
  __shared__ uint64_t fm[16];
  __shared__ int s_o1, s_k1;
  __shared__ uint64_t s_Ao, s_A1, s_S, s_target;
  const int t = threadIdx.x, b = blockIdx.x, lane = t & 63, wave = t >> 6;
  int64_t lo, hi;
  slice_of(a.n, b, lo, hi);
  // round trip 1: the slice's logits, the octave masses of every slice, M
  float z[kRS];
  load_slice<kRS, kSBThreads>(a, lo, hi, z);
  uint64_t os = 0;
#pragma unroll
  for (int k = 0; k < kSB / 4; ++k) os += w.oct[(int64_t)(wave * (kSB / 4) + k) * kOct + lane];
  red[wave][lane] = os;
  const float M = w.st->M, inv_t = a.inv_temperature;
  __syncthreads();
  // the boundary octave: lane l of the first wave takes octave 63 - l (top down)
  if (t < 64) {
    const int o = kOct - 1 - t;
    const uint64_t v = (red[0][o] + red[1][o]) + (red[2][o] + red[3][o]);
    const uint64_t inc = wave_incl_u64(v);  // mass of octaves >= o
    const uint64_t S = readlane64(inc, 63);
    uint64_t target = (uint64_t)ceil((double)a.top_p * (double)S);
    if (target < 1) target = 1;
    if (target > S) target = S;
    if (t == 0) {
      s_S = S;
      s_target = target;
      s_o1 = -1;
      s_k1 = 0;
    }
    if (S > 0 && inc - v < target && inc >= target) {  // unique: inc is non-decreasing in t
      s_o1 = o;
      s_Ao = inc - v;
      s_A1 = inc - v;
    }
  }
  __syncthreads();
  const int o1 = s_o1;
  if (o1 < 0) {  // no positive mass (all logits NaN): the select kernel reports token 0
    if (b == 0 && t == 0) {
      w.st->S = 0;
      w.st->target = 0;
      w.st->A1 = 0;
      w.st->j1 = -1;
    }
    return;
  }
  const uint64_t S = s_S, target = s_target;
  // round trip 2: the 16 bins of octave o1 of every slice (lane = slice, wave = 4 bins) ...
  uint64_t fmv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) fmv[k] = w.hist[(int64_t)lane * kBins + o1 * 16 + wave * 4 + k];
  // ... while the slice's keys are computed
  uint32_t key[kRS];
#pragma unroll
  for (int r = 0; r < kRS; ++r) key[r] = tok_key(z[r], inv_t, M);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t tm = wave_sum_u64(fmv[k]);
    if (lane == 0) fm[wave * 4 + k] = tm;
  }
  __syncthreads();
  // the boundary bin within o1: lane l of the first wave takes bin 15 - l of the octave
  if (t < 64) {
    const uint64_t v = t < 16 ? fm[15 - t] : 0;
    const uint64_t inc = s_Ao + wave_incl_u64(v);
    if (t < 16 && inc - v < target && inc >= target) {
      s_k1 = 15 - t;
      s_A1 = inc - v;
    }
  }
  __syncthreads();
  const int j1 = o1 * 16 + s_k1;
  uint64_t above = 0;
  bool f[kRS];
#pragma unroll
  for (int r = 0; r < kRS; ++r) {
    const bool act = lo + r * kSBThreads + t < hi;
    const int bin = key_bin(key[r]);
    if (act && bin > j1) above += key_mass(key[r]);
    f[r] = act && bin == j1;
  }
  uint32_t rank[kRS], tot;
  batch_rank<kSBThreads, kRS, false>(f, rank, tab, &tot);
#pragma unroll
  for (int r = 0; r < kRS; ++r)
    if (f[r]) w.cand[(int64_t)b * kSliceMax + rank[r]] = key[r];
  const uint64_t above_tot = block_sum_u64<kSBThreads>(above, tab2);
  if (t == 0) {
    w.above[b] = above_tot;
    w.ccount[b] = tot;
  }
  if (b == 0 && t == 0) {
    w.st->S = S;
    w.st->target = target;
    w.st->A1 = s_A1;
    w.st->j1 = j1;
  }
}

// The digit whose mass above it is below `target` and with it reaches `target`, among
// h[0 .. NB), and that mass above (NB / kFinal consecutive bins per thread, from the top).  tab is
// free again on return.
template <int NB>
__device__ inline void select_digit(const uint64_t* h, uint64_t target, uint64_t* tab, int* s_d,
                                    uint64_t* s_above) {
  constexpr int BPT = NB > kFinal ? NB / kFinal : 1;
  static_assert(NB <= kFinal || BPT * kFinal == NB, "whole bins per thread");
  const int t = threadIdx.x;
  uint64_t hv[BPT], loc = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    hv[k] = t * BPT + k < NB ? h[NB - 1 - (t * BPT + k)] : 0;
    loc += hv[k];
  }
  uint64_t v[1] = {loc}, ex[1], tot;
  batch_excl<kFinal, 1, false>(v, ex, tab, &tot);
  uint64_t above = ex[0];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    if (t * BPT + k < NB && above < target && above + hv[k] >= target) {
      *s_d = NB - 1 - (t * BPT + k);
      *s_above = above;
    }
    above += hv[k];
  }
  __syncthreads();
}

// The slice whose candidates hold position c: off[blk] <= c < off[blk + 1].
__device__ inline int cand_slice(const uint32_t* off, uint32_t c) {
  int lo = 0, hi = kSB;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= c) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ---- k_sample_select: k*, take, N, the draw, and the token ----
__global__ __launch_bounds__(kFinal) void k_sample_select(SampleArgs a, SampleWs w) {
  __shared__ uint32_t ck[kCandLds];
  __shared__ uint64_t h[1024];
  constexpr int kTab = (kRC > kRW ? kRC : kRW) * (kFinal / 64) + 1;
  __shared__ uint64_t tabA[kTab];
  __shared__ uint64_t tabB[kTab];
  __shared__ uint32_t off[kSB + 1];
  __shared__ uint64_t nb[kSB];
  __shared__ uint32_t tb[kSB];
  __shared__ int s_d, s_blk, s_more;
  __shared__ uint64_t s_above, s_dd;
  __shared__ uint32_t s_tb;
  __shared__ int64_t s_pick;
  const int t = threadIdx.x;
  // round trip 1: the state, the slices' masses above j1 and candidate counts, and the first
  // kSpec candidates of every slice whatever their counts
  const SampleState st = *w.st;
  const uint64_t ab = t < kSB ? w.above[t] : 0;
  const uint32_t cc = t < kSB ? w.ccount[t] : 0;
  const int sl = t / kTPS, su = t % kTPS;
  uint32_t spec[kSPT];
#pragma unroll
  for (int r = 0; r < kSPT; ++r) spec[r] = w.cand[(int64_t)sl * kSliceMax + su + kTPS * r];
  if (st.j1 < 0) {
    if (t == 0) *a.out = 0;
    return;
  }
  const int j1 = st.j1;
  if (t < 64) {  // the first candidate of each slice: exclusive scan of the counts
    const uint64_t inc = wave_incl_u64(cc);
    off[t] = (uint32_t)(inc - cc);
    if (t == 63) off[kSB] = (uint32_t)inc;
    nb[t] = 0;
    tb[t] = 0;
    const bool more = __ballot(cc > (uint32_t)kSpec) != 0;
    if (t == 0) s_more = more;
  }
  for (int j = t; j < 1024; j += kFinal) h[j] = 0;
  if (t == 0) {
    s_pick = -1;
    s_d = 0;
    s_above = 0;
  }
  __syncthreads();
  // the candidates in index order: into LDS, or (beyond kCandLds) compacted into the workspace
  const uint32_t C1 = off[kSB];
  const bool in_lds = C1 <= (uint32_t)kCandLds;
  uint32_t* dst = in_lds ? ck : w.cmp;
  {
    const uint32_t o = off[sl], cnt = off[sl + 1] - o;
#pragma unroll
    for (int r = 0; r < kSPT; ++r) {
      const uint32_t u = su + kTPS * r;
      if (u < cnt) dst[o + u] = spec[r];
    }
  }
  if (s_more) {  // slices with more than kSpec candidates
    for (uint32_t base = 0; base < C1; base += kRC * kFinal) {
      uint32_t kk[kRC];
      int64_t src[kRC];
#pragma unroll
      for (int r = 0; r < kRC; ++r) {
        const uint32_t c = base + r * kFinal + t;
        src[r] = -1;
        if (c < C1) {
          const int blk = cand_slice(off, c);
          const uint32_t u = c - off[blk];
          if (u >= (uint32_t)kSpec) src[r] = (int64_t)blk * kSliceMax + u;
        }
      }
#pragma unroll
      for (int r = 0; r < kRC; ++r) kk[r] = src[r] >= 0 ? w.cand[src[r]] : 0u;
#pragma unroll
      for (int r = 0; r < kRC; ++r)
        if (src[r] >= 0) dst[base + r * kFinal + t] = kk[r];
    }
  }
  __syncthreads();
  const uint32_t* ca = dst;
  // radix pass 1: key bits 18..9 of every candidate
  for (uint32_t base = 0; base < C1; base += kRC * kFinal) {
    uint32_t kk[kRC];
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const uint32_t c = base + r * kFinal + t;
      kk[r] = c < C1 ? ca[c] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const bool act = base + r * kFinal + t < C1;
      hist_add(h, nullptr, (kk[r] >> 9) & 1023u, act ? key_mass(kk[r]) : 0, act);
    }
  }
  __syncthreads();
  const uint64_t target2 = st.target - st.A1;
  select_digit<1024>(h, target2, tabA, &s_d, &s_above);
  const uint32_t d1 = (uint32_t)s_d;
  const uint64_t above2 = s_above;
  for (int j = t; j < 512; j += kFinal) h[j] = 0;
  __syncthreads();
  // radix pass 2: key bits 8..0 of the candidates in digit d1
  for (uint32_t base = 0; base < C1; base += kRC * kFinal) {
    uint32_t kk[kRC];
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const uint32_t c = base + r * kFinal + t;
      kk[r] = c < C1 ? ca[c] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const bool act = base + r * kFinal + t < C1 && ((kk[r] >> 9) & 1023u) == d1;
      hist_add(h, nullptr, kk[r] & 511u, act ? key_mass(kk[r]) : 0, act);
    }
  }
  __syncthreads();
  const uint64_t target3 = target2 - above2;
  select_digit<512>(h, target3, tabA, &s_d, &s_above);
  const uint32_t d2 = (uint32_t)s_d;
  const uint64_t above3 = s_above;
  const uint32_t kstar = ((uint32_t)(j1 - 1 + kBinBase) << 19) | (d1 << 9) | d2;
  const uint64_t A = st.A1 + above2 + above3;
  const uint64_t qs = max(key_mass(kstar), (uint64_t)1);
  const uint64_t take = (st.target - A + qs - 1) / qs;
  const uint64_t N = A + take * qs;
  // the draw d = floor(u N), u = (Philox word 0 >> 8) / 2^24, in exact integer arithmetic
  const int pos = a.desc ? a.desc->pos : a.pos_arg;
  uint32_t ctr[4] = {(uint32_t)pos, 0u, 0u, 0u};
  philox4x32_10(ctr, (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
  const uint64_t u24 = ctr[0] >> 8;
  const uint64_t d = ((u24 * (N >> 32)) << 8) + ((u24 * (N & 0xFFFFFFFFull)) >> 24);
  // nucleus mass and ties at k* of each slice among the candidates (index order = array order)
  uint32_t trun = 0;
  for (uint32_t base = 0; base < C1; base += kRC * kFinal) {
    uint32_t kk[kRC];
    bool tie[kRC];
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const uint32_t c = base + r * kFinal + t;
      kk[r] = c < C1 ? ca[c] : 0u;
      tie[r] = c < C1 && kk[r] == kstar;
    }
    uint32_t rank[kRC], ttot;
    batch_rank<kFinal, kRC>(tie, rank, tabA, &ttot);
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const uint32_t c = base + r * kFinal + t;
      const bool act = c < C1;
      const bool in = act && (kk[r] > kstar || (tie[r] && trun + rank[r] < take));
      const int blk = act ? cand_slice(off, c) : 0;
      hist_add(nb, nullptr, blk, in ? key_mass(kk[r]) : 0, in);
      hist_add(nullptr, tb, blk, 0, tie[r]);
    }
    trun += ttot;
  }
  __syncthreads();
  // the slice that holds the draw (lane = slice)
  if (t < 64) {
    const uint64_t m = nb[t] + ab;
    const uint64_t inc = wave_incl_u64(m);
    const uint64_t tinc = wave_incl_u64(tb[t]);
    if (t == 0) s_blk = -1;
    if (m > 0 && d >= inc - m && d < inc) {
      s_blk = t;
      s_dd = d - (inc - m);
      s_tb = (uint32_t)(tinc - tb[t]);
    }
  }
  __syncthreads();
  if (s_blk < 0) {  // cannot happen: the slices' masses sum to N > d
    if (t == 0) *a.out = 0;
    return;
  }
  // round trip 2: index-order scan of that slice
  int64_t lo, hi;
  slice_of(a.n, s_blk, lo, hi);
  float z[kRW];
  load_slice<kRW, kFinal>(a, lo, hi, z);
  const float M = st.M, inv_t = a.inv_temperature;
  uint32_t key[kRW];
  bool tie[kRW];
  uint64_t vgt[kRW], exg[kRW];
#pragma unroll
  for (int r = 0; r < kRW; ++r) {
    const bool act = lo + r * kFinal + t < hi;
    key[r] = act ? tok_key(z[r], inv_t, M) : 0u;
    tie[r] = act && key[r] == kstar;
    vgt[r] = act && key[r] > kstar ? key_mass(key[r]) : 0;
  }
  // exclusive prefix of the mass above k* and ranks of the ties, in index order; the ties in
  // the nucleus are the first `avail` of this slice
  uint32_t rank[kRW];
  batch_excl_rank<kFinal, kRW>(vgt, exg, tie, rank, tabB, tabA);
  const uint64_t tb0 = s_tb, dd = s_dd;
  const uint64_t avail = take > tb0 ? take - tb0 : 0;
#pragma unroll
  for (int r = 0; r < kRW; ++r) {
    const bool tin = tie[r] && rank[r] < avail;
    const uint64_t ex = exg[r] + qs * min((uint64_t)rank[r], avail);
    const uint64_t v = vgt[r] + (tin ? qs : 0);
    if (v > 0 && ex <= dd && dd < ex + v) s_pick = lo + r * kFinal + t;
  }
  __syncthreads();
  if (t == 0) *a.out = (int32_t)(s_pick >= 0 ? s_pick : lo);
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  if (!a.ws || a.n < 1 || a.n > kSB * kSliceMax) return hipErrorInvalidValue;
  const SampleWs w = carve_ws(a.ws, a.n);
  if (!a.part_val) hipLaunchKernelGGL(k_sample_max, dim3(kSB), dim3(kSBThreads), 0, s, a, w);
  hipLaunchKernelGGL(k_sample_hist, dim3(kSB), dim3(kSBThreads), 0, s, a, w);
  hipLaunchKernelGGL(k_sample_gather, dim3(kSB), dim3(kSBThreads), 0, s, a, w);
  hipLaunchKernelGGL(k_sample_select, dim3(1), dim3(kFinal), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace qd

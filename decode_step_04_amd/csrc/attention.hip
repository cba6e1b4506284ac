// attention.hip - split-KV causal GQA decode attention over a paged KV cache.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
//
// What is computed ([Qwen3-runtime] §2.5-2.6): for each query head h, with kv head
// g = h / (Hq / Hkv), scores s_j = q_h . k_j / sqrt(D) over positions j < ctx, and
// out_h = sum_j softmax(s)_j v_j.
//
// k_attn: one work-group (4 waves) per (kv head g, partition), a partition being part_tokens
// consecutive positions (whole 16-token pages).
//   - Loads are ordered for the shortest dependent chain: ctx, the partition's block-table
//     entries (read ahead of ctx; every entry below bt_len is a valid page number) and the QKV
//     rows are requested together, then each wave requests its first K/V page tile before doing
//     anything else, so HBM latency overlaps the prologue.
//   - Fused prologue (model path, [Qwen3-runtime] §2.3-2.4, §7.1-7.2): the work-group RMS-
//     normalises and rotates the G = Hq/Hkv query heads of g (one wave per head: lane l holds
//     the RoPE pair (l, l + D/2), so the norm is one wave reduction and the rotation needs no
//     data exchange).  The work-group whose partition holds the new position also normalises and
//     rotates K of head g, stores K and V at (bt[pos/16], pos%16) -- the paged append -- and uses
//     the same values in registers for that slot.
//   - Page loop ([Qwen3-runtime] §10.1-10.2): each wave takes every 4th page; a 16 x D page tile
//     of one head is contiguous and read with 16-byte loads, and all G heads use the same K/V
//     registers, so each K/V byte is read once for the whole query group ([Qwen3-runtime] §2.5).
//     fp32 (m, l, acc) state per head ([ETE], the online-softmax passage).  Three page loops:
//       * D = 128, bf16 K/V, G = 4 or 8: the dot products run on the matrix cores, with the fp32
//         query and probabilities each split into two bf16 parts (the comment at the loop gives
//         the layout); non-temporal page loads (every byte is used once).
//       * D = 128, bf16 K/V, G = 1 or 2: transposed scores on the vector ALUs (TrGeo) -- with one
//         or two heads the per-page VALU work is small and its shorter dependency chain measured
//         faster than the matrix-core loop.
//       * Other shapes (fp32 K/V, D = 64, other G): lane l holds EPL consecutive dims of one
//         token per load (token row l / LPT); scores are reduced over the LPT lanes of a token
//         with DPP and each token row keeps its own state.
//   - Rows, then waves (LDS), are combined exactly ([Qwen3-runtime] §9.1).  With one partition
//     the normalised output is written directly (the short path of §10.1); otherwise the
//     unnormalised state goes to scratch for k_attn_merge.
// k_attn_merge: one work-group per (query head, 32 dims): M = max m_p, w_p = 2^(m_p - M),
// out = sum w_p acc_p / sum w_p l_p.
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

// Matrix-core operands (bf16 K/V, D = 128)
typedef __bf16 mf_bf8 __attribute__((ext_vector_type(8)));
typedef short mf_s4 __attribute__((ext_vector_type(4)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u4 __attribute__((ext_vector_type(4)));


// Per-head RMSNorm (when `norm`) and rotate-half RoPE of one D-vector by one wave; lane l holds
// the pair (x0, x1) = (v[l], v[l + D/2]) and its gammas (g0, g1) (zeros for l >= D/2) and gets
// the rotated pair.
// Branch-free, so that the compiler keeps the gamma loads where they are issued.
template <int D>
__device__ __forceinline__ void norm_rope(float x0, float x1, bool norm, float g0, float g1,
                                          float eps, float2 cs, float& y0, float& y1) {
  const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
  const float rinv = norm ? __builtin_amdgcn_rsqf(ss / (float)D + eps) : 1.0f;
  x0 = norm ? x0 * rinv * g0 : x0;
  x1 = norm ? x1 * rinv * g1 : x1;
  y0 = x0 * cs.x - x1 * cs.y;
  y1 = x1 * cs.x + x0 * cs.y;
}

// Merges the (m, l, acc) states of the lane pairs (l, l ^ OFF): M = max, each side rescaled by
// 2^(m - M).  Both lanes of a pair end with the same merged state.
template <int OFF, int G, int EPL>
__device__ __forceinline__ void combine_rows(float (&m)[G], float (&l)[G], float (&acc)[G][EPL]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ma, mb, la, lb;
    lane_pair<OFF>(m[h], ma, mb);
    lane_pair<OFF>(l[h], la, lb);
    const float mx = fmaxf(ma, mb);
    const float ca = fast_exp2(ma - mx), cb = fast_exp2(mb - mx);
    l[h] = fmaf(la, ca, lb * cb);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float aa, ab;
      lane_pair<OFF>(acc[h][e], aa, ab);
      acc[h][e] = fmaf(aa, ca, ab * cb);
    }
    m[h] = mx;
  }
}

// ---- transposed scores (D = 128, bf16 K/V: 16 lanes per token, 4 tokens per lane and page) ----
// After the per-lane partial dot products, a lane holds NV = 4G partial scores (head h, token
// slot i at index 4h + i), each a partial sum over the lane's 8 dims.  A transpose-reduce over
// the 16 lanes of a row halves the values at each of four lane pairings (xor 8, 7, 3, 1, deciding
// by bit 3, 2, 1, 0 of the lane in the row which half a lane keeps), so that every lane ends
// with complete scores of its own (head, slot) -- one softmax exponential per score instead of
// one in each of the 16 lanes of the token.  With fewer than 16 values the last pairings are
// plain sums, and lanes that differ only in those bits hold duplicates.
template <int G>
struct TrGeo {
  static constexpr int NV = 4 * G;                                   // partial scores per lane
  static constexpr int H = NV >= 16 ? 4 : NV == 8 ? 3 : NV == 4 ? 2 : 1;  // halving pairings
  static constexpr int NVF = NV >> H;                                // complete scores per lane
  static constexpr int DUP = (1 << (4 - H)) - 1;                     // duplicate-lane bits
  static constexpr int GS = (4 / NVF) << (4 - H);                    // lanes of one head in a row
  // lane in the row holding score index v, and its slot there
  static constexpr int lane_of(int v) { return (v / NVF) << (4 - H); }
  static constexpr int slot_of(int v) { return v % NVF; }
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "head groups of 1, 2, 4 or 8");
};


// One pairing of the transpose-reduce over the first CNT values: lanes x and x ^ (pairing) both
// form a + a' and b + b' for each pair (a, b) = (v[k], v[CNT/2 + k]), and keep the first when
// `hi` is clear; with CNT <= 1 the single value is summed with its partner's.
template <int CTRL, int CNT, int N>
__device__ __forceinline__ void tr_step(float (&v)[N], bool hi) {
  if constexpr (CNT > 1) {
    constexpr int HF = CNT / 2;
#pragma unroll
    for (int k = 0; k < HF; ++k) {
      const float sa = v[k] + dpp<CTRL>(v[k]);
      const float sb = v[HF + k] + dpp<CTRL>(v[HF + k]);
      v[k] = hi ? sb : sa;
    }
  } else {
    v[0] += dpp<CTRL>(v[0]);
  }
}

template <int NV>
__device__ __forceinline__ void transpose_reduce16(float (&v)[NV], int c) {
  tr_step<0x128, NV>(v, (c & 8) != 0);        // xor 8
  tr_step<0x141, NV / 2>(v, (c & 4) != 0);    // xor 7 (half mirror)
  tr_step<0x1B, NV / 4>(v, (c & 2) != 0);     // xor 3 (quad mirror)
  tr_step<0xB1, NV / 8>(v, (c & 1) != 0);     // xor 1
}

// The score of index v (head v / 4, slot v % 4) for every lane of the row: read from the lane
// of the row that owns it (DPP row broadcast, gfx950 row_newbcast).  v is a compile-time index
// after unrolling.
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<0x150 + L>(x);
}

template <int G>
__device__ __forceinline__ float bcast_slot(const float (&sv)[4 * G], int v) {
  using Tg = TrGeo<G>;
  const int ln = Tg::lane_of(v), k = Tg::slot_of(v);
  const float x = Tg::NVF == 1 ? sv[0] : (k == 0 ? sv[0] : sv[1]);
  switch (ln) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
  }
}

// maximum over aligned groups of GS lanes of a row (GS = 1, 2, 4, 8 or 16)
template <int GS>
__device__ __forceinline__ float group_max_any(float v) {
  if constexpr (GS >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (GS >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (GS >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (GS >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

constexpr int kAttnWaves = 4;  // waves per work-group of k_attn (8 measured slower at both shapes)
constexpr int kAttnThreads = kAttnWaves * kWave;

// The matrix-core page loop of the plain (not fused) kernel fits in 128 registers for groups of
// 4: four work-groups per CU instead of three (long contexts launch more than three per CU).  The
// fused kernel would spill at that bound, and G = 8 is held to three by its LDS.
template <int D, bool KVB, int G, bool FUSED>
constexpr int attn_waves_per_simd() {
  return !FUSED && D == 128 && KVB && G == 4 ? 4 : 1;
}

template <int D, bool KVB, int G, bool FUSED>
__global__ __launch_bounds__(kAttnThreads) __attribute__((
    amdgpu_waves_per_eu(attn_waves_per_simd<D, KVB, G, FUSED>()))) void k_attn(AttnArgs a) {
  using Gm = Geo<D, KVB>;
  constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TPI = Gm::TPI, NI = Gm::NI, ELEM = Gm::ELEM;
  constexpr int HALF = D / 2;
  constexpr int NW = kAttnWaves, NT = kAttnThreads;
  constexpr int NPH = kMaxPartTokens / kPage / NW;  // block-table entries per wave, read ahead
  constexpr int QT = (G + NW - 1) / NW;             // query heads per wave in the prologue
  // 128-dim bf16 pages: matrix-core pages for head groups of 4 and 8; transposed scores on the
  // vector ALUs for groups of 1 and 2 (at that width the VALU work per page is small and the
  // shorter dependency chain per page wins)
  constexpr bool MF = D == 128 && KVB && (G == 4 || G == 8);
  constexpr bool TR = D == 128 && KVB && (G == 1 || G == 2);
  constexpr int VROW = D + 16;      // LDS row of a staged V page, in bf16 (288 bytes)
  __shared__ float sq[G][D];        // scaled query heads
  __shared__ __attribute__((aligned(16))) uint16_t svp[MF ? NW * kPage * VROW : 1];
  // matrix-core pages: the scaled query heads split into bf16 hi = bf16(q) and lo = bf16(q - hi).
  // Rows of 288 bytes: with 256 (a whole bank cycle) every column's 16-byte operand read of a
  // k-step sat on the same four banks.  rocprofv3's SQ_LDS_BANK_CONFLICT at G = 4 (8B shape, 8K
  // positions): 426K stall cycles per launch with 256-byte rows, 98K with 288; the launch time
  // did not change (the page loop waits on memory, not on the LDS)
  constexpr int QROW = MF ? D + 16 : D;
  __shared__ __attribute__((aligned(16))) uint16_t sqb[MF ? G : 1][2][QROW];
  auto put_q = [&](int h, int d, float x) {
    sq[h][d] = x;
    if constexpr (MF) {
      const uint16_t hb = f32_to_bf16(x);
      sqb[h][0][d] = hb;
      sqb[h][1][d] = f32_to_bf16(x - bf16_to_f32(hb));
    }
  };
  __shared__ float skv[2][D];       // K and V of the new token (as stored)
  // matrix-core pages of the fused kernel: the same K and V as bf16, patched into their page
  __shared__ __attribute__((aligned(16))) uint16_t skvb[MF && FUSED ? 2 : 1][D];
  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];

  // Matrix-core pages take the wave index as a scalar: its block-table entries, pages and token
  // ranges are then wave-uniform values (scalar loads and registers, uniform branches), which
  // the 128-register budget needs.  (The other paths measured faster without.)
  const int lane = threadIdx.x & 63;
  const int wave = MF ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int hkv = a.n_kv_heads;
  const int g = blockIdx.x % hkv;
  const int pi = blockIdx.x / hkv;
  const int part = a.part_tokens;
  const int ppp = part / kPage;                  // pages per partition
  const int pg_first = pi * ppp;

  // ---- independent loads: block-table entries, ctx, the QKV rows of the prologue.  Every load
  //      of the kernel is issued unconditionally (an unused one reads a valid clamped address and
  //      its value is discarded): loads complete in order, and with no load under a branch each
  //      wait the compiler inserts covers exactly the loads its consumer needs ----
  int phys[NPH];
  const int npw = (ppp + NW - 1 - wave) / NW;    // pages of this wave in a full partition
#pragma unroll
  for (int j = 0; j < NPH; ++j) {
    const int idx = pg_first + wave + NW * j;
    const bool ok = j < npw && idx < a.bt_len;   // bt_len >= 1: entry 0 always exists
    const int v = a.block_table[ok ? idx : 0];
    phys[j] = ok ? v : 0;
  }
  constexpr int QP = (G * D + NT - 1) / NT;      // op path: query values per thread
  float qx0[QT], qx1[QT];                        // fused path: this wave's query heads wave + NW t
  float kx0 = 0.f, kx1 = 0.f, vx0 = 0.f, vx1 = 0.f;
  float gq0 = 0.f, gq1 = 0.f, gk0 = 0.f, gk1 = 0.f;  // Q/K-norm gammas of this lane's pair
  float qop[QP];
  const bool qk_norm = a.q_gamma != nullptr;
  const int hl = lane & (HALF - 1);              // lanes >= D/2 read lane - D/2, then zero it
  const bool lo_half = lane < HALF;
  float2 cs = make_float2(1.f, 0.f);              // (cos, sin) of this lane's pair at pos
  if constexpr (FUSED) {
    cs = reinterpret_cast<const float2*>(a.rope_step)[hl];
    const float* gqs = qk_norm ? a.q_gamma : a.qkv;
    const float* gks = qk_norm ? a.k_gamma : a.qkv;
    gq0 = gqs[hl];
    gq1 = gqs[hl + HALF];
    gk0 = gks[hl];
    gk1 = gks[hl + HALF];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int h = wave + NW * t;
      const float* src = a.qkv + (int64_t)(g * G + (h < G ? h : 0)) * D;
      qx0[t] = src[hl];
      qx1[t] = src[hl + HALF];
    }
    const float* ks = a.qkv + (int64_t)(a.n_q_heads + g) * D;
    const float* vs = a.qkv + (int64_t)(a.n_q_heads + hkv + g) * D;
    kx0 = ks[hl];
    kx1 = ks[hl + HALF];
    vx0 = vs[hl];
    vx1 = vs[hl + HALF];
  } else {
#pragma unroll
    for (int t = 0; t < QP; ++t) {
      const int i = threadIdx.x + NT * t;
      const int idx = g * G * D + (i < G * D ? i : 0);
      qop[t] = a.q_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[idx])
                        : static_cast<const float*>(a.q)[idx];
    }
  }
  // the context length last: scalar loads are waited for all at once, so the loads above are
  // issued before the wait for this one
  const int ctx = a.desc ? a.desc->ctx : a.ctx_arg;
  const int pos = ctx - 1;
  const int np = n_parts_for(ctx, part);
  // Surplus partitions (a graph captured for a longer context) run through with empty ranges
  // and store nothing; returning early instead would let the compiler move the loads above
  // below that branch, behind the context load.
  const bool live = pi < np;
  const int tok0 = pi * part;
  const int tok1 = min(ctx, tok0 + part);
  const int pg1 = (tok1 + kPage - 1) / kPage;    // one past the last page of the partition
  const bool has_new = FUSED && (pos >= tok0) && (pos < tok1);

  // ---- the page of the new token, then this wave's first page tile (page 0's when the wave has
  //      none; those values are never used) ----
  int64_t phys_new = 0;
  if constexpr (FUSED) phys_new = a.block_table[pos / kPage];
  const int64_t tile_bytes = (int64_t)kPage * D * ELEM;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  // pages are requested one ahead of the one being computed, in two alternating register sets
  // (separate arrays: indexing one array by set would make the compiler move registers)
  uint4 k0[NI], v0[NI], k1[NI], v1[NI];
  int t0, t1;  // physical page of each set
  int pg = pg_first + wave;
  const int gh = live ? g : 0;
  // Matrix-core pages read K as the A operand of v_mfma_f32_16x16x32_bf16: load ks of lane l is
  // token l % 16, dims 32 ks + 8 (l / 16) .. + 7 (64 contiguous bytes per token and load).
  const int64_t kmf = ((int64_t)(lane & 15) * D + 8 * (lane >> 4)) * ELEM;
  // The address is computed from a page number chosen by a select (not a select of two
  // addresses), so the compiler cannot fold a re-request into a copy of another set's registers.
  // Matrix-core pages use non-temporal loads: each byte of the pages is read once (measured 10 %
  // faster at 128K positions than cached loads; on the transposed-score path they measured
  // slower inside the decode step).
  auto load16 = [](const char* p) {
    const mf_u4 x = MF ? __builtin_nontemporal_load(reinterpret_cast<const mf_u4*>(p))
                       : *reinterpret_cast<const mf_u4*>(p);
    return make_uint4(x[0], x[1], x[2], x[3]);
  };
  auto request = [&](uint4 (&kd)[NI], uint4 (&vd)[NI], int& td, int ph) {
    td = ph;
    const int64_t tile = ((int64_t)ph * hkv + gh) * tile_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kd[i] = load16(kbase + tile + (MF ? kmf + 64 * i : (int64_t)(i * kWave + lane) * 16));
#pragma unroll
    for (int i = 0; i < NI; ++i) vd[i] = load16(vbase + tile + (int64_t)(i * kWave + lane) * 16);
  };
  // a surplus partition reads page 0 of head 0 (cached after the first), not HBM
  request(k0, v0, t0, live ? phys[0] : 0);
  if (!lo_half) {
#pragma unroll
    for (int t = 0; t < QT; ++t) qx0[t] = qx1[t] = 0.f;
    kx0 = kx1 = vx0 = vx1 = 0.f;
    gq0 = gq1 = gk0 = gk1 = 0.f;
    cs = make_float2(1.f, 0.f);
  }

  // ---- prologue: query heads (and the new K/V) into LDS.  Every wave computes every norm and
  //      rotation (cheap) and stores only what it owns: with the values used unconditionally the
  //      compiler keeps their loads ahead of the page loads, instead of moving them into the
  //      branch that would use them ----
  if constexpr (FUSED) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int h = wave + NW * t;
      float y0, y1;
      norm_rope<D>(qx0[t], qx1[t], qk_norm, gq0, gq1, a.eps, cs, y0, y1);
      if (a.round_q) {
        y0 = round_bf16(y0);
        y1 = round_bf16(y1);
      }
      if (h < G && lane < HALF) {
        put_q(h, lane, y0 * a.qscale);
        put_q(h, lane + HALF, y1 * a.qscale);
      }
    }
    float y0, y1;
    norm_rope<D>(kx0, kx1, qk_norm, gk0, gk1, a.eps, cs, y0, y1);
    float v0 = vx0, v1 = vx1;
    if constexpr (KVB) {
      y0 = round_bf16(y0); y1 = round_bf16(y1); v0 = round_bf16(v0); v1 = round_bf16(v1);
    }
    if (has_new && wave == NW - 1 && lane < HALF) {
      const int64_t off = ((phys_new * hkv + g) * kPage + pos % kPage) * D + lane;
      if constexpr (KVB) {
        uint16_t* kp = static_cast<uint16_t*>(a.k_pool);
        uint16_t* vp = static_cast<uint16_t*>(a.v_pool);
        kp[off] = f32_to_bf16(y0); kp[off + HALF] = f32_to_bf16(y1);
        vp[off] = f32_to_bf16(v0); vp[off + HALF] = f32_to_bf16(v1);
      } else {
        float* kp = static_cast<float*>(a.k_pool);
        float* vp = static_cast<float*>(a.v_pool);
        kp[off] = y0; kp[off + HALF] = y1;
        vp[off] = v0; vp[off + HALF] = v1;
      }
      skv[0][lane] = y0; skv[0][lane + HALF] = y1;
      skv[1][lane] = v0; skv[1][lane + HALF] = v1;
      if constexpr (MF && FUSED) {
        skvb[0][lane] = f32_to_bf16(y0); skvb[0][lane + HALF] = f32_to_bf16(y1);
        skvb[1][lane] = f32_to_bf16(v0); skvb[1][lane + HALF] = f32_to_bf16(v1);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < QP; ++t) {
      const int i = threadIdx.x + NT * t;
      if (i < G * D) put_q(i / D, i % D, qop[t] * a.qscale);
    }
  }
  __syncthreads();

  const int dsub = (lane % LPT) * EPL;
  const int trow = lane / LPT;
  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] = sq[h][dsub + e];
  // Fully unrolled page loops below: every step's code follows the previous one's with no loop
  // back-edge, so each wait counts exactly the loads in flight (a loop makes the compiler drain
  // all loads before entering it).  One page per step: request the wave's next page (on the last
  // page the current one again, served by the caches, so that no load sits under a branch), then
  // compute the current one; the two register sets alternate between the steps (copying an
  // in-flight load's registers would make the compiler wait for it).
  if constexpr (MF) {
    // Matrix-core pages.  Scores S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = the page's 16 tokens
    // x 32 dims, B = 32 dims x 16 columns), then O^T += V^T P^T on v_mfma_f32_16x16x16_bf16
    // (A = 16 dims x the page's 16 tokens, B = P^T).  The query and the probabilities are fp32,
    // the operands bf16: each is split into a rounded part and the rounded rest (x = hi + lo to
    // about 2^-17 relative), and column 2h of B carries hi of head h, column 2h + 1 lo of head h
    // (columns from 2G on are zero).  Lane l receives the scores of tokens 4 (l / 16) + j (j < 4) of
    // column l % 16; a lane adds its partner column's value (DPP lane xor 1, applied to every lane:
    // a DPP read under a lane-dependent branch would see its partner disabled), so both lanes of
    // a head hold its complete scores and run the same softmax, each producing its own part of
    // P -- which is already the B operand of the second product (its keys are 4 (l / 16) + j, the
    // same tokens).  The running maximum of a head is reduced over the four
    // rows, so the whole page shares it.  V is staged row-major in the wave's LDS tile and read as
    // V^T with ds_read_b64_tr_b16.  O^T lands with lane l holding dims 16 T + 4 (l / 16) + j of
    // column l % 16; the hi and lo columns are added at the end.  The appended token (pos) goes
    // through the same products: on its page, its K and V as stored (from LDS) replace what the
    // page load returned (the load may have been issued before the append).
    const int c = lane & 15, r = lane >> 4;
    const bool hi_col = (c & 1) == 0, used = c < 2 * G;
    const int hc = used ? c >> 1 : 0;              // head of this lane's column
    uint16_t* vw = svp + wave * kPage * VROW;
    // this lane's B operand of the scores: dims 32 ks + 8 (l / 16) .. + 7 of its column's part
    // (columns from 2G on repeat head 0; their scores are never used)
    const uint16_t* qrow = &sqb[hc][c & 1][8 * r];
    float mL = -1e30f, lL = 0.f;
    mf_f4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mf_f4{0.f, 0.f, 0.f, 0.f};
    const int pg_new = has_new ? pos / kPage : -1;  // page of the appended token (wave-uniform)
    const int slot_new = pos % kPage;

    auto page_step = [&](const uint4 (&ck)[NI], const uint4 (&cv)[NI], int tc, uint4 (&nk)[NI],
                         uint4 (&nv)[NI], int& tn, int ph1) {
      // the query operand is re-read from LDS on every page (an empty asm with a memory
      // clobber keeps the compiler from holding it in registers across the pages)
      asm volatile("" ::: "memory");
      request(nk, nv, tn, (pg + NW < pg1) ? ph1 : tc);
      mf_u4 kk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = mf_u4{ck[ks].x, ck[ks].y, ck[ks].z, ck[ks].w};
      if (FUSED && pg == pg_new) {
        // the appended token's K replaces its row (lanes l % 16 == slot)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const mf_u4 x = *reinterpret_cast<const mf_u4*>(&skvb[0][32 * ks + 8 * r]);
          kk[ks] = c == slot_new ? x : kk[ks];
        }
      }
      mf_f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(mf_bf8, kk[ks]),
            __builtin_bit_cast(mf_bf8, *reinterpret_cast<const mf_u4*>(qrow + 32 * ks)), st, 0,
            0, 0);
      float s[4], pmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = st[j] + dpp<kDppXor1>(st[j]);
        const int tok = pg * kPage + 4 * r + j;
        s[j] = (used && tok < tok1) ? x : -INFINITY;
        pmax = fmaxf(pmax, s[j]);
      }
      {
        float lo, hi;
        lane_pair<16>(pmax, lo, hi);
        pmax = fmaxf(lo, hi);
        lane_pair<32>(pmax, lo, hi);
        pmax = fmaxf(lo, hi);
      }
      const float mnew = fmaxf(mL, pmax);
      if (__builtin_amdgcn_ballot_w64(mnew > mL) != 0) {  // wave-uniform
        const float cL = fast_exp2(mL - mnew);
        lL *= cL;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= cL;
        mL = mnew;
      }
      mf_s4 pb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(s[j] - mL);     // 0 for masked tokens and unused columns
        lL += p;
        const float ph = round_bf16(p);
        pb[j] = (short)f32_to_bf16(hi_col ? ph : p - ph);
      }
      // V row-major into the wave's tile: load i of lane l is token 4 i + l / 16, dims 8 (l % 16)
      // (then the appended token's row, written after, so it wins).  Staged only now: the wait
      // for V's loads would otherwise hold up the scores, which need only K (the empty asm keeps
      // the compiler from moving the stores up).
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<mf_u4*>(vw + (4 * i + r) * VROW + 8 * c) =
            mf_u4{cv[i].x, cv[i].y, cv[i].z, cv[i].w};
      if (FUSED && pg == pg_new && r == 0)
        *reinterpret_cast<mf_u4*>(vw + slot_new * VROW + 8 * c) =
            *reinterpret_cast<const mf_u4*>(&skvb[1][8 * c]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const mf_s4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) mf_s4*)(vw + (4 * r + (c >> 2)) * VROW + 16 * t +
                                                       4 * (c & 3)));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[t], 0, 0, 0);
      }
      pg += NW;
    };
#pragma unroll
    for (int jj = 0; jj < NPH; ++jj) {
      if (pg >= pg1) break;
      const int ph1 = jj + 1 < NPH ? phys[jj + 1 < NPH ? jj + 1 : 0] : 0;
      if (jj % 2 == 0)
        page_step(k0, v0, t0, k1, v1, t1, ph1);
      else
        page_step(k1, v1, t1, k0, v0, t0, ph1);
    }
    float lsum;
    {
      float lo, hi;
      lane_pair<16>(lL, lo, hi);
      lane_pair<32>(lo + hi, lo, hi);
      lsum = lo + hi;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t][j] += dpp<kDppXor1>(acc[t][j]);
    if (hi_col && used) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<mf_f4*>(&sm_acc[wave][hc][16 * t + 4 * r]) = acc[t];
      if (r == 0) {
        sm_m[wave][hc] = mL;
        sm_l[wave][hc] = lsum;
      }
    }
  } else if constexpr (TR) {
    // Transposed scores (TrGeo): each lane owns NVF complete scores -- head hL, token slots
    // iK[k] of its row -- so the softmax runs once per score.  The running maximum of each head
    // is shared by the whole wave (page maxima are reduced over the head's lanes and the rows),
    // so the accumulators of the four rows need no rescaling against each other, and a page
    // whose maxima do not grow skips the rescaling altogether (a wave-uniform branch).  The
    // appended token (pos) is left out of the pages and folded in once afterwards.
    using Tg = TrGeo<G>;
    constexpr int NV = Tg::NV, NVF = Tg::NVF;
    const int c = lane & 15;                       // lane in its 16-lane row; trow = lane >> 4
    const int vbase = (c >> (4 - Tg::H)) * NVF;    // score index of slot 0 of this lane
    const int hL = vbase >> 2;                     // its head
    const bool nondup = (c & Tg::DUP) == 0;        // counts its scores (duplicates do not)
    auto first_lane = [](int h) { return Tg::lane_of(4 * h); };
    float mL = -1e30f, lL = 0.f, acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    const int tlim = has_new ? pos : tok1;         // the appended token comes after the pages

    auto page_step = [&](const uint4 (&ck)[NI], const uint4 (&cv)[NI], int tc, uint4 (&nk)[NI],
                         uint4 (&nv)[NI], int& tn, int ph1) {
      request(nk, nv, tn, (pg + NW < pg1) ? ph1 : tc);
      // partial scores over the lane's 8 dims, then the transpose-reduce over the row
      float sv[NV];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[EPL];
        widen16<KVB, EPL>(ck[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], kf[e], p);
          sv[4 * h + i] = p;
        }
      }
      transpose_reduce16<NV>(sv, c);
      float pmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        const int tok = pg * kPage + ((vbase + k) & 3) * TPI + trow;
        sv[k] = tok < tlim ? sv[k] : -INFINITY;
        pmax = fmaxf(pmax, sv[k]);
      }
      pmax = group_max_any<Tg::GS>(pmax);
      {
        float lo, hi;
        lane_pair<16>(pmax, lo, hi);
        pmax = fmaxf(lo, hi);
        lane_pair<32>(pmax, lo, hi);
        pmax = fmaxf(lo, hi);
      }
      const float mnew = fmaxf(mL, pmax);
      if (__builtin_amdgcn_ballot_w64(mnew > mL) != 0) {  // wave-uniform
        const float cL = fast_exp2(mL - mnew);
        lL *= cL;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ch = lane_value(cL, first_lane(h));
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= ch;
        }
        mL = mnew;
      }
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        sv[k] = fast_exp2(sv[k] - mL);
        lL += sv[k];
      }
      // P V: the probability of (head h, slot i) comes from the lane of the row that owns it
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[EPL];
        widen16<KVB, EPL>(cv[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pb = bcast_slot<G>(sv, 4 * h + i);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pb, vf[e], acc[h][e]);
        }
      }
      pg += NW;
    };
#pragma unroll
    for (int jj = 0; jj < NPH; ++jj) {
      if (pg >= pg1) break;
      const int ph1 = jj + 1 < NPH ? phys[jj + 1 < NPH ? jj + 1 : 0] : 0;
      if (jj % 2 == 0)
        page_step(k0, v0, t0, k1, v1, t1, ph1);
      else
        page_step(k1, v1, t1, k0, v0, t0, ph1);
    }
    // the appended token, folded into wave 0's state (its K and V as stored, from LDS)
    if (has_new && wave == 0) {
      float sh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], skv[0][dsub + e], p);
        sh[h] = lanes_sum<16>(p);
      }
      float sL = sh[0];
#pragma unroll
      for (int h = 1; h < G; ++h) sL = hL == h ? sh[h] : sL;
      const float mnew = fmaxf(mL, sL);
      const float cL = fast_exp2(mL - mnew), pL = fast_exp2(sL - mnew);
      lL = fmaf(lL, cL, lane == first_lane(hL) ? pL : 0.f);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ch = lane_value(cL, first_lane(h));
        const float ph = trow == 0 ? lane_value(pL, first_lane(h)) : 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(acc[h][e], ch, ph * skv[1][dsub + e]);
      }
      mL = mnew;
    }
    // the four rows share each head's maximum: their accumulators add up as they are
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float lo, hi;
        lane_pair<16>(acc[h][e], lo, hi);
        lane_pair<32>(lo + hi, lo, hi);
        acc[h][e] = lo + hi;
      }
    float lh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lh[h] = wave_sum(hL == h && nondup ? lL : 0.f);
    if (trow == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_acc[wave][h][dsub + e] = acc[h][e];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sm_m[wave][h] = lane_value(mL, first_lane(h));
        sm_l[wave][h] = lh[h];
      }
    }
  } else {
    float m[G], l[G], acc[G][EPL];
  #pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -1e30f;
      l[h] = 0.f;
  #pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }

    auto page_step = [&](const uint4 (&ck)[NI], const uint4 (&cv)[NI], int tc, uint4 (&nk)[NI],
                         uint4 (&nv)[NI], int& tn, int ph1) {
      request(nk, nv, tn, (pg + NW < pg1) ? ph1 : tc);
      // scores from K first; V is still arriving (loads complete in order)
      float s[G][NI];
  #pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[EPL];
        widen16<KVB, EPL>(ck[i], kf);
        const int tok = pg * kPage + i * TPI + trow;
        if (has_new && tok == pos) {  // the appended slot: use the values just computed
  #pragma unroll
          for (int e = 0; e < EPL; ++e) kf[e] = skv[0][dsub + e];
        }
  #pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = 0.f;
  #pragma unroll
          for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], kf[e], p);
          p = lanes_sum<LPT>(p);
          s[h][i] = (tok < tok1) ? p : -INFINITY;
        }
      }
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
          s[h][i] = fast_exp2(s[h][i] - mx);
          l[h] += s[h][i];
        }
        m[h] = mx;
      }
  #pragma unroll
      for (int i = 0; i < NI; ++i) {
        float vf[EPL];
        widen16<KVB, EPL>(cv[i], vf);
        const int tok = pg * kPage + i * TPI + trow;
        if (has_new && tok == pos) {
  #pragma unroll
          for (int e = 0; e < EPL; ++e) vf[e] = skv[1][dsub + e];
        }
  #pragma unroll
        for (int h = 0; h < G; ++h)
  #pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(s[h][i], vf[e], acc[h][e]);
      }
      pg += NW;
    };
  #pragma unroll
    for (int jj = 0; jj < NPH; ++jj) {
      if (pg >= pg1) break;
      const int ph1 = jj + 1 < NPH ? phys[jj + 1 < NPH ? jj + 1 : 0] : 0;
      if (jj % 2 == 0)
        page_step(k0, v0, t0, k1, v1, t1, ph1);
      else
        page_step(k1, v1, t1, k0, v0, t0, ph1);
    }

    // combine the token rows of the wave (lanes with equal dims), exact rescaling
    if constexpr (LPT <= 8) combine_rows<8, G, EPL>(m, l, acc);
    if constexpr (LPT <= 16) combine_rows<16, G, EPL>(m, l, acc);
    combine_rows<32, G, EPL>(m, l, acc);
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
  }
  __syncthreads();

  // combine the waves; threads cover (head, dim) pairs
  for (int idx = threadIdx.x; idx < G * D; idx += NT) {
    const int h = idx / D, r = idx % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = fast_exp2(sm_m[w][h] - M);
      L = fmaf(sm_l[w][h], c, L);
      O = fmaf(sm_acc[w][h][r], c, O);
    }
    const int hq = g * G + h;
    if (!live) {
      // nothing to store
    } else if (np == 1 && !a.to_partials) {
      const float o = O / L;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[hq * D + r] = f32_to_bf16(o);
      else
        static_cast<float*>(a.out)[hq * D + r] = o;
    } else {
      const int64_t slot = (int64_t)hq * a.max_parts + a.part_base + pi;
      a.part_acc[slot * D + r] = O;
      if (r == 0) {
        a.part_ml[slot * 2 + 0] = M;
        a.part_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// One work-group of NW waves per (query head, 64 dims); lane l of every wave owns dim l of the
// block.  NW = 1 when the scratch holds at most CH partitions per head, else 4.
// Partitions are folded in chunks of CH: lane j < CH holds the (m, l) pair of partition p0 + j,
// so the chunk maximum and the denominator are wave reductions, and every lane reads the weights
// from the lanes that hold them.  Wave w takes the chunks w, w + 4, ...; its first chunk is
// requested before the context length is known (every slot below max_parts is valid scratch;
// slots at or past the step's partition count hold stale bits and are masked by selects), so a
// merge of up to CH partitions is one memory round trip after launch, done by wave 0 alone with
// no LDS and no barrier.  Longer merges (NW = 4) request each chunk of a wave while folding the one
// before, in two alternating register sets, and combine the four waves' states through LDS.  The
// running sums are rescaled to each chunk's maximum (exact up to rounding).
constexpr int kMergeChunk = 32;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_merge(AttnArgs a) {
  constexpr int CH = kMergeChunk;
  __shared__ float s_m[NW], s_l[NW], s_o[NW][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = blockIdx.x;
  const int dim = blockIdx.y * 64 + lane;
  const int maxp = a.max_parts;
  const int64_t base = (int64_t)hq * maxp;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + base;
  const float* acc = a.part_acc + base * D + dim;
  // In the chunk loop an empty asm with a memory clobber keeps the compiler from moving a chunk's
  // loads down to their use in the following fold, which would serialise the chunks; it emits no
  // instruction.
  auto request = [&](float2& mv, float (&pv)[CH], int p0, int last) {
    mv = ml[min(p0 + (lane & (CH - 1)), last)];
#pragma unroll
    for (int j = 0; j < CH; ++j) pv[j] = acc[(int64_t)min(p0 + j, last) * D];
    if constexpr (NW > 1) asm volatile("" ::: "memory");
  };
  float2 mlA, mlB;
  float pA[CH], pB[CH];
  request(mlA, pA, wave * CH, maxp - 1);
  const int ctx = a.desc ? a.desc->ctx : a.ctx_arg;
  const int np = n_parts_for(ctx, a.part_tokens);
  float M = -1e30f, L = 0.f, O = 0.f;
  auto fold = [&](const float2& mv, const float (&pv)[CH], int p0) {
    const bool ok = lane < CH && p0 + lane < np;
    const float mx = fmaxf(M, wave_max(ok ? mv.x : -1e30f));
    const float w = ok ? fast_exp2(mv.x - mx) : 0.f;
    const float c = fast_exp2(M - mx);
    L = fmaf(L, c, wave_sum(ok ? w * mv.y : 0.f));
    O *= c;
#pragma unroll
    for (int j = 0; j < CH; ++j) O = fmaf(lane_value(w, j), p0 + j < np ? pv[j] : 0.f, O);
    M = mx;
  };
  auto store = [&](float o) {
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[hq * D + dim] = f32_to_bf16(o);
    else
      static_cast<float*>(a.out)[hq * D + dim] = o;
  };
  if (NW == 1 || np <= CH) {  // uniform; with one partition the partition kernel wrote the output
    if (wave == 0 && (np > 1 || a.to_partials)) {
      fold(mlA, pA, 0);
      store(O / L);
    }
    return;
  }
  constexpr int STEP = NW * CH;
  int p0 = wave * CH;
  if (p0 < np) {  // wave-uniform
    request(mlB, pB, p0 + STEP, np - 1);
    fold(mlA, pA, p0);
    for (p0 += STEP; p0 < np;) {
      request(mlA, pA, p0 + STEP, np - 1);
      fold(mlB, pB, p0);
      p0 += STEP;
      if (p0 >= np) break;
      request(mlB, pB, p0 + STEP, np - 1);
      fold(mlA, pA, p0);
      p0 += STEP;
    }
  }
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = L;
  }
  s_o[wave][lane] = O;
  __syncthreads();
  if (wave == 0) {
    float mx = s_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_m[w]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = fast_exp2(s_m[w] - mx);  // 0 for a wave that had no partition
      lt = fmaf(s_l[w], c, lt);
      ot = fmaf(s_o[w][lane], c, ot);
    }
    store(ot / lt);
  }
}

template <int D, bool KVB, bool FUSED>
static hipError_t launch_dkf(int group, const AttnArgs& a, int grid_parts, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv_heads * grid_parts)), block(kAttnThreads);
  switch (group) {
    case 1: hipLaunchKernelGGL((k_attn<D, KVB, 1, FUSED>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn<D, KVB, 2, FUSED>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn<D, KVB, 3, FUSED>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn<D, KVB, 4, FUSED>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_attn<D, KVB, 5, FUSED>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_attn<D, KVB, 6, FUSED>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_attn<D, KVB, 7, FUSED>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_attn<D, KVB, 8, FUSED>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int head_dim, bool kv_bf16, int group, bool fused, const AttnArgs& a,
                            int grid_parts, hipStream_t s) {
  if (head_dim == 64) {
    if (kv_bf16) return fused ? launch_dkf<64, true, true>(group, a, grid_parts, s)
                              : launch_dkf<64, true, false>(group, a, grid_parts, s);
    return fused ? launch_dkf<64, false, true>(group, a, grid_parts, s)
                 : launch_dkf<64, false, false>(group, a, grid_parts, s);
  }
  if (kv_bf16) return fused ? launch_dkf<128, true, true>(group, a, grid_parts, s)
                            : launch_dkf<128, true, false>(group, a, grid_parts, s);
  return fused ? launch_dkf<128, false, true>(group, a, grid_parts, s)
               : launch_dkf<128, false, false>(group, a, grid_parts, s);
}

hipError_t launch_attention_merge(int head_dim, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_q_heads, (unsigned)(head_dim / 64));
  const bool one = a.max_parts <= kMergeChunk;  // every possible partition fits one chunk
  if (head_dim == 64) {
    if (one)
      hipLaunchKernelGGL((k_attn_merge<64, 1>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_merge<64, 4>), grid, dim3(256), 0, s, a);
  } else {
    if (one)
      hipLaunchKernelGGL((k_attn_merge<128, 1>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_merge<128, 4>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace qd

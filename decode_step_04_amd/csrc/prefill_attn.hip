// prefill_attn.hip - causal GQA attention of P new tokens over the paged cache, on the matrix
// cores.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
//
// FlashAttention-style ([ETE], the batched-prefill next step; the (m, l, acc) state of
// [Qwen3-runtime] §9.1 / [ETE] online softmax, per query row).  Query t of the prompt sees keys
// 0 .. pos0 + t.  This file is built with the IEEE mode off and without NaN semantics (inputs are
// finite; -inf stands for a masked score), so the max reductions compile to v_max3 without
// canonicalising every operand.
//
// A work-group of 8 waves takes 64 rows of kv head g, each row a (query, head of the KV group)
// pair, query-major (BQ = 64 / G queries).  Keys go in blocks of 64 (four pages), two blocks per
// step: waves 0-3 take the even block and waves 4-7 the odd one, each wave 16 rows, and the two
// halves' (m, l, acc) states are merged through LDS at the end (exact up to rounding, as the
// split-KV merge of the decode path).  Every thread loads 16-byte chunks of both blocks' K and V
// two steps ahead into registers and writes them row-major into one of two LDS buffers; one
// barrier per step.  A thread's chunks sit at fixed offsets inside fixed pages of the step, so
// outside the last step a load is a scalar page base plus a constant 32-bit lane offset.
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims of K from LDS (16 contiguous
//     bytes per lane), B = the wave's 16 query rows (held in registers).  Lane l receives keys
//     4(l/16) + e of each 16-key tile for query row l % 16, so each lane holds 16 of the block's
//     64 keys for one row: the row maximum is 16 local values and two lane swaps
//     (v_permlane16/32_swap), and the rescale of a row's accumulator uses the lane's own factor.
//   P = 2^(S - m) is rounded to bf16 (the MFMA operand type) and is already the B operand of
//     O^T += V^T P^T: lane l's 8 values of a 32-key half are keys 4(l/16) + e and 16 + 4(l/16) + e,
//     and the A operand (V^T, 16 dims x the same 8 keys) comes from the row-major V tile through
//     ds_read_b64_tr_b16.  In each 16-lane group that instruction returns to lane i element
//     i % 4 of the 8 bytes addressed by lane 4e + i / 4, as its e-th value (checked on MI355X):
//     lanes 4e .. 4e+3 address the 16 dims of key row e, so lane i gets dim i of 4 key rows.
//   The denominator is one more MFMA per half with an A operand of ones: every row of that tile
//     is the column sum of the rounded P, so l adds exactly the values the output averages, and
//     each lane receives its own row's sum.
//   The output O^T lands with lane l holding dims 4(l/16) + e of query row l % 16.
// A work-group takes query blocks nb-1-x and x (the causal work of the pair is the same for every
// x), heaviest first; the work-group index runs kv head fastest, so with 8 XCDs dispatched round
// robin one kv head's work-groups share an XCD (and its L2 copy of that head's K and V).
// LDS rows (D = 128): K and V both D + 16 bf16, 288 bytes, chosen by measurement with rocprofv3's
// SQ_LDS_BANK_CONFLICT on MI355X (2048-token prefill, 0.6B shape).  K rows of 272 bytes, the
// layout that is conflict-free if a 16-byte read is served 16 consecutive lanes at a time,
// stalled the LDS for about two thirds of its active cycles; 288-byte rows stalled it for none
// (the kernel 6.6 % faster).  V rows of 272 or 320 bytes doubled the stalls, and 288 bytes (the
// 8-byte transposed reads of a 16-lane group then cover 4 rows x 32 contiguous bytes, each row 32
// bytes further along the banks) had none.  For D = 64, K rows stay D + 8.
#include "common.h"
#include "launch.h"

namespace qd {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf8 frag(const uint16_t* p) {
  return __builtin_bit_cast(bf8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf8 frag_tr(const uint16_t* p0, const uint16_t* p1) {
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p1));
  return __builtin_bit_cast(bf8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4 mfma(bf8 a, bf8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(512) void k_prefill_attn(PrefillAttnArgs a) {
  constexpr int BQ = 64 / G;     // queries per query block
  constexpr int ROWS = BQ * G;   // active rows (64 unless G does not divide 64)
  constexpr int KB = 64;         // keys per block
  constexpr int KS = D / 32;     // MFMA k-steps over D
  constexpr int ND = D / 16;     // 16-dim tiles of the output
  constexpr int KP = D == 128 ? D + 16 : D + 8;  // LDS row stride of K, in bf16
  constexpr int VP = D + 16;     // LDS row stride of V, in bf16
  constexpr int CPK = D / 8;     // 16-byte chunks per key row
  constexpr int CL = 2 * KB * CPK / 512;  // chunks of K (and of V) per thread per step
  constexpr int MW = 4 * ND + 2;          // floats per lane of the merge: acc, m, l
  __shared__ __align__(16) uint16_t kt[2][2][KB][KP];
  __shared__ __align__(16) uint16_t vt[2][2][KB][VP];
  static_assert(sizeof(kt) >= 4 * MW * 64 * sizeof(float), "merge area");
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int half = wave >> 2;                      // 0: even key blocks, 1: odd ones
  const int r16 = lane & 15, q4 = lane >> 4;
  const int hq = a.n_q_heads, hkv = a.n_kv_heads;
  const int g = (int)(blockIdx.x % (unsigned)hkv);
  const int x = (int)(blockIdx.x / (unsigned)hkv);
  const int nb = (a.p + BQ - 1) / BQ;
  const float NEG = -INFINITY;
  const int64_t head_stride = (int64_t)kPage * D;  // one head's page tile, in elements
  const int row = (wave & 3) * 16 + r16;           // this lane's query row in the block
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)g * head_stride * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)g * head_stride * 2;
  const int64_t page_bytes = (int64_t)hkv * head_stride * 2;  // one page of every head
  // this thread's chunk u of a step: idx = t + 512 u is 16 bytes at dim 8 (idx % CPK) of key
  // kl = idx / CPK of the step's 128 (block kl / 64 of the pair), in page kl / 16 of the step
  // (the same for the whole wave) at byte offset off[u] of that page's head tile
  uint32_t off[CL];
  int jpg[CL];
#pragma unroll
  for (int u = 0; u < CL; ++u) {
    const int idx = t + 512 * u, kl = idx / CPK, c = idx % CPK;
    off[u] = (uint32_t)(((kl % kPage) * D + 8 * c) * 2);
    jpg[u] = __builtin_amdgcn_readfirstlane(kl / kPage);
  }
  bf8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  for (int pass = 0; pass < 2; ++pass) {
    const int qb = pass == 0 ? nb - 1 - x : x;
    if (pass == 1) {
      if (qb >= nb - 1 - x) break;  // an odd count's middle block runs once (uniform)
      __syncthreads();              // the first block's merge has read its LDS area
    }
    // block-level scalars (readfirstlane marks them wave-uniform for the compiler)
    const int t0 = __builtin_amdgcn_readfirstlane(qb * BQ);
    const int nq = min(BQ, a.p - t0);              // valid queries of the block (>= 1)
    const int kend = __builtin_amdgcn_readfirstlane(a.pos0 + t0 + nq);  // keys 0 .. kend-1
    const int last = kend - 1;
    const int qfirst = a.pos0 + t0;                // position of the block's first query
    const bool active = row < ROWS && row / G < nq;
    const int qpos = active ? qfirst + row / G : -1;   // an inactive row sees no key
    bf8 qf[KS];
    {
      const int qa = min(row < ROWS ? row / G : 0, nq - 1), ha = row % G;
      const uint16_t* qrow = a.q + ((int64_t)(t0 + qa) * hq + g * G + ha) * D + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = frag(qrow + 32 * ks);
    }
    // m: the row's running maximum (log2 units); ol: its denominator (every element the same)
    float m = -1e30f;
    f32x4 o[ND], ol = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nblk = (kend + KB - 1) / KB;
    const int nstep = (nblk + 1) / 2;
    // page numbers without a memory round trip in the loop: lane l holds page l of the current
    // chunk of 64 pages (8 steps); the next chunk is loaded a whole chunk ahead.  Pages past the
    // last visible one are clamped to it (every entry below npages is valid).
    const int npages = (kend + kPage - 1) / kPage;
    int pc = a.block_table[min(lane, npages - 1)], pn = 0;
    u32x4 kc0[CL], vc0[CL], kc1[CL], vc1[CL];
    auto fetch = [&](int st, u32x4 (&kc)[CL], u32x4 (&vc)[CL]) __attribute__((always_inline)) {
      const int key0 = st * 2 * KB;
      if (key0 + 2 * KB - 1 <= last) {  // wave-uniform: no key of the step is clamped
#pragma unroll
        for (int u = 0; u < CL; ++u) {
          const int64_t ph = __builtin_amdgcn_readlane(pc, (8 * st + jpg[u]) & 63);
          kc[u] = *reinterpret_cast<const u32x4*>(kbase + ph * page_bytes + off[u]);
          vc[u] = *reinterpret_cast<const u32x4*>(vbase + ph * page_bytes + off[u]);
        }
      } else {  // the last step: keys past `last` read key `last` (a wave's keys share a page)
#pragma unroll
        for (int u = 0; u < CL; ++u) {
          const int idx = t + 512 * u, kl = idx / CPK, c = idx % CPK;
          const int key = min(key0 + kl, last);
          const int pidx = __builtin_amdgcn_readfirstlane(key / kPage) & 63;
          const int64_t ph = __builtin_amdgcn_readlane(pc, pidx);
          const uint32_t lo = (uint32_t)(((key % kPage) * D + 8 * c) * 2);
          kc[u] = *reinterpret_cast<const u32x4*>(kbase + ph * page_bytes + lo);
          vc[u] = *reinterpret_cast<const u32x4*>(vbase + ph * page_bytes + lo);
        }
      }
    };
    auto stage = [&](int buf, const u32x4 (&kc)[CL], const u32x4 (&vc)[CL])
                     __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < CL; ++u) {
        const int idx = t + 512 * u, kl = idx / CPK, c = idx % CPK;
        *reinterpret_cast<u32x4*>(&kt[buf][kl / KB][kl % KB][8 * c]) = kc[u];
        *reinterpret_cast<u32x4*>(&vt[buf][kl / KB][kl % KB][8 * c]) = vc[u];
      }
    };
    // one 64-key block of this wave's half: keys key0 .. key0 + 63 in LDS tile (buf, half)
    auto compute = [&](int key0, int buf) __attribute__((always_inline)) {
      // S^T for the four 16-key tiles, the k-steps outermost so that four independent
      // accumulators separate dependent MFMAs
      f32x4 sc[4];
#pragma unroll
      for (int kt4 = 0; kt4 < 4; ++kt4) sc[kt4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kt4 = 0; kt4 < 4; ++kt4)
          sc[kt4] = mfma(frag(&kt[buf][half][16 * kt4 + r16][32 * ks + 8 * q4]), qf[ks], sc[kt4]);
      // online softmax of row `row` over keys key0 + 16 kt4 + 4 q4 + e: the maximum on the
      // unscaled scores (qscale > 0), the scale folded into the exponent's fma
      if (key0 + KB - 1 > qfirst) {
        const int rel = qpos - key0 - 4 * q4;   // key offset 16 kt4 + e is visible iff <= rel
#pragma unroll
        for (int kt4 = 0; kt4 < 4; ++kt4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * kt4 + e > rel) sc[kt4][e] = NEG;
      }
      float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
      for (int kt4 = 1; kt4 < 4; ++kt4)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[kt4][0], sc[kt4][1]), fmaxf(sc[kt4][2], sc[kt4][3])));
      float lo, hi;
      lane_pair<16>(mx, lo, hi);
      mx = fmaxf(lo, hi);
      lane_pair<32>(mx, lo, hi);
      mx = fmaxf(lo, hi) * a.qscale;
      const float mn = fmaxf(m, mx);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      const bool grew = mn != m;
      m = mn;
      bf8 pb[2];
#pragma unroll
      for (int kt4 = 0; kt4 < 4; ++kt4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pb[kt4 >> 1][4 * (kt4 & 1) + e] =
              (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[kt4][e], a.qscale, -mn));
      if (__ballot(grew) != 0) {  // wave-uniform; when no row's maximum grew every factor is 1
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) o[nd] *= corr;
        ol *= corr;
      }
      // O^T += V^T P^T and l += 1^T P^T, one 32-key half at a time
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = 32 * h + 4 * q4 + (r16 >> 2);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const int dc = 16 * nd + 4 * (r16 & 3);
          o[nd] = mfma(frag_tr(&vt[buf][half][kr][dc], &vt[buf][half][kr + 16][dc]), pb[h], o[nd]);
        }
        ol = mfma(ones, pb[h], ol);
      }
    };
    auto step = [&](int st, u32x4 (&kc)[CL], u32x4 (&vc)[CL]) __attribute__((always_inline)) {
      const int buf = st & 1;
      if ((st & 7) == 0 && st + 8 < nstep)   // wave-uniform
        pn = a.block_table[min(((st >> 3) + 1) * 64 + lane, npages - 1)];
      if (((st + 2) & 7) == 0) pc = pn;       // the step fetched next opens a new chunk
      stage(buf, kc, vc);
      if (st + 2 < nstep) fetch(st + 2, kc, vc);
      __syncthreads();
      const int kb = 2 * st + half;
      if (kb < nblk) compute(kb * KB, buf);   // wave-uniform
    };
    fetch(0, kc0, vc0);
    if (nstep > 1) fetch(1, kc1, vc1);
    for (int st = 0; st < nstep; st += 2) {
      step(st, kc0, vc0);
      if (st + 1 >= nstep) break;
      step(st + 1, kc1, vc1);
    }

    // merge the odd-block half into the even one: lane-major floats, [wave & 3][MW][64]
    __syncthreads();  // every wave is done with the K/V tiles
    float* mg = reinterpret_cast<float*>(&kt[0][0][0][0]) + (wave & 3) * MW * 64 + lane;
    if (half == 1) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
#pragma unroll
        for (int e = 0; e < 4; ++e) mg[(4 * nd + e) * 64] = o[nd][e];
      mg[4 * ND * 64] = m;
      mg[(4 * ND + 1) * 64] = ol[0];
    }
    __syncthreads();
    if (half == 0) {
      const float m1 = mg[4 * ND * 64], l1 = mg[(4 * ND + 1) * 64];
      const float mn = fmaxf(m, m1);
      const float c0 = __builtin_amdgcn_exp2f(m - mn), c1 = __builtin_amdgcn_exp2f(m1 - mn);
      const float lsum = fmaf(ol[0], c0, l1 * c1);
      if (active) {
        const float inv = 1.0f / lsum;
        uint16_t* orow = a.out + ((int64_t)(t0 + row / G) * hq + g * G + row % G) * D + 4 * q4;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(o[nd][e], c0, mg[(4 * nd + e) * 64] * c1) * inv;
          uint2 w;
          w.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          w.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *reinterpret_cast<uint2*>(orow + 16 * nd) = w;
        }
      }
    }
  }
}

template <int D>
hipError_t launch_pa(int group, const PrefillAttnArgs& a, hipStream_t s) {
  const unsigned hk = (unsigned)a.n_kv_heads;
  switch (group) {
#define QD_PA(G)                                                                                 \
  case G:                                                                                        \
    hipLaunchKernelGGL((k_prefill_attn<D, G>),                                                   \
                       dim3((unsigned)(((a.p + 64 / G - 1) / (64 / G) + 1) / 2) * hk), dim3(512), \
                       0, s, a);                                                                 \
    break;
    QD_PA(1) QD_PA(2) QD_PA(3) QD_PA(4) QD_PA(5) QD_PA(6) QD_PA(7) QD_PA(8)
#undef QD_PA
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attn(int head_dim, int group, const PrefillAttnArgs& a, hipStream_t s) {
  if (a.p <= 0) return hipSuccess;
  return head_dim == 64 ? launch_pa<64>(group, a, s) : launch_pa<128>(group, a, s);
}

}  // namespace qd

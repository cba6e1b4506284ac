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
#include <utility>

#include "common.h"
#include "launch.h"

namespace qd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// EPI_ROPE epilogue: the product tile (BM tokens x one 128-dim head of the QKV row) goes to LDS;
// wave w then takes tokens w BM/4 .. +BM/4-1.  The RMSNorm sums of squares of those rows are
// split over the lanes (64 / (BM/4) lanes per row, each a contiguous slice, then combined), so
// each row's 1/sqrt is computed once; then row by row lane l takes the RoPE pair (l, l + 64) with
// the row's factor read from the lane that holds it, and stores Q as bf16 rows or K / V into the
// paged pool (the operations of k_prefill_rope, the sum of squares in another order).
template <int BM, int BN, int WM, int WN, int NI, int NJ, typename Acc>
__device__ __forceinline__ void rope_epilogue(const GemmArgs& a, const Acc (&acc)[NI][NJ],
                                              float* tile, int m0, int n0, int wave, int lane) {
  constexpr int TS = BN + 4, HALF = 64, D = 128;
  const int r32 = lane & 31;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (wave >> 1) * WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = (wave & 1) * WN + 32 * j + r32;
        tile[row * TS + col] = acc[i][j][r];
      }
  __syncthreads();
  const PrefillRopeArgs& ra = a.rope;
  const int hq = ra.n_q_heads, hkv = ra.n_kv_heads;
  const int hh = n0 / D;               // head of the QKV row: Q heads, then K, then V
  const bool is_q = hh < hq, is_v = hh >= hq + hkv;
  const int g = is_q ? 0 : (is_v ? hh - hq - hkv : hh - hq);
  const float* gam = is_v ? nullptr : (is_q ? ra.q_gamma : ra.k_gamma);
  const float g0 = gam != nullptr ? gam[lane] : 0.f, g1 = gam != nullptr ? gam[lane + HALF] : 0.f;
  // every row's (cos, sin) and page number are requested before the first row is processed
  // (rows past the end read the last row's, and store nothing)
  constexpr int RPW = BM / 4;
  constexpr int LPR = 64 / RPW, SPAN = D / LPR;   // lanes per row, columns per lane
  const int r0 = wave * RPW;
  float2 cs[RPW];
  int pg[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int pos = ra.pos0 + min(m0 + r0 + q, a.m - 1);
    cs[q] = reinterpret_cast<const float2*>(ra.table)[(int64_t)pos * HALF + lane];
    pg[q] = ra.block_table[pos / kPage];
  }
  // lane l sums the squares of columns (l / RPW) SPAN .. +SPAN-1 of row r0 + l % RPW; the LPR
  // partial sums of a row are combined (lanes l, l + RPW, ...) and lane q < RPW keeps row q's
  // 1 / rms
  float rinv = 1.f;
  if (gam != nullptr) {  // uniform
    const float* tr = tile + (r0 + (lane % RPW)) * TS + (lane / RPW) * SPAN;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < SPAN; ++c) ss = fmaf(tr[c], tr[c], ss);
    if constexpr (LPR >= 4) ss += __shfl_xor(ss, 2 * RPW);
    ss += __shfl_xor(ss, RPW);
    rinv = 1.0f / sqrtf(ss / (float)D + ra.eps);
  }
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int rr = r0 + q, t = m0 + rr;
    if (t >= a.m) break;  // wave-uniform
    float x0 = tile[rr * TS + lane], x1 = tile[rr * TS + lane + HALF];
    const int pos = ra.pos0 + t;
    const int64_t off = (((int64_t)pg[q] * hkv + g) * kPage + pos % kPage) * D + lane;
    if (is_v) {
      ra.v_pool[off] = f32_to_bf16(x0);
      ra.v_pool[off + HALF] = f32_to_bf16(x1);
      continue;
    }
    if (gam != nullptr) {
      const float ri = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rinv), q));
      x0 = x0 * ri * g0;
      x1 = x1 * ri * g1;
    }
    const float y0 = x0 * cs[q].x - x1 * cs[q].y;
    const float y1 = x1 * cs[q].x + x0 * cs[q].y;
    if (is_q) {
      const int64_t o = ((int64_t)t * hq + hh) * D + lane;
      ra.q_out[o] = f32_to_bf16(y0);
      ra.q_out[o + HALF] = f32_to_bf16(y1);
    } else {
      ra.k_pool[off] = f32_to_bf16(y0);
      ra.k_pool[off + HALF] = f32_to_bf16(y1);
    }
  }
}

// k_gemm_lds: the same product and epilogues with the operand tiles staged in LDS, on
// v_mfma_f32_32x32x16_bf16 (on MI355X it sustains about 1.3x the rate of the 16x16x32 form: 2.15
// against 1.62 PFLOP/s in a register-only loop).  For one 32 x 32 x 16 step lane l supplies
// A[row l % 32][k 8(l/32) .. +7] and W[row l % 32][k 8(l/32) .. +7] and receives
// C[row 8(r/4) + 4(l/32) + r % 4][col l % 32], r < 16 (layout checked on MI355X).  A work-group
// of 4 waves computes BM rows (128 or 64) against BN weight rows (128 or 64) in K steps of 64.
// Each thread moves 16-byte chunks (8 threads per 128-byte row segment) of A[BM x 64] and
// W[BN x 64]: a step's chunks are requested PF steps ahead into one of PF register sets and
// written into one of two LDS buffers the step before their MFMAs; one barrier per step.  LDS
// rows are padded to 72 bf16 (144 bytes): the 16-byte fragment reads of 16 consecutive rows at
// one k offset fall in distinct banks.  Wave w owns rows (w / 2) BM/2 .. +BM/2-1 and weight rows
// (w % 2) BN/2 .. +BN/2-1 of the tile.  For SWIGLU (BN = 128) a wave's 64 weight rows are 32 gate
// rows and the matching 32 up rows, so g and u of an output meet in the same lanes.  For ROPE
// (BN = 128 = head_dim) the fp32 tile is staged in LDS and each wave takes BM / 4 of its rows
// (tokens), one at a time, with the lane layout and arithmetic of k_prefill_rope.
template <int EPI, int BM, int BN, int PF>
__global__ __launch_bounds__(256) void k_gemm_lds(GemmArgs a) {
  constexpr int BK = 64, LDR = BK + 8;
  constexpr int WM = BM / 2, WN = BN / 2;   // rows and weight rows per wave
  constexpr int NI = WM / 32, NJ = WN / 32; // their 32-row blocks
  constexpr int AL = BM * BK / 8 / 256;     // 16-byte loads per thread per step
  constexpr int BL = BN * BK / 8 / 256;
  constexpr int TS = BN + 4;                // ROPE: fp32 row stride of the staged tile
  static_assert(EPI != EPI_SWIGLU || NJ == 2, "SWIGLU pairs one gate and one up block per wave");
  static_assert(EPI != EPI_ROPE || BN == 128, "ROPE tiles are one 128-dim head");
  static_assert(EPI != EPI_ROPE || BM * TS * 4 <= 2 * (BM + BN) * LDR * 2, "ROPE tile in LDS");
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDR];
  uint16_t (*sa)[BM * LDR] = reinterpret_cast<uint16_t (*)[BM * LDR]>(smem);
  uint16_t (*sb)[BN * LDR] = reinterpret_cast<uint16_t (*)[BN * LDR]>(smem + 2 * BM * LDR);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int M = a.m, N = a.n, K = a.k;
  const int m0 = blockIdx.y * BM;
  const int nout = EPI == EPI_SWIGLU ? BN / 2 : BN;   // output columns per work-group
  const int n0 = blockIdx.x * nout;
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  // this thread's loads: row t / 8 + 32 r of a tile, 16 bytes at k offset 8 (t % 8); source rows
  // past the end are clamped (their results are discarded)
  const int trow = t >> 3, tkc = (t & 7) * 8;
  auto wrow = [&](int row) __attribute__((always_inline)) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int h = row / WN, q = row % WN;
      const int col = min(n0 + h * (WN / 2) + q % (WN / 2), N - 1);
      return q < WN / 2 ? col : N + col;
    } else {
      return min(n0 + row, N - 1);
    }
  };
  const uint16_t* pa[AL];
  const uint16_t* pb[BL];
#pragma unroll
  for (int r = 0; r < AL; ++r) pa[r] = A + (int64_t)min(m0 + trow + 32 * r, M - 1) * K + tkc;
#pragma unroll
  for (int r = 0; r < BL; ++r) pb[r] = W + (int64_t)wrow(trow + 32 * r) * K + tkc;
  u32x4 ra[PF][AL], rb[PF][BL];
  auto gload = [&](int set, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < AL; ++r) ra[set][r] = *reinterpret_cast<const u32x4*>(pa[r] + kt * BK);
#pragma unroll
    for (int r = 0; r < BL; ++r) rb[set][r] = *reinterpret_cast<const u32x4*>(pb[r] + kt * BK);
  };
  auto lstore = [&](int set, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < AL; ++r)
      *reinterpret_cast<u32x4*>(&sa[st][(trow + 32 * r) * LDR + tkc]) = ra[set][r];
#pragma unroll
    for (int r = 0; r < BL; ++r)
      *reinterpret_cast<u32x4*>(&sb[st][(trow + 32 * r) * LDR + tkc]) = rb[set][r];
  };
  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  const int r32 = lane & 31, kq = (lane >> 5) * 8;
  const int arow = (wave >> 1) * WM + r32, brow = (wave & 1) * WN + r32;
  auto compute = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 fa[NI], fb[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &sa[st][(arow + 32 * i) * LDR + ks + kq]));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &sb[st][(brow + 32 * j) * LDR + ks + kq]));
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt lives in register set kt % PF from its request until it is written to LDS; steps
  // 0 .. PF-1 are requested first, step 0 goes to LDS, and its set takes step PF
  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (s < nk) gload(s, s);
  lstore(0, 0);
  if (PF < nk) gload(0, PF);
  __syncthreads();
  for (int k0 = 0; k0 < nk; k0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int kt = k0 + s;
      if (kt >= nk) break;
      compute(kt & 1);
      const int nx = kt + 1, set = (s + 1) % PF;   // step nx is in register set nx % PF
      if (nx < nk) {
        lstore(set, nx & 1);
        if (nx + PF < nk) gload(set, nx + PF);
      }
      __syncthreads();
    }
  }

  if constexpr (EPI == EPI_ROPE) {
    rope_epilogue<BM, BN, WM, WN, NI, NJ>(a, acc, reinterpret_cast<float*>(smem), m0, n0, wave,
                                          lane);
    return;
  }
  // epilogue: lane holds C[row 32 i + 8 (r/4) + 4 (l/32) + r % 4 of the wave][weight row
  // 32 j + l % 32]
  const int mw = m0 + (wave >> 1) * WM;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mw + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        const int n = n0 + (wave & 1) * (WN / 2) + r32;
        if (n >= N) continue;
        const float g = acc[i][0][r], u = acc[i][1][r];
        const float v = g / (1.0f + expf(-g)) * u;
        static_cast<uint16_t*>(a.y)[(int64_t)m * N + n] = f32_to_bf16(v);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = n0 + (wave & 1) * WN + 32 * j + r32;
          if (n >= N) continue;
          const float v = acc[i][j][r];
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

// k_gemm_dma: the STORE, RESID and SWIGLU products with the operand tiles moved straight from
// global memory into LDS (gfx950 global_load_lds_dwordx4: each lane names its own 16-byte source,
// the wave's 64 chunks land at consecutive 16-byte slots of a wave-uniform LDS address), so no
// register staging, no LDS store instructions and no VGPRs held for tiles in flight.
//   - Tiles of K are 64 wide (128-byte rows, 8 chunks).  Row r of a tile keeps its chunk c at slot
//     c ^ ((r / 2) % 8): the 32 x 32 x 16 fragment read of 16 consecutive rows at one k offset then
//     covers all 64 banks once (two rows per 256 bytes, eight slot positions).
//   - NS stages, each its own __shared__ array (the compiler tracks direct-to-LDS loads per LDS
//     object, so reading one stage does not wait for the loads into the others).  Step kt waits
//     for its own stage with an explicit vmcnt (the loads of the NS - 2 later tiles may stay in
//     flight), meets the other waves at a plain s_barrier (a __syncthreads would drain every load
//     in flight), requests tile kt + NS - 1 into the stage freed by step kt - 1, and computes.
//     Past the last tile the requests re-read the last one, so the count of loads in flight is
//     the same at every step.
//   - The loop body is U steps (the compiler drains all loads at the loop head, once per U).
//   - Wave w of a WGM x WGN grid owns rows (w / WGN) BM/WGM .. and weight rows (w % WGN) BN/WGN ..;
//     the epilogues are those of k_gemm_lds (SWIGLU needs 64 weight rows per wave: 32 gate, 32 up).
// Measured on MI355X (2048 rows, N 24576, K 4096, fp32 out, weights cold in HBM): 426 us with
// 256 x 256 tiles and 8 waves, against about 555 us for 128 x 128 tiles (either kernel).  With
// 128 x 128 and smaller tiles it is no faster than register staging inside the prefill.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}

// Stage S of a tile kind (ID: 0 for A, 1 for W) of SZ bf16: one LDS object per stage.
template <int ID, int S, int SZ>
__device__ __forceinline__ uint16_t* gemm_stage() {
  __shared__ __attribute__((aligned(1024))) uint16_t buf[SZ];
  return buf;
}

// f(integral_constant<int, I>) for I = 0 .. N-1, in order
template <class F, int... I>
__device__ __forceinline__ void for_each_const(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

template <int EPI, int BM, int BN, int NS, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm_dma(GemmArgs a) {
  constexpr int BK = 64, CPR = BK * 2 / 16, RPB = 64 / CPR, RPP = 256 / (BK * 2);
  constexpr int NW = WGM * WGN;
  constexpr int AL = BM / RPB / NW, BL = BN / RPB / NW;   // 1 KiB loads per wave per tile
  constexpr int WM = BM / WGM, WN = BN / WGN, NI = WM / 32, NJ = WN / 32;
  constexpr int U = NS == 3 ? 18 : 16;                     // steps per loop iteration
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  static_assert(AL * RPB * NW == BM && BL * RPB * NW == BN && NI >= 1 && NJ >= 1, "tile split");
  static_assert(EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_SWIGLU, "epilogue");
  static_assert(EPI != EPI_SWIGLU || NJ == 2, "SWIGLU pairs one gate and one up block per wave");
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int M = a.m, N = a.n, K = a.k;
  const int m0 = blockIdx.y * BM;
  const int nout = EPI == EPI_SWIGLU ? BN / 2 : BN;   // output columns per work-group
  const int n0 = blockIdx.x * nout;
  const int nk = K / BK;
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  auto wrow = [&](int row) __attribute__((always_inline)) {
    if constexpr (EPI == EPI_SWIGLU) {
      const int h = row / WN, q = row % WN;
      const int col = min(n0 + h * (WN / 2) + q % (WN / 2), N - 1);
      return q < WN / 2 ? col : N + col;
    } else {
      return min(n0 + row, N - 1);
    }
  };
  // this lane's chunk of load r: tile row (r NW + wave) RPB + lane / CPR, slot lane % CPR, which
  // holds source chunk slot ^ swizzle(row); rows past the end are clamped (results discarded)
  const int lrow = lane / CPR, slot = lane % CPR;
  const uint16_t* pa[AL];
  const uint16_t* pb[BL];
#pragma unroll
  for (int r = 0; r < AL; ++r) {
    const int row = (r * NW + wave) * RPB + lrow;
    pa[r] = A + (int64_t)min(m0 + row, M - 1) * K + (slot ^ ((row / RPP) % CPR)) * 8;
  }
#pragma unroll
  for (int r = 0; r < BL; ++r) {
    const int row = (r * NW + wave) * RPB + lrow;
    pb[r] = W + (int64_t)wrow(row) * K + (slot ^ ((row / RPP) % CPR)) * 8;
  }
  auto request = [&](auto stage, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    uint16_t* sa = gemm_stage<0, S, BM * BK>();
    uint16_t* sb = gemm_stage<1, S, BN * BK>();
    kt = min(kt, nk - 1);
#pragma unroll
    for (int r = 0; r < AL; ++r)
      __builtin_amdgcn_global_load_lds((const void*)(pa[r] + kt * BK),
                                       (__attribute__((address_space(3))) void*)(sa + (r * NW + wave) * 512),
                                       16, 0, 0);
#pragma unroll
    for (int r = 0; r < BL; ++r)
      __builtin_amdgcn_global_load_lds((const void*)(pb[r] + kt * BK),
                                       (__attribute__((address_space(3))) void*)(sb + (r * NW + wave) * 512),
                                       16, 0, 0);
  };
  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  const int r32 = lane & 31, kq = lane >> 5;
  const int arow = (wave / WGN) * WM + r32, brow = (wave % WGN) * WN + r32;
  auto frag = [&](const uint16_t* base, int row, int ks) __attribute__((always_inline)) {
    const int c = (2 * ks + kq) ^ ((row / RPP) % CPR);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + row * BK + 8 * c));
  };
  auto compute = [&](auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const uint16_t* sa = gemm_stage<0, S, BM * BK>();
    const uint16_t* sb = gemm_stage<1, S, BN * BK>();
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[NI], fb[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) fa[i] = frag(sa, arow + 32 * i, ks);
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = frag(sb, brow + 32 * j, ks);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  for_each_const([&](auto st) { request(st, decltype(st)::value); },
                 std::make_integer_sequence<int, NS - 1>{});
  for (int k0 = 0; k0 < nk; k0 += U) {
    bool done = false;
    for_each_const(
        [&](auto u) {
          constexpr int UI = decltype(u)::value;
          const int kt = k0 + UI;
          done = done || kt >= nk;
          if (done) return;
          wait_vmcnt<(NS - 2) * (AL + BL)>();   // this step's tile has landed (this wave's part)
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();         // ... every wave's part, and step kt - 1 is done
          asm volatile("" ::: "memory");
          request(std::integral_constant<int, (UI + NS - 1) % NS>{}, kt + NS - 1);
          compute(std::integral_constant<int, UI % NS>{});
        },
        std::make_integer_sequence<int, U>{});
  }

  // epilogue: lane holds C[row 32 i + 8 (r/4) + 4 (l/32) + r % 4 of the wave][weight row
  // 32 j + l % 32]
  const int mw = m0 + (wave / WGN) * WM;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mw + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= M) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        const int n = n0 + (wave % WGN) * (WN / 2) + r32;
        if (n >= N) continue;
        const float g = acc[i][0][r], u = acc[i][1][r];
        const float v = g / (1.0f + expf(-g)) * u;
        static_cast<uint16_t*>(a.y)[(int64_t)m * N + n] = f32_to_bf16(v);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = n0 + (wave % WGN) * WN + 32 * j + r32;
          if (n >= N) continue;
          const float v = acc[i][j][r];
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

// The largest tile that still gives two work-groups per CU (512), else the smallest (SWIGLU tiles
// keep 128 weight rows: 64 gate and 64 up).
template <int EPI>
static void launch_gemm_lds(const GemmArgs& a, hipStream_t s) {
  const int64_t wide = EPI == EPI_SWIGLU ? 2 : 1;  // weight rows per output column
  auto wgs = [&](int bm, int bn) {
    return ((a.n * wide + bn - 1) / bn) * (int64_t)((a.m + bm - 1) / bm);
  };
  auto grid = [&](int bm, int bn) {
    return dim3((unsigned)((a.n * wide + bn - 1) / bn), (unsigned)((a.m + bm - 1) / bm));
  };
#ifdef QD_GEMM_SWEEP
  QD_GEMM_SWEEP
#endif
  if (EPI == EPI_SWIGLU || EPI == EPI_ROPE || wgs(128, 128) >= 512) {
    if ((EPI == EPI_SWIGLU || EPI == EPI_ROPE) && wgs(128, 128) < 512)
      hipLaunchKernelGGL((k_gemm_lds<EPI, 64, 128, 1>), grid(64, 128), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_lds<EPI, 128, 128, 1>), grid(128, 128), dim3(256), 0, s, a);
  } else if constexpr (EPI != EPI_SWIGLU && EPI != EPI_ROPE) {
    if (wgs(64, 128) >= 512)
      hipLaunchKernelGGL((k_gemm_lds<EPI, 64, 128, 1>), grid(64, 128), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_lds<EPI, 64, 64, 1>), grid(64, 64), dim3(256), 0, s, a);
  }
}

// Products with at least 512 tiles of 256 x 256 (weight rows per output column: 2 for SWIGLU) take
// the direct-to-LDS kernel with 8 waves (128 KiB of LDS: one work-group per CU); the others keep
// the register-staged kernel, which measured as fast or faster on them in the prefill (smaller
// tiles are bound by the latency of the first weight bytes, not by the operand traffic).
template <int EPI>
static bool launch_gemm_dma(const GemmArgs& a, hipStream_t s) {
  const int64_t wide = EPI == EPI_SWIGLU ? 2 : 1;
  const int64_t tiles = ((a.n * wide + 255) / 256) * (int64_t)((a.m + 255) / 256);
  if (tiles < 512) return false;
  const dim3 grid((unsigned)((a.n * wide + 255) / 256), (unsigned)((a.m + 255) / 256));
  hipLaunchKernelGGL((k_gemm_dma<EPI, 256, 256, 2, 2, 4>), grid, dim3(512), 0, s, a);
  return true;
}

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.m <= 0 || a.n <= 0) return hipSuccess;
  if (a.k % 32 || a.k < 32) return hipErrorInvalidValue;
  if (a.k % 64 == 0) {
    switch (epi) {
      case EPI_STORE:
        if (!launch_gemm_dma<EPI_STORE>(a, s)) launch_gemm_lds<EPI_STORE>(a, s);
        break;
      case EPI_RESID:
        if (!launch_gemm_dma<EPI_RESID>(a, s)) launch_gemm_lds<EPI_RESID>(a, s);
        break;
      case EPI_ROPE:
        if (a.n % 128) return hipErrorInvalidValue;
        launch_gemm_lds<EPI_ROPE>(a, s);
        break;
      default:
        if (!launch_gemm_dma<EPI_SWIGLU>(a, s)) launch_gemm_lds<EPI_SWIGLU>(a, s);
        break;
    }
    return hipGetLastError();
  }
  if (epi == EPI_ROPE) return hipErrorInvalidValue;
  const int ncols = epi == EPI_SWIGLU ? 64 : 128;
  const dim3 grid((unsigned)((a.n + ncols - 1) / ncols), (unsigned)((a.m + 127) / 128));
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemm<EPI_STORE>), grid, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm<EPI_RESID>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm<EPI_SWIGLU>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

// ---- embedding rows of the P prompt tokens ([ETE]: the block pipeline starts from each token's
//      embedding row) -----
__global__ __launch_bounds__(256) void k_embed_rows(const void* table, int table_bf16,
                                                    const int32_t* tokens, int d, int vocab,
                                                    float* x, StepDesc* desc) {
  const int t = blockIdx.x;
  const int tok = tokens[t];
  const bool bad = tok < 0 || tok >= vocab;
  if (bad && threadIdx.x == 0 && desc != nullptr) desc->error = 1;
  const int64_t base = bad ? 0 : (int64_t)tok * d;
  for (int i = threadIdx.x; i < d; i += 256) {
    float v = 0.f;
    if (!bad) v = table_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(table)[base + i])
                             : static_cast<const float*>(table)[base + i];
    x[(int64_t)t * d + i] = v;
  }
}

hipError_t launch_embed_rows(const void* table, int table_bf16, const int32_t* tokens, int n,
                             int d, int vocab, float* x, StepDesc* desc, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed_rows, dim3((unsigned)n), dim3(256), 0, s, table, table_bf16, tokens,
                     d, vocab, x, desc);
  return hipGetLastError();
}

// ---- Q/K RMSNorm + RoPE + paged K/V append for P tokens ([Qwen3-runtime] §2.3-2.4, §7.1-7.2) -----
// One wave per (head, token): lane l < D/2 holds the pair (l, l + D/2) of the head's row, as the
// decode path does.  Q is stored normalised and rotated, rounded to bf16, not yet scaled; K and V
// go to slot pos % 16 of page bt[pos / 16].
template <int D>
__global__ __launch_bounds__(64) void k_prefill_rope(PrefillRopeArgs a) {
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x, hh = blockIdx.x, t = blockIdx.y;
  const int hq = a.n_q_heads, hkv = a.n_kv_heads;
  const int pos = a.pos0 + t;
  const bool act = lane < HALF;
  const int hl = lane & (HALF - 1);
  const bool is_q = hh < hq;
  const int g = hh - hq;
  const float* row = a.qkv + (int64_t)t * (hq + 2 * hkv) * D;
  const float* src = row + (int64_t)(is_q ? hh : hq + g) * D;
  float x0 = act ? src[hl] : 0.f, x1 = act ? src[hl + HALF] : 0.f;
  const float* gam = is_q ? a.q_gamma : a.k_gamma;
  if (gam != nullptr) {
    const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
    const float rinv = 1.0f / sqrtf(ss / (float)D + a.eps);
    x0 = x0 * rinv * gam[hl];
    x1 = x1 * rinv * gam[hl + HALF];
  }
  if (!act) return;
  const float2 cs = reinterpret_cast<const float2*>(a.table)[(int64_t)pos * HALF + lane];
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x1 * cs.x + x0 * cs.y;
  if (is_q) {
    const int64_t o = ((int64_t)t * hq + hh) * D + lane;
    a.q_out[o] = f32_to_bf16(y0);
    a.q_out[o + HALF] = f32_to_bf16(y1);
    return;
  }
  const int64_t phys = a.block_table[pos / kPage];
  const int64_t off = ((phys * hkv + g) * kPage + pos % kPage) * D + lane;
  const float* vs = row + (int64_t)(hq + hkv + g) * D;
  a.k_pool[off] = f32_to_bf16(y0);
  a.k_pool[off + HALF] = f32_to_bf16(y1);
  a.v_pool[off] = f32_to_bf16(vs[lane]);
  a.v_pool[off + HALF] = f32_to_bf16(vs[lane + HALF]);
}

hipError_t launch_prefill_rope(int head_dim, const PrefillRopeArgs& a, hipStream_t s) {
  if (a.p <= 0) return hipSuccess;
  const dim3 grid((unsigned)(a.n_q_heads + a.n_kv_heads), (unsigned)a.p);
  if (head_dim == 64)
    hipLaunchKernelGGL((k_prefill_rope<64>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k_prefill_rope<128>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace qd

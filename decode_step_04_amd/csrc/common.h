// common.h - device primitives and kernel argument blocks shared by the HIP kernels (gfx950).
//
// Wave64 throughout.  Reductions use DPP row operations inside each 16-lane row and
// v_readlane across rows, so they need every lane of the wave active (callers reduce in
// converged code, idle lanes contributing the neutral element).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

constexpr int kWave = 64;
constexpr int kPage = 16;  // tokens per KV page

// Weight storage types of the GEMV (values equal the public qdec_dtype codes): fp32, bf16, int8
// codes with a per-row scale, int8 codes with a scale per 128-value group, and int4 codes (two
// per byte, offset-binary, even element in the low nibble) with a scale per 128-value group.
enum WType : int { W_F32 = 0, W_BF16 = 1, W_I8 = 2, W_I8G = 3, W_I4G = 4 };
constexpr int kQGroup = 128;  // values per scale of the group-wise types

// ---- bf16 <-> fp32 -------------------------------------------------------------------------
// bf16 is the upper half of an fp32 word: widening is a 16-bit shift.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.  Branch-free.
// Round to nearest even (ties to even, overflow to infinity, NaN stays NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// ---- DPP wave reductions ---------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of a group gets the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  if (N >= 8) v += dpp<kDppHalfMirror>(v);
  if (N >= 16) v += dpp<kDppMirror>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  if (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Full-wave sum; the result is wave-uniform.  Fixed association order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// The two values of the lane pair (l, l ^ OFF), OFF = 8, 16 or 32: `lo` from the lane with bit
// OFF clear, `hi` from the lane with it set, identical on both lanes of the pair.  OFF = 8 uses
// a DPP rotation by 8 inside each 16-lane row; 16 and 32 use the gfx950 lane-swap instructions
// (v_permlane16_swap exchanges odd rows of its first operand with even rows of its second,
// v_permlane32_swap the upper half of the first with the lower half of the second), so no
// exchange goes through LDS.
template <int OFF>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "pair distance");
  const uint32_t u = __float_as_uint(v);
  if constexpr (OFF == 8) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    const bool upper = (__lane_id() & 8) != 0;
    lo = upper ? o : v;
    hi = upper ? v : o;
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}

// ---- split-KV partition sizing (shared by the host launcher and the kernels) -----------------
// Fixed partitions when part_fixed > 0; otherwise the partition length grows with the context
// so that Hkv * n_part stays near target_wgs work-groups, between 64 and kMaxPartTokens tokens.
// Partitions are at most kMaxPartTokens long (the attention kernel reads a partition's
// block-table entries ahead, 8 pages per wave).
constexpr int kMaxPartTokens = 512;
__host__ __device__ inline int part_tokens_for(int ctx, int part_fixed, int n_kv_heads,
                                               int target_wgs) {
  if (part_fixed > 0) return part_fixed;
  long long want = ((long long)ctx * n_kv_heads + target_wgs - 1) / target_wgs;
  int p = (int)(((want + 63) / 64) * 64);
  p = p < 64 ? 64 : p;
  return p > kMaxPartTokens ? kMaxPartTokens : p;
}
__host__ __device__ inline int n_parts_for(int ctx, int part_tokens) {
  return (ctx + part_tokens - 1) / part_tokens;
}

// ---- kernel argument blocks (passed by value) -----------------------------------------------

// Step descriptor in device memory: written by the embedding kernel, read by the later kernels
// of the step, so a replayed graph needs only the embedding node's arguments updated.
struct StepDesc {
  int32_t pos;
  int32_t ctx;    // pos + 1
  int32_t error;  // sticky: 1 after an out-of-range token id
  int32_t pad;
};

struct GemvArgs {
  const void* w;          // [rows x k] (rows = n, or 2n for SwiGLU: gate rows then up rows)
  const float* scale;     // fp32 scales: [rows] (W_I8) or [rows][k / 128] (W_I8G, W_I4G)
  const void* x;          // input vector [k]; the raw fp32 residual when gamma != nullptr
  int32_t x_bf16;         // x element type
  int32_t round_h;        // round the normalised input to bf16 (16-bit activations)
  const float* gamma;     // RMSNorm gamma [k], or nullptr for no norm prologue
  float eps;
  int32_t y_bf16;         // output element type for EPI_STORE / EPI_SWIGLU
  void* y;                // output [n]
  float* resid;           // EPI_RESID: resid[n] += W x
  float* hidden_copy;     // optional: work-group 0 copies the raw input x here
  float* part_val;        // optional (EPI_STORE): per-work-group largest rounded output ...
  int32_t* part_idx;      // ... and its lowest row index (-1 when none)
  int32_t part_cap;       // entries of part_val / part_idx: the launcher refuses a plan with more
                          // work-groups (each writes the entry of its index)
  int64_t n;              // output rows
  int64_t k;              // input length
  int32_t split;          // waves sharing one row group along K (set by the launcher)
};

// Prefill GEMM Y[m x n] = A[m x k] . W[n x k]^T with bf16 A and W (row-major, k contiguous).

struct AttnArgs {
  // fused (model) path: the query heads and the new K/V come from the QKV projection output
  const float* qkv;           // [(Hq + 2 Hkv) D] fp32
  const float* q_gamma;       // [D] or nullptr (no Q/K norm)
  const float* k_gamma;
  float eps;
  const float* rope_table;    // [max_pos][D/2][2] (cos, sin)
  const float* rope_step;     // [D/2][2]: the row of rope_table at this step's pos
  int32_t round_q;            // round the rotated query to bf16 (16-bit activations)
  // op path: the rotated query heads are given
  const void* q;              // [Hq x D] (bf16 or fp32)
  int32_t q_bf16;
  void* k_pool;               // [P][Hkv][16][D] (bf16 or fp32); appended to on the fused path
  void* v_pool;
  const int32_t* block_table;
  int32_t bt_len;             // entries that may be read ahead of ctx (all valid page numbers)
  const StepDesc* desc;       // ctx from here when non-null
  int32_t ctx_arg;            // ctx when desc == nullptr
  int32_t n_q_heads, n_kv_heads;
  int32_t part_tokens;        // partition length, a multiple of 64
  int32_t max_parts;          // scratch stride (partitions per head)
  int32_t part_base;          // scratch slot of this launch's partition 0 (tiles of a longer context)
  int32_t to_partials;        // always write (m, l, acc), even for a single partition; the merge
                              // then normalises a lone partition too
  float* part_acc;            // [Hq][max_parts][D] unnormalised accumulators
  float* part_ml;             // [Hq][max_parts][2]: running max (log2 units) and denominator
  void* out;                  // [Hq x D]
  int32_t out_bf16;
  float qscale;               // log2(e) / sqrt(D)
};

struct RopeAppendArgs {
  const float* qkv;           // [(Hq + 2 Hkv) D] fp32
  const float* q_gamma;       // [D] or nullptr (no Q/K norm)
  const float* k_gamma;
  float eps;
  const float* table;         // [max_pos][D/2][2] (cos, sin)
  const StepDesc* desc;
  int32_t pos_arg;
  void* q_out;
  int32_t q_bf16;
  void* k_pool;
  void* v_pool;
  int32_t kv_bf16;
  const int32_t* block_table;
  int32_t n_q_heads, n_kv_heads;
};

// Batched prefill: Q/K RMSNorm + RoPE + paged K/V append of P tokens, and causal attention.
struct PrefillRopeArgs {
  const float* qkv;           // [P][(Hq + 2 Hkv) D] fp32
  const float* q_gamma;       // [D] or nullptr (no Q/K norm)
  const float* k_gamma;
  float eps;
  const float* table;         // [max_pos][D/2][2] (cos, sin)
  uint16_t* q_out;            // [P][Hq][D] bf16 (normalised, rotated, not scaled)
  uint16_t* k_pool;           // [pages][Hkv][16][D] bf16
  uint16_t* v_pool;
  const int32_t* block_table;
  int32_t pos0, p, n_q_heads, n_kv_heads;
};

struct GemmArgs {
  const void* a;          // [m x k] bf16
  const void* w;          // [n x k] bf16 ([2n x k] for SwiGLU: gate rows, then up rows)
  void* y;                // EPI_STORE: [m x n] fp32 or bf16; EPI_SWIGLU: [m x n] bf16
  int32_t y_bf16;
  float* resid;           // EPI_RESID: resid[m x n] += A W^T
  int32_t m, n, k;        // k % 32 == 0
  PrefillRopeArgs rope;   // EPI_ROPE: where the rows go (its qkv field is unused)
};

struct PrefillAttnArgs {
  const uint16_t* q;          // [P][Hq][D] bf16
  const uint16_t* k_pool;     // [pages][Hkv][16][D] bf16, holding positions 0 .. pos0 + P - 1
  const uint16_t* v_pool;
  const int32_t* block_table;
  uint16_t* out;              // [P][Hq][D] bf16
  int32_t pos0, p, n_q_heads, n_kv_heads;
  float qscale;               // log2(e) / sqrt(D)
};

// Temperature + top-p sampling of one token from logits[n].
struct SampleArgs {
  const void* logits;         // [n] bf16 or fp32
  int32_t x_bf16;
  int64_t n;
  float inv_temperature;      // 1 / T, T > 0
  float top_p;                // (0, 1]
  uint64_t seed;              // Philox key
  const StepDesc* desc;       // position from here when non-null (graph replay) ...
  int32_t pos_arg;            // ... else this one; the Philox counter
  int32_t* out;               // the sampled token
  const float* part_val;      // optional: maxima of disjoint parts of the stored logits that
  int32_t n_parts;            //   together cover all of them (the LM head's argmax partials)
  void* ws;                   // sample_workspace_bytes(n) bytes, 256-byte aligned
};

struct EmbedArgs {
  const void* table;          // [V x d] (bf16 or fp32), used when emb == nullptr
  int32_t table_bf16;
  const void* emb;            // caller's embedding row (act dtype) or nullptr
  const int32_t* token;       // device token id
  float* x;                   // [d] fp32 residual stream
  StepDesc* desc;             // written: pos, ctx (nullable)
  const float* rope_table;    // [max_pos][half][2] (nullable)
  float* rope_step;           // written: row pos of rope_table (the attention kernel reads it
  int32_t rope_half;          // without waiting for the descriptor)
  int32_t pos;
  int32_t vocab;
  int32_t d;
};

}  // namespace qd

// launch.h - host-side launchers of the HIP kernels (internal to the library).
//
// Each launcher enqueues one kernel on `stream` and returns hipGetLastError() of the launch.
// Shapes have been validated by the caller (runtime.hip); the launchers only derive grids.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace qd {

// EPI_ROPE (prefill QKV, head_dim 128): the Q/K norm, RoPE and paged K/V append of
// k_prefill_rope applied to each 128-column tile (one head) of the product in the epilogue
enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ROPE = 3 };

// The RMSNorm prologue stages x * gamma in LDS: norm GEMVs take inputs of at most this length.
constexpr int64_t kGemvNormMaxK = 16384;
hipError_t launch_gemv(int wtype, int epi, bool norm, const GemvArgs& a, hipStream_t s);
// Number of work-groups (= partial argmax slots) launch_gemv uses for this shape.
int gemv_partials(int wtype, int epi, int64_t n, int64_t k);
// Whether launch_gemv handles this shape: k a multiple of the lane vector (and of 128 for the
// group-wise types) and each wave's K-slice within 8 wave-wide loads (k <= 8192 fp32, 16384
// bf16, 32768 int8 or int4 weights).
bool gemv_supported(int wtype, int epi, int64_t n, int64_t k);
// Final reduction of per-work-group (value, index) partials to the argmax.
hipError_t launch_argmax_partials(const float* val, const int32_t* idx, int n, int32_t* out,
                                  hipStream_t s);

// Split-KV attention over `grid_parts` partitions per KV head (surplus ones exit early); `fused`
// adds the Q/K norm + RoPE + K/V append prologue.
hipError_t launch_attention(int head_dim, bool kv_bf16, int group, bool fused, const AttnArgs& a,
                            int grid_parts, hipStream_t s);
// Exact merge of the partitions (a no-op when the context fits one partition).
hipError_t launch_attention_merge(int head_dim, const AttnArgs& a, hipStream_t s);
constexpr int kMaxMergeParts = 8192;  // partitions per head the split-KV scratch layout allows

hipError_t launch_rope_append(int head_dim, const RopeAppendArgs& a, hipStream_t s);
// Prefill GEMM on MFMA (epi: EPI_STORE, EPI_RESID or EPI_SWIGLU); k % 32 == 0.
hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s);
// Prefill: Q/K norm + RoPE + paged append of P tokens; causal GQA attention on the matrix cores.
hipError_t launch_prefill_rope(int head_dim, const PrefillRopeArgs& a, hipStream_t s);
hipError_t launch_prefill_attn(int head_dim, int group, const PrefillAttnArgs& a, hipStream_t s);
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);
// Temperature + top-p sampling (one 1024-thread work-group).
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);
int64_t sample_workspace_bytes(int64_t n);
const void* embed_kernel_fn();

hipError_t launch_argmax(const void* x, int x_bf16, int64_t n, int32_t* out, hipStream_t s);
hipError_t launch_quantize(const void* w, int src_bf16, int8_t* q, float* scale, int64_t n,
                           int64_t k, hipStream_t s);
// Group-wise quantisation, 128-value groups: bits = 8 (int8 codes [n][k]) or 4 (packed int4
// [n][k / 2]); scale [n][k / 128].  k % 128 == 0.
hipError_t launch_quantize_groups(const void* w, int src_bf16, int bits, void* q, float* scale,
                                  int64_t n, int64_t k, hipStream_t s);
hipError_t launch_kv_copy(void* pool, void* linear, const int32_t* block_table, int pos0, int n,
                          int n_kv_heads, int head_dim, int elem, int to_pool, hipStream_t s);
hipError_t launch_rope_table(float* table, int max_pos, int head_dim, float theta, hipStream_t s);
// bytes % 16 == 0; at most max_wgs work-groups (4096 fill the chip; a few dozen saturate the host
// link when src is mapped host memory)
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s,
                       int max_wgs = 4096);
hipError_t launch_convert(void* dst, int dst_type, const void* src, int src_type, int64_t n,
                          hipStream_t s);
hipError_t launch_rmsnorm(const float* x, const float* gamma, float eps, void* y, int y_bf16,
                          int n, hipStream_t s);
// RMSNorm of `rows` consecutive rows of n values (one work-group per row).
hipError_t launch_rmsnorm_rows(const float* x, const float* gamma, float eps, void* y, int y_bf16,
                               int n, int rows, hipStream_t s);
// Prefill embedding: x[t] = E[tokens[t]] widened to fp32 for t < n; a bad id gives a zero row and
// sets desc->error.
hipError_t launch_embed_rows(const void* table, int table_bf16, const int32_t* tokens, int n,
                             int d, int vocab, float* x, StepDesc* desc, hipStream_t s);

}  // namespace qd

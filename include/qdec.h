/*
 * qdec.h - C ABI of the batch-1 GQA decode-step library for AMD Instinct MI355X (gfx950).
 *
 * The library runs one decode step of a Llama/Qwen3-style grouped-query-attention transformer
 * (one new token, batch 1) entirely in hand-written HIP kernels on one GPU.  Every entry point
 * takes plain pointers and sizes; no torch or HIP types appear here (a stream is passed as an
 * opaque `void*` holding a hipStream_t, NULL meaning the legacy default stream).
 *
 * Sources the operations follow (cited by page title and section):
 *   [Qwen3-runtime]  "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化"
 *                    (chengzipai.xyz, a Qwen3-0.6B CUDA runtime).  Sections 0.1-14.6.
 *   [ETE]            "EdgeTransformerEngine" (thomasli.cn/cuda-engine.html), a hand-written
 *                    Llama-style CUDA engine behind an extern "C" DLL.
 *   [DSV4-stream]    "【DGX Spark 实战】面向 128GB 统一内存的DeepSeek-V4 流式推理引擎设计及实现"
 *                    (cnblogs.com), only for its graph-capture lessons (issues 9, 12, 14; 7.7).
 *
 * General rules, for every function below:
 *   - Return value: a qdec_status.  Nothing throws, aborts or exits across the ABI.
 *   - Validation happens on the host before anything is enqueued; a call that fails
 *     validation enqueues nothing and changes no state.
 *   - A failing HIP runtime call yields QDEC_E_HIP; the HIP error string is kept for
 *     qdec_last_error().  Faults inside a kernel are asynchronous and surface at the caller's
 *     next synchronisation of the stream (as for any HIP kernel).
 *   - Work is enqueued on the caller's stream and the call returns without synchronising
 *     (unless a function says otherwise).  Buffers passed in must stay valid until the
 *     enqueued work has completed.  The library never uses another stream for step work.
 *   - "device" pointers are HIP device allocations on the context's device; "host" pointers are
 *     ordinary host memory.
 *   - A context is not thread-safe: one host thread at a time.
 *   - Matrices are row-major [rows x cols] with cols (the input dimension K) contiguous; a
 *     projection computes y[n] = sum_k W[n][k] * x[k].
 */
#ifndef QDEC_H
#define QDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDEC_ABI_VERSION 1

typedef enum qdec_status {
  QDEC_OK = 0,
  QDEC_E_INVAL = 1,        /* bad argument: NULL/misaligned pointer, bad size, bad enum value */
  QDEC_E_UNSUPPORTED = 2,  /* valid request the library does not implement (capability gate) */
  QDEC_E_STATE = 3,        /* call made in the wrong state (e.g. step before all weights uploaded) */
  QDEC_E_RANGE = 4,        /* position/context outside max_context or the block table */
  QDEC_E_NOMEM = 5,        /* device allocation failed at create */
  QDEC_E_HIP = 6           /* a HIP runtime call failed */
} qdec_status;

/* Storage types.  [ETE] (the bf16 storage passage) and [Qwen3-runtime] §0.1: bf16 is a storage
 * format; every product and reduction is done in fp32.  QDEC_I8_ROW is W8A16 with one fp32 scale
 * per output row (symmetric, codes in [-127, 127]; [ETE], the int8 quantisation passage). */
/* QDEC_I8_G128 and QDEC_I4_G128 keep one fp32 scale per 128-value group of a row
 * ([Qwen3-runtime] §13.1: the W8A16 kernel walks a row in 128-value groups, each with its own
 * scale; [ETE] names 4-bit codes as the next step).  Per group: scale = max|w| / 127 (int8) or
 * / 7 (int4) in fp32, codes round-half-even(w / scale) clamped to [-127, 127] or [-7, 7].
 * Layouts, row-major [rows x cols]: I8_G128 codes are int8 [rows][cols]; I4_G128 codes are two per
 * byte, [rows][cols / 2], element 2j in the low nibble of byte j, each nibble stored as code + 8;
 * scales [rows][cols / 128].  cols % 128 == 0. */
typedef enum qdec_dtype {
  QDEC_F32 = 0, QDEC_BF16 = 1, QDEC_I8_ROW = 2, QDEC_I8_G128 = 3, QDEC_I4_G128 = 4
} qdec_dtype;

/* Model and cache geometry.  [Qwen3-runtime] §1.1 (shapes), §2.1-2.7 (the layer), §3.3 (KV). */
typedef struct qdec_config {
  int32_t n_layers;       /* transformer blocks, >= 1 */
  int32_t hidden;         /* d: residual width, multiple of 64 */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 8 ([Qwen3-runtime] §2.5) */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t ffn;            /* F: SwiGLU inner width, multiple of 64 */
  int32_t vocab;          /* V */
  int32_t tied_lm_head;   /* 1: the LM head is the embedding table ([Qwen3-runtime] §1.1) */
  int32_t qk_norm;        /* 1: per-head RMSNorm of Q and K before RoPE ([Qwen3-runtime] §2.3) */
  float rms_eps;          /* RMSNorm epsilon, > 0 (1e-6 in [Qwen3-runtime] §2.1) */
  float rope_theta;       /* RoPE base, > 1 */
  int32_t proj_dtype;     /* qdec_dtype of the QKV, O, gate-up and down projections */
  int32_t lm_head_dtype;  /* qdec_dtype of the LM head */
  int32_t io_dtype;       /* QDEC_F32 | QDEC_BF16: the embedding table, a caller's token_embedding
                             and logits_out */
  int32_t act_dtype;      /* QDEC_F32 | QDEC_BF16: activations that cross an op boundary inside the
                             step (the normalised GEMV inputs, rotated Q, attention output, SwiGLU
                             output).  F32 keeps bf16 a storage format only ([ETE], the bf16
                             passage); BF16 rounds them as in [Qwen3-runtime] §0.1 (the "A16" of
                             W8A16).  The residual stream is always fp32. */
  int32_t kv_dtype;       /* QDEC_F32 | QDEC_BF16: KV-cache storage */
  int32_t page_size;      /* tokens per KV page; must be 16 */
  int32_t num_pages;      /* physical pages in the pool (each layer has its own pool of this size) */
  int32_t max_context;    /* positions 0 .. max_context-1 may be decoded; <= num_pages*page_size */
  int32_t partition_size; /* split-KV partition length in tokens (multiple of 64, at most 512),
                           * 0 = automatic (about one GPU-full of work-groups at max_context) */
  int32_t max_prefill;    /* most tokens one qdec_prefill call takes (its buffers are allocated
                           * at create); 0 = no prefill.  Prefill needs bf16 projections, io and
                           * KV. */
  int32_t weight_slots;   /* Where the layers' projections live.  0: device memory.  N in
                           * [1, n_layers]: layer streaming ([ETE], the "Layer streaming" passage):
                           * every layer's projections live in pinned host memory that the context
                           * allocates, and N device slots hold N layers at a time - layer l
                           * computes from slot l % N, a copy stream fills the slot for layer l+N
                           * once layer l has finished with it (buffer free), and layer l's kernels
                           * wait for their slot's copy (data ready); steps then run eagerly (no
                           * graph capture).  -1: the same pinned host copy, read by the kernels
                           * through its device mapping (no copies, no slots; graph capture
                           * allowed).  Gammas, embedding and LM head stay in device memory.
                           * Host-resident layers take no prefill (max_prefill 0). */
} qdec_config;

/* Supported dtype combinations (checked by qdec_config_validate):
 *   io F32  : proj, lm_head, act and kv all F32                                  (the fp32 path)
 *   io BF16 : proj and lm_head each BF16 | I8_ROW | I8_G128 | I4_G128, act F32 | BF16, kv BF16
 *             (bf16 / W8A16 / W4A16); the group-wise types need hidden, ffn and
 *             n_q_heads * head_dim to be multiples of 128 */

/* Weight slots for qdec_upload / qdec_upload_quantized.  Norm gammas are always stored fp32 (small
 * sensitive tensors stay fp32: [ETE], the int8 quantisation passage). */
typedef enum qdec_weight {
  QDEC_W_EMBED = 0,      /* [vocab x hidden] in io_dtype; global (layer ignored) */
  QDEC_W_LM_HEAD = 1,    /* [vocab x hidden] in lm_head_dtype; global.  With tied_lm_head the
                            slot is filled from QDEC_W_EMBED's upload and may not be uploaded. */
  QDEC_W_FINAL_NORM = 2, /* [hidden] fp32; global */
  QDEC_W_IN_NORM = 3,    /* [hidden] fp32, input RMSNorm of a layer ([Qwen3-runtime] §2.1) */
  QDEC_W_POST_NORM = 4,  /* [hidden] fp32, post-attention RMSNorm ([Qwen3-runtime] §2.7) */
  QDEC_W_Q_NORM = 5,     /* [head_dim] fp32, shared by all Q heads ([Qwen3-runtime] §2.3) */
  QDEC_W_K_NORM = 6,     /* [head_dim] fp32, shared by all K heads */
  QDEC_W_QKV = 7,        /* [(Hq+2*Hkv)*D x hidden]: Q rows, then K rows, then V rows
                            ([Qwen3-runtime] §2.2, packed along the output dimension) */
  QDEC_W_O = 8,          /* [hidden x Hq*D] ([Qwen3-runtime] §2.6) */
  QDEC_W_GATE_UP = 9,    /* [2*ffn x hidden]: gate rows 0..F-1, then up rows ([Qwen3-runtime] §2.7) */
  QDEC_W_DOWN = 10       /* [hidden x ffn] */
} qdec_weight;

typedef struct qdec_ctx qdec_ctx; /* opaque, owned by the library */

/* One decode step ([Qwen3-runtime] §3.2: one new token per step; [ETE] the GPU block pipeline).
 * All pointers are device pointers owned by the caller. */
typedef struct qdec_step {
  const void* token_embedding; /* [hidden] io_dtype input row, or NULL to gather EMBED[*token_id] */
  const int32_t* token_id;     /* device int32 token id (read on the device, so it may be the
                                  previous step's argmax_out); required if token_embedding is NULL.
                                  An id outside [0, vocab) yields a zero row and sets the device
                                  error flag read by qdec_device_error. */
  int32_t pos;                 /* 0-based position of the new token; attention covers 0..pos */
  int32_t reserved;            /* must be 0 */
  float* hidden_out;           /* optional [hidden] fp32: residual stream after the last layer */
  void* logits_out;            /* optional [vocab] io_dtype logits.  NULL together with
                                  argmax_out == NULL skips the final norm and LM head (the
                                  prompt-token trim of [ETE]) */
  int32_t* argmax_out;         /* optional device int32: the next token.  With temperature 0,
                                  the index of the largest logit (the lowest index winning ties;
                                  NaN logits never win); with temperature > 0, a token sampled
                                  as qdec_op_sample does from the step's logits, with this
                                  step's pos as the Philox counter */
  float temperature;           /* 0: greedy; > 0 (finite): sampling temperature */
  float top_p;                 /* sampling only: nucleus mass, in (0, 1] */
  uint64_t seed;               /* sampling only: Philox key.  A captured graph keeps the
                                  temperature, top_p and seed of its template step */
} qdec_step;

/* Sizes and byte counts derived from a config.  [Qwen3-runtime] §1.1 (parameter count),
 * §3.3 (KV bytes 2*Hkv*D*elem per layer-token), §4.1 (weight bytes streamed per token). */
typedef struct qdec_info {
  int64_t params_per_layer;        /* matrices + the four gammas of one layer */
  int64_t params_total;            /* all layers + embedding + final norm (+ LM head if untied) */
  int64_t layer_matrix_bytes;      /* bytes of all layers' matrices as stored (codes if quantised) */
  int64_t layer_scale_bytes;       /* fp32 scales of quantised layer matrices (0 otherwise) */
  int64_t lm_head_bytes;           /* LM head as stored, scales included */
  int64_t kv_bytes_per_layer_token;
  int64_t kv_pool_bytes;           /* n_layers * 2 * num_pages * page_size * Hkv * D * elem */
  int64_t device_bytes;            /* device memory qdec_create allocates for this config (from
                                      qdec_info_get: what the context did allocate) */
  int32_t partition_tokens;        /* split-KV partition length in effect */
  int32_t max_partitions;          /* ceil(max_context / partition_tokens) */
} qdec_info;

/* Algorithmic HBM bytes of one decode step at context T (pos = T-1), per kernel class and in
 * total: weights and scales read once, the embedding row, gammas, T keys and values read per
 * layer, one key and value written per layer, logits written.  Split-KV scratch traffic is
 * listed separately (overhead, not part of total). */
typedef struct qdec_bytes {
  int64_t embed, qkv, rope_append, attention, merge, o_proj, gate_up, down, lm_head, argmax;
  int64_t total;
  int64_t scratch;
} qdec_bytes;

/* ---- configuration (host only; callable without a GPU) ----------------------------------- */

/* Capability gate ([ETE] lists silent wrong results on unsupported head_dim and unread fields as
 * its worst failure, and proposes a load-time check).  Returns QDEC_OK, QDEC_E_INVAL (malformed)
 * or QDEC_E_UNSUPPORTED (well-formed but not implemented); writes a NUL-terminated reason into
 * msg[0..len) when msg != NULL. */
qdec_status qdec_config_validate(const qdec_config* cfg, char* msg, size_t len);

/* Fills *out for a valid config. */
qdec_status qdec_config_info(const qdec_config* cfg, qdec_info* out);

/* Algorithmic bytes of one step at context `context` (1 <= context <= max_context).
 * with_logits = 0 leaves out the final norm, LM head and argmax. */
qdec_status qdec_bytes_model(const qdec_config* cfg, int32_t context, int32_t with_logits,
                             qdec_bytes* out);

/* ---- context lifecycle --------------------------------------------------------------------- */

/* Validates cfg, selects `device`, and allocates every device buffer the context will ever use:
 * weights, KV pool, block table, RoPE cos/sin table, split-KV scratch, activations and the step
 * descriptor ([Qwen3-runtime] §5.2: nothing is allocated on the decode path).  The KV pool is
 * filled with zeros.  On failure *out is NULL and nothing stays allocated. */
qdec_status qdec_create(const qdec_config* cfg, int32_t device, qdec_ctx** out);

/* Frees everything the context owns (synchronises the device first).  NULL is ignored. */
void qdec_destroy(qdec_ctx* ctx);

/* Last error message of ctx (or of the calling thread's last context-free call when ctx is
 * NULL).  The string is owned by the library and valid until the next call. */
const char* qdec_last_error(const qdec_ctx* ctx);

/* Human-readable name of a status code (static storage). */
const char* qdec_status_string(qdec_status s);

/* Info for the context's config (same as qdec_config_info, plus the partition size in effect). */
qdec_status qdec_info_get(const qdec_ctx* ctx, qdec_info* out);

/* ---- weights ------------------------------------------------------------------------------- */

/* Copies one weight tensor into the context, converting to the slot's storage dtype:
 * F32->BF16 rounds to nearest even, BF16->F32 widens exactly, F32|BF16 -> I8_ROW quantises each
 * row on the device (scale = max|row| / 127 in fp32, code = round-half-even(w / scale) clamped to
 * [-127, 127], zero rows get scale 0 and zero codes), F32|BF16 -> I8_G128 | I4_G128 quantises
 * each 128-value group the same way (qdec_dtype).  `src` is [rows x cols] of src_dtype
 * (QDEC_F32 or QDEC_BF16), contiguous; rows/cols must equal the slot's shape.  `layer` selects the
 * block for per-layer slots (ignored for global ones).  A host source (src_is_device = 0) is
 * accepted only when no conversion is needed.  Uploading QDEC_W_EMBED with tied_lm_head also
 * fills the LM head (quantising it when lm_head_dtype is quantised).  Asynchronous on `stream`,
 * except for a projection of a host-resident layer (weight_slots != 0): that one is converted in
 * device staging memory and copied to the layer's pinned host copy before the call returns, so it
 * must not overlap a decode step. */
qdec_status qdec_upload(qdec_ctx* ctx, int32_t layer, int32_t which, const void* src,
                        int32_t src_dtype, int64_t rows, int64_t cols, int32_t src_is_device,
                        void* stream);

/* Copies pre-quantised codes and fp32 scales, in the layouts of the slot's dtype (qdec_dtype),
 * into a quantised slot (I8_ROW, I8_G128 or I4_G128); QDEC_E_INVAL for another slot dtype or a
 * shape mismatch.  Asynchronous on `stream`; a host source is copied synchronously; a projection
 * of a host-resident layer goes through device staging to the layer's host copy, synchronously. */
qdec_status qdec_upload_quantized(qdec_ctx* ctx, int32_t layer, int32_t which, const void* codes,
                                  const float* scales, int64_t rows, int64_t cols,
                                  int32_t src_is_device, void* stream);

/* qdec_upload_quantized for an I8_ROW slot only: codes [rows x cols] int8, scales [rows]. */
qdec_status qdec_upload_i8(qdec_ctx* ctx, int32_t layer, int32_t which, const int8_t* codes,
                           const float* scales, int64_t rows, int64_t cols, int32_t src_is_device,
                           void* stream);

/* Pointers of a stored weight slot (for read-back in tests): *data receives the matrix as stored,
 * *scales the fp32 scales (NULL unless quantised).  Device pointers, except for the projections
 * of a host-resident layer (weight_slots != 0), whose storage is the context's pinned host copy
 * (its device mapping when weight_slots = -1). */
qdec_status qdec_weight_ptr(const qdec_ctx* ctx, int32_t layer, int32_t which, void** data,
                            float** scales);

/* ---- paged KV cache ([Qwen3-runtime] §7.2: logical page -> physical page via a block table) -- */

/* Physical layout of each layer's pool (element offsets; elem = 4 or 2 bytes by kv_dtype):
 *   K of (position p, kv head g, dim r) at
 *     ((bt[p / page_size] * Hkv + g) * page_size + p % page_size) * D + r
 *   from the layer's K base; V likewise from its V base.  One page of one head is a contiguous
 *   page_size x D tile. */

/* Copies the block table (host int32[n_logical], entry i = physical page of logical page i) to
 * the device.  Entries must be distinct and in [0, num_pages); n_logical * page_size must cover
 * max_context or later steps beyond the mapped range fail with QDEC_E_RANGE.  Synchronous with
 * respect to the host buffer (it may be freed on return). */
qdec_status qdec_kv_set_block_table(qdec_ctx* ctx, const int32_t* table, int32_t n_logical,
                                    void* stream);

/* Writes n logical positions pos0..pos0+n-1 of one layer: k, v are device [n x Hkv x D] arrays
 * in kv_dtype, scattered into the pool through the block table (pre-filling a context). */
qdec_status qdec_kv_write(qdec_ctx* ctx, int32_t layer, int32_t pos0, int32_t n, const void* k,
                          const void* v, void* stream);

/* Reads n logical positions back into device [n x Hkv x D] arrays (inverse of qdec_kv_write). */
qdec_status qdec_kv_read(qdec_ctx* ctx, int32_t layer, int32_t pos0, int32_t n, void* k, void* v,
                         void* stream);

/* Raw device base pointers of a layer's K and V pools (layout above). */
qdec_status qdec_kv_pool_ptr(const qdec_ctx* ctx, int32_t layer, void** k_pool, void** v_pool);

/* ---- the decode step ----------------------------------------------------------------------- */

/* Enqueues one decode step on `stream` ([Qwen3-runtime] §2.1-2.7 for one token; [ETE] pipeline):
 * embedding -> per layer { RMSNorm + QKV projection, Q/K RMSNorm + RoPE + paged K/V append at
 * `pos`, split-KV causal GQA attention over 0..pos with an exact partition merge, O projection +
 * residual, RMSNorm + gate-up projection + SwiGLU, down projection + residual } -> optional
 * final RMSNorm + LM head + argmax.  Allocates nothing and does not synchronise.  Requires every
 * weight slot uploaded (QDEC_E_STATE), a block table mapping pos (QDEC_E_RANGE), and
 * 0 <= pos < max_context (QDEC_E_RANGE). */
qdec_status qdec_decode_step(qdec_ctx* ctx, const qdec_step* step, void* stream);

/* Batched prefill of n_tokens prompt tokens at positions pos0 .. pos0 + n_tokens - 1 ([ETE], the
 * batched-prefill next step: GEMMs on the matrix cores and FlashAttention-style causal attention
 * over the paged cache, which it fills).  It computes what n_tokens decode steps would, with the
 * 16-bit activation policy (act_dtype BF16) at every op boundary: the GEMM inputs, the rotated
 * queries, the attention output and the SwiGLU output are bf16; the residual stream stays fp32.
 * token_ids: device [n_tokens]; an id outside [0, vocab) gives a zero row and sets the device
 * error flag.  Outputs, each optional, are those of the last token: hidden_out [hidden] fp32
 * (the residual stream after the last layer), logits_out [vocab] of io_dtype, argmax_out.
 * Requires max_prefill >= n_tokens >= 1 (QDEC_E_INVAL), every weight slot uploaded
 * (QDEC_E_STATE), and a block table mapping pos0 + n_tokens - 1 < max_context (QDEC_E_RANGE).
 * Allocates nothing and does not synchronise. */
qdec_status qdec_prefill(qdec_ctx* ctx, const int32_t* token_ids, int32_t n_tokens, int32_t pos0,
                         float* hidden_out, void* logits_out, int32_t* argmax_out, void* stream);

/* Captures the step described by `templ` (its buffers, not its pos) into a HIP graph whose
 * kernels read pos from a device descriptor, and sizes the split-KV grid for max_context
 * ([Qwen3-runtime] §5.2 static buffers, §14.5 graph replay; [DSV4-stream] issue 14: capture
 * executes nothing, so it writes no KV).  Replaces any previously captured graph. */
qdec_status qdec_graph_capture(qdec_ctx* ctx, const qdec_step* templ, void* stream);

/* Launches the captured graph on `stream` for position `pos` (same checks as qdec_decode_step).
 * Produces bit-identical results to qdec_decode_step with the template's buffers. */
qdec_status qdec_graph_replay(qdec_ctx* ctx, int32_t pos, void* stream);

/* Drops the captured graph, if any. */
qdec_status qdec_graph_reset(qdec_ctx* ctx);

/* Synchronises `stream` and reports the device error flag (1 if a kernel saw an out-of-range
 * token id since the last call), then clears it. */
qdec_status qdec_device_error(qdec_ctx* ctx, int32_t* flag, void* stream);

/* ---- per-kernel timing with HIP events (eager steps only) ---------------------------------- */

/* Kernel classes of the step, for the event profiler and qdec_bytes. */
typedef enum qdec_kclass {
  QDEC_K_EMBED = 0, QDEC_K_QKV = 1, QDEC_K_ROPE_APPEND = 2, QDEC_K_ATTENTION = 3, QDEC_K_MERGE = 4,
  QDEC_K_O_PROJ = 5, QDEC_K_GATE_UP = 6, QDEC_K_DOWN = 7, QDEC_K_LM_HEAD = 8, QDEC_K_ARGMAX = 9,
  QDEC_K_COUNT = 10
} qdec_kclass;

/* enable = 1: later qdec_decode_step calls record a HIP event pair around every kernel launch,
 * on the step's stream.  enable = 0 turns it off and clears the totals. */
qdec_status qdec_profile_enable(qdec_ctx* ctx, int32_t enable);

/* Waits for the events of the last profiled step and adds their elapsed times to the running
 * totals; then copies the totals out: ms[k] = summed milliseconds and launches[k] = launch count
 * for each class k < QDEC_K_COUNT (either pointer may be NULL). */
qdec_status qdec_profile_collect(qdec_ctx* ctx, double* ms, int64_t* launches);

/* Enqueues `reps` launches of one kernel class of the step (QDEC_K_QKV .. QDEC_K_ARGMAX, not
 * QDEC_K_EMBED or QDEC_K_ROPE_APPEND) exactly as qdec_decode_step launches it for `layer` with
 * the buffers and pos of `step` (same arguments, grid and data; the kernels read pos from the
 * step descriptor the last embedding kernel wrote, so run a step at the same pos first).
 * layer = -1 cycles through the layers (launch i uses layer i % n_layers), so consecutive
 * launches read different weights and KV pools, as in a step, instead of finding the previous
 * launch's data in the caches.  Meant for timing one kernel in isolation, for example inside a
 * captured graph.  Side effects are those of repeating the kernel: O and down projections add
 * into the residual stream on every launch, and the attention kernel re-appends the K/V row of
 * pos.  QDEC_E_INVAL for a bad class, layer < -1, layer >= n_layers or reps < 1. */
qdec_status qdec_profile_kernel(qdec_ctx* ctx, int32_t kclass, int32_t layer, int32_t reps,
                                const qdec_step* step, void* stream);

/* ---- op-level entry points on caller-owned device buffers ---------------------------------- */

/* y = W x for one row-major matrix ([Qwen3-runtime] §4.1: M = 1 is a GEMV; §13.1 W8A16).
 * w: [n x k] of w_dtype (F32, BF16, or quantised codes with w_scale: [n] fp32 row scales for
 * I8_ROW, [n][k / 128] group scales for I8_G128 / I4_G128 (qdec_dtype), whose k must be a
 * multiple of 128; w_scale must be NULL otherwise).  x: [k] of x_dtype (F32 | BF16).  y: [n] of
 * y_dtype (F32 | BF16, the fp32 sum rounded to nearest even).  A row must fill whole 16-byte
 * vectors (k a multiple of 4 fp32, 8 bf16, 16 int8 or 32 int4 values) and k be at most
 * 8192 (F32 weights), 16384 (BF16) or 32768 (int8 / int4): the kernel keeps each wave's slice of x
 * in registers (QDEC_E_UNSUPPORTED beyond).  w and x 16-byte aligned, y and w_scale 4-byte
 * aligned (QDEC_E_INVAL otherwise). */
qdec_status qdec_op_gemv(const void* w, int32_t w_dtype, const float* w_scale, const void* x,
                         int32_t x_dtype, void* y, int32_t y_dtype, int64_t n, int64_t k,
                         void* stream);

/* Per-row symmetric int8 quantisation (the rule of qdec_upload): w [n x k] F32|BF16 ->
 * codes [n x k] int8, scales [n] fp32.  k % 16 == 0. */
qdec_status qdec_op_quantize_rows(const void* w, int32_t w_dtype, int8_t* codes, float* scales,
                                  int64_t n, int64_t k, void* stream);

/* Epilogues of qdec_op_gemm. */
typedef enum qdec_gemm_epilogue {
  QDEC_GEMM_STORE = 0,   /* y = A W^T, [m x n] of y_dtype (F32 | BF16) */
  QDEC_GEMM_RESID = 1,   /* resid[m x n] (fp32) += A W^T */
  QDEC_GEMM_SWIGLU = 2   /* W is [2n x k] (n gate rows, then n up rows); y = silu(g) * u, BF16 */
} qdec_gemm_epilogue;

/* Prefill GEMM on the matrix cores ([ETE], the batched-prefill next step: the [1, hidden] GEMVs
 * become [P, hidden] GEMMs): A [m x k] and W [n x k] bf16 row-major (k contiguous, the weight
 * layout of qdec_upload), fp32 accumulation.  k a positive multiple of 32; a and w 16-byte
 * aligned.  QDEC_E_INVAL for bad sizes, dtypes or pointers. */
qdec_status qdec_op_gemm(const void* a, const void* w, void* y, int32_t y_dtype, float* resid,
                         int32_t epilogue, int32_t m, int32_t n, int32_t k, void* stream);

/* Causal GQA attention of n_tokens new tokens at positions pos0 .. pos0 + n_tokens - 1 over a
 * bf16 paged cache that already holds positions 0 .. pos0 + n_tokens - 1 ([ETE], the
 * FlashAttention-style prefill next step; [Qwen3-runtime] §2.5-2.6 per token, §7.2 paging).
 * q: [n_tokens][n_q_heads][head_dim] bf16, normalised and rotated (not scaled); pools
 * [pages][n_kv_heads][16][head_dim] bf16; block_table maps every position below
 * pos0 + n_tokens; out: [n_tokens][n_q_heads][head_dim] bf16.  Query t attends to keys
 * 0 .. pos0 + t with scores q.k / sqrt(head_dim) on the matrix cores (bf16 operands, fp32
 * softmax state; the probabilities are rounded to bf16 as the second product's operand).
 * head_dim 64 or 128; n_q_heads / n_kv_heads <= 8; q and pools 16-byte aligned. */
qdec_status qdec_op_prefill_attention(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, int32_t pos0, int32_t n_tokens,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      void* out, void* stream);

/* Temperature + top-p (nucleus) sampling of one token from logits [n] (F32 | BF16), n <= 2^18
 * ([ETE], whose limitations passage names greedy-only decoding).  p = softmax(logits /
 * temperature); the nucleus is the shortest prefix of the tokens ordered by p descending (ties:
 * lower index first) whose mass reaches top_p; the token is the nucleus member, in index order,
 * at which the cumulative nucleus mass first exceeds u times the nucleus mass, u in [0, 1) being
 * the top 24 bits of the first word of Philox4x32-10 (Salmon et al., SC 2011) with key (seed
 * low, seed high) and counter (position, 0, 0, 0).  Probabilities are summed as exact 64-bit
 * fixed-point integers (2^-40 per unit of the largest), so the result is deterministic; NaN
 * logits are never drawn (all NaN: token 0).  temperature > 0 and finite, 0 < top_p <= 1,
 * position >= 0; workspace: device memory of at least qdec_op_sample_workspace(n) bytes,
 * 256-byte aligned, owned by the caller; calls that share a workspace must not overlap.  *out on
 * the device. */
qdec_status qdec_op_sample(const void* logits, int32_t dtype, int64_t n, float temperature,
                           float top_p, uint64_t seed, int32_t position, void* workspace,
                           size_t workspace_bytes, int32_t* out, void* stream);

/* Bytes of device workspace qdec_op_sample needs for n logits (1 <= n <= 2^18): per-slice
 * histograms, their sum and the boundary candidates, all rewritten by every call. */
qdec_status qdec_op_sample_workspace(int64_t n, size_t* bytes);

/* Group-wise quantisation (the rule of qdec_upload for I8_G128 / I4_G128): w [n x k] F32|BF16 ->
 * codes and scales [n][k / 128] in the layouts of dst_dtype (qdec_dtype).  k % 128 == 0; w
 * 8-byte aligned, codes and scales 4-byte aligned. */
qdec_status qdec_op_quantize_groups(const void* w, int32_t w_dtype, int32_t dst_dtype, void* codes,
                                    float* scales, int64_t n, int64_t k, void* stream);

/* y = x / sqrt(mean(x^2) + eps) * gamma ([Qwen3-runtime] §2.1), x fp32 [n], y [n] of y_dtype. */
qdec_status qdec_op_rmsnorm(const float* x, const float* gamma, float eps, void* y,
                            int32_t y_dtype, int32_t n, void* stream);

/* Fills the RoPE table: table[p][i] = (cos(p*theta^(-2i/D)), sin(...)) for p < max_pos,
 * i < D/2, as fp32 pairs, angles evaluated in fp64 ([Qwen3-runtime] §2.4). */
qdec_status qdec_op_rope_table(float* table, int32_t max_pos, int32_t head_dim, float theta,
                               void* stream);

/* The fused per-head step of [Qwen3-runtime] §7.1-7.2: from the QKV projection output
 * qkv fp32 [(Hq+2Hkv)*D], RMSNorm each Q and K head over D (when q_gamma/k_gamma != NULL),
 * rotate pairs (r, r+D/2) by pos * theta_r using `table`, write the rotated Q to q_out
 * ([Hq*D] of q_dtype) and write the rotated K and the raw V of position pos into the pools
 * (layout above) through block_table. */
qdec_status qdec_op_qk_norm_rope_append(const float* qkv, const float* q_gamma,
                                        const float* k_gamma, float eps, const float* table,
                                        int32_t pos, void* q_out, int32_t q_dtype, void* k_pool,
                                        void* v_pool, int32_t kv_dtype,
                                        const int32_t* block_table, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                        void* stream);

/* Bytes of workspace qdec_op_attention needs for these sizes (0 when one partition suffices). */
qdec_status qdec_op_attention_workspace(int32_t ctx_len, int32_t n_q_heads, int32_t head_dim,
                                        int32_t partition_size, size_t* bytes);

/* Causal GQA decode attention of one query per head over positions 0..ctx_len-1
 * ([Qwen3-runtime] §2.5-2.6, §9.1, §10.1-10.2): q [Hq x D] of q_dtype; k_pool/v_pool one layer's
 * pools of kv_dtype (layout above); query head h reads kv head h / (Hq/Hkv); scores scaled by
 * 1/sqrt(D); each partition of partition_size tokens (multiple of 64 up to 512; 0 = automatic) keeps an
 * fp32 online-softmax state (m, l, acc) and the partitions are merged exactly.  out [Hq x D] of
 * out_dtype.  workspace: device buffer of at least qdec_op_attention_workspace() bytes, 256-byte
 * aligned (may be NULL when that size is 0). */
qdec_status qdec_op_attention(const void* q, int32_t q_dtype, const void* k_pool,
                              const void* v_pool, int32_t kv_dtype, const int32_t* block_table,
                              int32_t ctx_len, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* out,
                              int32_t out_dtype, void* stream);

/* qdec_op_attention without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The split-KV partials go to a static device scratch array of 16 MiB that each GPU the library
 * runs on holds until the process ends; the call itself allocates nothing.  Runs on the current
 * device (stream must belong to it); the first call on a device looks up that device's scratch
 * address.  Calls that overlap on one GPU share its scratch and race: order them on one stream or
 * serialise them.  QDEC_E_RANGE when the partials (Hq x partitions x (D + 2) x 4 bytes, the size
 * qdec_op_attention_workspace reports) exceed 16 MiB; other arguments as qdec_op_attention. */
qdec_status qdec_op_attention_noalloc(const void* q, int32_t q_dtype, const void* k_pool,
                                      const void* v_pool, int32_t kv_dtype,
                                      const int32_t* block_table, int32_t ctx_len,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t page_size, int32_t partition_size, void* out,
                                      int32_t out_dtype, void* stream);

/* Index of the largest of n values of x_dtype (F32|BF16), lowest index on ties, NaN ignored
 * (-1 if every value is NaN); out: device int32. */
qdec_status qdec_op_argmax(const void* x, int32_t x_dtype, int64_t n, int32_t* out, void* stream);

/* Streams `bytes` (multiple of 16, 16-byte aligned pointers) from src to dst with the library's
 * own copy kernel: the reference point for achievable bandwidth and for scaling HBM counters. */
qdec_status qdec_op_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* ---- Attention over host-resident K/V: tiles copied in, double-buffered ------------------------
 * [ETE] KV-offload passage: the history K/V stay in host memory; one tile of positions at a time
 * is copied into a device tile buffer, a tile pass folds it into (m, l, acc) state kept in global
 * memory, and a last pass normalises (acc / l), so device memory is fixed by the tile, not the
 * context.  [ETE] next-steps list: give the tiles several buffers with the event pattern of its
 * layer streaming - a tile's compute waits for that tile's copy (data ready), and a copy into a
 * buffer waits for the compute that last read it (buffer free).
 *
 * Each tile is a whole number of split-KV partitions.  A tile launch writes the (m, l, acc) of its
 * partitions into the slots the resident path uses for them, and one exact merge ends the call,
 * so the result is qdec_op_attention's on the same K/V and partition length (bit for bit when the
 * context spans two or more partitions).  Copies run on the object's own stream (default
 * priority), kernels on the caller's.  With n_slots = 0 nothing is copied: pinned host memory is
 * mapped into the GPU's address space, and the split-KV kernel streams the pages over the host
 * link itself, every partition at once (partition_size 0 then sizes partitions for max_context). */
typedef struct qdec_offload qdec_offload;

typedef struct qdec_offload_config {
  int32_t device;
  int32_t n_q_heads, n_kv_heads, head_dim; /* Hq % Hkv == 0, Hq / Hkv <= 8; head_dim 64 or 128 */
  int32_t kv_dtype;                        /* QDEC_F32 | QDEC_BF16 */
  int32_t max_context;                     /* positions one call may cover, >= 1 */
  int32_t tile_tokens;                     /* positions per copy: a multiple of 64, 64 .. 65536 */
  int32_t n_slots;                         /* device tile buffers, 1 .. 8 (1: copy, then compute);
                                              0: no copies - the split-KV kernel reads the pinned
                                              host pages through their device mapping */
  int32_t partition_size;                  /* 0 = automatic, else a multiple of 64 up to 512 that
                                              divides tile_tokens */
} qdec_offload_config;

/* Validates cfg and allocates everything a call needs: n_slots K and V tile buffers, the (m, l,
 * acc) partials for max_context, the copy stream and the events.  *out is NULL on failure. */
qdec_status qdec_offload_create(const qdec_offload_config* cfg, qdec_offload** out);
/* Waits for the object's copies, then frees it.  NULL is a no-op. */
void qdec_offload_destroy(qdec_offload* o);
/* Device bytes the object holds, and the partition length in effect. */
qdec_status qdec_offload_info(const qdec_offload* o, int64_t* device_bytes,
                              int32_t* partition_tokens);

/* Causal GQA decode attention (as qdec_op_attention) of q [Hq x D] (device, q_dtype F32|BF16)
 * over positions 0 .. ctx_len-1 (1 <= ctx_len <= max_context) whose K and V are in host memory:
 * host_k / host_v hold ceil(ctx_len / 16) pages in position order, page p = positions 16p ..
 * 16p+15 laid out [Hkv][16][D] of kv_dtype (the device pool's page layout), and must be pinned
 * (qdec_host_alloc or another hipHostMalloc'd block; pageable memory is rejected).  out [Hq x D]
 * on the device, out_dtype F32|BF16.  The call enqueues and returns: the host pages must stay
 * unchanged, and out unread, until the caller's stream has passed it.  Calls on one object are
 * ordered among themselves (each waits for the previous call's work); issue them from one host
 * thread. */
qdec_status qdec_offload_attention(qdec_offload* o, const void* q, int32_t q_dtype,
                                   const void* host_k, const void* host_v, int32_t ctx_len,
                                   void* out, int32_t out_dtype, void* stream);

/* The enqueue order qdec_offload_attention uses for n_tiles tiles over n_slots buffers, as
 * records of four int32 (kind, tile, slot, other): kind 0 = the copy stream waits for the compute
 * of tile `other` (buffer free), 1 = copy tile into slot, 2 = the compute stream waits for the
 * copy of tile `other` (data ready), 3 = compute tile from slot, 4 = merge (tile, slot -1).
 * Writes at most cap records; *n gets the number the schedule has.  Needs no GPU. */
qdec_status qdec_offload_schedule(int32_t n_tiles, int32_t n_slots, int32_t* records,
                                  int32_t cap, int32_t* n);

/* Pinned host memory (hipHostMalloc) for host-resident K/V; freed by qdec_host_free. */
qdec_status qdec_host_alloc(size_t bytes, void** ptr);
qdec_status qdec_host_free(void* ptr);

#ifdef __cplusplus
}
#endif

#endif /* QDEC_H */

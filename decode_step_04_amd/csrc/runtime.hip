// runtime.hip - the C ABI of include/qdec.h: validation, context lifecycle, uploads, paged KV,
// the decode-step driver, HIP graph capture/replay, the event profiler and op-level entry points.
//
// [Qwen3-runtime] = the page "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化".
// [ETE] = the page "EdgeTransformerEngine".
//
// Rules kept here ([Qwen3-runtime] §5.1-5.2; [ETE], its list of limitations):
//   - every argument is validated on the host before anything is enqueued;
//   - every HIP call is checked and mapped to QDEC_E_HIP with its message;
//   - all device memory is allocated in qdec_create; the step only enqueues kernels on the
//     caller's stream, so it can be captured and replayed at fixed addresses.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "launch.h"
#include "qdec.h"

#define QDEC_API extern "C" __attribute__((visibility("default")))

using namespace qd;

namespace {

thread_local std::string g_err;  // last error of context-free calls on this thread

// Split-KV work-groups aimed for when partitions are automatic: one per CU.  Each wave then
// streams several pages with the next one requested ahead, which measured faster than one page
// per wave on four times as many work-groups (less per-wave prologue and combine work, fewer
// partitions to merge).
inline int target_wgs(int /*n_q_heads*/, int /*n_kv_heads*/) { return 256; }
constexpr int kMaxTargetWgs = 256;
// work-groups of the copy kernel that fills a weight slot from mapped host memory
constexpr int kSlotCopyWgs = 64;
constexpr int kNumSlots = 11;

qdec_status fail(std::string* dst, qdec_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (dst) *dst = buf;
  g_err = buf;
  return s;
}

int elem_size(int dtype) { return dtype == QDEC_F32 ? 4 : dtype == QDEC_BF16 ? 2 : 1; }
// Storage of a [rows x cols] matrix of a weight dtype: code bytes, and fp32 scales (one per row for
// I8_ROW, one per 128-value group for the group-wise types).
static bool is_quant(int dt) { return dt == QDEC_I8_ROW || dt == QDEC_I8_G128 || dt == QDEC_I4_G128; }
static bool is_grouped(int dt) { return dt == QDEC_I8_G128 || dt == QDEC_I4_G128; }
static int64_t code_bytes(int dt, int64_t rows, int64_t cols) {
  return dt == QDEC_I4_G128 ? rows * (cols / 2) : rows * cols * elem_size(dt);
}
static int64_t scale_count(int dt, int64_t rows, int64_t cols) {
  return dt == QDEC_I8_ROW ? rows : is_grouped(dt) ? rows * (cols / kQGroup) : 0;
}
// GEMV weight type of a storage dtype (the codes coincide)
static int wt_of(int32_t dt) { return dt; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Mat {
  void* data = nullptr;
  float* scale = nullptr;
  int64_t rows = 0, cols = 0;
  int dtype = QDEC_F32;
  int64_t bytes() const { return code_bytes(dtype, rows, cols) + scale_count(dtype, rows, cols) * 4; }
};

struct Layer {
  Mat qkv, o, gu, down;
  float* in_norm = nullptr;
  float* post_norm = nullptr;
  float* q_norm = nullptr;
  float* k_norm = nullptr;
  void* k_pool = nullptr;
  void* v_pool = nullptr;
};

// Split-KV partition length of a context: the configured one, or the length that gives about
// target_wgs (kv head, partition) work-groups at max_context (a multiple of 64, at least 64).
int model_part_tokens(const qdec_config& c) {
  return c.partition_size > 0
             ? c.partition_size
             : part_tokens_for(c.max_context, 0, c.n_kv_heads, target_wgs(c.n_q_heads, c.n_kv_heads));
}
int64_t model_max_parts(const qdec_config& c) {
  const int p = model_part_tokens(c);
  return (c.max_context + p - 1) / p;
}
// Device block-table entries: enough for every page a partition may look up ahead of ctx.
int64_t block_table_entries(const qdec_config& c) {
  return std::max<int64_t>(c.num_pages, model_max_parts(c) * (model_part_tokens(c) / kPage));
}

// One record of the offload schedule (kinds as in qdec_offload_schedule).
struct OffloadOp {
  int kind, tile, slot, other;
};
enum { OFF_WAIT_FREE = 0, OFF_COPY = 1, OFF_WAIT_READY = 2, OFF_COMPUTE = 3, OFF_MERGE = 4 };

// Tile i uses buffer i % n_slots.  Its copy may start once the compute of the tile that last used
// that buffer (i - n_slots) has finished, and its compute once its own copy has finished.
void offload_schedule(int n_tiles, int n_slots, std::vector<OffloadOp>* ops) {
  ops->clear();
  for (int i = 0; i < n_tiles; ++i) {
    const int slot = i % n_slots;
    if (i >= n_slots) ops->push_back({OFF_WAIT_FREE, i, slot, i - n_slots});
    ops->push_back({OFF_COPY, i, slot, -1});
    ops->push_back({OFF_WAIT_READY, i, slot, i});
    ops->push_back({OFF_COMPUTE, i, slot, -1});
  }
  ops->push_back({OFF_MERGE, -1, -1, -1});
}
}  // namespace

struct qdec_ctx {
  qdec_config cfg{};
  int device = 0;
  int part_tokens = 64;
  int max_parts = 1;
  int32_t bt_entries = 0;
  std::vector<void*> allocs;
  int64_t device_bytes = 0;
  Mat embed, lm;
  bool lm_alias = false;
  float* final_norm = nullptr;
  std::vector<Layer> layers;
  int32_t* block_table = nullptr;
  int32_t n_logical = 0;
  float* rope = nullptr;
  float* rope_step = nullptr;  // [D/2] (cos, sin) of the current step's pos
  float* x = nullptr;
  float* qkv = nullptr;
  void* attn = nullptr;
  void* act = nullptr;
  void* logits = nullptr;
  float* part_acc = nullptr;
  float* part_ml = nullptr;
  // prefill buffers for max_prefill tokens (absent when max_prefill = 0)
  float* px = nullptr;        // [P][d] fp32 residual streams
  void* ph = nullptr;         // [P][d] bf16 normalised GEMM inputs
  float* pqkv = nullptr;      // [P][(Hq + 2 Hkv) D] fp32
  void* pq = nullptr;         // [P][Hq][D] bf16 rotated queries
  void* pattn = nullptr;      // [P][Hq D] bf16 attention outputs
  void* pact = nullptr;       // [P][F] bf16 SwiGLU outputs
  float* am_val = nullptr;    // per-work-group partial argmax of the LM head
  int32_t* am_idx = nullptr;
  void* sample_ws = nullptr;  // temperature / top-p sampling (vocab <= 2^18)
  int am_parts = 0;
  StepDesc* desc = nullptr;
  // layer streaming (weight_slots > 0): the layers' projection Mats point into host_layers
  // (pinned host memory, one block of layer_block bytes per layer); slots[s] holds the device
  // Mats of slot s (one block each, the same layout)
  std::vector<Layer> slots;
  bool direct_weights = false;  // weight_slots = -1: kernels read the mapped host copy; slots[0]
                                // is only the upload staging area
  void* host_layers = nullptr;
  char* host_layers_dev = nullptr;  // the device's address of host_layers (its mapping)
  int64_t layer_block = 0;
  hipStream_t copy_stream = nullptr;
  std::vector<hipEvent_t> ev_copied, ev_computed;  // per slot: data ready, buffer free
  std::vector<OffloadOp> wops;
  std::vector<uint8_t> uploaded;  // (n_layers + 1) x kNumSlots; row n_layers = global slots
  std::string err;
  // graph of everything after the embedding kernel
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;
  qdec_step graph_templ{};
  // event profiler
  bool prof = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_class;
  int ev_used = 0;
  double prof_ms[QDEC_K_COUNT] = {};
  int64_t prof_n[QDEC_K_COUNT] = {};

  qdec_status hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return QDEC_OK;
    return fail(&err, QDEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
  }
  template <typename T>
  qdec_status alloc(T** p, int64_t bytes, const char* what) {
    *p = nullptr;
    if (bytes <= 0) return QDEC_OK;
    void* d = nullptr;
    hipError_t e = hipMalloc(&d, (size_t)bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(&err, QDEC_E_NOMEM, "hipMalloc of %lld bytes for %s failed: %s",
                  (long long)bytes, what, hipGetErrorString(e));
    }
    allocs.push_back(d);
    device_bytes += bytes;
    *p = static_cast<T*>(d);
    return QDEC_OK;
  }
  uint8_t& slot(int layer, int which) { return uploaded[(size_t)layer * kNumSlots + which]; }
  bool act_bf16() const { return cfg.act_dtype == QDEC_BF16; }
  bool io_bf16() const { return cfg.io_dtype == QDEC_BF16; }
  bool kv_bf16() const { return cfg.kv_dtype == QDEC_BF16; }
};

// =====================================================================================
// configuration
// =====================================================================================

static qdec_status validate(const qdec_config* c, std::string* why) {
  if (!c) return fail(why, QDEC_E_INVAL, "config is NULL");
  if (c->n_layers < 1 || c->n_layers > 4096)
    return fail(why, QDEC_E_INVAL, "n_layers %d out of [1, 4096]", c->n_layers);
  if (c->hidden <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0)
    return fail(why, QDEC_E_INVAL, "sizes must be positive");
  if (c->hidden % 64 || c->ffn % 64)
    return fail(why, QDEC_E_UNSUPPORTED, "hidden (%d) and ffn (%d) must be multiples of 64",
                c->hidden, c->ffn);
  if (c->hidden > 16384 || c->ffn > 16384)
    return fail(why, QDEC_E_UNSUPPORTED, "hidden and ffn are limited to 16384");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(why, QDEC_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are implemented",
                c->head_dim);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(why, QDEC_E_INVAL, "n_q_heads %d is not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > 8)
    return fail(why, QDEC_E_UNSUPPORTED, "more than 8 query heads per KV head");
  if ((int64_t)c->n_q_heads * c->head_dim > 16384)
    return fail(why, QDEC_E_UNSUPPORTED, "n_q_heads * head_dim is limited to 16384");
  if (c->vocab > (1 << 30)) return fail(why, QDEC_E_UNSUPPORTED, "vocab above 2^30");
  if ((c->tied_lm_head != 0 && c->tied_lm_head != 1) || (c->qk_norm != 0 && c->qk_norm != 1))
    return fail(why, QDEC_E_INVAL, "tied_lm_head and qk_norm must be 0 or 1");
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps))
    return fail(why, QDEC_E_INVAL, "rms_eps must be positive and finite");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta))
    return fail(why, QDEC_E_INVAL, "rope_theta must be finite and above 1");
  auto dt_ok = [](int d) { return d >= QDEC_F32 && d <= QDEC_I4_G128; };
  if (!dt_ok(c->proj_dtype) || !dt_ok(c->lm_head_dtype) || !dt_ok(c->io_dtype) ||
      !dt_ok(c->act_dtype) || !dt_ok(c->kv_dtype))
    return fail(why, QDEC_E_INVAL, "unknown dtype value");
  if (is_quant(c->act_dtype) || is_quant(c->io_dtype) || is_quant(c->kv_dtype))
    return fail(why, QDEC_E_UNSUPPORTED, "io, act and kv dtypes must be F32 or BF16");
  if ((is_grouped(c->proj_dtype) &&
       (c->hidden % kQGroup || c->ffn % kQGroup || (c->n_q_heads * c->head_dim) % kQGroup)) ||
      (is_grouped(c->lm_head_dtype) && c->hidden % kQGroup))
    return fail(why, QDEC_E_UNSUPPORTED,
                "group-wise weights need every projection's input length to be a multiple of 128");
  if (c->io_dtype == QDEC_F32) {
    if (c->proj_dtype != QDEC_F32 || c->lm_head_dtype != QDEC_F32 || c->kv_dtype != QDEC_F32 ||
        c->act_dtype != QDEC_F32)
      return fail(why, QDEC_E_UNSUPPORTED,
                  "the fp32 path needs fp32 projections, LM head, activations and KV");
  } else {
    if (c->proj_dtype == QDEC_F32 || c->lm_head_dtype == QDEC_F32 || c->kv_dtype != QDEC_BF16)
      return fail(why, QDEC_E_UNSUPPORTED,
                  "the bf16 path needs bf16 or quantised projections / LM head and a bf16 KV cache");
  }
  if (c->page_size != kPage)
    return fail(why, QDEC_E_UNSUPPORTED, "page_size %d: only 16 is implemented", c->page_size);
  if (c->num_pages < 1 || c->max_context < 1)
    return fail(why, QDEC_E_INVAL, "num_pages and max_context must be positive");
  if ((int64_t)c->num_pages * kPage < c->max_context)
    return fail(why, QDEC_E_INVAL, "max_context %d exceeds num_pages * page_size", c->max_context);
  if (c->max_context > (1 << 24)) return fail(why, QDEC_E_UNSUPPORTED, "max_context above 2^24");
  if (c->partition_size < 0 || c->partition_size % 64 || c->partition_size > kMaxPartTokens)
    return fail(why, QDEC_E_INVAL, "partition_size must be 0 or a multiple of 64 up to %d",
                kMaxPartTokens);
  if (c->max_prefill < 0 || c->max_prefill > (1 << 16))
    return fail(why, QDEC_E_INVAL, "max_prefill must be in [0, 65536]");
  if (c->max_prefill > 0 &&
      (c->proj_dtype != QDEC_BF16 || c->io_dtype != QDEC_BF16 || c->kv_dtype != QDEC_BF16))
    return fail(why, QDEC_E_UNSUPPORTED,
                "prefill runs bf16 GEMMs on the matrix cores: it needs bf16 projections, io and KV");
  if (model_max_parts(*c) > kMaxMergeParts)
    return fail(why, QDEC_E_UNSUPPORTED, "more than %d split-KV partitions at max_context",
                kMaxMergeParts);
  if (c->weight_slots < -1 || c->weight_slots > c->n_layers)
    return fail(why, QDEC_E_INVAL, "weight_slots %d out of [-1, n_layers = %d]", c->weight_slots,
                c->n_layers);
  if (c->weight_slots != 0 && c->max_prefill > 0)
    return fail(why, QDEC_E_UNSUPPORTED, "host-resident layers (weight_slots != 0) run decode "
                "steps only: max_prefill must be 0");
  {
    const int wp = wt_of(c->proj_dtype);
    const int wl = wt_of(c->lm_head_dtype);
    const int64_t d = c->hidden, f = c->ffn, qd = (int64_t)c->n_q_heads * c->head_dim,
                  nqkv = (int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
    if (!gemv_supported(wp, EPI_STORE, nqkv, d) || !gemv_supported(wp, EPI_RESID, d, qd) ||
        !gemv_supported(wp, EPI_SWIGLU, f, d) || !gemv_supported(wp, EPI_RESID, d, f) ||
        !gemv_supported(wl, EPI_STORE, c->vocab, d))
      return fail(why, QDEC_E_UNSUPPORTED,
                  "a projection's input length exceeds what the GEMV keeps in registers "
                  "(8192 fp32, 16384 bf16, 32768 int8 or int4 values)");
    if (d > kGemvNormMaxK)
      return fail(why, QDEC_E_UNSUPPORTED, "hidden size %lld above %lld (the fused RMSNorm stages "
                  "the normalised input in LDS)", (long long)d, (long long)kGemvNormMaxK);
  }
  return QDEC_OK;
}

static void fill_info(const qdec_config& c, qdec_info* o) {
  const int64_t d = c.hidden, hq = c.n_q_heads, hkv = c.n_kv_heads, hd = c.head_dim, f = c.ffn,
                v = c.vocab, L = c.n_layers;
  const int64_t mats = (hq + 2 * hkv) * hd * d + d * hq * hd + 2 * f * d + d * f;
  const int64_t rows = (hq + 2 * hkv) * hd + d + 2 * f + d;
  const int64_t norms = 2 * d + (c.qk_norm ? 2 * hd : 0);
  memset(o, 0, sizeof *o);
  o->params_per_layer = mats + norms;
  o->params_total = L * (mats + norms) + v * d * (c.tied_lm_head ? 1 : 2) + d;
  o->layer_matrix_bytes = L * code_bytes(c.proj_dtype, 1, mats);
  // scales: per row (I8_ROW), or per 128-value group (every projection's k is a multiple of 128)
  o->layer_scale_bytes = c.proj_dtype == QDEC_I8_ROW ? L * rows * 4
                         : is_grouped(c.proj_dtype) ? L * (mats / kQGroup) * 4 : 0;
  o->lm_head_bytes = code_bytes(c.lm_head_dtype, v, d) + scale_count(c.lm_head_dtype, v, d) * 4;
  o->kv_bytes_per_layer_token = 2 * hkv * hd * elem_size(c.kv_dtype);
  o->kv_pool_bytes = L * 2 * (int64_t)c.num_pages * kPage * hkv * hd * elem_size(c.kv_dtype);
  const int64_t mp = model_max_parts(c);
  o->partition_tokens = model_part_tokens(c);
  o->max_partitions = (int32_t)mp;
  const int ae = elem_size(c.act_dtype), ie = elem_size(c.io_dtype);
  const bool lm_alias = c.tied_lm_head && c.lm_head_dtype == c.io_dtype;
  // host-resident layers (weight_slots != 0) keep their projections in pinned host memory and
  // hold max(1, slots) layer-sized device blocks instead
  const int64_t nslot = c.weight_slots < 0 ? 1 : c.weight_slots;
  const int64_t layer_dev = c.weight_slots == 0
                                ? o->layer_matrix_bytes + o->layer_scale_bytes
                                : nslot * ((o->layer_matrix_bytes + o->layer_scale_bytes) / L);
  o->device_bytes = v * d * ie + (lm_alias ? 0 : o->lm_head_bytes) + d * 4 +
                    layer_dev + L * norms * 4 + o->kv_pool_bytes +
                    block_table_entries(c) * 4 + (int64_t)c.max_context * (hd / 2) * 8 + d * 4 +
                    (hq + 2 * hkv) * hd * 4 + 2 * hq * hd * ae + f * ae + v * ie +
                    hq * mp * hd * 4 + hq * mp * 8 + (int64_t)sizeof(StepDesc) +
                    (int64_t)c.max_prefill * (d * 6 + (hq + 2 * hkv) * hd * 4 + 4 * hq * hd + 2 * f) +
                    (v <= (int64_t(1) << 18) ? sample_workspace_bytes(v) : 0);
}

QDEC_API qdec_status qdec_config_validate(const qdec_config* cfg, char* msg, size_t len) {
  std::string why;
  qdec_status s = validate(cfg, &why);
  if (msg && len) {
    snprintf(msg, len, "%s", s == QDEC_OK ? "ok" : why.c_str());
  }
  return s;
}

QDEC_API qdec_status qdec_config_info(const qdec_config* cfg, qdec_info* out) {
  if (!out) return fail(nullptr, QDEC_E_INVAL, "out is NULL");
  qdec_status s = validate(cfg, nullptr);
  if (s != QDEC_OK) return s;
  fill_info(*cfg, out);
  return QDEC_OK;
}

QDEC_API qdec_status qdec_bytes_model(const qdec_config* c, int32_t context, int32_t with_logits,
                                      qdec_bytes* o) {
  if (!o) return fail(nullptr, QDEC_E_INVAL, "out is NULL");
  qdec_status s = validate(c, nullptr);
  if (s != QDEC_OK) return s;
  if (context < 1 || context > c->max_context)
    return fail(nullptr, QDEC_E_RANGE, "context %d outside [1, %d]", context, c->max_context);
  const int64_t d = c->hidden, hq = c->n_q_heads, hkv = c->n_kv_heads, hd = c->head_dim,
                f = c->ffn, v = c->vocab, L = c->n_layers, T = context;
  const int64_t ke = elem_size(c->kv_dtype), ae = elem_size(c->io_dtype);
  const int pt = c->proj_dtype;
  // weight + scale bytes of a [rows x cols] projection
  auto wb = [&](int64_t rows, int64_t cols) {
    return code_bytes(pt, rows, cols) + scale_count(pt, rows, cols) * 4;
  };
  memset(o, 0, sizeof *o);
  o->embed = d * ae;
  o->qkv = L * (wb((hq + 2 * hkv) * hd, d) + d * 4);
  // the attention kernel also normalises/rotates Q and K and appends the new K/V row
  o->rope_append = 0;
  o->attention = L * (T * 2 * hkv * hd * ke + (c->qk_norm ? 2 * hd * 4 : 0) + 2 * hkv * hd * ke);
  o->merge = 0;
  o->o_proj = L * wb(d, hq * hd);
  o->gate_up = L * (wb(2 * f, d) + d * 4);
  o->down = L * wb(d, f);
  if (with_logits) {
    o->lm_head = code_bytes(c->lm_head_dtype, v, d) + scale_count(c->lm_head_dtype, v, d) * 4 +
                 d * 4 + v * ae;
    o->argmax = 0;  // reduces per-work-group partials written by the LM head
  }
  o->total = o->embed + o->qkv + o->rope_append + o->attention + o->o_proj + o->gate_up + o->down +
             o->lm_head;
  const int64_t np = n_parts_for(context, model_part_tokens(*c));
  o->scratch = np > 1 ? L * hq * np * (hd + 2) * 4 * 2 : 0;
  return QDEC_OK;
}

// =====================================================================================
// lifecycle
// =====================================================================================

QDEC_API const char* qdec_status_string(qdec_status s) {
  switch (s) {
    case QDEC_OK: return "ok";
    case QDEC_E_INVAL: return "invalid argument";
    case QDEC_E_UNSUPPORTED: return "unsupported";
    case QDEC_E_STATE: return "wrong state";
    case QDEC_E_RANGE: return "out of range";
    case QDEC_E_NOMEM: return "out of device memory";
    case QDEC_E_HIP: return "HIP error";
  }
  return "unknown status";
}

QDEC_API const char* qdec_last_error(const qdec_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_err.c_str();
}

static void release(qdec_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  if (c->gexec) (void)hipGraphExecDestroy(c->gexec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
  for (hipEvent_t e : c->ev_copied) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->ev_computed) (void)hipEventDestroy(e);
  if (c->host_layers) (void)hipHostFree(c->host_layers);
  for (void* p : c->allocs) (void)hipFree(p);
  delete c;
}

QDEC_API void qdec_destroy(qdec_ctx* ctx) { release(ctx); }

QDEC_API qdec_status qdec_create(const qdec_config* cfg, int32_t device, qdec_ctx** out) {
  if (!out) return fail(nullptr, QDEC_E_INVAL, "out is NULL");
  *out = nullptr;
  std::string why;
  qdec_status s = validate(cfg, &why);
  if (s != QDEC_OK) return s;
  int ndev = 0;
  hipError_t he = hipGetDeviceCount(&ndev);
  if (he != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(nullptr, QDEC_E_HIP, "no HIP device: %s", hipGetErrorString(he));
  }
  if (device < 0 || device >= ndev)
    return fail(nullptr, QDEC_E_INVAL, "device %d out of [0, %d)", device, ndev);
  he = hipSetDevice(device);
  if (he != hipSuccess) return fail(nullptr, QDEC_E_HIP, "hipSetDevice: %s", hipGetErrorString(he));

  qdec_ctx* c = new qdec_ctx();
  c->cfg = *cfg;
  c->device = device;
  c->part_tokens = model_part_tokens(*cfg);
  c->max_parts = (int)model_max_parts(*cfg);
  c->bt_entries = (int32_t)block_table_entries(*cfg);
  const int64_t d = cfg->hidden, hq = cfg->n_q_heads, hkv = cfg->n_kv_heads, hd = cfg->head_dim,
                f = cfg->ffn, v = cfg->vocab, L = cfg->n_layers;
  const int ae = elem_size(cfg->act_dtype), ie = elem_size(cfg->io_dtype);
  c->uploaded.assign((size_t)(L + 1) * kNumSlots, 0);

#define TRY(x)                  \
  do {                          \
    qdec_status s_ = (x);       \
    if (s_ != QDEC_OK) {        \
      g_err = c->err;           \
      release(c);               \
      return s_;                \
    }                           \
  } while (0)

  auto make_mat = [&](Mat& m, int64_t rows, int64_t cols, int dtype, const char* what) {
    m.rows = rows;
    m.cols = cols;
    m.dtype = dtype;
    qdec_status st = c->alloc(&m.data, code_bytes(dtype, rows, cols), what);
    if (st == QDEC_OK && is_quant(dtype))
      st = c->alloc(&m.scale, scale_count(dtype, rows, cols) * 4, what);
    return st;
  };

  TRY(make_mat(c->embed, v, d, cfg->io_dtype, "embedding"));
  c->lm_alias = cfg->tied_lm_head && cfg->lm_head_dtype == cfg->io_dtype;
  if (c->lm_alias)
    c->lm = c->embed;
  else
    TRY(make_mat(c->lm, v, d, cfg->lm_head_dtype, "LM head"));
  TRY(c->alloc(&c->final_norm, d * 4, "final norm"));
  c->layers.resize((size_t)L);
  const int64_t pool_bytes = (int64_t)cfg->num_pages * kPage * hkv * hd * elem_size(cfg->kv_dtype);
  // one layer's projections (codes, then scales, each 256-byte aligned) carved out of a block
  auto carve = [&](Layer& ly, char* base) {
    int64_t off = 0;
    auto one = [&](Mat& m, int64_t rows, int64_t cols) {
      m.rows = rows;
      m.cols = cols;
      m.dtype = cfg->proj_dtype;
      m.data = base ? base + off : nullptr;
      off += (code_bytes(m.dtype, rows, cols) + 255) / 256 * 256;
      m.scale = (base && is_quant(m.dtype)) ? reinterpret_cast<float*>(base + off) : nullptr;
      off += (scale_count(m.dtype, rows, cols) * 4 + 255) / 256 * 256;
    };
    one(ly.qkv, (hq + 2 * hkv) * hd, d);
    one(ly.o, d, hq * hd);
    one(ly.gu, 2 * f, d);
    one(ly.down, d, f);
    return off;
  };
  if (cfg->weight_slots != 0) {
    Layer probe;
    c->layer_block = carve(probe, nullptr);
    const size_t host_bytes = (size_t)c->layer_block * (size_t)L;
    hipError_t eh = hipHostMalloc(&c->host_layers, host_bytes, hipHostMallocDefault);
    if (eh != hipSuccess) {
      (void)hipGetLastError();
      c->host_layers = nullptr;
      fail(&c->err, QDEC_E_NOMEM, "hipHostMalloc of %zu bytes for the streamed layers: %s",
           host_bytes, hipGetErrorString(eh));
      g_err = c->err;
      release(c);
      return QDEC_E_NOMEM;
    }
    c->direct_weights = cfg->weight_slots < 0;
    c->slots.resize(c->direct_weights ? 1 : (size_t)cfg->weight_slots);
    for (auto& sl : c->slots) {
      char* blk = nullptr;
      TRY(c->alloc(&blk, c->layer_block, "weight slot"));
      carve(sl, blk);
    }
    // the device's address of the pinned host block: the slot copies read it (streaming), or
    // the kernels do (direct)
    void* mapped = nullptr;
    TRY(c->hip(hipHostGetDevicePointer(&mapped, c->host_layers, 0),
               "hipHostGetDevicePointer (host-resident layers)"));
    if (!mapped || !aligned(mapped, 256)) {
      fail(&c->err, QDEC_E_HIP, "host-resident layers have no aligned device mapping");
      g_err = c->err;
      release(c);
      return QDEC_E_HIP;
    }
    c->host_layers_dev = static_cast<char*>(mapped);
    char* host_base = c->direct_weights ? c->host_layers_dev : static_cast<char*>(c->host_layers);
    for (int64_t l = 0; l < L; ++l)
      carve(c->layers[(size_t)l], host_base + l * c->layer_block);
    TRY(c->hip(hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking),
               "hipStreamCreateWithFlags (weight copies)"));
    for (int i = 0; i < (c->direct_weights ? 0 : cfg->weight_slots); ++i) {
      hipEvent_t a = nullptr, b = nullptr;
      TRY(c->hip(hipEventCreateWithFlags(&a, hipEventDisableTiming), "hipEventCreate"));
      c->ev_copied.push_back(a);
      TRY(c->hip(hipEventCreateWithFlags(&b, hipEventDisableTiming), "hipEventCreate"));
      c->ev_computed.push_back(b);
    }
  }
  for (auto& ly : c->layers) {
    if (cfg->weight_slots == 0) {
      TRY(make_mat(ly.qkv, (hq + 2 * hkv) * hd, d, cfg->proj_dtype, "QKV"));
      TRY(make_mat(ly.o, d, hq * hd, cfg->proj_dtype, "O"));
      TRY(make_mat(ly.gu, 2 * f, d, cfg->proj_dtype, "gate-up"));
      TRY(make_mat(ly.down, d, f, cfg->proj_dtype, "down"));
    }
    TRY(c->alloc(&ly.in_norm, d * 4, "norm"));
    TRY(c->alloc(&ly.post_norm, d * 4, "norm"));
    if (cfg->qk_norm) {
      TRY(c->alloc(&ly.q_norm, hd * 4, "q norm"));
      TRY(c->alloc(&ly.k_norm, hd * 4, "k norm"));
    }
    TRY(c->alloc(&ly.k_pool, pool_bytes, "K pool"));
    TRY(c->alloc(&ly.v_pool, pool_bytes, "V pool"));
    TRY(c->hip(hipMemset(ly.k_pool, 0, (size_t)pool_bytes), "hipMemset K pool"));
    TRY(c->hip(hipMemset(ly.v_pool, 0, (size_t)pool_bytes), "hipMemset V pool"));
  }
  // zero-filled: every entry is a valid page number, so the attention kernel may read entries
  // ahead of the context
  TRY(c->alloc(&c->block_table, (int64_t)c->bt_entries * 4, "block table"));
  TRY(c->hip(hipMemset(c->block_table, 0, (size_t)c->bt_entries * 4), "hipMemset block table"));
  TRY(c->alloc(&c->rope, (int64_t)cfg->max_context * (hd / 2) * 8, "RoPE table"));
  TRY(c->alloc(&c->rope_step, (hd / 2) * 8, "RoPE row of the step"));
  TRY(c->alloc(&c->x, d * 4, "residual"));
  TRY(c->alloc(&c->qkv, (hq + 2 * hkv) * hd * 4, "qkv"));
  TRY(c->alloc(&c->attn, hq * hd * ae, "attention output"));
  TRY(c->alloc(&c->act, f * ae, "SwiGLU output"));
  TRY(c->alloc(&c->logits, v * ie, "logits"));
  c->am_parts = gemv_partials(wt_of(cfg->lm_head_dtype), EPI_STORE, v, d);
  TRY(c->alloc(&c->am_val, (int64_t)c->am_parts * 4, "argmax partials"));
  TRY(c->alloc(&c->am_idx, (int64_t)c->am_parts * 4, "argmax partials"));
  if (v <= (int64_t(1) << 18))
    TRY(c->alloc(&c->sample_ws, sample_workspace_bytes(v), "sampling workspace"));
  TRY(c->alloc(&c->part_acc, hq * (int64_t)c->max_parts * hd * 4, "split-KV scratch"));
  TRY(c->alloc(&c->part_ml, hq * (int64_t)c->max_parts * 8, "split-KV scratch"));
  if (cfg->max_prefill > 0) {
    const int64_t P = cfg->max_prefill;
    TRY(c->alloc(&c->px, P * d * 4, "prefill residual"));
    TRY(c->alloc(&c->ph, P * d * 2, "prefill GEMM input"));
    TRY(c->alloc(&c->pqkv, P * (hq + 2 * hkv) * hd * 4, "prefill qkv"));
    TRY(c->alloc(&c->pq, P * hq * hd * 2, "prefill queries"));
    TRY(c->alloc(&c->pattn, P * hq * hd * 2, "prefill attention output"));
    TRY(c->alloc(&c->pact, P * f * 2, "prefill SwiGLU output"));
  }
  TRY(c->alloc(&c->desc, (int64_t)sizeof(StepDesc), "step descriptor"));
  TRY(c->hip(hipMemset(c->desc, 0, sizeof(StepDesc)), "hipMemset descriptor"));
  TRY(c->hip(launch_rope_table(c->rope, cfg->max_context, (int)hd, cfg->rope_theta, nullptr),
             "RoPE table kernel"));
  TRY(c->hip(hipDeviceSynchronize(), "hipDeviceSynchronize after create"));
#undef TRY
  *out = c;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_info_get(const qdec_ctx* ctx, qdec_info* out) {
  if (!ctx || !out) return fail(nullptr, QDEC_E_INVAL, "NULL argument");
  fill_info(ctx->cfg, out);
  out->device_bytes = ctx->device_bytes;  // what this context did allocate
  return QDEC_OK;
}

// =====================================================================================
// weights
// =====================================================================================

static bool is_global(int which) {
  return which == QDEC_W_EMBED || which == QDEC_W_LM_HEAD || which == QDEC_W_FINAL_NORM;
}

// Resolves a slot to a matrix or a gamma vector and its expected shape.
static qdec_status resolve(qdec_ctx* c, int32_t layer, int32_t which, Mat** mat, float** vec,
                           int64_t* rows, int64_t* cols) {
  *mat = nullptr;
  *vec = nullptr;
  if (which < 0 || which >= kNumSlots) return fail(&c->err, QDEC_E_INVAL, "unknown weight slot %d", which);
  if (!is_global(which) && (layer < 0 || layer >= c->cfg.n_layers))
    return fail(&c->err, QDEC_E_INVAL, "layer %d out of [0, %d)", layer, c->cfg.n_layers);
  const int64_t d = c->cfg.hidden, hd = c->cfg.head_dim;
  Layer* ly = is_global(which) ? nullptr : &c->layers[(size_t)layer];
  switch (which) {
    case QDEC_W_EMBED: *mat = &c->embed; break;
    case QDEC_W_LM_HEAD: *mat = &c->lm; break;
    case QDEC_W_FINAL_NORM: *vec = c->final_norm; *rows = 1; *cols = d; return QDEC_OK;
    case QDEC_W_IN_NORM: *vec = ly->in_norm; *rows = 1; *cols = d; return QDEC_OK;
    case QDEC_W_POST_NORM: *vec = ly->post_norm; *rows = 1; *cols = d; return QDEC_OK;
    case QDEC_W_Q_NORM:
    case QDEC_W_K_NORM:
      if (!c->cfg.qk_norm) return fail(&c->err, QDEC_E_INVAL, "qk_norm is off: no Q/K gamma slot");
      *vec = which == QDEC_W_Q_NORM ? ly->q_norm : ly->k_norm;
      *rows = 1;
      *cols = hd;
      return QDEC_OK;
    case QDEC_W_QKV: *mat = &ly->qkv; break;
    case QDEC_W_O: *mat = &ly->o; break;
    case QDEC_W_GATE_UP: *mat = &ly->gu; break;
    default: *mat = &ly->down; break;
  }
  *rows = (*mat)->rows;
  *cols = (*mat)->cols;
  return QDEC_OK;
}

static qdec_status copy_in(qdec_ctx* c, void* dst, const void* src, int64_t bytes, int src_dev,
                           hipStream_t s) {
  return c->hip(hipMemcpyAsync(dst, src, (size_t)bytes,
                               src_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s),
                "hipMemcpyAsync (upload)");
}

// Fills `m` from src of src_dtype (conversion or quantisation on the device).
static qdec_status fill_mat(qdec_ctx* c, Mat& m, const void* src, int src_dtype, int src_dev,
                            hipStream_t s) {
  const int64_t n = m.rows * m.cols;
  if (m.dtype == src_dtype) return copy_in(c, m.data, src, n * elem_size(src_dtype), src_dev, s);
  if (!src_dev)
    return fail(&c->err, QDEC_E_UNSUPPORTED,
                "converting a host source needs a device copy first (src_is_device = 1)");
  if (m.dtype == QDEC_I8_ROW)
    return c->hip(launch_quantize(src, src_dtype == QDEC_BF16, static_cast<int8_t*>(m.data),
                                  m.scale, m.rows, m.cols, s),
                  "quantize kernel");
  if (is_grouped(m.dtype))
    return c->hip(launch_quantize_groups(src, src_dtype == QDEC_BF16,
                                         m.dtype == QDEC_I8_G128 ? 8 : 4, m.data, m.scale, m.rows,
                                         m.cols, s),
                  "group quantize kernel");
  return c->hip(launch_convert(m.data, m.dtype == QDEC_BF16 ? W_BF16 : W_F32, src,
                               src_dtype == QDEC_BF16 ? W_BF16 : W_F32, n, s),
                "convert kernel");
}

// Layer streaming: a layer's projection lives in pinned host memory.  Uploads go through the
// same projection of slot 0 (device staging, where conversion and quantisation run), then to
// the host copy; the call waits for both, since slot 0 is reused.
static bool streamed(const qdec_ctx* c, int which) {
  return !c->slots.empty() && (which == QDEC_W_QKV || which == QDEC_W_O ||
                               which == QDEC_W_GATE_UP || which == QDEC_W_DOWN);
}
static Mat& stage_of(qdec_ctx* c, int which) {
  Layer& s0 = c->slots[0];
  return which == QDEC_W_QKV ? s0.qkv : which == QDEC_W_O ? s0.o : which == QDEC_W_GATE_UP ? s0.gu
                                                                                          : s0.down;
}
static qdec_status stage_to_host(qdec_ctx* c, const Mat& stage, Mat& host, hipStream_t s) {
  // (the host copy's address may be its device mapping: the runtime resolves the direction)
  qdec_status st = c->hip(hipMemcpyAsync(host.data, stage.data,
                                         (size_t)code_bytes(stage.dtype, stage.rows, stage.cols),
                                         hipMemcpyDefault, s),
                          "hipMemcpyAsync (streamed layer to host)");
  if (st == QDEC_OK && stage.scale)
    st = c->hip(hipMemcpyAsync(host.scale, stage.scale,
                               (size_t)scale_count(stage.dtype, stage.rows, stage.cols) * 4,
                               hipMemcpyDefault, s),
                "hipMemcpyAsync (streamed layer scales to host)");
  if (st == QDEC_OK) st = c->hip(hipStreamSynchronize(s), "hipStreamSynchronize (upload)");
  return st;
}

QDEC_API qdec_status qdec_upload(qdec_ctx* c, int32_t layer, int32_t which, const void* src,
                                 int32_t src_dtype, int64_t rows, int64_t cols,
                                 int32_t src_is_device, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (!src) return fail(&c->err, QDEC_E_INVAL, "src is NULL");
  if (src_dtype != QDEC_F32 && src_dtype != QDEC_BF16)
    return fail(&c->err, QDEC_E_INVAL, "src_dtype must be F32 or BF16");
  if (src_is_device && !aligned(src, 16))
    return fail(&c->err, QDEC_E_INVAL, "device source must be 16-byte aligned");
  Mat* m;
  float* vec;
  int64_t er, ec;
  qdec_status st = resolve(c, layer, which, &m, &vec, &er, &ec);
  if (st != QDEC_OK) return st;
  if (rows != er || cols != ec)
    return fail(&c->err, QDEC_E_INVAL, "shape %lldx%lld, expected %lldx%lld", (long long)rows,
                (long long)cols, (long long)er, (long long)ec);
  if (which == QDEC_W_LM_HEAD && c->cfg.tied_lm_head)
    return fail(&c->err, QDEC_E_INVAL, "tied LM head: upload QDEC_W_EMBED instead");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return st;
  const int lrow = is_global(which) ? c->cfg.n_layers : layer;
  if (vec) {
    if (src_dtype == QDEC_F32)
      st = copy_in(c, vec, src, cols * 4, src_is_device, s);
    else if (!src_is_device)
      return fail(&c->err, QDEC_E_UNSUPPORTED, "bf16 gamma from the host needs a device copy");
    else
      st = c->hip(launch_convert(vec, W_F32, src, W_BF16, cols, s), "convert kernel");
    if (st == QDEC_OK) c->slot(lrow, which) = 1;
    return st;
  }
  if (m->dtype == QDEC_I8_ROW && m->cols % 16)
    return fail(&c->err, QDEC_E_UNSUPPORTED, "int8 rows need cols %% 16 == 0");
  if (is_grouped(m->dtype) && m->cols % kQGroup)
    return fail(&c->err, QDEC_E_UNSUPPORTED, "group-wise rows need cols %% 128 == 0");
  if (streamed(c, which)) {
    Mat& stage = stage_of(c, which);
    st = fill_mat(c, stage, src, src_dtype, src_is_device, s);
    if (st == QDEC_OK) st = stage_to_host(c, stage, *m, s);
    if (st == QDEC_OK) c->slot(lrow, which) = 1;
    return st;
  }
  st = fill_mat(c, *m, src, src_dtype, src_is_device, s);
  if (st != QDEC_OK) return st;
  c->slot(lrow, which) = 1;
  if (which == QDEC_W_EMBED && c->cfg.tied_lm_head) {
    if (!c->lm_alias) {
      st = fill_mat(c, c->lm, src, src_dtype, src_is_device, s);
      if (st != QDEC_OK) return st;
    }
    c->slot(lrow, QDEC_W_LM_HEAD) = 1;
  }
  return QDEC_OK;
}

QDEC_API qdec_status qdec_upload_quantized(qdec_ctx* c, int32_t layer, int32_t which,
                                           const void* codes, const float* scales, int64_t rows,
                                           int64_t cols, int32_t src_is_device, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (!codes || !scales) return fail(&c->err, QDEC_E_INVAL, "codes/scales NULL");
  Mat* m;
  float* vec;
  int64_t er, ec;
  qdec_status st = resolve(c, layer, which, &m, &vec, &er, &ec);
  if (st != QDEC_OK) return st;
  if (!m || !is_quant(m->dtype)) return fail(&c->err, QDEC_E_INVAL, "slot is not quantised");
  if (which == QDEC_W_LM_HEAD && c->cfg.tied_lm_head && c->lm_alias)
    return fail(&c->err, QDEC_E_INVAL, "tied LM head aliases the embedding");
  if (rows != er || cols != ec) return fail(&c->err, QDEC_E_INVAL, "shape mismatch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return st;
  Mat* dst = streamed(c, which) ? &stage_of(c, which) : m;
  if ((st = copy_in(c, dst->data, codes, code_bytes(m->dtype, rows, cols), src_is_device, s)) !=
      QDEC_OK)
    return st;
  if ((st = copy_in(c, dst->scale, scales, scale_count(m->dtype, rows, cols) * 4, src_is_device,
                    s)) != QDEC_OK)
    return st;
  if (dst != m && (st = stage_to_host(c, *dst, *m, s)) != QDEC_OK) return st;
  c->slot(is_global(which) ? c->cfg.n_layers : layer, which) = 1;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_upload_i8(qdec_ctx* c, int32_t layer, int32_t which,
                                    const int8_t* codes, const float* scales, int64_t rows,
                                    int64_t cols, int32_t src_is_device, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  Mat* m;
  float* vec;
  int64_t er, ec;
  qdec_status st = resolve(c, layer, which, &m, &vec, &er, &ec);
  if (st != QDEC_OK) return st;
  if (!m || m->dtype != QDEC_I8_ROW) return fail(&c->err, QDEC_E_INVAL, "slot is not int8-row");
  return qdec_upload_quantized(c, layer, which, codes, scales, rows, cols, src_is_device, stream);
}

QDEC_API qdec_status qdec_weight_ptr(const qdec_ctx* c0, int32_t layer, int32_t which,
                                     void** data, float** scales) {
  qdec_ctx* c = const_cast<qdec_ctx*>(c0);
  if (!c || !data) return fail(nullptr, QDEC_E_INVAL, "NULL argument");
  Mat* m;
  float* vec;
  int64_t r, k;
  qdec_status st = resolve(c, layer, which, &m, &vec, &r, &k);
  if (st != QDEC_OK) return st;
  *data = m ? m->data : vec;
  if (scales) *scales = m ? m->scale : nullptr;
  return QDEC_OK;
}

// =====================================================================================
// paged KV
// =====================================================================================

QDEC_API qdec_status qdec_kv_set_block_table(qdec_ctx* c, const int32_t* table, int32_t n_logical,
                                             void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (!table) return fail(&c->err, QDEC_E_INVAL, "table is NULL");
  if (n_logical < 1 || n_logical > c->cfg.num_pages)
    return fail(&c->err, QDEC_E_INVAL, "n_logical %d out of [1, %d]", n_logical, c->cfg.num_pages);
  std::vector<uint8_t> used((size_t)c->cfg.num_pages, 0);
  for (int i = 0; i < n_logical; ++i) {
    const int32_t p = table[i];
    if (p < 0 || p >= c->cfg.num_pages)
      return fail(&c->err, QDEC_E_INVAL, "block_table[%d] = %d out of [0, %d)", i, p,
                  c->cfg.num_pages);
    if (used[(size_t)p]) return fail(&c->err, QDEC_E_INVAL, "physical page %d mapped twice", p);
    used[(size_t)p] = 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  qdec_status st;
  if ((st = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return st;
  if ((st = c->hip(hipMemcpyAsync(c->block_table, table, (size_t)n_logical * 4,
                                  hipMemcpyHostToDevice, s),
                   "hipMemcpyAsync (block table)")) != QDEC_OK)
    return st;
  if ((st = c->hip(hipStreamSynchronize(s), "hipStreamSynchronize")) != QDEC_OK) return st;
  c->n_logical = n_logical;
  return QDEC_OK;
}

static qdec_status kv_copy(qdec_ctx* c, int32_t layer, int32_t pos0, int32_t n, void* k, void* v,
                           void* stream, int to_pool) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(&c->err, QDEC_E_INVAL, "layer out of range");
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16))
    return fail(&c->err, QDEC_E_INVAL, "k/v must be non-NULL and 16-byte aligned");
  if (pos0 < 0 || n < 0) return fail(&c->err, QDEC_E_INVAL, "negative position or count");
  if (c->n_logical == 0) return fail(&c->err, QDEC_E_STATE, "no block table set");
  if ((int64_t)pos0 + n > (int64_t)c->n_logical * kPage || (int64_t)pos0 + n > c->cfg.max_context)
    return fail(&c->err, QDEC_E_RANGE, "positions [%d, %d) not mapped", pos0, pos0 + n);
  if (n == 0) return QDEC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  qdec_status st;
  if ((st = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return st;
  const Layer& ly = c->layers[(size_t)layer];
  const int es = elem_size(c->cfg.kv_dtype);
  if ((st = c->hip(launch_kv_copy(ly.k_pool, k, c->block_table, pos0, n, c->cfg.n_kv_heads,
                                  c->cfg.head_dim, es, to_pool, s),
                   "kv copy kernel")) != QDEC_OK)
    return st;
  return c->hip(launch_kv_copy(ly.v_pool, v, c->block_table, pos0, n, c->cfg.n_kv_heads,
                               c->cfg.head_dim, es, to_pool, s),
                "kv copy kernel");
}

QDEC_API qdec_status qdec_kv_write(qdec_ctx* c, int32_t layer, int32_t pos0, int32_t n,
                                   const void* k, const void* v, void* stream) {
  return kv_copy(c, layer, pos0, n, const_cast<void*>(k), const_cast<void*>(v), stream, 1);
}

QDEC_API qdec_status qdec_kv_read(qdec_ctx* c, int32_t layer, int32_t pos0, int32_t n, void* k,
                                  void* v, void* stream) {
  return kv_copy(c, layer, pos0, n, k, v, stream, 0);
}

QDEC_API qdec_status qdec_kv_pool_ptr(const qdec_ctx* c, int32_t layer, void** k_pool,
                                      void** v_pool) {
  if (!c || !k_pool || !v_pool) return fail(nullptr, QDEC_E_INVAL, "NULL argument");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(nullptr, QDEC_E_INVAL, "layer out of range");
  *k_pool = c->layers[(size_t)layer].k_pool;
  *v_pool = c->layers[(size_t)layer].v_pool;
  return QDEC_OK;
}

// =====================================================================================
// the decode step
// =====================================================================================

static qdec_status check_step(qdec_ctx* c, const qdec_step* st, bool check_pos) {
  if (!st) return fail(&c->err, QDEC_E_INVAL, "step is NULL");
  if (st->reserved != 0) return fail(&c->err, QDEC_E_INVAL, "step.reserved must be 0");
  if (!(st->temperature >= 0.f) || !std::isfinite(st->temperature))
    return fail(&c->err, QDEC_E_INVAL, "temperature must be >= 0 and finite");
  if (st->temperature > 0.f) {
    if (!(st->top_p > 0.f) || st->top_p > 1.f)
      return fail(&c->err, QDEC_E_INVAL, "top_p must be in (0, 1] when sampling");
    if (c->cfg.vocab > (1 << 18))
      return fail(&c->err, QDEC_E_UNSUPPORTED, "sampling supports vocab <= 2^18");
  }
  if (!st->token_embedding && !st->token_id)
    return fail(&c->err, QDEC_E_INVAL, "need token_embedding or token_id");
  if (st->token_embedding && !aligned(st->token_embedding, 4))
    return fail(&c->err, QDEC_E_INVAL, "token_embedding misaligned");
  if (st->hidden_out && !aligned(st->hidden_out, 16))
    return fail(&c->err, QDEC_E_INVAL, "hidden_out must be 16-byte aligned");
  if (st->logits_out && !aligned(st->logits_out, 4))
    return fail(&c->err, QDEC_E_INVAL, "logits_out misaligned");
  const int L = c->cfg.n_layers;
  for (int l = 0; l <= L; ++l)
    for (int w = 0; w < kNumSlots; ++w) {
      bool need;
      if (l == L)
        need = is_global(w);
      else
        need = !is_global(w) && (c->cfg.qk_norm || (w != QDEC_W_Q_NORM && w != QDEC_W_K_NORM));
      if (need && !c->slot(l, w))
        return fail(&c->err, QDEC_E_STATE, "weight slot %d of layer %d not uploaded", w,
                    l == L ? -1 : l);
    }
  if (c->n_logical == 0) return fail(&c->err, QDEC_E_STATE, "no block table set");
  if (check_pos) {
    if (st->pos < 0 || st->pos >= c->cfg.max_context)
      return fail(&c->err, QDEC_E_RANGE, "pos %d outside [0, %d)", st->pos, c->cfg.max_context);
    if (st->pos / kPage >= c->n_logical)
      return fail(&c->err, QDEC_E_RANGE, "pos %d beyond the block table (%d pages)", st->pos,
                  c->n_logical);
  }
  return QDEC_OK;
}

// Records one launch for the event profiler (eager steps only).
struct ProfScope {
  qdec_ctx* c;
  hipStream_t s;
  int cls;
  bool on;
  ProfScope(qdec_ctx* c_, hipStream_t s_, int cls_, bool graph)
      : c(c_), s(s_), cls(cls_), on(c_->prof && !graph && c_->ev_used + 2 <= (int)c_->ev.size()) {
    if (on) (void)hipEventRecord(c->ev[(size_t)c->ev_used], s);
  }
  void done() {
    if (!on) return;
    (void)hipEventRecord(c->ev[(size_t)c->ev_used + 1], s);
    c->ev_class[(size_t)c->ev_used / 2] = cls;
    c->ev_used += 2;
  }
};

// Launches one kernel of the step: class `cls` of layer `l` (the LM head and argmax ignore l).
// grid_parts is the number of split-KV partitions the attention grid covers.
static hipError_t launch_class(qdec_ctx* c, const qdec_step* st, int cls, int64_t l,
                               int grid_parts, hipStream_t s) {
  const qdec_config& k = c->cfg;
  const int64_t d = k.hidden, hq = k.n_q_heads, hkv = k.n_kv_heads, hd = k.head_dim, f = k.ffn;
  const bool ab = c->act_bf16();
  const int wt = wt_of(k.proj_dtype);
  const Layer& ly = c->layers[(size_t)l];
  // the projections: the layer's own, or (layer streaming) those of its slot l % N
  const Layer& wm = (c->slots.empty() || c->direct_weights)
                        ? ly
                        : c->slots[(size_t)(l % (int64_t)c->slots.size())];
  switch (cls) {
    case QDEC_K_QKV: {
      GemvArgs g{};
      g.w = wm.qkv.data;
      g.scale = wm.qkv.scale;
      g.x = c->x;
      g.gamma = ly.in_norm;
      g.eps = k.rms_eps;
      g.round_h = ab;
      g.y = c->qkv;
      g.y_bf16 = 0;
      g.n = (hq + 2 * hkv) * hd;
      g.k = d;
      return launch_gemv(wt, EPI_STORE, true, g, s);
    }
    case QDEC_K_ATTENTION:
    case QDEC_K_MERGE: {
      AttnArgs at{};
      at.qkv = c->qkv;
      at.q_gamma = ly.q_norm;
      at.k_gamma = ly.k_norm;
      at.eps = k.rms_eps;
      at.rope_table = c->rope;
      at.rope_step = c->rope_step;
      at.round_q = ab;
      at.k_pool = ly.k_pool;
      at.v_pool = ly.v_pool;
      at.block_table = c->block_table;
      at.bt_len = c->bt_entries;
      at.desc = c->desc;
      at.n_q_heads = (int)hq;
      at.n_kv_heads = (int)hkv;
      at.part_tokens = c->part_tokens;
      at.max_parts = c->max_parts;
      at.part_acc = c->part_acc;
      at.part_ml = c->part_ml;
      at.out = c->attn;
      at.out_bf16 = ab;
      at.qscale = (float)(1.4426950408889634 / std::sqrt((double)hd));
      if (cls == QDEC_K_MERGE) return launch_attention_merge((int)hd, at, s);
      return launch_attention((int)hd, c->kv_bf16(), (int)(hq / hkv), true, at, grid_parts, s);
    }
    case QDEC_K_O_PROJ: {
      GemvArgs o{};
      o.w = wm.o.data;
      o.scale = wm.o.scale;
      o.x = c->attn;
      o.x_bf16 = ab;
      o.resid = c->x;
      o.n = d;
      o.k = hq * hd;
      return launch_gemv(wt, EPI_RESID, false, o, s);
    }
    case QDEC_K_GATE_UP: {
      GemvArgs gu{};
      gu.w = wm.gu.data;
      gu.scale = wm.gu.scale;
      gu.x = c->x;
      gu.gamma = ly.post_norm;
      gu.eps = k.rms_eps;
      gu.round_h = ab;
      gu.y = c->act;
      gu.y_bf16 = ab;
      gu.n = f;
      gu.k = d;
      return launch_gemv(wt, EPI_SWIGLU, true, gu, s);
    }
    case QDEC_K_DOWN: {
      GemvArgs dn{};
      dn.w = wm.down.data;
      dn.scale = wm.down.scale;
      dn.x = c->act;
      dn.x_bf16 = ab;
      dn.resid = c->x;
      dn.n = d;
      dn.k = f;
      return launch_gemv(wt, EPI_RESID, false, dn, s);
    }
    case QDEC_K_LM_HEAD: {
      const int lt = wt_of(k.lm_head_dtype);
      GemvArgs h{};
      h.w = c->lm.data;
      h.scale = c->lm.scale;
      h.x = c->x;
      h.gamma = c->final_norm;
      h.eps = k.rms_eps;
      h.round_h = ab;
      h.y = st->logits_out ? st->logits_out : c->logits;
      h.y_bf16 = c->io_bf16();
      h.hidden_copy = st->hidden_out;
      if (st->argmax_out) {  // the sampler takes its maximum from these too
        h.part_val = c->am_val;
        h.part_idx = c->am_idx;
        h.part_cap = c->am_parts;
      }
      h.n = k.vocab;
      h.k = d;
      return launch_gemv(lt, EPI_STORE, true, h, s);
    }
    case QDEC_K_ARGMAX: {
      if (!(st->temperature > 0.f))
        return launch_argmax_partials(c->am_val, c->am_idx, c->am_parts, st->argmax_out, s);
      SampleArgs sa{};
      sa.logits = st->logits_out ? st->logits_out : c->logits;
      sa.x_bf16 = c->io_bf16();
      sa.n = k.vocab;
      sa.inv_temperature = 1.0f / st->temperature;
      sa.top_p = st->top_p;
      sa.seed = st->seed;
      sa.desc = c->desc;
      sa.out = st->argmax_out;
      sa.part_val = c->am_val;
      sa.n_parts = c->am_parts;
      sa.ws = c->sample_ws;
      return launch_sample(sa, s);
    }
    default:
      return hipErrorInvalidValue;
  }
}

// Enqueues every kernel of the step after the embedding.  In graph mode the split-KV grid covers
// max_context (surplus work-groups exit at once) and the merge always runs; the kernels take
// ctx from the device descriptor in both modes, so eager and replayed steps compute the same
// values.
static qdec_status enqueue_layers(qdec_ctx* c, const qdec_step* st, int pos, hipStream_t s,
                                  bool graph) {
  const int np = n_parts_for(pos + 1, c->part_tokens);
  const int grid_parts = graph ? c->max_parts : np;
  qdec_status rs;
#define LAUNCH(cls, l)                                                                    \
  do {                                                                                    \
    ProfScope ps_(c, s, cls, graph);                                                      \
    if ((rs = c->hip(launch_class(c, st, cls, l, grid_parts, s), #cls)) != QDEC_OK) return rs; \
    ps_.done();                                                                           \
  } while (0)
  auto layer = [&](int64_t l) -> qdec_status {
    LAUNCH(QDEC_K_QKV, l);
    LAUNCH(QDEC_K_ATTENTION, l);
    if (graph || np > 1) LAUNCH(QDEC_K_MERGE, l);
    LAUNCH(QDEC_K_O_PROJ, l);
    LAUNCH(QDEC_K_GATE_UP, l);
    LAUNCH(QDEC_K_DOWN, l);
    return QDEC_OK;
  };
  if (c->slots.empty() || c->direct_weights) {
    for (int64_t l = 0; l < c->cfg.n_layers; ++l)
      if ((rs = layer(l)) != QDEC_OK) return rs;
  } else {
    // Layer streaming ([ETE], the "Layer streaming" passage): layer l runs from slot l % N.  Its
    // copy (host block of layer l -> slot) waits for the compute that last used the slot
    // (buffer free: layer l - N of this step, or for the first N layers the previous step's last
    // user of the slot), and its kernels wait for that copy (data ready).
    offload_schedule((int)c->cfg.n_layers, (int)c->slots.size(), &c->wops);
    for (const OffloadOp& op : c->wops) {
      hipError_t e = hipSuccess;
      switch (op.kind) {
        case OFF_WAIT_FREE:
          e = hipStreamWaitEvent(c->copy_stream, c->ev_computed[(size_t)op.slot], 0);
          break;
        case OFF_COPY: {
          if (op.tile < (int)c->slots.size())  // the previous step's last use of the slot
            e = hipStreamWaitEvent(c->copy_stream, c->ev_computed[(size_t)op.slot], 0);
          // the library's copy kernel on 64 work-groups reads the mapped host block: enough
          // requests in flight for the link, and a kernel launch, not a DMA transfer, between
          // two copies
          const Layer& dst = c->slots[(size_t)op.slot];
          const char* src = c->host_layers_dev + op.tile * c->layer_block;
          if (e == hipSuccess)
            e = launch_copy(dst.qkv.data, src, c->layer_block, c->copy_stream, kSlotCopyWgs);
          if (e == hipSuccess) e = hipEventRecord(c->ev_copied[(size_t)op.slot], c->copy_stream);
          break;
        }
        case OFF_WAIT_READY:
          e = hipStreamWaitEvent(s, c->ev_copied[(size_t)op.slot], 0);
          break;
        case OFF_COMPUTE:
          if ((rs = layer(op.tile)) != QDEC_OK) return rs;
          e = hipEventRecord(c->ev_computed[(size_t)op.slot], s);
          break;
        default:
          break;
      }
      if ((rs = c->hip(e, "layer streaming")) != QDEC_OK) return rs;
    }
  }
  if (st->logits_out || st->argmax_out) {
    LAUNCH(QDEC_K_LM_HEAD, 0);
    if (st->argmax_out) LAUNCH(QDEC_K_ARGMAX, 0);
  } else if (st->hidden_out) {
    if ((rs = c->hip(launch_copy(st->hidden_out, c->x, c->cfg.hidden * 4, s), "hidden copy")) !=
        QDEC_OK)
      return rs;
  }
#undef LAUNCH
  return QDEC_OK;
}

static qdec_status enqueue_embed(qdec_ctx* c, const qdec_step* st, int pos, hipStream_t s) {
  EmbedArgs e{};
  e.table = c->embed.data;
  e.table_bf16 = c->io_bf16();
  e.emb = st->token_embedding;
  e.token = st->token_id;
  e.x = c->x;
  e.desc = c->desc;
  e.rope_table = c->rope;
  e.rope_step = c->rope_step;
  e.rope_half = c->cfg.head_dim / 2;
  e.pos = pos;
  e.vocab = c->cfg.vocab;
  e.d = c->cfg.hidden;
  ProfScope ps(c, s, QDEC_K_EMBED, false);
  qdec_status r = c->hip(launch_embed(e, s), "embedding kernel");
  if (r == QDEC_OK) ps.done();
  return r;
}

QDEC_API qdec_status qdec_decode_step(qdec_ctx* c, const qdec_step* st, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  qdec_status r = check_step(c, st, true);
  if (r != QDEC_OK) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  if (c->prof) c->ev_used = 0;
  if ((r = enqueue_embed(c, st, st->pos, s)) != QDEC_OK) return r;
  return enqueue_layers(c, st, st->pos, s, false);
}

QDEC_API qdec_status qdec_prefill(qdec_ctx* c, const int32_t* token_ids, int32_t n, int32_t pos0,
                                  float* hidden_out, void* logits_out, int32_t* argmax_out,
                                  void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  const qdec_config& k = c->cfg;
  if (!token_ids) return fail(&c->err, QDEC_E_INVAL, "token_ids is NULL");
  if (k.max_prefill == 0) return fail(&c->err, QDEC_E_INVAL, "created with max_prefill = 0");
  if (n < 1 || n > k.max_prefill)
    return fail(&c->err, QDEC_E_INVAL, "n_tokens %d outside [1, %d]", n, k.max_prefill);
  if (hidden_out && !aligned(hidden_out, 16))
    return fail(&c->err, QDEC_E_INVAL, "hidden_out must be 16-byte aligned");
  if (logits_out && !aligned(logits_out, 4)) return fail(&c->err, QDEC_E_INVAL, "logits_out misaligned");
  if (pos0 < 0 || (int64_t)pos0 + n > k.max_context)
    return fail(&c->err, QDEC_E_RANGE, "positions %d .. %d outside [0, %d)", pos0, pos0 + n - 1,
                k.max_context);
  // the weight and block-table checks of a decode step at the last position
  qdec_step probe{};
  probe.token_id = token_ids;
  probe.pos = pos0 + n - 1;
  qdec_status r = check_step(c, &probe, true);
  if (r != QDEC_OK) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  const int d = k.hidden, hq = k.n_q_heads, hkv = k.n_kv_heads, hd = k.head_dim, f = k.ffn;
  const int nqkv = (hq + 2 * hkv) * hd;
#define P_TRY(call, what)                                \
  do {                                                   \
    if ((r = c->hip((call), what)) != QDEC_OK) return r; \
  } while (0)
  P_TRY(launch_embed_rows(c->embed.data, c->io_bf16(), token_ids, n, d, k.vocab, c->px, c->desc, s),
        "prefill embedding");
  for (int l = 0; l < k.n_layers; ++l) {
    const Layer& ly = c->layers[(size_t)l];
    GemmArgs g{};
    g.m = n;
    P_TRY(launch_rmsnorm_rows(c->px, ly.in_norm, k.rms_eps, c->ph, 1, d, n, s), "prefill norm");
    g.a = c->ph;
    g.w = ly.qkv.data;
    g.y = c->pqkv;
    g.y_bf16 = 0;
    g.n = nqkv;
    g.k = d;
    PrefillRopeArgs pr{};
    pr.qkv = c->pqkv;
    pr.q_gamma = ly.q_norm;
    pr.k_gamma = ly.k_norm;
    pr.eps = k.rms_eps;
    pr.table = c->rope;
    pr.q_out = static_cast<uint16_t*>(c->pq);
    pr.k_pool = static_cast<uint16_t*>(ly.k_pool);
    pr.v_pool = static_cast<uint16_t*>(ly.v_pool);
    pr.block_table = c->block_table;
    pr.pos0 = pos0;
    pr.p = n;
    pr.n_q_heads = hq;
    pr.n_kv_heads = hkv;
    if (hd == 128 && d % 64 == 0) {  // one 128-column tile per head: norm, RoPE, append in the epilogue
      g.rope = pr;
      P_TRY(launch_gemm(EPI_ROPE, g, s), "prefill qkv gemm + rope/append");
    } else {
      P_TRY(launch_gemm(EPI_STORE, g, s), "prefill qkv gemm");
      P_TRY(launch_prefill_rope(hd, pr, s), "prefill rope/append");
    }
    PrefillAttnArgs pa{};
    pa.q = static_cast<const uint16_t*>(c->pq);
    pa.k_pool = static_cast<const uint16_t*>(ly.k_pool);
    pa.v_pool = static_cast<const uint16_t*>(ly.v_pool);
    pa.block_table = c->block_table;
    pa.out = static_cast<uint16_t*>(c->pattn);
    pa.pos0 = pos0;
    pa.p = n;
    pa.n_q_heads = hq;
    pa.n_kv_heads = hkv;
    pa.qscale = (float)(1.4426950408889634 / std::sqrt((double)hd));
    P_TRY(launch_prefill_attn(hd, hq / hkv, pa, s), "prefill attention");
    g.a = c->pattn;
    g.w = ly.o.data;
    g.y = nullptr;
    g.resid = c->px;
    g.n = d;
    g.k = hq * hd;
    P_TRY(launch_gemm(EPI_RESID, g, s), "prefill o gemm");
    P_TRY(launch_rmsnorm_rows(c->px, ly.post_norm, k.rms_eps, c->ph, 1, d, n, s), "prefill norm");
    g.a = c->ph;
    g.w = ly.gu.data;
    g.y = c->pact;
    g.y_bf16 = 1;
    g.resid = nullptr;
    g.n = f;
    g.k = d;
    P_TRY(launch_gemm(EPI_SWIGLU, g, s), "prefill gate-up gemm");
    g.a = c->pact;
    g.w = ly.down.data;
    g.y = nullptr;
    g.resid = c->px;
    g.n = d;
    g.k = f;
    P_TRY(launch_gemm(EPI_RESID, g, s), "prefill down gemm");
  }
  // the last token: hidden state, final norm + LM head + argmax (the decode path's GEMV)
  float* xl = c->px + (int64_t)(n - 1) * d;
  if (logits_out || argmax_out) {
    GemvArgs h{};
    h.w = c->lm.data;
    h.scale = c->lm.scale;
    h.x = xl;
    h.gamma = c->final_norm;
    h.eps = k.rms_eps;
    h.round_h = 1;
    h.y = logits_out ? logits_out : c->logits;
    h.y_bf16 = c->io_bf16();
    h.hidden_copy = hidden_out;
    if (argmax_out) {
      h.part_val = c->am_val;
      h.part_idx = c->am_idx;
      h.part_cap = c->am_parts;
    }
    h.n = k.vocab;
    h.k = d;
    P_TRY(launch_gemv(wt_of(k.lm_head_dtype), EPI_STORE, true, h, s), "prefill LM head");
    if (argmax_out)
      P_TRY(launch_argmax_partials(c->am_val, c->am_idx, c->am_parts, argmax_out, s), "argmax");
  } else if (hidden_out) {
    P_TRY(launch_copy(hidden_out, xl, (int64_t)d * 4, s), "hidden copy");
  }
#undef P_TRY
  return QDEC_OK;
}

QDEC_API qdec_status qdec_graph_reset(qdec_ctx* c) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (c->gexec) (void)hipGraphExecDestroy(c->gexec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  c->gexec = nullptr;
  c->graph = nullptr;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_graph_capture(qdec_ctx* c, const qdec_step* templ, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (!c->slots.empty() && !c->direct_weights)
    return fail(&c->err, QDEC_E_UNSUPPORTED,
                "layer streaming (weight_slots > 0) runs its steps eagerly: no graph capture");
  qdec_status r = check_step(c, templ, false);
  if (r != QDEC_OK) return r;
  qdec_graph_reset(c);
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  if (!c->cap_stream &&
      (r = c->hip(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking),
                  "hipStreamCreateWithFlags")) != QDEC_OK)
    return r;
  // the capture stream must not start before earlier work on the caller's stream (uploads)
  if ((r = c->hip(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize")) !=
      QDEC_OK)
    return r;
  if ((r = c->hip(hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal),
                  "hipStreamBeginCapture")) != QDEC_OK)
    return r;
  qdec_status er = enqueue_layers(c, templ, 0, c->cap_stream, true);
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(c->cap_stream, &g);
  if (er != QDEC_OK) {
    if (g) (void)hipGraphDestroy(g);
    return er;
  }
  if ((r = c->hip(e, "hipStreamEndCapture")) != QDEC_OK) {
    if (g) (void)hipGraphDestroy(g);
    return r;
  }
  hipGraphExec_t ex = nullptr;
  if ((r = c->hip(hipGraphInstantiate(&ex, g, nullptr, nullptr, 0), "hipGraphInstantiate")) !=
      QDEC_OK) {
    (void)hipGraphDestroy(g);
    return r;
  }
  c->graph = g;
  c->gexec = ex;
  c->graph_templ = *templ;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_graph_replay(qdec_ctx* c, int32_t pos, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (!c->gexec) return fail(&c->err, QDEC_E_STATE, "no captured graph");
  qdec_step st = c->graph_templ;
  st.pos = pos;
  qdec_status r = check_step(c, &st, true);
  if (r != QDEC_OK) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  // the embedding kernel carries pos and runs in stream order ahead of the graph
  const bool prof = c->prof;
  c->prof = false;
  r = enqueue_embed(c, &st, pos, s);
  c->prof = prof;
  if (r != QDEC_OK) return r;
  return c->hip(hipGraphLaunch(c->gexec, s), "hipGraphLaunch");
}

QDEC_API qdec_status qdec_device_error(qdec_ctx* c, int32_t* flag, void* stream) {
  if (!c || !flag) return fail(nullptr, QDEC_E_INVAL, "NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  StepDesc h{};
  qdec_status r;
  if ((r = c->hip(hipMemcpyAsync(&h, c->desc, sizeof h, hipMemcpyDeviceToHost, s), "read flag")) !=
      QDEC_OK)
    return r;
  if ((r = c->hip(hipStreamSynchronize(s), "hipStreamSynchronize")) != QDEC_OK) return r;
  *flag = h.error;
  if (h.error) {
    const int32_t zero = 0;
    if ((r = c->hip(hipMemcpyAsync(&c->desc->error, &zero, 4, hipMemcpyHostToDevice, s),
                    "clear flag")) != QDEC_OK)
      return r;
    if ((r = c->hip(hipStreamSynchronize(s), "hipStreamSynchronize")) != QDEC_OK) return r;
  }
  return QDEC_OK;
}

// =====================================================================================
// event profiler
// =====================================================================================

QDEC_API qdec_status qdec_profile_enable(qdec_ctx* c, int32_t enable) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  qdec_status r;
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  for (int k = 0; k < QDEC_K_COUNT; ++k) {
    c->prof_ms[k] = 0;
    c->prof_n[k] = 0;
  }
  c->ev_used = 0;
  if (enable && c->ev.empty()) {
    const size_t n = 2 * (size_t)(8 * c->cfg.n_layers + 4);
    for (size_t i = 0; i < n; ++i) {
      hipEvent_t e;
      if ((r = c->hip(hipEventCreate(&e), "hipEventCreate")) != QDEC_OK) return r;
      c->ev.push_back(e);
    }
    c->ev_class.assign(n / 2, 0);
  }
  c->prof = enable != 0;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_profile_collect(qdec_ctx* c, double* ms, int64_t* launches) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  qdec_status r;
  for (int i = 0; i + 1 < c->ev_used; i += 2) {
    if ((r = c->hip(hipEventSynchronize(c->ev[(size_t)i + 1]), "hipEventSynchronize")) != QDEC_OK)
      return r;
    float t = 0.f;
    if ((r = c->hip(hipEventElapsedTime(&t, c->ev[(size_t)i], c->ev[(size_t)i + 1]),
                    "hipEventElapsedTime")) != QDEC_OK)
      return r;
    const int cls = c->ev_class[(size_t)i / 2];
    c->prof_ms[cls] += t;
    c->prof_n[cls] += 1;
  }
  c->ev_used = 0;
  for (int k = 0; k < QDEC_K_COUNT; ++k) {
    if (ms) ms[k] = c->prof_ms[k];
    if (launches) launches[k] = c->prof_n[k];
  }
  return QDEC_OK;
}

QDEC_API qdec_status qdec_profile_kernel(qdec_ctx* c, int32_t kclass, int32_t layer, int32_t reps,
                                         const qdec_step* st, void* stream) {
  if (!c) return fail(nullptr, QDEC_E_INVAL, "ctx is NULL");
  if (kclass < QDEC_K_QKV || kclass > QDEC_K_ARGMAX)
    return fail(&c->err, QDEC_E_INVAL, "kernel class %d cannot be replayed alone", kclass);
  if (layer < -1 || layer >= c->cfg.n_layers || reps < 1)
    return fail(&c->err, QDEC_E_INVAL, "bad layer or repetition count");
  qdec_status r = check_step(c, st, true);
  if (r != QDEC_OK) return r;
  if ((kclass == QDEC_K_LM_HEAD || kclass == QDEC_K_ARGMAX) && !st->argmax_out && !st->logits_out)
    return fail(&c->err, QDEC_E_INVAL, "the LM head needs logits_out or argmax_out");
  if (kclass == QDEC_K_ARGMAX && !st->argmax_out)
    return fail(&c->err, QDEC_E_INVAL, "argmax needs argmax_out");
  if (kclass == QDEC_K_ROPE_APPEND)
    return fail(&c->err, QDEC_E_INVAL, "Q/K norm, RoPE and append run inside the attention kernel");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((r = c->hip(hipSetDevice(c->device), "hipSetDevice")) != QDEC_OK) return r;
  const int np = n_parts_for(st->pos + 1, c->part_tokens);
  for (int i = 0; i < reps; ++i) {
    const int l = layer >= 0 ? layer : i % c->cfg.n_layers;
    if ((r = c->hip(launch_class(c, st, kclass, l, np, s), "profiled kernel")) != QDEC_OK) return r;
  }
  return QDEC_OK;
}

// =====================================================================================
// op-level entry points
// =====================================================================================



QDEC_API qdec_status qdec_op_gemv(const void* w, int32_t w_dtype, const float* w_scale,
                                  const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                                  int64_t n, int64_t k, void* stream) {
  if (!w || !x || !y) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (w_dtype < QDEC_F32 || w_dtype > QDEC_I4_G128) return fail(nullptr, QDEC_E_INVAL, "bad w_dtype");
  if (is_quant(w_dtype) != (w_scale != nullptr))
    return fail(nullptr, QDEC_E_INVAL, "w_scale is required for (and only for) quantised weights");
  if ((x_dtype != QDEC_F32 && x_dtype != QDEC_BF16) || (y_dtype != QDEC_F32 && y_dtype != QDEC_BF16))
    return fail(nullptr, QDEC_E_INVAL, "x/y dtype must be F32 or BF16");
  if (n < 1 || k < 1) return fail(nullptr, QDEC_E_INVAL, "n and k must be positive");
  if (code_bytes(w_dtype, 1, k) % 16) return fail(nullptr, QDEC_E_INVAL, "rows must be 16-byte multiples");
  if (is_grouped(w_dtype) && k % kQGroup)
    return fail(nullptr, QDEC_E_INVAL, "group-wise weights need k %% 128 == 0");
  if (!gemv_supported(wt_of(w_dtype), EPI_STORE, n, k))
    return fail(nullptr, QDEC_E_UNSUPPORTED,
                "k = %lld exceeds what the GEMV keeps in registers (8192 fp32, 16384 bf16, "
                "32768 int8 or int4 values)", (long long)k);
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || (w_scale && !aligned(w_scale, 4)))
    return fail(nullptr, QDEC_E_INVAL, "misaligned pointer (w and x 16-byte, y 4-byte)");
  GemvArgs a{};
  a.w = w;
  a.scale = w_scale;
  a.x = x;
  a.x_bf16 = x_dtype == QDEC_BF16;
  a.y = y;
  a.y_bf16 = y_dtype == QDEC_BF16;
  a.n = n;
  a.k = k;
  hipError_t e = launch_gemv(wt_of(w_dtype), EPI_STORE, false, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "gemv launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_quantize_rows(const void* w, int32_t w_dtype, int8_t* codes,
                                           float* scales, int64_t n, int64_t k, void* stream) {
  if (!w || !codes || !scales) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (w_dtype != QDEC_F32 && w_dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "bad w_dtype");
  if (n < 1 || k < 1 || k % 16) return fail(nullptr, QDEC_E_INVAL, "need n, k > 0 and k %% 16 == 0");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(nullptr, QDEC_E_INVAL, "misaligned pointer");
  hipError_t e = launch_quantize(w, w_dtype == QDEC_BF16, codes, scales, n, k,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "quantize launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_gemm(const void* a, const void* w, void* y, int32_t y_dtype,
                                  float* resid, int32_t epilogue, int32_t m, int32_t n, int32_t k,
                                  void* stream) {
  if (!a || !w) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (epilogue < QDEC_GEMM_STORE || epilogue > QDEC_GEMM_SWIGLU)
    return fail(nullptr, QDEC_E_INVAL, "bad epilogue");
  if (m < 1 || n < 1 || k < 32 || k % 32) return fail(nullptr, QDEC_E_INVAL, "need m, n > 0 and k a positive multiple of 32");
  if (epilogue == QDEC_GEMM_RESID ? !resid : !y) return fail(nullptr, QDEC_E_INVAL, "output is NULL");
  if (epilogue == QDEC_GEMM_STORE && y_dtype != QDEC_F32 && y_dtype != QDEC_BF16)
    return fail(nullptr, QDEC_E_INVAL, "y_dtype must be F32 or BF16");
  if (epilogue == QDEC_GEMM_SWIGLU && y_dtype != QDEC_BF16)
    return fail(nullptr, QDEC_E_INVAL, "the SwiGLU epilogue writes BF16");
  if (!aligned(a, 16) || !aligned(w, 16) || (y && !aligned(y, 4)) || (resid && !aligned(resid, 4)))
    return fail(nullptr, QDEC_E_INVAL, "misaligned pointer (a and w 16-byte)");
  GemmArgs g{};
  g.a = a;
  g.w = w;
  g.y = y;
  g.y_bf16 = y_dtype == QDEC_BF16;
  g.resid = resid;
  g.m = m;
  g.n = n;
  g.k = k;
  hipError_t e = launch_gemm(epilogue == QDEC_GEMM_STORE ? EPI_STORE
                             : epilogue == QDEC_GEMM_RESID ? EPI_RESID : EPI_SWIGLU,
                             g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "gemm launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_prefill_attention(const void* q, const void* k_pool,
                                               const void* v_pool, const int32_t* block_table,
                                               int32_t pos0, int32_t n_tokens, int32_t n_q_heads,
                                               int32_t n_kv_heads, int32_t head_dim, void* out,
                                               void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !out) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (head_dim != 64 && head_dim != 128) return fail(nullptr, QDEC_E_UNSUPPORTED, "head_dim");
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_q_heads / n_kv_heads > 8)
    return fail(nullptr, QDEC_E_INVAL, "bad head counts");
  if (pos0 < 0 || n_tokens < 1) return fail(nullptr, QDEC_E_INVAL, "need pos0 >= 0 and n_tokens >= 1");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 4))
    return fail(nullptr, QDEC_E_INVAL, "misaligned pointer (q and pools 16-byte)");
  PrefillAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.pos0 = pos0;
  a.p = n_tokens;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  hipError_t e = launch_prefill_attn(head_dim, n_q_heads / n_kv_heads, a,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "prefill attention launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_sample_workspace(int64_t n, size_t* bytes) {
  if (!bytes) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (n < 1 || n > (int64_t(1) << 18)) return fail(nullptr, QDEC_E_INVAL, "n must be in [1, 2^18]");
  *bytes = (size_t)sample_workspace_bytes(n);
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_sample(const void* logits, int32_t dtype, int64_t n, float temperature,
                                    float top_p, uint64_t seed, int32_t position, void* workspace,
                                    size_t workspace_bytes, int32_t* out, void* stream) {
  if (!logits || !out || !workspace) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (!aligned(workspace, 256)) return fail(nullptr, QDEC_E_INVAL, "workspace must be 256-byte aligned");
  if (dtype != QDEC_F32 && dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "bad dtype");
  if (n < 1 || n > (int64_t(1) << 18)) return fail(nullptr, QDEC_E_INVAL, "n must be in [1, 2^18]");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(nullptr, QDEC_E_INVAL, "temperature must be positive and finite");
  if (!(top_p > 0.f) || top_p > 1.f) return fail(nullptr, QDEC_E_INVAL, "top_p must be in (0, 1]");
  if (position < 0) return fail(nullptr, QDEC_E_INVAL, "position must be >= 0");
  if (workspace_bytes < (size_t)sample_workspace_bytes(n))
    return fail(nullptr, QDEC_E_INVAL, "workspace smaller than qdec_op_sample_workspace(n)");
  SampleArgs a{};
  a.logits = logits;
  a.x_bf16 = dtype == QDEC_BF16;
  a.n = n;
  a.inv_temperature = 1.0f / temperature;
  a.top_p = top_p;
  a.seed = seed;
  a.pos_arg = position;
  a.out = out;
  a.ws = workspace;
  hipError_t e = launch_sample(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "sample launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_quantize_groups(const void* w, int32_t w_dtype, int32_t dst_dtype,
                                             void* codes, float* scales, int64_t n, int64_t k,
                                             void* stream) {
  if (!w || !codes || !scales) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (w_dtype != QDEC_F32 && w_dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "bad w_dtype");
  if (!is_grouped(dst_dtype)) return fail(nullptr, QDEC_E_INVAL, "dst_dtype must be I8_G128 or I4_G128");
  if (n < 1 || k < 1 || k % kQGroup) return fail(nullptr, QDEC_E_INVAL, "need n, k > 0 and k %% 128 == 0");
  if (!aligned(w, 8) || !aligned(codes, 4) || !aligned(scales, 4))
    return fail(nullptr, QDEC_E_INVAL, "misaligned pointer (w 8-byte, codes and scales 4-byte)");
  hipError_t e = launch_quantize_groups(w, w_dtype == QDEC_BF16, dst_dtype == QDEC_I8_G128 ? 8 : 4,
                                        codes, scales, n, k, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "quantize launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_rmsnorm(const float* x, const float* gamma, float eps, void* y,
                                     int32_t y_dtype, int32_t n, void* stream) {
  if (!x || !gamma || !y) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (n < 1 || !(eps > 0.f)) return fail(nullptr, QDEC_E_INVAL, "need n > 0 and eps > 0");
  if (y_dtype != QDEC_F32 && y_dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "bad y_dtype");
  hipError_t e = launch_rmsnorm(x, gamma, eps, y, y_dtype == QDEC_BF16, n,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "rmsnorm launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_rope_table(float* table, int32_t max_pos, int32_t head_dim,
                                        float theta, void* stream) {
  if (!table) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (max_pos < 1 || (head_dim != 64 && head_dim != 128) || !(theta > 1.f))
    return fail(nullptr, QDEC_E_INVAL, "bad sizes");
  hipError_t e = launch_rope_table(table, max_pos, head_dim, theta, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "rope table launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_qk_norm_rope_append(
    const float* qkv, const float* q_gamma, const float* k_gamma, float eps, const float* table,
    int32_t pos, void* q_out, int32_t q_dtype, void* k_pool, void* v_pool, int32_t kv_dtype,
    const int32_t* block_table, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
    int32_t page_size, void* stream) {
  if (!qkv || !table || !q_out || !k_pool || !v_pool || !block_table)
    return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if ((q_gamma == nullptr) != (k_gamma == nullptr))
    return fail(nullptr, QDEC_E_INVAL, "q_gamma and k_gamma must both be set or both NULL");
  if (head_dim != 64 && head_dim != 128) return fail(nullptr, QDEC_E_UNSUPPORTED, "head_dim");
  if (page_size != kPage) return fail(nullptr, QDEC_E_UNSUPPORTED, "page_size must be 16");
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || pos < 0)
    return fail(nullptr, QDEC_E_INVAL, "bad head counts or position");
  if ((q_dtype != QDEC_F32 && q_dtype != QDEC_BF16) || (kv_dtype != QDEC_F32 && kv_dtype != QDEC_BF16))
    return fail(nullptr, QDEC_E_INVAL, "bad dtype");
  RopeAppendArgs a{};
  a.qkv = qkv;
  a.q_gamma = q_gamma;
  a.k_gamma = k_gamma;
  a.eps = eps;
  a.table = table;
  a.pos_arg = pos;
  a.q_out = q_out;
  a.q_bf16 = q_dtype == QDEC_BF16;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_bf16 = kv_dtype == QDEC_BF16;
  a.block_table = block_table;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  hipError_t e = launch_rope_append(head_dim, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "rope/append launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

static int op_part(int32_t ctx_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t partition_size) {
  return part_tokens_for(ctx_len, partition_size, n_kv_heads, target_wgs(n_q_heads, n_kv_heads));
}

// Workspace of the op-level attention with np partitions: accumulators, then (m, l) pairs, the
// second region 256-byte aligned.
struct AttnWs {
  int64_t acc_off, ml_off, bytes;
};
static AttnWs attn_ws(int64_t n_q_heads, int64_t np, int64_t head_dim) {
  AttnWs w;
  w.acc_off = 0;
  w.ml_off = (n_q_heads * np * head_dim * 4 + 255) / 256 * 256;
  w.bytes = w.ml_off + n_q_heads * np * 8;
  return w;
}

QDEC_API qdec_status qdec_op_attention_workspace(int32_t ctx_len, int32_t n_q_heads,
                                                 int32_t head_dim, int32_t partition_size,
                                                 size_t* bytes) {
  if (!bytes) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (ctx_len < 1 || n_q_heads < 1 || head_dim < 1 || partition_size < 0 || partition_size % 64 ||
      partition_size > kMaxPartTokens)
    return fail(nullptr, QDEC_E_INVAL, "bad sizes");
  // the automatic size depends on n_kv_heads; take the largest count it can produce (Hkv = 1)
  const int part = partition_size > 0 ? partition_size
                                      : part_tokens_for(ctx_len, 0, 1, kMaxTargetWgs);
  const int64_t np = n_parts_for(ctx_len, part);
  *bytes = np <= 1 ? 0 : (size_t)attn_ws(n_q_heads, np, head_dim).bytes;
  return QDEC_OK;
}

// Validates an op-level attention call and derives its partition length and count.
static qdec_status op_attention_check(const void* q, int32_t q_dtype, const void* k_pool,
                                      const void* v_pool, int32_t kv_dtype,
                                      const int32_t* block_table, int32_t ctx_len,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t page_size, int32_t partition_size, const void* out,
                                      int32_t out_dtype, int* part, int* np) {
  if (!q || !k_pool || !v_pool || !block_table || !out) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (head_dim != 64 && head_dim != 128) return fail(nullptr, QDEC_E_UNSUPPORTED, "head_dim");
  if (page_size != kPage) return fail(nullptr, QDEC_E_UNSUPPORTED, "page_size must be 16");
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_q_heads / n_kv_heads > 8)
    return fail(nullptr, QDEC_E_INVAL, "bad head counts");
  if (ctx_len < 1) return fail(nullptr, QDEC_E_INVAL, "ctx_len must be positive");
  if (partition_size < 0 || partition_size % 64 || partition_size > kMaxPartTokens)
    return fail(nullptr, QDEC_E_INVAL, "partition_size must be 0 or a multiple of 64 up to %d",
                kMaxPartTokens);
  if ((q_dtype != QDEC_F32 && q_dtype != QDEC_BF16) || (kv_dtype != QDEC_F32 && kv_dtype != QDEC_BF16) ||
      (out_dtype != QDEC_F32 && out_dtype != QDEC_BF16))
    return fail(nullptr, QDEC_E_INVAL, "bad dtype");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return fail(nullptr, QDEC_E_INVAL, "pools must be 16-byte aligned");
  *part = op_part(ctx_len, n_q_heads, n_kv_heads, partition_size);
  *np = n_parts_for(ctx_len, *part);
  if (*np > kMaxMergeParts)
    return fail(nullptr, QDEC_E_UNSUPPORTED, "more than %d partitions", kMaxMergeParts);
  return QDEC_OK;
}

// Enqueues the split-KV kernel (and the merge, with several partitions) of a checked call; the
// partials go to workspace (laid out as attn_ws describes).
static qdec_status op_attention_launch(const void* q, int32_t q_dtype, const void* k_pool,
                                       const void* v_pool, int32_t kv_dtype,
                                       const int32_t* block_table, int32_t ctx_len,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       int part, int np, void* workspace, void* out,
                                       int32_t out_dtype, void* stream) {
  const AttnWs ws = attn_ws(n_q_heads, np, head_dim);
  AttnArgs a{};
  a.q = q;
  a.q_bf16 = q_dtype == QDEC_BF16;
  a.k_pool = const_cast<void*>(k_pool);
  a.v_pool = const_cast<void*>(v_pool);
  a.block_table = block_table;
  a.bt_len = (ctx_len + kPage - 1) / kPage;  // the caller's table covers exactly the context
  a.desc = nullptr;
  a.ctx_arg = ctx_len;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.part_tokens = part;
  a.max_parts = np;
  char* wsb = static_cast<char*>(workspace);
  if (np > 1) {
    a.part_acc = reinterpret_cast<float*>(wsb + ws.acc_off);
    a.part_ml = reinterpret_cast<float*>(wsb + ws.ml_off);
  }
  a.out = out;
  a.out_bf16 = out_dtype == QDEC_BF16;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      launch_attention(head_dim, kv_dtype == QDEC_BF16, n_q_heads / n_kv_heads, false, a, np, s);
  if (e == hipSuccess && np > 1) e = launch_attention_merge(head_dim, a, s);
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "attention launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_attention(const void* q, int32_t q_dtype, const void* k_pool,
                                       const void* v_pool, int32_t kv_dtype,
                                       const int32_t* block_table, int32_t ctx_len,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                       int32_t page_size, int32_t partition_size, void* workspace,
                                       size_t workspace_bytes, void* out, int32_t out_dtype,
                                       void* stream) {
  int part = 0, np = 0;
  qdec_status r = op_attention_check(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len,
                                     n_q_heads, n_kv_heads, head_dim, page_size, partition_size,
                                     out, out_dtype, &part, &np);
  if (r != QDEC_OK) return r;
  const AttnWs ws = attn_ws(n_q_heads, np, head_dim);
  if (np > 1 && (!workspace || workspace_bytes < (size_t)ws.bytes || !aligned(workspace, 256)))
    return fail(nullptr, QDEC_E_INVAL, "workspace of %lld bytes (256-byte aligned) required",
                (long long)ws.bytes);
  return op_attention_launch(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len,
                             n_q_heads, n_kv_heads, head_dim, part, np, workspace, out, out_dtype,
                             stream);
}

// ---- the allocation-free variant of qdec_op_attention ---------------------------------------
// Its split-KV partials live in `scratch`, a file-scope device array of kNoAllocScratchBytes that
// every GPU the library runs on holds for the life of the process.  In host code the array's
// name is only a stand-in: the device address of each GPU's copy comes from hipGetSymbolAddress,
// taken once per device (with that device current) on the first call there, and only that
// address is ever handed to a kernel.  Calls on one GPU share its copy, so calls that overlap on
// one GPU race; nothing in it needs clearing (every slot a call reads, the same call writes first).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

// Device address of the current device's copy of `scratch`.
static qdec_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(nullptr, QDEC_E_UNSUPPORTED, "device %d beyond the %d the scratch table covers",
                dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, QDEC_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_attention_noalloc(const void* q, int32_t q_dtype, const void* k_pool,
                                               const void* v_pool, int32_t kv_dtype,
                                               const int32_t* block_table, int32_t ctx_len,
                                               int32_t n_q_heads, int32_t n_kv_heads,
                                               int32_t head_dim, int32_t page_size,
                                               int32_t partition_size, void* out,
                                               int32_t out_dtype, void* stream) {
  int part = 0, np = 0;
  qdec_status r = op_attention_check(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len,
                                     n_q_heads, n_kv_heads, head_dim, page_size, partition_size,
                                     out, out_dtype, &part, &np);
  if (r != QDEC_OK) return r;
  const AttnWs ws = attn_ws(n_q_heads, np, head_dim);
  if (np > 1 && (size_t)ws.bytes > kNoAllocScratchBytes)
    return fail(nullptr, QDEC_E_RANGE,
                "split-KV partials of %lld bytes exceed the %zu-byte static scratch (fewer query "
                "heads, a shorter context or longer partitions fit)",
                (long long)ws.bytes, kNoAllocScratchBytes);
  void* sp = nullptr;
  if (np > 1 && (r = scratch_address(&sp)) != QDEC_OK) return r;
  return op_attention_launch(q, q_dtype, k_pool, v_pool, kv_dtype, block_table, ctx_len,
                             n_q_heads, n_kv_heads, head_dim, part, np, sp, out, out_dtype, stream);
}

QDEC_API qdec_status qdec_op_argmax(const void* x, int32_t x_dtype, int64_t n, int32_t* out,
                                    void* stream) {
  if (!x || !out) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (x_dtype != QDEC_F32 && x_dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "bad dtype");
  if (n < 1 || n > (int64_t)1 << 31) return fail(nullptr, QDEC_E_INVAL, "n out of range");
  hipError_t e = launch_argmax(x, x_dtype == QDEC_BF16, n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "argmax launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_op_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (bytes < 0 || bytes % 16 || !aligned(dst, 16) || !aligned(src, 16))
    return fail(nullptr, QDEC_E_INVAL, "bytes and pointers must be multiples of 16");
  hipError_t e = launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "copy launch: %s", hipGetErrorString(e));
  return QDEC_OK;
}

// =====================================================================================
// attention over host-resident K/V: tiles copied into device buffers, double-buffered
// =====================================================================================

// (the copy / compute schedule, offload_schedule, is defined with the context above: layer
// streaming uses it too)
struct qdec_offload {
  qdec_offload_config cfg{};
  int part = 0;               // partition length
  int max_parts = 0;          // partials per head (stride)
  int tile_pages = 0;
  int64_t page_bytes = 0;     // one page of K (or V): Hkv * 16 * D * elem
  char* dev_k = nullptr;      // [n_slots][tile_pages] pages
  char* dev_v = nullptr;
  int32_t* bt = nullptr;      // identity page table of one buffer
  float* part_acc = nullptr;
  float* part_ml = nullptr;
  hipStream_t copy_stream = nullptr;
  hipEvent_t start = nullptr, done = nullptr;
  std::vector<hipEvent_t> copied, computed;
  bool called = false;
  int64_t device_bytes = 0;
  std::vector<OffloadOp> ops;
};

static void offload_free(qdec_offload* o) {
  if (!o) return;
  (void)hipSetDevice(o->cfg.device);
  if (o->copy_stream) (void)hipStreamSynchronize(o->copy_stream);
  for (hipEvent_t e : o->copied)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : o->computed)
    if (e) (void)hipEventDestroy(e);
  if (o->start) (void)hipEventDestroy(o->start);
  if (o->done) (void)hipEventDestroy(o->done);
  if (o->copy_stream) (void)hipStreamDestroy(o->copy_stream);
  for (void* p : {(void*)o->dev_k, (void*)o->dev_v, (void*)o->bt, (void*)o->part_acc,
                  (void*)o->part_ml})
    if (p) (void)hipFree(p);
  delete o;
}

QDEC_API qdec_status qdec_offload_create(const qdec_offload_config* cfg, qdec_offload** out) {
  if (!cfg || !out) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  *out = nullptr;
  const qdec_offload_config& c = *cfg;
  if (c.head_dim != 64 && c.head_dim != 128) return fail(nullptr, QDEC_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads || c.n_q_heads / c.n_kv_heads > 8)
    return fail(nullptr, QDEC_E_INVAL, "bad head counts");
  if (c.kv_dtype != QDEC_F32 && c.kv_dtype != QDEC_BF16) return fail(nullptr, QDEC_E_INVAL, "kv_dtype must be F32 or BF16");
  if (c.max_context < 1) return fail(nullptr, QDEC_E_INVAL, "max_context must be positive");
  if (c.tile_tokens < 64 || c.tile_tokens > 65536 || c.tile_tokens % 64)
    return fail(nullptr, QDEC_E_INVAL, "tile_tokens must be a multiple of 64 in [64, 65536]");
  if (c.n_slots < 0 || c.n_slots > 8) return fail(nullptr, QDEC_E_INVAL, "n_slots must be in [0, 8]");
  if (c.partition_size < 0 || c.partition_size % 64 || c.partition_size > kMaxPartTokens ||
      (c.partition_size > 0 && c.tile_tokens % c.partition_size))
    return fail(nullptr, QDEC_E_INVAL,
                "partition_size must be 0 or a multiple of 64 up to %d that divides tile_tokens",
                kMaxPartTokens);
  int part = c.partition_size;
  if (part == 0) {  // the resident path's choice for one tile (direct: for max_context), lowered
                    // until it divides the tile
    part = part_tokens_for(c.n_slots ? c.tile_tokens : c.max_context, 0, c.n_kv_heads,
                           target_wgs(c.n_q_heads, c.n_kv_heads));
    while (c.tile_tokens % part) part -= 64;
  }
  const int64_t max_parts = n_parts_for(c.max_context, part);
  if (max_parts > kMaxMergeParts)
    return fail(nullptr, QDEC_E_UNSUPPORTED, "more than %d partitions at max_context", kMaxMergeParts);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || c.device < 0 || c.device >= ndev)
    return fail(nullptr, QDEC_E_INVAL, "no such device");
  if (hipSetDevice(c.device) != hipSuccess) return fail(nullptr, QDEC_E_HIP, "hipSetDevice failed");
  qdec_offload* o = new qdec_offload();
  o->cfg = c;
  o->part = part;
  o->max_parts = (int)max_parts;
  o->tile_pages = c.tile_tokens / kPage;
  o->page_bytes = (int64_t)c.n_kv_heads * kPage * c.head_dim * elem_size(c.kv_dtype);
  const int64_t buf_bytes = (int64_t)c.n_slots * o->tile_pages * o->page_bytes;
  // identity page table: one buffer's pages, or (direct) every page of max_context
  const int bt_pages = c.n_slots ? o->tile_pages : (c.max_context + kPage - 1) / kPage;
  const AttnWs ws = attn_ws(c.n_q_heads, max_parts, c.head_dim);
  auto alloc = [&](void** p, int64_t bytes) {
    o->device_bytes += bytes;
    return hipMalloc(p, (size_t)bytes) == hipSuccess;
  };
  bool ok = (buf_bytes == 0 || (alloc((void**)&o->dev_k, buf_bytes) &&
                                 alloc((void**)&o->dev_v, buf_bytes))) &&
            alloc((void**)&o->bt, (int64_t)bt_pages * 4) &&
            alloc((void**)&o->part_acc, ws.ml_off) && alloc((void**)&o->part_ml, ws.bytes - ws.ml_off);
  if (ok) {
    std::vector<int32_t> ident(bt_pages);
    for (int j = 0; j < bt_pages; ++j) ident[j] = j;
    ok = hipMemcpy(o->bt, ident.data(), ident.size() * 4, hipMemcpyHostToDevice) == hipSuccess;
  }
  ok = ok && hipStreamCreateWithFlags(&o->copy_stream, hipStreamNonBlocking) == hipSuccess &&
       hipEventCreateWithFlags(&o->start, hipEventDisableTiming) == hipSuccess &&
       hipEventCreateWithFlags(&o->done, hipEventDisableTiming) == hipSuccess;
  o->copied.assign(c.n_slots, nullptr);
  o->computed.assign(c.n_slots, nullptr);
  for (int s = 0; ok && s < c.n_slots; ++s)
    ok = hipEventCreateWithFlags(&o->copied[s], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&o->computed[s], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    const hipError_t e = hipGetLastError();
    offload_free(o);
    return fail(nullptr, QDEC_E_NOMEM, "offload allocation failed: %s", hipGetErrorString(e));
  }
  *out = o;
  return QDEC_OK;
}

QDEC_API void qdec_offload_destroy(qdec_offload* o) { offload_free(o); }

QDEC_API qdec_status qdec_offload_info(const qdec_offload* o, int64_t* device_bytes,
                                       int32_t* partition_tokens) {
  if (!o) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (device_bytes) *device_bytes = o->device_bytes;
  if (partition_tokens) *partition_tokens = o->part;
  return QDEC_OK;
}

QDEC_API qdec_status qdec_offload_schedule(int32_t n_tiles, int32_t n_slots, int32_t* records,
                                           int32_t cap, int32_t* n) {
  if (!n || (cap > 0 && !records)) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  if (n_tiles < 1 || n_slots < 1 || n_slots > 8 || n_tiles > (1 << 24))
    return fail(nullptr, QDEC_E_INVAL, "bad tile or slot count");
  std::vector<OffloadOp> ops;
  offload_schedule(n_tiles, n_slots, &ops);
  *n = (int32_t)ops.size();
  for (int32_t i = 0; i < cap && i < (int32_t)ops.size(); ++i) {
    records[4 * i + 0] = ops[i].kind;
    records[4 * i + 1] = ops[i].tile;
    records[4 * i + 2] = ops[i].slot;
    records[4 * i + 3] = ops[i].other;
  }
  return QDEC_OK;
}

static bool pinned_host(const void* p) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // pageable memory: clear the error so no later call reports it
    return false;
  }
  return at.type == hipMemoryTypeHost;
}

QDEC_API qdec_status qdec_offload_attention(qdec_offload* o, const void* q, int32_t q_dtype,
                                            const void* host_k, const void* host_v,
                                            int32_t ctx_len, void* out, int32_t out_dtype,
                                            void* stream) {
  if (!o || !q || !host_k || !host_v || !out) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  const qdec_offload_config& c = o->cfg;
  if (ctx_len < 1 || ctx_len > c.max_context)
    return fail(nullptr, QDEC_E_RANGE, "ctx_len must be in [1, %d]", c.max_context);
  if ((q_dtype != QDEC_F32 && q_dtype != QDEC_BF16) || (out_dtype != QDEC_F32 && out_dtype != QDEC_BF16))
    return fail(nullptr, QDEC_E_INVAL, "bad dtype");
  if (hipSetDevice(c.device) != hipSuccess) return fail(nullptr, QDEC_E_HIP, "hipSetDevice failed");
  if (!pinned_host(host_k) || !pinned_host(host_v))
    return fail(nullptr, QDEC_E_INVAL, "host_k and host_v must be pinned host memory");
  void* dk = nullptr;  // direct mode: the device's address of the host pages
  void* dv = nullptr;
  if (c.n_slots == 0 &&
      (hipHostGetDevicePointer(&dk, const_cast<void*>(host_k), 0) != hipSuccess ||
       hipHostGetDevicePointer(&dv, const_cast<void*>(host_v), 0) != hipSuccess || !dk || !dv ||
       !aligned(dk, 16) || !aligned(dv, 16))) {
    (void)hipGetLastError();
    return fail(nullptr, QDEC_E_INVAL, "host_k and host_v must be device-mapped pinned memory");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n_tiles = (ctx_len + c.tile_tokens - 1) / c.tile_tokens;
  const int tile_parts = c.tile_tokens / o->part;
  const int64_t buf_bytes = (int64_t)o->tile_pages * o->page_bytes;
  AttnArgs a{};
  a.q = q;
  a.q_bf16 = q_dtype == QDEC_BF16;
  a.block_table = o->bt;
  a.desc = nullptr;
  a.n_q_heads = c.n_q_heads;
  a.n_kv_heads = c.n_kv_heads;
  a.part_tokens = o->part;
  a.max_parts = o->max_parts;
  a.part_acc = o->part_acc;
  a.part_ml = o->part_ml;
  a.to_partials = 1;
  a.out = out;
  a.out_bf16 = out_dtype == QDEC_BF16;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  const bool kvb = c.kv_dtype == QDEC_BF16;
  const int group = c.n_q_heads / c.n_kv_heads;
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
    return e == hipSuccess;
  };
  // the previous call's kernels (slots, partials) and everything before this call on the
  // caller's stream come first
  if (o->called) chk(hipStreamWaitEvent(s, o->done, 0));
  if (c.n_slots == 0) {  // direct: the split-KV kernel reads the mapped host pages itself
    AttnArgs t = a;
    t.k_pool = dk;
    t.v_pool = dv;
    t.bt_len = (ctx_len + kPage - 1) / kPage;
    t.ctx_arg = ctx_len;
    chk(launch_attention(c.head_dim, kvb, group, false, t, n_parts_for(ctx_len, o->part), s));
    chk(launch_attention_merge(c.head_dim, t, s));
    chk(hipEventRecord(o->done, s));
    o->called = true;
    if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "offload attention: %s", hipGetErrorString(e));
    return QDEC_OK;
  }
  // the tiles are copied by the library's copy kernel reading the pinned pages through their
  // device mapping (a kernel launch between two tiles instead of a DMA transfer's setup)
  if (hipHostGetDevicePointer(&dk, const_cast<void*>(host_k), 0) != hipSuccess ||
      hipHostGetDevicePointer(&dv, const_cast<void*>(host_v), 0) != hipSuccess || !dk || !dv ||
      !aligned(dk, 16) || !aligned(dv, 16)) {
    (void)hipGetLastError();
    return fail(nullptr, QDEC_E_INVAL, "host_k and host_v must be device-mapped pinned memory");
  }
  chk(hipEventRecord(o->start, s));
  chk(hipStreamWaitEvent(o->copy_stream, o->start, 0));
  offload_schedule(n_tiles, c.n_slots, &o->ops);
  for (const OffloadOp& op : o->ops) {
    if (e != hipSuccess) break;
    const int i = op.tile;
    const int64_t t0 = (int64_t)i * c.tile_tokens;
    const int len = i >= 0 ? (int)std::min<int64_t>(c.tile_tokens, ctx_len - t0) : 0;
    const int pages = (len + kPage - 1) / kPage;
    switch (op.kind) {
      case OFF_WAIT_FREE:
        chk(hipStreamWaitEvent(o->copy_stream, o->computed[op.slot], 0));
        break;
      case OFF_COPY: {
        const int64_t src = t0 / kPage * o->page_bytes, bytes = pages * o->page_bytes;
        chk(launch_copy(o->dev_k + op.slot * buf_bytes, static_cast<const char*>(dk) + src,
                        bytes, o->copy_stream, kSlotCopyWgs));
        chk(launch_copy(o->dev_v + op.slot * buf_bytes, static_cast<const char*>(dv) + src,
                        bytes, o->copy_stream, kSlotCopyWgs));
        chk(hipEventRecord(o->copied[op.slot], o->copy_stream));
        break;
      }
      case OFF_WAIT_READY:
        chk(hipStreamWaitEvent(s, o->copied[op.slot], 0));
        break;
      case OFF_COMPUTE: {
        AttnArgs t = a;
        t.k_pool = o->dev_k + op.slot * buf_bytes;
        t.v_pool = o->dev_v + op.slot * buf_bytes;
        t.bt_len = pages;
        t.ctx_arg = len;
        t.part_base = i * tile_parts;
        chk(launch_attention(c.head_dim, kvb, group, false, t, n_parts_for(len, o->part), s));
        chk(hipEventRecord(o->computed[op.slot], s));
        break;
      }
      case OFF_MERGE: {
        AttnArgs m = a;
        m.ctx_arg = ctx_len;
        chk(launch_attention_merge(c.head_dim, m, s));
        chk(hipEventRecord(o->done, s));
        break;
      }
    }
  }
  o->called = true;
  if (e != hipSuccess) return fail(nullptr, QDEC_E_HIP, "offload attention: %s", hipGetErrorString(e));
  return QDEC_OK;
}

QDEC_API qdec_status qdec_host_alloc(size_t bytes, void** ptr) {
  if (!ptr) return fail(nullptr, QDEC_E_INVAL, "NULL pointer");
  *ptr = nullptr;
  if (bytes == 0) return fail(nullptr, QDEC_E_INVAL, "bytes must be positive");
  if (hipHostMalloc(ptr, bytes, hipHostMallocDefault) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    *ptr = nullptr;
    return fail(nullptr, QDEC_E_NOMEM, "hipHostMalloc of %zu bytes: %s", bytes, hipGetErrorString(e));
  }
  return QDEC_OK;
}

QDEC_API qdec_status qdec_host_free(void* ptr) {
  if (ptr && hipHostFree(ptr) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return fail(nullptr, QDEC_E_HIP, "hipHostFree: %s", hipGetErrorString(e));
  }
  return QDEC_OK;
}

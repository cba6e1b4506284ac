/*
 * oracle.c - plain, slow CPU reference for the batch-1 GQA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry file and the
 * benchmark's CPU-baseline leg may load or call this library.  The HIP library never does, and
 * the two share no code, headers, tables or helpers.
 *
 * Arithmetic: every dot product, sum of squares and softmax sum is accumulated in fp64 and each
 * function returns fp64 results.  Stored tensors are read exactly as stored (bf16 widened by the
 * 16-bit shift, int8 codes as integers, fp32 as is).  Where the pages fix a narrower precision the
 * oracle applies it at the same place:
 *   - the quantisers compute their scales and codes in fp32 (scale = max|row| / 127 per row, or
 *     max|group| / 127 or / 7 per 128-value group);
 *   - the KV cache stores values rounded to its storage type (bf16 or fp32), and the logits are
 *     rounded to their output type;
 *   - when the step keeps bf16 activations at op boundaries ([Qwen3-runtime] §0.1: bf16 in and
 *     out, fp32 inside reductions), those tensors are rounded to bf16 at the same places.
 *
 * Sources, cited by page title and section:
 *   [Qwen3-runtime]  "从 Qwen3 数学到 CUDA Kernel：0.6B 推理运行时的完整实现与优化" (chengzipai.xyz)
 *   [ETE]            "EdgeTransformerEngine" (thomasli.cn/cuda-engine.html)
 *
 * Pins (what checks this file against something other than itself) live in the CPU tests:
 * library routines (torch rms_norm / silu / bfloat16 casts, numpy matmul, scipy softmax), closed
 * forms (complex-exponential RoPE, constant-vector RMSNorm), invariants (rotation norm, softmax
 * shift invariance, bijective paging) and brute force on tiny inputs.  Every exported function
 * below has at least one such pin; none is "parity unpinned".
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).  OpenMP only splits
 * independent output rows or heads across threads; each row's arithmetic order is sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2, OR_I8G = 3, OR_I4G = 4 };

/* Values per quantisation group of the group-wise formats ([Qwen3-runtime] §13.1: a warp walks a
 * row in 128-value groups, each with its own scale). */
#define OR_GROUP 128

/* ------------------------------------------------------------------------------------------ */
/* Number formats                                                                             */
/* ------------------------------------------------------------------------------------------ */

/* bf16 -> value: the bf16 bits are the upper half of an fp32 word ([ETE], the passage on bf16 as a
 * storage format: widening is a 16-bit left shift). */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Rounds a value to the nearest bf16 number, ties to even, directly from fp64 (8 significant
 * bits, fp32's exponent range; below 2^-126 the spacing is the subnormal step 2^-133).  Overflow
 * rounds to infinity.  This is a reading: the pages show only the widening direction. */
static double round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  double a = fabs(v);
  if (a < ldexp(1.0, -126)) return ldexp(nearbyint(ldexp(v, 133)), -133);
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
  double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
  if (fabs(r) >= ldexp(1.0, 128)) return v > 0 ? INFINITY : -INFINITY;
  return r;
}

static uint16_t bf16_bits_of(double rounded) {
  float f = (float)rounded; /* exact: rounded is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(rounded)) return (uint16_t)0x7FC0;
  return (uint16_t)(u >> 16);
}

static double round_f32(double v) { return (double)(float)v; }

/* Arithmetic mode.  0 (the default, and the reference every test compares against): every sum,
 * product and function in fp64.  1: plain fp32 -- every partial sum, every product that is not
 * fused into a sum, and every function value rounded to fp32, in the sequential order the loops
 * below state, as a straightforward fp32 implementation computes them.  The fp32 mode measures
 * how far a correct fp32 implementation of the same method lands from the fp64 result; with
 * 16-bit activations that distance is the method's own sensitivity to fp32 rounding, which the
 * tests use to bound the GPU's distance. */
static int g_fp32 = 0;
void or_set_fp32(int32_t on) { g_fp32 = on != 0; }
int32_t or_get_fp32(void) { return g_fp32; }

/* Threads that split independent rows and heads (timing only: each row's arithmetic is the same
 * sequential order whatever the count). */
#ifdef _OPENMP
#include <omp.h>
void or_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }
int32_t or_get_threads(void) { return omp_get_max_threads(); }
#else
void or_set_threads(int32_t n) { (void)n; }
int32_t or_get_threads(void) { return 1; }
#endif
static double F(double v) { return g_fp32 ? round_f32(v) : v; }

void or_round_bf16(const double* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
}

void or_to_bf16_bits(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_of(round_bf16(in[i]));
}

void or_bf16_bits_to_double(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_double(in[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Shapes and byte counts ([Qwen3-runtime] §1.1 and §3.3)                                      */
/* ------------------------------------------------------------------------------------------ */

/* Parameters of one layer: the packed QKV matrix (Q width Hq*D, K and V width Hkv*D each), the O
 * matrix, packed gate and up, down, the input and post-attention gammas and the per-head Q/K
 * gammas. */
int64_t or_params_per_layer(int64_t hidden, int64_t hq, int64_t hkv, int64_t d, int64_t ffn,
                            int32_t qk_norm) {
  int64_t q_w = hq * d, kv_w = hkv * d;
  int64_t mats = (q_w + 2 * kv_w) * hidden  /* W_q, W_k, W_v */
                 + hidden * q_w             /* W_o */
                 + 2 * ffn * hidden         /* W_gate, W_up */
                 + hidden * ffn;            /* W_down */
  int64_t norms = 2 * hidden + (qk_norm ? 2 * d : 0);
  return mats + norms;
}

/* All layers plus the embedding (counted once when the LM head is tied) plus the final norm. */
int64_t or_params_total(int64_t n_layers, int64_t hidden, int64_t hq, int64_t hkv, int64_t d,
                        int64_t ffn, int64_t vocab, int32_t tied, int32_t qk_norm) {
  return n_layers * or_params_per_layer(hidden, hq, hkv, d, ffn, qk_norm) +
         vocab * hidden * (tied ? 1 : 2) + hidden;
}

/* KV bytes of one layer and one token at batch 1: K and V (the first factor 2), Hkv heads of D
 * elements each, elem bytes per element ([Qwen3-runtime] §3.3). */
int64_t or_kv_bytes_per_layer_token(int64_t hkv, int64_t d, int64_t elem) {
  return 2 * hkv * d * elem;
}

/* ------------------------------------------------------------------------------------------ */
/* Elementwise pieces                                                                          */
/* ------------------------------------------------------------------------------------------ */

/* RMSNorm without mean subtraction ([Qwen3-runtime] §2.1): y = x / sqrt(mean(x^2) + eps) * gamma. */
void or_rmsnorm(const double* x, const float* gamma, int64_t n, double eps, double* y) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss = F(ss + x[i] * x[i]);
  double inv = F(1.0 / F(sqrt(F(F(ss / (double)n) + eps))));
  for (int64_t i = 0; i < n; ++i) y[i] = F(F(x[i] * inv) * (double)gamma[i]);
}

/* SiLU ([Qwen3-runtime] §2.7): silu(z) = z * sigmoid(z). */
static double silu(double z) { return F(z / F(1.0 + F(exp(-z)))); }

void or_silu(const double* z, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(z[i]);
}

/* Half-rotation RoPE at position pos ([Qwen3-runtime] §2.4): the two halves of a head vector are
 * paired, a = v[i], b = v[i + D/2], and rotated by the angle pos * theta_i with
 * theta_i = base^(-2i/D):  a' = a cos - b sin,  b' = b cos + a sin.  The frequency formula and the
 * sign convention were lost from the page; this is the reading taken. */
void or_rope(double* v, int32_t d, int64_t pos, double base) {
  int32_t h = d / 2;
  for (int32_t i = 0; i < h; ++i) {
    double ang = (double)pos * pow(base, -2.0 * (double)i / (double)d);
    double c = F(cos(ang)), s = F(sin(ang));
    double a = v[i], b = v[i + h];
    v[i] = F(a * c - F(b * s));
    v[i + h] = F(b * c + F(a * s));
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Projections ([Qwen3-runtime] §4.1: at batch 1 every linear layer is a GEMV)                   */
/* ------------------------------------------------------------------------------------------ */

/* Code of element c in row r of a group-wise matrix: an int8 byte (OR_I8G), or a nibble of the
 * packed int4 layout (OR_I4G: element c sits in byte c / 2 of the row, even c in the low nibble,
 * stored offset-binary as code + 8). */
static double group_code(const void* w, int32_t wt, int64_t k, int64_t r, int64_t c) {
  if (wt == OR_I8G) return (double)((const int8_t*)w)[r * k + c];
  const uint8_t b = ((const uint8_t*)w)[r * (k / 2) + c / 2];
  const int nib = (c % 2 == 0) ? (b & 0x0F) : (b >> 4);
  return (double)(nib - 8);
}

/* y[n] = sum_k W[n][k] x[k] for W of type wt (OR_F32, OR_BF16, OR_I8 codes, or the group-wise
 * OR_I8G / OR_I4G codes).  For OR_I8 the per-row scale multiplies the integer-weighted sum once:
 * y = s_n * sum_k q_nk x_k, which equals sum_k (q_nk s_n) x_k in exact arithmetic
 * ([Qwen3-runtime] §13.1, the group-scale step, read per row as [ETE] quantises per row).  For the
 * group-wise types the steps are those of [Qwen3-runtime] §13.1: each 128-value group's
 * integer-weighted partial sum is formed first, then multiplied by that group's scale
 * (scale[n][k / 128]) and added to the row total. */
void or_gemv(const void* w, int32_t wt, const float* scale, const double* x, int64_t n, int64_t k,
             double* y) {
  if (wt == OR_F32) {
    const float* W = (const float*)w;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      double s = 0.0;
      for (int64_t c = 0; c < k; ++c) s = F(s + (double)W[r * k + c] * x[c]);
      y[r] = s;
    }
  } else if (wt == OR_BF16) {
    const uint16_t* W = (const uint16_t*)w;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      double s = 0.0;
      for (int64_t c = 0; c < k; ++c) s = F(s + bf16_bits_to_double(W[r * k + c]) * x[c]);
      y[r] = s;
    }
  } else if (wt == OR_I8) {
    const int8_t* W = (const int8_t*)w;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      double s = 0.0;
      for (int64_t c = 0; c < k; ++c) s = F(s + (double)W[r * k + c] * x[c]);
      y[r] = F(s * (double)scale[r]);
    }
  } else {
    const int64_t ng = k / OR_GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      double total = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        double part = 0.0;
        for (int64_t c = g * OR_GROUP; c < (g + 1) * OR_GROUP; ++c)
          part = F(part + group_code(w, wt, k, r, c) * x[c]);
        total = F(total + F(part * (double)scale[r * ng + g]));
      }
      y[r] = total;
    }
  }
}

/* Symmetric per-row int8 quantisation ([ETE], the int8 passage: symmetric, one scale per row).
 * In fp32 as the scheme states: scale = max|w_row| / 127; code = w / scale rounded to nearest
 * (ties to even: a reading), clamped to [-127, 127].  A zero row gets scale 0 and zero codes. */
void or_quantize_rows(const float* w, int64_t n, int64_t k, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    const float* row = w + r * k;
    float mx = 0.0f;
    for (int64_t c = 0; c < k; ++c) {
      float a = fabsf(row[c]);
      if (a > mx) mx = a;
    }
    float sc = mx / 127.0f;
    s[r] = sc;
    for (int64_t c = 0; c < k; ++c) {
      float v = 0.0f;
      if (sc != 0.0f) {
        v = rintf(row[c] / sc);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
      }
      q[r * k + c] = (int8_t)v;
    }
  }
}

/* Group-wise symmetric quantisation: one fp32 scale per 128-value group of a row
 * ([Qwen3-runtime] §13.1 keeps a scale per row and group), with 8-bit codes (qmax = 127) or the
 * 4-bit codes [ETE] names as the next step (qmax = 7).  Within each group it is the per-row rule
 * above: scale = max|w| / qmax in fp32, code = w / scale rounded to nearest (ties to even),
 * clamped to [-qmax, qmax]; an all-zero group gets scale 0 and zero codes.  k % 128 == 0.
 * Storage: bits = 8, int8 codes [n][k]; bits = 4, two codes per byte [n][k / 2] (element c in
 * byte c / 2, even c in the low nibble, offset-binary code + 8).  s: [n][k / 128]. */
void or_quantize_groups(const float* w, int64_t n, int64_t k, int32_t bits, void* q, float* s) {
  const int64_t ng = k / OR_GROUP;
  const float qmax = bits == 8 ? 127.0f : 7.0f;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < ng; ++g) {
      const float* grp = w + r * k + g * OR_GROUP;
      float mx = 0.0f;
      for (int64_t c = 0; c < OR_GROUP; ++c) {
        float a = fabsf(grp[c]);
        if (a > mx) mx = a;
      }
      const float sc = mx / qmax;
      s[r * ng + g] = sc;
      for (int64_t c = 0; c < OR_GROUP; ++c) {
        float v = 0.0f;
        if (sc != 0.0f) {
          v = rintf(grp[c] / sc);
          if (v > qmax) v = qmax;
          if (v < -qmax) v = -qmax;
        }
        const int64_t e = g * OR_GROUP + c;  /* element index within the row */
        if (bits == 8) {
          ((int8_t*)q)[r * k + e] = (int8_t)v;
        } else {
          uint8_t* byte = (uint8_t*)q + r * (k / 2) + e / 2;
          const uint8_t nib = (uint8_t)((int)v + 8);
          if (e % 2 == 0)
            *byte = nib;  /* the even element comes first and starts the byte */
          else
            *byte = (uint8_t)(*byte | (nib << 4));
        }
      }
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Attention ([Qwen3-runtime] §2.5-2.6, §9.1; [ETE] the online-softmax passage)                */
/* ------------------------------------------------------------------------------------------ */

/* The plain definition, two passes.  q: [hq][d]; K, V: logical [t][hkv][d] (values as stored).
 * Query head h reads kv head h / (hq / hkv) ([Qwen3-runtime] §2.5).  Scores s_j = q.k_j / sqrt(d)
 * over every key j < t (the causal range of the new token); softmax with the maximum subtracted;
 * out = sum_j p_j v_j. */
void or_attention(const double* q, const float* K, const float* V, int64_t t, int32_t hq,
                  int32_t hkv, int32_t d, double* out) {
  int32_t group = hq / hkv;
  double rs = sqrt((double)d);
#pragma omp parallel for schedule(dynamic)
  for (int32_t h = 0; h < hq; ++h) {
    int32_t g = h / group;
    const double* qh = q + (int64_t)h * d;
    double* s = (double*)malloc(sizeof(double) * (size_t)(t > 0 ? t : 1));
    double mx = -INFINITY;
    for (int64_t j = 0; j < t; ++j) {
      const float* kj = K + (j * hkv + g) * d;
      double dot = 0.0;
      for (int32_t r = 0; r < d; ++r) dot = F(dot + qh[r] * (double)kj[r]);
      s[j] = F(dot / F(rs));
      if (s[j] > mx) mx = s[j];
    }
    double* o = out + (int64_t)h * d;
    for (int32_t r = 0; r < d; ++r) o[r] = 0.0;
    double den = 0.0;
    for (int64_t j = 0; j < t; ++j) {
      double w = F(exp(F(s[j] - mx)));
      den = F(den + w);
      const float* vj = V + (j * hkv + g) * d;
      for (int32_t r = 0; r < d; ++r) o[r] = F(o[r] + w * (double)vj[r]);
    }
    for (int32_t r = 0; r < d; ++r) o[r] = F(o[r] / den);
    free(s);
  }
}

/* One online-softmax update of the state (m, l, acc) with a new score and value row
 * ([ETE], the (m, l, acc) passage; [Qwen3-runtime] §9.1, the scalar state update). */
static void online_update(double score, const float* v, int32_t d, double* m, double* l,
                          double* acc) {
  double nm = score > *m ? score : *m;
  double old_scale = exp(*m - nm);
  double new_scale = exp(score - nm);
  *l = *l * old_scale + new_scale;
  for (int32_t r = 0; r < d; ++r) acc[r] = acc[r] * old_scale + (double)v[r] * new_scale;
  *m = nm;
}

/* State of one contiguous range [j0, j1) of keys for query head h: m starts at -1e30, l and acc
 * at 0 ([ETE]: the initialisation kernel's values). */
static void partition_state(const double* qh, const float* K, const float* V, int64_t j0,
                            int64_t j1, int32_t g, int32_t hkv, int32_t d, double* m, double* l,
                            double* acc) {
  double rs = sqrt((double)d);
  *m = -1e30;
  *l = 0.0;
  for (int32_t r = 0; r < d; ++r) acc[r] = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    const float* kj = K + (j * hkv + g) * d;
    double dot = 0.0;
    for (int32_t r = 0; r < d; ++r) dot += qh[r] * (double)kj[r];
    online_update(dot / rs, V + (j * hkv + g) * d, d, m, l, acc);
  }
}

/* Single-pass online form over all t keys, then out = acc / l ([ETE]: the finalisation kernel). */
void or_attention_online(const double* q, const float* K, const float* V, int64_t t, int32_t hq,
                         int32_t hkv, int32_t d, double* out) {
  int32_t group = hq / hkv;
  for (int32_t h = 0; h < hq; ++h) {
    double m, l;
    double* o = out + (int64_t)h * d;
    partition_state(q + (int64_t)h * d, K, V, 0, t, h / group, hkv, d, &m, &l, o);
    for (int32_t r = 0; r < d; ++r) o[r] /= l;
  }
}

/* Split form ([Qwen3-runtime] §9.1, §10.2): keys cut into contiguous partitions of `part`
 * positions, each reduced to (m_p, l_p, o_p) with o_p unnormalised; then M = max_p m_p, each state
 * rescaled by exp(m_p - M), L = sum l_p e^(m_p-M), O = sum o_p e^(m_p-M), out = O / L. */
void or_attention_partitioned(const double* q, const float* K, const float* V, int64_t t,
                              int32_t hq, int32_t hkv, int32_t d, int64_t part, double* out) {
  int32_t group = hq / hkv;
  int64_t np = (t + part - 1) / part;
  double* ms = (double*)malloc(sizeof(double) * (size_t)np);
  double* ls = (double*)malloc(sizeof(double) * (size_t)np);
  double* os = (double*)malloc(sizeof(double) * (size_t)(np * d));
  for (int32_t h = 0; h < hq; ++h) {
    for (int64_t p = 0; p < np; ++p) {
      int64_t j0 = p * part, j1 = j0 + part < t ? j0 + part : t;
      partition_state(q + (int64_t)h * d, K, V, j0, j1, h / group, hkv, d, &ms[p], &ls[p],
                      os + p * d);
    }
    double M = -INFINITY;
    for (int64_t p = 0; p < np; ++p)
      if (ms[p] > M) M = ms[p];
    double L = 0.0;
    double* o = out + (int64_t)h * d;
    for (int32_t r = 0; r < d; ++r) o[r] = 0.0;
    for (int64_t p = 0; p < np; ++p) {
      double w = exp(ms[p] - M);
      L += ls[p] * w;
      for (int32_t r = 0; r < d; ++r) o[r] += os[p * d + r] * w;
    }
    for (int32_t r = 0; r < d; ++r) o[r] /= L;
  }
  free(ms);
  free(ls);
  free(os);
}

/* ------------------------------------------------------------------------------------------ */
/* Paged KV addressing ([Qwen3-runtime] §7.2: logical page = p / page, slot = p % page, physical  */
/* page from the block table).  The intra-page layout is not on the page; the reading taken is  */
/* one contiguous page x D tile per (physical page, kv head).                                   */
/* ------------------------------------------------------------------------------------------ */

int64_t or_pool_offset(int32_t pos, int32_t head, int32_t r, const int32_t* block_table,
                       int32_t hkv, int32_t d, int32_t page) {
  int64_t phys = block_table[pos / page];
  int64_t slot = pos % page;
  return ((phys * hkv + head) * page + slot) * d + r;
}

/* Places logical rows [n][hkv][d] (elem bytes each, copied bit for bit) of positions
 * pos0..pos0+n-1 into a pool buffer by or_pool_offset. */
void or_pool_scatter(const void* logical, int32_t elem, int32_t pos0, int32_t n,
                     const int32_t* block_table, int32_t hkv, int32_t d, int32_t page,
                     void* pool) {
  const unsigned char* src = (const unsigned char*)logical;
  unsigned char* dst = (unsigned char*)pool;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t g = 0; g < hkv; ++g)
      for (int32_t r = 0; r < d; ++r) {
        int64_t off = or_pool_offset(pos0 + i, g, r, block_table, hkv, d, page);
        memcpy(dst + off * elem, src + (((int64_t)i * hkv + g) * d + r) * elem, (size_t)elem);
      }
}

/* ------------------------------------------------------------------------------------------ */
/* Sampling beyond greedy ([ETE] names temperature and top-p as missing; the method is the     */
/* usual one, read plainly)                                                                    */
/* ------------------------------------------------------------------------------------------ */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011): ten rounds, each multiplying words 0 and 2 of the
 * counter by 0xD2511F53 and 0xCD9E8D57 into 64-bit products, the new counter being
 * (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key is bumped by the
 * Weyl constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    if (r < 9) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform draw of a sampling step: Philox4x32-10 with key (seed low, seed high) and counter
 * (position, 0, 0, 0); u = (first word >> 8) * 2^-24, in [0, 1). */
double or_sample_uniform(uint64_t seed, int64_t pos) {
  const uint32_t ctr[4] = {(uint32_t)pos, 0u, 0u, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  or_philox4x32_10(ctr, key, out);
  return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

/* Temperature + top-p (nucleus) sampling of one token from logits[n], by definition:
 *   p_i = softmax(logits / temperature)_i (temperature > 0);
 *   the nucleus is the shortest prefix of the tokens ordered by p descending (ties: lower index
 *   first) whose probability mass reaches top_p (the token that reaches it is included);
 *   the draw is the nucleus token, in index order, at which the cumulative nucleus mass first
 *   exceeds u times the nucleus mass (the order of this inverse-CDF walk is a reading: any fixed
 *   order gives the same distribution, and index order needs no sort).
 * Returns the token index; writes the nucleus size and mass to *nsize / *nmass when non-NULL. */
static const double* g_sort_p;
static int cmp_desc(const void* a, const void* b) {
  const int64_t i = *(const int64_t*)a, j = *(const int64_t*)b;
  if (g_sort_p[i] > g_sort_p[j]) return -1;
  if (g_sort_p[i] < g_sort_p[j]) return 1;
  return i < j ? -1 : (i > j ? 1 : 0);
}
int64_t or_sample(const double* logits, int64_t n, double temperature, double top_p, double u,
                  int64_t* nsize, double* nmass) {
  double mx = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (logits[i] / temperature > mx) mx = logits[i] / temperature;
  double* p = (double*)malloc((size_t)n * sizeof(double));
  int64_t* idx = (int64_t*)malloc((size_t)n * sizeof(int64_t));
  unsigned char* in = (unsigned char*)calloc((size_t)n, 1);
  double z = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    p[i] = exp(logits[i] / temperature - mx);
    z += p[i];
  }
  for (int64_t i = 0; i < n; ++i) {
    p[i] /= z;
    idx[i] = i;
  }
  g_sort_p = p;
  qsort(idx, (size_t)n, sizeof(int64_t), cmp_desc);
  double mass = 0.0;
  int64_t k = 0;
  while (k < n) {
    mass += p[idx[k]];
    in[idx[k]] = 1;
    ++k;
    if (mass >= top_p) break;
  }
  double target = u * mass, cum = 0.0;
  int64_t pick = idx[0];
  for (int64_t i = 0; i < n; ++i) {
    if (!in[i]) continue;
    cum += p[i];
    pick = i;
    if (cum > target) break;
  }
  if (nsize) *nsize = k;
  if (nmass) *nmass = mass;
  free(p);
  free(idx);
  free(in);
  return pick;
}

/* ------------------------------------------------------------------------------------------ */
/* One decode step of the whole model                                                          */
/* ------------------------------------------------------------------------------------------ */

typedef struct or_model {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t qk_norm;
  int32_t embed_type, proj_type, lm_type; /* OR_F32 / OR_BF16 / OR_I8 / OR_I8G / OR_I4G */
  int32_t act_bf16;                       /* 1: bf16 rounding of op-boundary activations */
  int32_t kv_bf16;                        /* 1: the KV cache stores bf16 values, else fp32 */
  int32_t logits_bf16;                    /* 1: logits are returned as bf16 values, else fp32 */
  int32_t max_ctx;
  double eps, theta;
  const void* embed;
  const void* lm_head;
  const float* lm_scale;
  const float* final_norm;
  const void* const* qkv;
  const float* const* qkv_scale;
  const void* const* o;
  const float* const* o_scale;
  const void* const* gate_up;
  const float* const* gate_up_scale;
  const void* const* down;
  const float* const* down_scale;
  const float* const* in_norm;
  const float* const* post_norm;
  const float* const* q_norm;
  const float* const* k_norm;
  float* const* k_cache; /* per layer, logical [max_ctx][Hkv][D] */
  float* const* v_cache;
} or_model;

static double act_round(const or_model* m, double v) { return m->act_bf16 ? round_bf16(v) : v; }
static double kv_round(const or_model* m, double v) {
  return m->kv_bf16 ? round_bf16(v) : round_f32(v);
}

/* The step of [ETE] (its GPU block pipeline) with the math of [Qwen3-runtime] §2.1-2.7:
 *   x = E[token] (or the given embedding row)
 *   per layer:  h = RMSNorm(x, g_in);  [q|k|v] = W_qkv h  (Q rows, then K, then V)
 *               per Q and K head: RMSNorm over D (when qk_norm), then RoPE at pos
 *               append k, v at logical position pos (so attention covers 0..pos)
 *               o_h = attention(q_h, K[0..pos], V[0..pos]) for every Q head
 *               x += W_o concat(o_h)
 *               h2 = RMSNorm(x, g_post);  [g|u] = W_gu h2;  a = silu(g) * u;  x += W_down a
 *   hidden = x;  logits = W_lm RMSNorm(x, g_final);  argmax = lowest index of the maximum.
 * With act_bf16, activations crossing an op boundary are rounded to bf16 ([Qwen3-runtime] §0.1):
 * each RMSNorm output that feeds a projection, the rotated Q, the attention output and the
 * SwiGLU output; without it they stay fp64 (bf16 only as a storage format, [ETE]).  K/V are
 * stored by kv_round.  The logits are rounded to their output type (bf16 or fp32) before the
 * argmax, so the greedy decision is taken on the values returned.
 * Returns 0, or -1 on a bad argument. */
int32_t or_decode_step(const or_model* m, int32_t token, const double* emb, int32_t pos,
                       double* hidden_out, double* logits_out, int32_t* argmax_out) {
  const int64_t dm = m->hidden, hq = m->n_q_heads, hkv = m->n_kv_heads, d = m->head_dim;
  const int64_t f = m->ffn, v = m->vocab;
  const int64_t qw = hq * d, kw = hkv * d, nqkv = qw + 2 * kw;
  if (pos < 0 || pos >= m->max_ctx || d > 256) return -1;
  if (!emb && (token < 0 || token >= v)) return -1;

  double* x = (double*)calloc((size_t)dm, sizeof(double));
  double* h = (double*)malloc(sizeof(double) * (size_t)(dm > f ? dm : f));
  double* qkv = (double*)malloc(sizeof(double) * (size_t)nqkv);
  double* att = (double*)malloc(sizeof(double) * (size_t)qw);
  double* y = (double*)malloc(sizeof(double) * (size_t)(dm > 2 * f ? dm : 2 * f));
  double* a = (double*)malloc(sizeof(double) * (size_t)f);

  if (emb) {
    for (int64_t i = 0; i < dm; ++i) x[i] = emb[i];
  } else if (m->embed_type == OR_BF16) {
    const uint16_t* E = (const uint16_t*)m->embed;
    for (int64_t i = 0; i < dm; ++i) x[i] = bf16_bits_to_double(E[(int64_t)token * dm + i]);
  } else {
    const float* E = (const float*)m->embed;
    for (int64_t i = 0; i < dm; ++i) x[i] = (double)E[(int64_t)token * dm + i];
  }

  for (int32_t l = 0; l < m->n_layers; ++l) {
    /* attention block */
    or_rmsnorm(x, m->in_norm[l], dm, m->eps, h);
    for (int64_t i = 0; i < dm; ++i) h[i] = act_round(m, h[i]);
    or_gemv(m->qkv[l], m->proj_type, m->qkv_scale ? m->qkv_scale[l] : NULL, h, nqkv, dm, qkv);

    double* q = qkv;            /* [hq][d] */
    double* kx = qkv + qw;      /* [hkv][d] */
    double* vx = qkv + qw + kw; /* [hkv][d] */
    double tmp[256];
    for (int64_t hh = 0; hh < hq; ++hh) {
      double* qh = q + hh * d;
      if (m->qk_norm) {
        or_rmsnorm(qh, m->q_norm[l], d, m->eps, tmp);
        memcpy(qh, tmp, sizeof(double) * (size_t)d);
      }
      or_rope(qh, (int32_t)d, pos, m->theta);
      for (int64_t r = 0; r < d; ++r) qh[r] = act_round(m, qh[r]);
    }
    float* kc = m->k_cache[l];
    float* vc = m->v_cache[l];
    for (int64_t g = 0; g < hkv; ++g) {
      double* kh = kx + g * d;
      if (m->qk_norm) {
        or_rmsnorm(kh, m->k_norm[l], d, m->eps, tmp);
        memcpy(kh, tmp, sizeof(double) * (size_t)d);
      }
      or_rope(kh, (int32_t)d, pos, m->theta);
      for (int64_t r = 0; r < d; ++r) {
        kc[((int64_t)pos * hkv + g) * d + r] = (float)kv_round(m, kh[r]);
        vc[((int64_t)pos * hkv + g) * d + r] = (float)kv_round(m, vx[g * d + r]);
      }
    }
    or_attention(q, kc, vc, (int64_t)pos + 1, (int32_t)hq, (int32_t)hkv, (int32_t)d, att);
    for (int64_t i = 0; i < qw; ++i) att[i] = act_round(m, att[i]);
    or_gemv(m->o[l], m->proj_type, m->o_scale ? m->o_scale[l] : NULL, att, dm, qw, y);
    for (int64_t i = 0; i < dm; ++i) x[i] = F(x[i] + y[i]);

    /* MLP block */
    or_rmsnorm(x, m->post_norm[l], dm, m->eps, h);
    for (int64_t i = 0; i < dm; ++i) h[i] = act_round(m, h[i]);
    or_gemv(m->gate_up[l], m->proj_type, m->gate_up_scale ? m->gate_up_scale[l] : NULL, h, 2 * f,
            dm, y);
    for (int64_t i = 0; i < f; ++i) a[i] = act_round(m, F(silu(y[i]) * y[f + i]));
    or_gemv(m->down[l], m->proj_type, m->down_scale ? m->down_scale[l] : NULL, a, dm, f, y);
    for (int64_t i = 0; i < dm; ++i) x[i] = F(x[i] + y[i]);
  }

  if (hidden_out)
    for (int64_t i = 0; i < dm; ++i) hidden_out[i] = x[i];

  if (logits_out || argmax_out) {
    double* lg = (double*)malloc(sizeof(double) * (size_t)v);
    or_rmsnorm(x, m->final_norm, dm, m->eps, h);
    for (int64_t i = 0; i < dm; ++i) h[i] = act_round(m, h[i]);
    or_gemv(m->lm_head, m->lm_type, m->lm_scale, h, v, dm, lg);
    for (int64_t i = 0; i < v; ++i) lg[i] = m->logits_bf16 ? round_bf16(lg[i]) : round_f32(lg[i]);
    if (argmax_out) {
      int32_t best = -1;
      for (int64_t i = 0; i < v; ++i)
        if (!isnan(lg[i]) && (best < 0 || lg[i] > lg[best])) best = (int32_t)i;
      *argmax_out = best;
    }
    if (logits_out) memcpy(logits_out, lg, sizeof(double) * (size_t)v);
    free(lg);
  }
  free(x);
  free(h);
  free(qkv);
  free(att);
  free(y);
  free(a);
  return 0;
}

/* Index of the largest value, the lowest index on ties, NaN never chosen (-1 if all NaN). */
int64_t or_argmax(const double* x, int64_t n) {
  int64_t best = -1;
  for (int64_t i = 0; i < n; ++i)
    if (!isnan(x[i]) && (best < 0 || x[i] > x[best])) best = i;
  return best;
}

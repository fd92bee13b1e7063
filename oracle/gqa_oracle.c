/*
 * Plain fp64 CPU oracle for one incremental decoding step of grouped-query
 * attention against a per-sequence KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path (the
 * HIP library under gqa_kv_cache_decode_amd/csrc) shares no code, header,
 * table or constant with this file.
 *
 * Sources (web pages; see the oracle package docstring for the full list):
 *   [MQA-review]   "Fast Transformer Decoding: One Write-Head is All You Need"
 *                  paper review (velog): §2.1 Dot-Product Attention,
 *                  §2.4 Multi-head Attention (Incremental), §3 Multi Query
 *                  Attention.
 *   [GQA-lesson]   "TF2 GQA" lesson (ttlab): the g-knob table (g = h is MHA,
 *                  1 < g < h is GQA, g = 1 is MQA), the h mod g = 0 rule, the
 *                  cache element-count formula, the multiplication counts and
 *                  the lab description (contiguous query-head groups, K/V
 *                  repeated per query head).
 *   [LLM-inf-05]   "LLM inference 05" notes (albangk): the prefill/decode
 *                  table, the per-layer decode pseudocode (push K, push V,
 *                  then attend) and the bytes-per-token arithmetic.
 *
 * What is computed is the plain definition, written out with no blocking,
 * fusion or reordering:
 *   for every sequence b and query head i (G = h/g query heads per KV head,
 *   j = floor(i / G)):
 *     s_t   = scale * sum_k q[b,i,k] * K[b,j,t,k]          t < L_b
 *     w_t   = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
 *     o[v]  = sum_t w_t * V[b,j,t,v]
 * Subtracting the maximum logit leaves the softmax unchanged mathematically
 * and keeps exp() finite; it is the one reading added to the pages' softmax.
 *
 * Element types: 0 = IEEE fp32, 1 = bf16 given as raw 16-bit patterns (the
 * upper half of an fp32). Both are widened to double exactly.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fused
 * multiply-add contraction, so every product and sum is one double rounding).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_GROUPS (-2)
#define ORC_ERR_UNSUPPORTED (-3)
#define ORC_ERR_CAPACITY (-4)

static size_t elem_size(int dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/* Exact widening of one stored element to double. */
static double widen(const void* base, size_t idx, int dtype) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * Cache element count for one model: 2 (K and V) x layers x KV heads x
 * length x head dimension [GQA-lesson, section on what shrinks and what
 * does not]. The query-head count does not appear.
 */
int64_t oracle_kv_cache_elems(int64_t layers, int64_t kv_heads, int64_t length,
                              int64_t head_dim) {
  return 2 * layers * kv_heads * length * head_dim;
}

/*
 * Bytes one token leaves in the cache: 2 x layers x KV heads x head dim x
 * bytes per element [LLM-inf-05, memory arithmetic under "more depth"].
 */
int64_t oracle_kv_bytes_per_token(int64_t layers, int64_t kv_heads,
                                  int64_t head_dim, int64_t elem_bytes) {
  return oracle_kv_cache_elems(layers, kv_heads, 1, head_dim) * elem_bytes;
}

/*
 * Append one token per sequence: the new key and value rows of every KV head
 * are stored at position lens[b] and the length grows by one
 * [MQA-review §2.4 and §3: the new row is concatenated on the position axis;
 * LLM-inf-05 decode pseudocode: push K, push V, then attend].
 *
 * Caches are [b][g][cap][d_k] and [b][g][cap][d_v]; k_new is [b][g][d_k] and
 * v_new is [b][g][d_v]; all in the same element type. The copy is of raw
 * bits. Returns ORC_ERR_CAPACITY (and changes nothing) if any
 * lens[b] is outside [0, cap).
 */
int oracle_kv_append(void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, int32_t* lens, int b, int g, int d_k,
                     int d_v, int cap, int dtype) {
  if (!k_cache || !v_cache || !k_new || !v_new || !lens) return ORC_ERR_ARG;
  if (b <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 || cap <= 0) return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  for (int s = 0; s < b; ++s)
    if (lens[s] < 0 || lens[s] >= cap) return ORC_ERR_CAPACITY;
  const size_t es = elem_size(dtype);
  char* kc = (char*)k_cache;
  char* vc = (char*)v_cache;
  for (int s = 0; s < b; ++s) {
    const size_t pos = (size_t)lens[s];
    for (int j = 0; j < g; ++j) {
      const size_t head = (size_t)s * g + j;
      memcpy(kc + ((head * cap + pos) * d_k) * es,
             (const char*)k_new + head * d_k * es, (size_t)d_k * es);
      memcpy(vc + ((head * cap + pos) * d_v) * es,
             (const char*)v_new + head * d_v * es, (size_t)d_v * es);
    }
    lens[s] = (int32_t)(pos + 1);
  }
  return ORC_OK;
}

/*
 * One decoding step of attention for every (sequence, query head).
 *
 * q is [b][h][d_k]; caches are [b][g][cap][d]; lens[b] is the number of
 * cached positions attended by sequence b (the token appended this step
 * included, [LLM-inf-05 decode description: the new position mixes all
 * earlier positions and itself]). out is [b][h][d_v] in double.
 *
 * Query head i reads KV head j = floor(i / (h/g)): query heads form contiguous
 * groups of h/g, which is the same as repeating each KV head h/g times along
 * the head axis [GQA-lesson, lab description; g-knob table]. h must be a
 * multiple of g [GQA-lesson, divisibility rule]; otherwise ORC_ERR_GROUPS.
 *
 * Per row: logits (k contraction of [MQA-review §2.1]), softmax, and the
 * weighted sum over positions (the v contraction of §2.1). A sequence with
 * lens[b] == 0 attends nothing and gets an all-zero output.
 *
 * weights (optional, may be NULL) receives w_t as [b][h][cap] (entries
 * t >= lens[b] are set to 0). mul_count (optional) receives the number of
 * multiplications performed by the two contractions, counted as they happen
 * (the scale multiply and the softmax are not counted, following the
 * per-term multiplication counts of [GQA-lesson]).
 *
 * threads: OpenMP threads over the independent (b, i) rows (<= 0: default).
 */
int oracle_decode_attention(double* out, double* weights, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* lens, int b, int h, int g, int d_k,
                            int d_v, int cap, float scale, int dtype,
                            int64_t* mul_count, int threads) {
  if (!out || !q || !k_cache || !v_cache || !lens) return ORC_ERR_ARG;
  if (b <= 0 || h <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 || cap <= 0)
    return ORC_ERR_ARG;
  if (h % g != 0) return ORC_ERR_GROUPS;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  for (int s = 0; s < b; ++s)
    if (lens[s] < 0 || lens[s] > cap) return ORC_ERR_CAPACITY;

  const int G = h / g;
  const double dscale = (double)scale;
  const long rows = (long)b * h;
  int64_t muls = 0;
  int failed = 0;
  const int nthreads = threads > 0 ? threads : omp_get_max_threads();

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(+ : muls) reduction(| : failed)
  for (long r = 0; r < rows; ++r) {
    const int s = (int)(r / h);
    const int i = (int)(r % h);
    const int j = i / G;
    const int L = lens[s];
    double* o = out + (size_t)r * d_v;
    double* wrow = weights ? weights + (size_t)r * cap : NULL;
    for (int v = 0; v < d_v; ++v) o[v] = 0.0;
    if (wrow)
      for (int t = 0; t < cap; ++t) wrow[t] = 0.0;
    if (L == 0) continue;

    double* logit = (double*)malloc(sizeof(double) * (size_t)L);
    if (!logit) {
      failed = 1;
      continue;
    }
    const size_t qoff = (size_t)r * d_k;
    const size_t kvhead = (size_t)s * g + j;

    /* logits: contraction over the key dimension, in index order */
    for (int t = 0; t < L; ++t) {
      const size_t krow = (kvhead * cap + t) * d_k;
      double acc = 0.0;
      for (int k = 0; k < d_k; ++k) {
        acc += widen(q, qoff + k, dtype) * widen(k_cache, krow + k, dtype);
        muls += 1;
      }
      logit[t] = dscale * acc;
    }

    /* softmax over positions, max-subtracted */
    double mx = logit[0];
    for (int t = 1; t < L; ++t)
      if (logit[t] > mx) mx = logit[t];
    double z = 0.0;
    for (int t = 0; t < L; ++t) {
      logit[t] = exp(logit[t] - mx);
      z += logit[t];
    }
    for (int t = 0; t < L; ++t) logit[t] = logit[t] / z;
    if (wrow)
      for (int t = 0; t < L; ++t) wrow[t] = logit[t];

    /* weighted sum of value rows, in position order */
    for (int t = 0; t < L; ++t) {
      const size_t vrow = (kvhead * cap + t) * d_v;
      for (int v = 0; v < d_v; ++v) {
        o[v] += logit[t] * widen(v_cache, vrow + v, dtype);
        muls += 1;
      }
    }
    free(logit);
  }
  if (mul_count) *mul_count = muls;
  return failed ? ORC_ERR_ARG : ORC_OK;
}

/*
 * The same attention computed over a split of every sequence's positions
 * into consecutive chunks: each chunk's state is computed on its own (m =
 * its largest logit, l = sum over its positions of exp(s_t - m), o[v] = sum
 * of exp(s_t - m) V[t][v]) and the states are combined with M = max_c m_c:
 *   out[v] = sum_c exp(m_c - M) o_c[v] / sum_c exp(m_c - M) l_c.
 * This is the softmax of [MQA-review §2.1] written over a union of position
 * sets (a chunk with no positions is skipped); it equals the direct form in
 * exact arithmetic and is the split-and-merge a split-K schedule performs.
 * bounds is [b][n_chunks + 1]: chunk c of sequence s covers positions
 * [bounds[s][c], bounds[s][c + 1]), with bounds[s][0] = 0, non-decreasing,
 * and bounds[s][n_chunks] = lens[s] (ORC_ERR_ARG otherwise). Logits and
 * sums run in index order within a chunk, chunks in order.
 */
int oracle_decode_attention_chunked(double* out, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* lens, const int32_t* bounds, int n_chunks, int b, int h,
                                    int g, int d_k, int d_v, int cap, float scale, int dtype, int threads) {
  if (!out || !q || !k_cache || !v_cache || !lens || !bounds || n_chunks <= 0) return ORC_ERR_ARG;
  if (b <= 0 || h <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 || cap <= 0) return ORC_ERR_ARG;
  if (h % g != 0) return ORC_ERR_GROUPS;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  for (int s = 0; s < b; ++s) {
    if (lens[s] < 0 || lens[s] > cap) return ORC_ERR_CAPACITY;
    const int32_t* bs = bounds + (size_t)s * (n_chunks + 1);
    if (bs[0] != 0 || bs[n_chunks] != lens[s]) return ORC_ERR_ARG;
    for (int c = 0; c < n_chunks; ++c)
      if (bs[c + 1] < bs[c]) return ORC_ERR_ARG;
  }
  const int G = h / g;
  const double dscale = (double)scale;
  const long rows = (long)b * h;
  int failed = 0;
  const int nthreads = threads > 0 ? threads : omp_get_max_threads();

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
  for (long r = 0; r < rows; ++r) {
    const int s = (int)(r / h);
    const int i = (int)(r % h);
    const int j = i / G;
    const int32_t* bs = bounds + (size_t)s * (n_chunks + 1);
    double* o = out + (size_t)r * d_v;
    for (int v = 0; v < d_v; ++v) o[v] = 0.0;
    if (lens[s] == 0) continue;
    double* cm = (double*)malloc(sizeof(double) * (size_t)n_chunks);
    double* cl = (double*)malloc(sizeof(double) * (size_t)n_chunks);
    double* co = (double*)malloc(sizeof(double) * (size_t)n_chunks * d_v);
    if (!cm || !cl || !co) {
      free(cm);
      free(cl);
      free(co);
      failed = 1;
      continue;
    }
    const size_t qoff = (size_t)r * d_k;
    const size_t kvhead = (size_t)s * g + j;
    /* each chunk on its own */
    for (int c = 0; c < n_chunks; ++c) {
      double* oc = co + (size_t)c * d_v;
      for (int v = 0; v < d_v; ++v) oc[v] = 0.0;
      cl[c] = 0.0;
      cm[c] = 0.0;
      const int t0 = bs[c], t1 = bs[c + 1];
      if (t1 == t0) continue;
      double* logit = (double*)malloc(sizeof(double) * (size_t)(t1 - t0));
      if (!logit) {
        failed = 1;
        continue;
      }
      for (int t = t0; t < t1; ++t) {
        const size_t krow = (kvhead * cap + t) * d_k;
        double acc = 0.0;
        for (int k = 0; k < d_k; ++k) acc += widen(q, qoff + k, dtype) * widen(k_cache, krow + k, dtype);
        logit[t - t0] = dscale * acc;
      }
      double mx = logit[0];
      for (int t = 1; t < t1 - t0; ++t)
        if (logit[t] > mx) mx = logit[t];
      cm[c] = mx;
      for (int t = t0; t < t1; ++t) {
        const double e = exp(logit[t - t0] - mx);
        cl[c] += e;
        const size_t vrow = (kvhead * cap + t) * d_v;
        for (int v = 0; v < d_v; ++v) oc[v] += e * widen(v_cache, vrow + v, dtype);
      }
      free(logit);
    }
    /* combine the chunks' states */
    double M = 0.0;
    int any = 0;
    for (int c = 0; c < n_chunks; ++c)
      if (bs[c + 1] > bs[c] && (!any || cm[c] > M)) {
        M = cm[c];
        any = 1;
      }
    double den = 0.0;
    for (int c = 0; c < n_chunks; ++c) {
      if (bs[c + 1] == bs[c]) continue;
      const double wgt = exp(cm[c] - M);
      den += wgt * cl[c];
      for (int v = 0; v < d_v; ++v) o[v] += wgt * co[(size_t)c * d_v + v];
    }
    for (int v = 0; v < d_v; ++v) o[v] /= den;
    free(cm);
    free(cl);
    free(co);
  }
  return failed ? ORC_ERR_ARG : ORC_OK;
}

/*
 * A projection of the new token's vector by a weight matrix
 * [MQA-review §2.4: q = x P_q, k = x P_k, v = x P_v for the incremental step,
 * and y = o P_o after the attention; §3: P_k and P_v lose the head axis for
 * MQA]. The matrix is given output-major: w[o][k] is the weight from input
 * feature k to output feature o, so
 *   y[r][o] = sum_k x[r][k] * w[o][k]      r < rows, o < n_out,
 * with the sum over k in index order. x, w in the element type dtype; y in
 * double.
 */
int oracle_linear(double* y, const void* x, const void* w, int rows, int n_in, int n_out, int dtype) {
  if (!y || !x || !w || rows <= 0 || n_in <= 0 || n_out <= 0) return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < rows; ++r) {
    for (int o = 0; o < n_out; ++o) {
      double acc = 0.0;
      for (int k = 0; k < n_in; ++k)
        acc += widen(x, (size_t)r * n_in + k, dtype) * widen(w, (size_t)o * n_in + k, dtype);
      y[(size_t)r * n_out + o] = acc;
    }
  }
  return ORC_OK;
}

/*
 * A double rounded once to bf16 (8 significant bits, fp32's exponent range,
 * subnormals down to 2^-133), nearest even; returned as the bf16 bit pattern.
 * The value is scaled by a power of two so that its last kept bit is the
 * units place, rounded to an integer by nearbyint (the default rounding
 * mode, nearest even), and scaled back; both scalings are exact.
 */
static uint16_t double_to_bf16(double x) {
  if (isnan(x)) return (uint16_t)0x7fc0u;
  const uint16_t sign = signbit(x) ? (uint16_t)0x8000u : (uint16_t)0u;
  const double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int lsb = e - 8;
  if (lsb < -133) lsb = -133;
  const double v = ldexp(nearbyint(ldexp(a, -lsb)), lsb);
  if (v >= 0x1p128) return (uint16_t)(sign | 0x7f80u);
  const float f = (float)v; /* exact: at most 8 significant bits, in fp32's range */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (u >> 16));
}

/*
 * Store doubles in an element type, each rounded once to the nearest value of
 * that type (ties to even; a NaN stays a NaN): fp32 by the C conversion,
 * bf16 by double_to_bf16. Used where a value the step produces is held in
 * the activation type before the next operation reads it.
 */
void oracle_store(void* dst, const double* src, size_t n, int dtype) {
  for (size_t i = 0; i < n; ++i) {
    if (dtype == ORC_F32) ((float*)dst)[i] = (float)src[i];
    else ((uint16_t*)dst)[i] = double_to_bf16(src[i]);
  }
}

/*
 * Mean-fold of KV heads: turn a cache (or a key/value projection) with g_src
 * KV heads into one with g_dst heads by averaging each contiguous group of
 * F = g_src / g_dst heads [GQA-lesson, on merging the groups of a trained
 * multi-head model: the KV heads of a group are averaged, and the lab folds
 * the KV heads of contiguous groups by their mean]:
 *   dst[b][j][t][c] = (sum_{f<F} src[b][j*F + f][t][c]) / F
 * for t < rows_b and c < d, the sum in head order in double, the quotient
 * rounded once to the element type (nearest even). rows_b = lens[b] when
 * lens is given, else max_rows for every b. Rows of dst from rows_b on are
 * not written. src is [b][g_src][cap_src][d], dst is [b][g_dst][cap_dst][d].
 * A projection matrix [g*d_k][d_model] is the case b = 1, cap = d_k, d =
 * d_model, lens = NULL, max_rows = d_k.
 */
int oracle_fold_heads(void* dst, const void* src, const int32_t* lens, int b, int g_src, int g_dst, int cap_src,
                      int cap_dst, int d, int max_rows, int dtype) {
  if (!dst || !src || b <= 0 || g_src <= 0 || g_dst <= 0 || cap_src <= 0 || cap_dst <= 0 || d <= 0 ||
      max_rows < 0)
    return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  if (g_src % g_dst != 0) return ORC_ERR_GROUPS;
  if (max_rows > cap_src || max_rows > cap_dst) return ORC_ERR_CAPACITY;
  if (lens)
    for (int s = 0; s < b; ++s)
      if (lens[s] < 0 || lens[s] > max_rows) return ORC_ERR_CAPACITY;
  const int F = g_src / g_dst;
#pragma omp parallel for collapse(2) schedule(static)
  for (int s = 0; s < b; ++s) {
    for (int j = 0; j < g_dst; ++j) {
      const int rows = lens ? lens[s] : max_rows;
      for (int t = 0; t < rows; ++t) {
        for (int c = 0; c < d; ++c) {
          double sum = 0.0;
          for (int f = 0; f < F; ++f)
            sum += widen(src, (((size_t)s * g_src + (size_t)j * F + f) * cap_src + t) * d + c, dtype);
          const double mean = sum / F;
          const size_t o = (((size_t)s * g_dst + j) * cap_dst + t) * d + c;
          if (dtype == ORC_F32) ((float*)dst)[o] = (float)mean;
          else ((uint16_t*)dst)[o] = double_to_bf16(mean);
        }
      }
    }
  }
  return ORC_OK;
}

/* double_to_bf16 over an array (for its own pins). */
void oracle_round_bf16(uint16_t* dst, const double* src, size_t n) {
  for (size_t i = 0; i < n; ++i) dst[i] = double_to_bf16(src[i]);
}

/*
 * Paged caches. The pages name block-table caches (the "LLM inference 05"
 * notes point to vLLM's paged cache) but give no layout; the plain reading
 * taken here: a pool of blocks of B positions, pool[n][j][r][c] holding row r
 * of KV head j in block n, and a table [b][max_blocks] naming, for sequence
 * s, the block of positions n*B .. n*B + B - 1. A paged cache stands for the
 * contiguous cache whose row t of head j is pool[table[s][t / B]][j][t % B];
 * attention over it is the attention above over that cache.
 */

/*
 * Gather the rows t < lens[s] of every sequence from a pool into a
 * contiguous cache dst [b][g][cap][d] (rows from lens[s] on are not
 * written). ORC_ERR_ARG if a table entry needed is outside [0, num_blocks),
 * ORC_ERR_CAPACITY if a length exceeds cap or max_blocks * B.
 */
int oracle_gather_paged(void* dst, const void* pool, const int32_t* table, const int32_t* lens, int b, int g,
                        int block_size, int max_blocks, int num_blocks, int cap, int d, int dtype) {
  if (!dst || !pool || !table || !lens || b <= 0 || g <= 0 || block_size <= 0 || max_blocks <= 0 ||
      num_blocks <= 0 || cap <= 0 || d <= 0)
    return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  const size_t es = elem_size(dtype);
  for (int s = 0; s < b; ++s) {
    const int L = lens[s];
    if (L < 0 || L > cap || (int64_t)L > (int64_t)max_blocks * block_size) return ORC_ERR_CAPACITY;
    for (int t = 0; t < L; ++t) {
      const int blk = table[(size_t)s * max_blocks + t / block_size];
      if (blk < 0 || blk >= num_blocks) return ORC_ERR_ARG;
    }
  }
  for (int s = 0; s < b; ++s)
    for (int j = 0; j < g; ++j)
      for (int t = 0; t < lens[s]; ++t) {
        const int blk = table[(size_t)s * max_blocks + t / block_size];
        const size_t src_row = ((size_t)blk * g + j) * block_size + t % block_size;
        const size_t dst_row = ((size_t)s * g + j) * cap + t;
        memcpy((char*)dst + dst_row * d * es, (const char*)pool + src_row * d * es, d * es);
      }
  return ORC_OK;
}

/*
 * Append to a paged cache: the new rows of sequence s go to position lens[s]
 * (row lens[s] % B of block table[s][lens[s] / B]) and the length grows by
 * one [MQA-review §2.4; LLM-inf-05 decode pseudocode]. ORC_ERR_CAPACITY (and
 * nothing changed) if a length is outside [0, max_blocks * B), ORC_ERR_ARG if
 * the block it needs is outside the pool.
 */
int oracle_kv_append_paged(void* k_pool, void* v_pool, const void* k_new, const void* v_new, int32_t* lens,
                           const int32_t* table, int b, int g, int d_k, int d_v, int block_size, int max_blocks,
                           int num_blocks, int dtype) {
  if (!k_pool || !v_pool || !k_new || !v_new || !lens || !table || b <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 ||
      block_size <= 0 || max_blocks <= 0 || num_blocks <= 0)
    return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  const size_t es = elem_size(dtype);
  for (int s = 0; s < b; ++s) {
    if (lens[s] < 0 || (int64_t)lens[s] >= (int64_t)max_blocks * block_size) return ORC_ERR_CAPACITY;
    const int blk = table[(size_t)s * max_blocks + lens[s] / block_size];
    if (blk < 0 || blk >= num_blocks) return ORC_ERR_ARG;
  }
  for (int s = 0; s < b; ++s) {
    const int p = lens[s];
    const int blk = table[(size_t)s * max_blocks + p / block_size];
    for (int j = 0; j < g; ++j) {
      const size_t row = ((size_t)blk * g + j) * block_size + p % block_size;
      memcpy((char*)k_pool + row * d_k * es, (const char*)k_new + ((size_t)s * g + j) * d_k * es, d_k * es);
      memcpy((char*)v_pool + row * d_v * es, (const char*)v_new + ((size_t)s * g + j) * d_v * es, d_v * es);
    }
    lens[s] = p + 1;
  }
  return ORC_OK;
}

/*
 * Append n new tokens per sequence: token r's key and value rows go to
 * position lens[s] + r, then the length grows by n [MQA-review §2.3, the
 * batched form that processes n positions of a sequence in one step; §2.4
 * for the concatenation on the position axis]. k_new is [b][n][g][d_k],
 * v_new [b][n][g][d_v]. ORC_ERR_CAPACITY (and nothing changed) if some
 * lens[s] + n exceeds cap or a length is negative.
 */
int oracle_kv_append_multi(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t* lens, int b,
                           int n, int g, int d_k, int d_v, int cap, int dtype) {
  if (!k_cache || !v_cache || !k_new || !v_new || !lens || b <= 0 || n <= 0 || g <= 0 || d_k <= 0 || d_v <= 0 ||
      cap <= 0)
    return ORC_ERR_ARG;
  if (dtype != ORC_F32 && dtype != ORC_BF16) return ORC_ERR_UNSUPPORTED;
  for (int s = 0; s < b; ++s)
    if (lens[s] < 0 || (int64_t)lens[s] + n > cap) return ORC_ERR_CAPACITY;
  const size_t es = elem_size(dtype);
  for (int s = 0; s < b; ++s) {
    for (int r = 0; r < n; ++r) {
      const int pos = lens[s] + r;
      for (int j = 0; j < g; ++j) {
        const size_t src = (((size_t)s * n + r) * g + j);
        const size_t dst = ((size_t)s * g + j) * cap + pos;
        memcpy((char*)k_cache + dst * d_k * es, (const char*)k_new + src * d_k * es, d_k * es);
        memcpy((char*)v_cache + dst * d_v * es, (const char*)v_new + src * d_v * es, d_v * es);
      }
    }
    lens[s] += n;
  }
  return ORC_OK;
}

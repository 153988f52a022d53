/*
 * CPU oracle for MLA decode over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path (the HIP library)
 * neither links nor calls it, and shares no code with it.
 *
 * What it computes (the plain definition, in float64):
 *   The running example of the TileLang notes ("TileLang: bridging programmability
 *   and performance in modern neural kernels", section "A complete example:
 *   two-stage optimisation of FlashMLA") is MLA decoding as two chained GEMMs:
 *   S = Q . KV^T, then O = softmax(S) . KV restricted to the value columns.
 *   The pages do not write out MLA's mathematics; the problem statement the
 *   library implements fixes the rest:
 *     - one latent KV row per cached token, D_QK = 576 wide (512 latent + 64 rope),
 *       shared by all query heads; its first D_V = 512 dims are the value row;
 *     - rows are stored in pages of PAGE tokens, block_table[b][j] names the
 *       page holding tokens [j*PAGE, (j+1)*PAGE) of sequence b;
 *     - cache_seqlens[b] counts every cached token of sequence b, including the
 *       q_len new ones; with causal masking query t sees positions
 *       p <= cache_seqlens[b] - q_len + t;
 *     - scores are scale * (q . k) over all 576 dims; the softmax is exact;
 *     - lse is the natural log of sum_p exp(score_p).
 *   For each output row this file gathers the visible keys, forms every score
 *   with a naive loop, takes the maximum (pass 1), then the shifted exponentials,
 *   their sum and the weighted sum of value rows (pass 2), and divides.
 *   No blocking, no online rescaling, no reordering beyond that.
 *
 * Precision: inputs (float32 or bf16 bit patterns) are widened exactly to double;
 * all arithmetic is double.  Built without -ffast-math (the V4 note on precision
 * and bitwise alignment asks for IEEE behaviour by default).
 *
 * Degenerate rows: a row with no visible key gets out = 0 and lse = -inf.
 *
 * Attention sinks (optional).  The TileLang notes list an attention-sink variant of
 * MHA a few lines away from the standard kernel (main results table and the
 * programmability remarks after it) without writing it out.  Reading taken: head h
 * has one sink logit sigma_h that takes part in the softmax like an extra key with
 * score sigma_h (already in score units: not multiplied by `scale`) and a value row
 * of zeros.  So, with the sink, the weights are exp(s_p) / (exp(sigma_h) +
 * sum_q exp(s_q)), out is their sum over the real value rows, and lse is the natural
 * log of that whole denominator.  A row with no visible key then gets out = 0 and
 * lse = sigma_h; sigma_h = -inf is the plain decode.
 *
 * Sparse (top-k) decode (optional).  The DeepSeek-V4 TileLang note mentions the
 * dynamic sparse attention of DeepSeek models (TileLang's limits on it) without the
 * details.  Reading taken: each (b, t) has a list of topk logical token positions of
 * sequence b, shared by all heads, with -1 marking an unused entry; the row attends to
 * exactly the listed tokens, once per entry, in place of its causal range.  An entry
 * below -1 or at or past cache_seqlens[b] is an input fault (ORACLE_ERR_PAGE).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_PAGE 2     /* a visible token maps to a page outside the pool */
#define ORACLE_ERR_ALLOC 3

/* dtype codes: 0 = float32 values, 1 = bf16 bit patterns (uint16) */
static double load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Visible keys for query t of a sequence holding `seqlen` tokens. */
static int64_t visible(int64_t seqlen, int32_t q_len, int32_t t, int32_t causal) {
  int64_t n = seqlen;
  if (causal && q_len > 1) n = seqlen - q_len + 1 + t;
  return n < 0 ? 0 : n;
}

/*
 * Decode the requested rows.
 *   sinks        per-head sink logits [heads] (double), or NULL for none
 *   indices      sparse token lists [batch, q_len, topk] int32, or NULL (dense); needs causal 0
 *   q            [batch, q_len, heads, d_qk]           (dtype)
 *   kv           [num_pages, page, d_qk]               (dtype)
 *   block_table  int32, row b at block_table + b*bt_stride
 *   rows         flat row ids r = (b*q_len + t)*heads + h, or NULL for all rows in order
 *   out          [n_rows, d_v] double,  lse [n_rows] double
 *   n_threads    <= 0: OpenMP default
 * Returns ORACLE_OK or an error code (nothing is written past the first bad row's slot).
 */
int mla_oracle_decode(const void* q, const void* kv, int32_t dtype,
                      const int32_t* block_table, int64_t bt_stride,
                      const int32_t* cache_seqlens,
                      int32_t batch, int32_t q_len, int32_t heads,
                      int64_t num_pages, int32_t page, int32_t d_qk, int32_t d_v,
                      int32_t causal, double scale, const double* sinks,
                      const int32_t* indices, int32_t topk,
                      const int64_t* rows, int64_t n_rows,
                      double* out, double* lse, int32_t n_threads) {
  if (!q || !kv || !block_table || !cache_seqlens || !out || !lse) return ORACLE_ERR_ARG;
  if (dtype != 0 && dtype != 1) return ORACLE_ERR_ARG;
  if (batch < 0 || q_len < 1 || heads < 1 || page < 1 || d_v < 1 || d_v > d_qk) return ORACLE_ERR_ARG;
  if (indices && (topk < 1 || causal)) return ORACLE_ERR_ARG;
  const int64_t total_rows = (int64_t)batch * q_len * heads;
  if (rows == NULL) n_rows = total_rows;
  int err = ORACLE_OK;
#ifdef _OPENMP
  const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#else
  const int nt = 1;
  (void)n_threads;
#endif

#pragma omp parallel num_threads(nt)
  {
    /* per-thread scratch: scores of one row, and its gathered key positions */
    int64_t max_tokens = 0;
    for (int32_t b = 0; b < batch; ++b)
      if (cache_seqlens[b] > max_tokens) max_tokens = cache_seqlens[b];
    if (indices && topk > max_tokens) max_tokens = topk;
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_tokens > 0 ? max_tokens : 1));
    int64_t* kbase = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_tokens > 0 ? max_tokens : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)d_v);
    if (!s || !kbase || !acc) {
#pragma omp atomic write
      err = ORACLE_ERR_ALLOC;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      int seen;
#pragma omp atomic read
      seen = err;
      if (seen != ORACLE_OK) continue;
      const int64_t r = rows ? rows[i] : i;
      if (r < 0 || r >= total_rows) {
#pragma omp atomic write
        err = ORACLE_ERR_ARG;
        continue;
      }
      const int32_t b = (int32_t)(r / ((int64_t)q_len * heads));
      const int32_t t = (int32_t)((r / heads) % q_len);
      const int32_t h = (int32_t)(r % heads);
      const double sink = sinks ? sinks[h] : -INFINITY;
      const int has_sink = sink > -INFINITY || isnan(sink);
      int64_t n = visible(cache_seqlens[b], q_len, t, causal);
      double* o = out + i * d_v;

      /* gather: element offset of each visible key row inside kv (dense: positions
         0 .. n-1; sparse: the listed positions, in list order) */
      int bad = 0;
      const int32_t* list = indices ? indices + ((int64_t)b * q_len + t) * topk : NULL;
      if (list) {
        n = 0;
        for (int32_t k = 0; k < topk && !bad; ++k) {
          const int64_t p = list[k];
          if (p == -1) continue;
          if (p < 0 || p >= cache_seqlens[b]) { bad = 1; break; }
          const int64_t pg = block_table[b * bt_stride + p / page];
          if (pg < 0 || pg >= num_pages) { bad = 1; break; }
          kbase[n++] = (pg * page + p % page) * (int64_t)d_qk;
        }
      }
      for (int64_t p = 0; p < n && !list; ++p) {
        const int64_t pg = block_table[b * bt_stride + p / page];
        if (pg < 0 || pg >= num_pages) { bad = 1; break; }
        kbase[p] = (pg * page + p % page) * (int64_t)d_qk;
      }
      if (bad) {
#pragma omp atomic write
        err = ORACLE_ERR_PAGE;
        continue;
      }
      if (n == 0 && !has_sink) {
        for (int32_t d = 0; d < d_v; ++d) o[d] = 0.0;
        lse[i] = -INFINITY;
        continue;
      }
      /* scores s_p = scale * sum_d q[d] k_p[d] */
      const int64_t qbase = r * (int64_t)d_qk;
      for (int64_t p = 0; p < n; ++p) {
        double dot = 0.0;
        for (int32_t d = 0; d < d_qk; ++d)
          dot += load_elem(q, dtype, qbase + d) * load_elem(kv, dtype, kbase[p] + d);
        s[p] = scale * dot;
      }
      /* pass 1: maximum score (the sink counts as one more score) */
      double m = has_sink ? sink : s[0];
      for (int64_t p = 0; p < n; ++p)
        if (s[p] > m) m = s[p];
      /* pass 2: shifted exponentials, their sum, and the weighted sum of value rows;
         the sink adds its exponential to the sum and nothing to the values */
      double l = has_sink ? exp(sink - m) : 0.0;
      for (int32_t d = 0; d < d_v; ++d) acc[d] = 0.0;
      for (int64_t p = 0; p < n; ++p) {
        const double w = exp(s[p] - m);
        l += w;
        for (int32_t d = 0; d < d_v; ++d) acc[d] += w * load_elem(kv, dtype, kbase[p] + d);
      }
      for (int32_t d = 0; d < d_v; ++d) o[d] = acc[d] / l;
      lse[i] = m + log(l);
    }
    free(s);
    free(kbase);
    free(acc);
  }
  return err;
}

/* Number of threads an OpenMP parallel region here would use (for reporting). */
int32_t mla_oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

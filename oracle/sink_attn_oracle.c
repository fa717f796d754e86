/*
 * Sink-attention oracle: a plain, slow fp64 CPU implementation of what the
 * GPU library computes.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load this file's library.
 * The product path never calls it and shares no code, header or constant
 * with it.
 *
 * What is computed (GPT-OSS on Day 0, Perplexity; section "Attention: GQA
 * with attention sinks" and section "Sink attention" under "Kernels for
 * GPT-OSS"):
 *
 *   Every query head h owns one pretrained scalar, its sink sigma_h, which
 *   takes part in that head's softmax.  The formula on the page was lost in
 *   extraction; the reading taken here is the plainest one that the rest of
 *   the section supports: the sink is one extra logit placed beside the
 *   scaled scores q.k_j of the row, the softmax runs over scores and sink
 *   together, and the sink's column carries no value vector:
 *
 *     z      = { tau * q.k_j : j in J }  U  { sigma_h }
 *     M      = max(z)
 *     Z      = exp(sigma_h - M) + sum_{j in J} exp(tau*q.k_j - M)
 *     o      = sum_{j in J} exp(tau*q.k_j - M) / Z * v_j
 *     lse    = M + ln Z                       (natural log)
 *
 *   A constant bias added to every score would cancel inside the softmax,
 *   so the sink must be its own column.  The section's online form (running
 *   maximum started at the sink, running denominator started at 1) is the
 *   same quantity: exp(sigma - m0) = 1 when m0 = sigma.
 *
 *   GQA (same section heading): query head h reads KV head g = h / G with
 *   G = Hq / Hkv (contiguous groups; a convention, the page names no map).
 *
 *   Allowed key set J for query t of request b, whose absolute position is
 *   p = kv_len[b] - qlen[b] + t (the new tokens are the last qlen of the
 *   kv_len keys):  causal -> j <= p;  non-causal -> every j < kv_len[b].
 *   A decode query (qlen 1) therefore sees all kv_len keys.
 *
 *   Draft (tree) mask ("Accelerating Sonar Through Speculation", Perplexity,
 *   section "EAGLE": tree-shaped drafts are checked with custom attention
 *   masks).  When draft_mask is given, the qlen new tokens of a request are
 *   its drafted tokens and the mask replaces causality among them: row t may
 *   see every prefix key j < P = kv_len - qlen, and drafted key P + i
 *   (i < qlen) exactly when bit i of draft_mask[row] is set.  Bits at or
 *   above qlen are ignored.  The causal flag is not consulted.
 *
 *   Split-KV (same section: work is parallelised along the KV length and
 *   the sink may enter only the first chunk): a partial restricts J to a
 *   key window and includes the sink only when asked; merging partials by
 *   their log-sum-exp recovers the unsplit row (sa_oracle_merge).
 *
 * Everything runs in three literal passes per (query row, head): scores and
 * their maximum, the exponential sum, the weighted value sum.  No online
 * rescaling, no tiling.  Inputs are bf16 bit patterns (the values the GPU
 * reads); each is widened exactly to double.
 *
 * Data layout of the buffers read here (the library's documented format):
 *   q            bf16 [total_q, Hq, D], request b owns rows
 *                qo_indptr[b] .. qo_indptr[b+1]
 *   contiguous   k, v bf16 [total_kv, Hkv, D], request b owns tokens
 *                kv_indptr[b] .. kv_indptr[b+1]
 *   paged        k, v bf16 [num_pages, Hkv, page_size, D]; request b's
 *                token j lives in page page_indices[kv_indptr[b] + j /
 *                page_size], slot j % page_size
 *   kv_len       [B] valid keys per request (NULL: contiguous indptr gap)
 *   sinks        fp32 [Hq], NULL means no sink (sigma = -inf)
 *   draft_mask   uint64 [total_q] or NULL (no draft mask)
 *   out          double [total_q, Hq, D];  lse double [total_q, Hq]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  const uint16_t* q;
  const int32_t* qo_indptr;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_indptr;
  const int32_t* page_indices;
  const int32_t* kv_len;
  const float* sinks;
  const uint64_t* draft_mask; /* [total_q] or NULL */
  int batch, hq, hkv, d, page_size, causal;
  double sm_scale;
  int64_t key_begin, key_end; /* key window [key_begin, key_end) */
  int include_sink;
} ctx_t;

static double bf16_to_double(uint16_t bits) {
  union { uint32_t u; float f; } x;
  x.u = ((uint32_t)bits) << 16;
  return (double)x.f;
}

static int64_t request_kv_len(const ctx_t* c, int b) {
  if (c->kv_len) return c->kv_len[b];
  return (int64_t)c->kv_indptr[b + 1] - c->kv_indptr[b];
}

/* Address of key/value row j of request b for KV head g (layout above). */
static int64_t kv_row_offset(const ctx_t* c, int b, int64_t j, int g) {
  if (!c->page_indices) {
    int64_t tok = (int64_t)c->kv_indptr[b] + j;
    return (tok * c->hkv + g) * c->d;
  }
  int64_t page = c->page_indices[(int64_t)c->kv_indptr[b] + j / c->page_size];
  int64_t slot = j % c->page_size;
  return ((page * c->hkv + g) * c->page_size + slot) * c->d;
}

/* Request that owns query row `row` (qo_indptr is non-decreasing). */
static int request_of_row(const ctx_t* c, int64_t row) {
  int lo = 0, hi = c->batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (c->qo_indptr[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* Allowed key range [j0, j1) of query row `row` of request b. */
static void key_range(const ctx_t* c, int b, int64_t row, int64_t* j0, int64_t* j1) {
  int64_t L = request_kv_len(c, b);
  int64_t qlen = (int64_t)c->qo_indptr[b + 1] - c->qo_indptr[b];
  int64_t t = row - c->qo_indptr[b];
  int64_t hi = L;
  if (c->causal && !c->draft_mask) {
    int64_t p = L - qlen + t;  /* absolute position of the query */
    hi = p + 1 < L ? p + 1 : L;
    if (hi < 0) hi = 0;
  }
  int64_t lo = 0;
  if (c->key_begin > lo) lo = c->key_begin;
  if (c->key_end < hi) hi = c->key_end;
  if (hi < lo) hi = lo;
  *j0 = lo;
  *j1 = hi;
}

/* Whether key j of request b is in the allowed set of row `row` beyond its
 * key range: only a draft mask removes keys inside [j0, j1). */
static int key_allowed(const ctx_t* c, int b, int64_t row, int64_t j) {
  if (!c->draft_mask) return 1;
  int64_t L = request_kv_len(c, b);
  int64_t qlen = (int64_t)c->qo_indptr[b + 1] - c->qo_indptr[b];
  int64_t i = j - (L - qlen); /* index among the drafted tokens */
  if (i < 0) return 1;        /* a prefix key */
  if (i >= qlen || i >= 64) return 0;
  return (int)((c->draft_mask[row] >> i) & 1u);
}

/*
 * One (query row, head): the definition above in three passes.
 * `scores` is caller scratch of at least (j1 - j0) doubles.
 * If `weights` is non-NULL it receives the softmax weight of every allowed
 * key (length j1 - j0) and *w_sink the sink's weight.
 */
static void one_row(const ctx_t* c, int64_t row, int h, double* scores,
                    double* o, double* lse, double* weights, double* w_sink) {
  const int D = c->d;
  const int G = c->hq / c->hkv;
  const int g = h / G;
  const int b = request_of_row(c, row);
  int64_t j0, j1;
  key_range(c, b, row, &j0, &j1);
  const uint16_t* qrow = c->q + (row * c->hq + h) * (int64_t)D;
  const double sigma = (c->include_sink && c->sinks) ? (double)c->sinks[h] : -INFINITY;

  /* pass 1: scaled scores and the maximum over scores and sink */
  double M = sigma;
  for (int64_t j = j0; j < j1; ++j) {
    if (!key_allowed(c, b, row, j)) { scores[j - j0] = -INFINITY; continue; }
    const uint16_t* krow = c->k + kv_row_offset(c, b, j, g);
    double dot = 0.0;
    for (int x = 0; x < D; ++x) dot += bf16_to_double(qrow[x]) * bf16_to_double(krow[x]);
    double s = c->sm_scale * dot;
    scores[j - j0] = s;
    if (s > M) M = s;
  }
  for (int x = 0; x < D; ++x) o[x] = 0.0;
  if (weights) for (int64_t j = j0; j < j1; ++j) weights[j - j0] = 0.0;
  if (w_sink) *w_sink = 0.0;

  if (M == -INFINITY) { /* no keys and no sink: empty softmax */
    *lse = -INFINITY;
    return;
  }
  if (M == INFINITY) {  /* an infinite sink takes all of the mass */
    *lse = INFINITY;
    if (w_sink) *w_sink = 1.0;
    return;
  }

  /* pass 2: the denominator, sink term included once */
  double Z = exp(sigma - M);
  for (int64_t j = j0; j < j1; ++j)
    if (scores[j - j0] != -INFINITY) Z += exp(scores[j - j0] - M);

  /* pass 3: weighted sum of values; the sink column has no value */
  for (int64_t j = j0; j < j1; ++j) {
    if (scores[j - j0] == -INFINITY) continue; /* a masked-out key */
    double p = exp(scores[j - j0] - M) / Z;
    if (weights) weights[j - j0] = p;
    const uint16_t* vrow = c->v + kv_row_offset(c, b, j, g);
    for (int x = 0; x < D; ++x) o[x] += p * bf16_to_double(vrow[x]);
  }
  if (w_sink) *w_sink = exp(sigma - M) / Z;
  *lse = M + log(Z);
}

static int64_t max_kv_len(const ctx_t* c) {
  int64_t m = 0;
  for (int b = 0; b < c->batch; ++b) {
    int64_t L = request_kv_len(c, b);
    if (L > m) m = L;
  }
  return m;
}

static int check_ctx(const ctx_t* c) {
  if (!c->q || !c->qo_indptr || !c->k || !c->v || !c->kv_indptr) return -1;
  if (c->batch < 1 || c->hq < 1 || c->hkv < 1 || c->d < 1) return -2;
  if (c->hq % c->hkv) return -3;
  if (c->page_indices && c->page_size < 1) return -4;
  if (c->page_indices && !c->kv_len) return -5;
  return 0;
}

/* Evaluate the rows listed in (rows[i], heads[i]), i < n; writes
 * out[i*D ...] and lse[i].  Returns 0, or a negative code on bad args. */
static int run_rows(const ctx_t* c, const int64_t* rows, const int32_t* heads,
                    int64_t n, double* out, double* lse, int nthreads) {
  int rc = check_ctx(c);
  if (rc) return rc;
  const int64_t Lmax = max_kv_len(c);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
      if (scores) one_row(c, rows[i], heads[i], scores, out + i * c->d, lse + i, NULL, NULL);
    }
    free(scores);
  }
  return failed ? -9 : 0;
}

#define CTX_ARGS                                                              \
  const uint16_t *q, const int32_t *qo_indptr, const uint16_t *k,             \
      const uint16_t *v, const int32_t *kv_indptr,                            \
      const int32_t *page_indices, const int32_t *kv_len, const float *sinks, \
      int batch, int hq, int hkv, int d, int page_size, double sm_scale,      \
      int causal, const uint64_t *draft_mask

#define CTX_INIT(c)                                                     \
  ctx_t c;                                                              \
  memset(&c, 0, sizeof c);                                              \
  c.q = q; c.qo_indptr = qo_indptr; c.k = k; c.v = v;                   \
  c.kv_indptr = kv_indptr; c.page_indices = page_indices;               \
  c.kv_len = kv_len; c.sinks = sinks; c.batch = batch; c.hq = hq;       \
  c.hkv = hkv; c.d = d; c.page_size = page_size; c.sm_scale = sm_scale; \
  c.causal = causal; c.draft_mask = draft_mask;                         \
  c.key_begin = 0; c.key_end = INT64_MAX;                               \
  c.include_sink = 1

/*
 * Partial attention over the key window [key_begin, key_end) intersected
 * with each row's allowed keys, with the sink included iff include_sink.
 * key_begin = 0, key_end = INT64_MAX, include_sink = 1 is the full method.
 * Every (row, head) of the batch is written: out [total_q, Hq, D],
 * lse [total_q, Hq].
 */
int sa_oracle_partial(CTX_ARGS, int64_t key_begin, int64_t key_end, int include_sink,
                      double* out, double* lse, int nthreads) {
  CTX_INIT(c);
  c.key_begin = key_begin;
  c.key_end = key_end;
  c.include_sink = include_sink;
  if (check_ctx(&c)) return check_ctx(&c);
  const int64_t total_q = qo_indptr[batch];
  const int64_t n = total_q * hq;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  int32_t* heads = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!rows || !heads) { free(rows); free(heads); return -9; }
  for (int64_t i = 0; i < n; ++i) { rows[i] = i / hq; heads[i] = (int32_t)(i % hq); }
  int rc = run_rows(&c, rows, heads, n, out, lse, nthreads);
  free(rows);
  free(heads);
  return rc;
}

/* The full method over every (row, head). */
int sa_oracle_attend(CTX_ARGS, double* out, double* lse, int nthreads) {
  return sa_oracle_partial(q, qo_indptr, k, v, kv_indptr, page_indices, kv_len, sinks,
                           batch, hq, hkv, d, page_size, sm_scale, causal, draft_mask,
                           0, INT64_MAX, 1, out, lse, nthreads);
}

/* The full method on a sample: (rows[i], heads[i]) for i < n.
 * out [n, D], lse [n]. */
int sa_oracle_attend_rows(CTX_ARGS, const int64_t* rows, const int32_t* heads, int64_t n,
                          double* out, double* lse, int nthreads) {
  CTX_INIT(c);
  return run_rows(&c, rows, heads, n, out, lse, nthreads);
}

/* Softmax weights of one (row, head): weights[j - j0] for allowed keys
 * j0 <= j < j1 (written to *j0_out, *j1_out) and the sink's weight. */
int sa_oracle_row_weights(CTX_ARGS, int64_t row, int h, double* weights, double* w_sink,
                          int64_t* j0_out, int64_t* j1_out, double* o, double* lse) {
  CTX_INIT(c);
  int rc = check_ctx(&c);
  if (rc) return rc;
  int b = request_of_row(&c, row);
  key_range(&c, b, row, j0_out, j1_out);
  int64_t len = *j1_out - *j0_out;
  double* scores = (double*)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
  if (!scores) return -9;
  one_row(&c, row, h, scores, o, lse, weights, w_sink);
  free(scores);
  return 0;
}

/*
 * Merge of split-KV partials by their log-sum-exp (the same section
 * parallelises along the KV length and requires the sink to sit in one
 * chunk only; the rule that recombines the chunks is the standard one):
 *   L   = max_c lse_c
 *   w_c = exp(lse_c - L)
 *   o   = sum_c w_c o_c / sum_c w_c ;  lse = L + ln sum_c w_c
 * Each partial o_c is already normalised by its own denominator.  All
 * chunks empty (L = -inf) gives o = 0, lse = -inf; a chunk at +inf (an
 * infinite sink) takes all of the weight.
 * o_parts [N, H, S, D], lse_parts [N, H, S]; out [N, H, D], lse [N, H].
 */
int sa_oracle_merge(const double* o_parts, const double* lse_parts, int64_t n_rows,
                    int heads, int splits, int d, double* out, double* lse) {
  if (!o_parts || !lse_parts || !out || !lse) return -1;
  if (n_rows < 0 || heads < 1 || splits < 1 || d < 1) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows * heads; ++i) {
    const double* ls = lse_parts + i * splits;
    const double* os = o_parts + i * splits * (int64_t)d;
    double* o = out + i * d;
    double L = -INFINITY;
    for (int s = 0; s < splits; ++s) if (ls[s] > L) L = ls[s];
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    if (L == -INFINITY) { lse[i] = -INFINITY; continue; }
    double W = 0.0;
    for (int s = 0; s < splits; ++s) {
      double w;
      if (L == INFINITY) w = (ls[s] == INFINITY) ? 1.0 : 0.0;
      else w = exp(ls[s] - L);
      W += w;
      for (int x = 0; x < d; ++x) o[x] += w * os[s * (int64_t)d + x];
    }
    for (int x = 0; x < d; ++x) o[x] /= W;
    lse[i] = (L == INFINITY) ? INFINITY : L + log(W);
  }
  return 0;
}

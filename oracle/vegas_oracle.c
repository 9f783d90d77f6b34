/*
 * vegas_oracle.c -- plain, slow, fp64 CPU oracle for the attention work of one
 * decode iteration of Vegas ("Vegas: Self-Speculative Decoding with
 * Verification-Guided Sparse Attention", technical summary pages).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (each function cites the passage it follows):
 *   oracle_verify     full causal attention of the gamma+1 verify rows over the
 *                     whole cache; exports the pre-softmax logits of the first
 *                     draft row (row 0) and of the bonus row (row gamma).
 *   oracle_aggregate  one score per prefix position: the sum of the exported
 *                     logits over the exported rows and all query heads.
 *   oracle_topk       the k-subset of prefix positions maximising the summed
 *                     score (exactly the k largest scores, because the
 *                     objective is additive over positions).
 *   oracle_sparse     attention of the draft rows restricted to the selected
 *                     positions plus the causal tail after the prefix.
 *
 * Arithmetic is fp64 throughout.  Inputs are read exactly: bf16 values are
 * widened bit-for-bit (a bf16 is the top 16 bits of an IEEE binary32), f32
 * values are converted to double.  Loops run in logical-position order, so
 * the result does not depend on how pages are placed in memory.
 *
 * Layouts (row-major):
 *   q          [B][nrows][Hq][D]            dtype 0 = f32, 1 = bf16 bits
 *   k_cache    [num_slots][Hkv][D]           slot = page_table[b][pos/ps]*ps + pos%ps
 *   v_cache    [num_slots][Hkv][D]
 *   page_table [B][max_pages] int32
 * Query head h reads KV head h / (Hq/Hkv) (consecutive query heads share a KV head).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* ------------------------------------------------------------------ helpers */

static double load_elem(const void *base, int dtype, size_t idx) {
  if (dtype == 1) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* Logical position -> physical slot of a page-size-`ps` paged cache.  The
 * Implementation section of the pages passes token indices as page indices of
 * a page-size-1 PagedAttention call; a slot is exactly such a page-size-1
 * index into the cache viewed as [num_slots][Hkv][D]. */
static long long slot_of(const int32_t *page_table, int max_pages, int ps, int b, long long pos) {
  int32_t page = page_table[(size_t)b * max_pages + (size_t)(pos / ps)];
  if (page < 0) return -1;
  return (long long)page * ps + pos % ps;
}

typedef struct {
  int nunits;
  void *(*fn)(void *, int);
  void *ctx;
  int nthreads;
  int next;
  pthread_mutex_t mu;
  int err;
} pool_t;

typedef struct {
  pool_t *pool;
} worker_arg;

static void *pool_worker(void *p) {
  pool_t *pool = ((worker_arg *)p)->pool;
  for (;;) {
    pthread_mutex_lock(&pool->mu);
    int u = pool->next++;
    pthread_mutex_unlock(&pool->mu);
    if (u >= pool->nunits) break;
    if (pool->fn(pool->ctx, u) != NULL) {
      pthread_mutex_lock(&pool->mu);
      pool->err = 1;
      pthread_mutex_unlock(&pool->mu);
    }
  }
  return NULL;
}

/* Run fn(ctx, u) for u in [0, nunits) on up to nthreads threads (0 = all cores). */
static int run_units(int nunits, void *(*fn)(void *, int), void *ctx, int nthreads) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > nunits) nthreads = nunits;
  if (nthreads < 1) nthreads = 1;
  pool_t pool = {nunits, fn, ctx, nthreads, 0, PTHREAD_MUTEX_INITIALIZER, 0};
  worker_arg wa = {&pool};
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return ORACLE_ENOMEM;
  int started = 0;
  for (int t = 0; t < nthreads - 1; ++t)
    if (pthread_create(&th[started], NULL, pool_worker, &wa) == 0) ++started;
  pool_worker(&wa);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  return pool.err ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_num_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* Softmax-weighted sum over an explicit list of logical key positions.
 * logits[i] = scale * q . K[pos[i]]; p_i = exp(l_i - max l) / sum_i exp(l_i - max l);
 * out = sum_i p_i V[pos[i]].  Writes the n logits to `l` (caller-sized). */
static int attend(const double *q, int D, int dtype, double scale, const void *k_cache,
                  const void *v_cache, int Hkv, int g, const long long *slots, long long n,
                  double *l, double *out) {
  if (n <= 0) return ORACLE_EINVAL;
  for (long long i = 0; i < n; ++i) {
    if (slots[i] < 0) return ORACLE_EINVAL;
    size_t base = ((size_t)slots[i] * (size_t)Hkv + (size_t)g) * (size_t)D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * load_elem(k_cache, dtype, base + (size_t)d);
    l[i] = scale * dot;
  }
  double m = l[0];
  for (long long i = 1; i < n; ++i)
    if (l[i] > m) m = l[i];
  double z = 0.0;
  for (long long i = 0; i < n; ++i) z += exp(l[i] - m);
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (long long i = 0; i < n; ++i) {
    double p = exp(l[i] - m) / z;
    size_t base = ((size_t)slots[i] * (size_t)Hkv + (size_t)g) * (size_t)D;
    for (int d = 0; d < D; ++d) out[d] += p * load_elem(v_cache, dtype, base + (size_t)d);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ verify */

typedef struct {
  int B, Hq, Hkv, D, ps, max_pages, dtype, gamma, max_prefix;
  double scale;
  const void *q, *k_cache, *v_cache;
  const int32_t *page_table, *prefix_len;
  double *out, *logits, *group, *logits_all;
} verify_ctx;

/* One thread unit: every verify row of query head h of sequence b. */
static void *verify_unit(void *vctx, int unit) {
  verify_ctx *c = (verify_ctx *)vctx;
  int b = unit / c->Hq, h = unit % c->Hq;
  int G = c->Hq / c->Hkv, R = c->gamma + 1, D = c->D, g = h / G;
  long long P = c->prefix_len[b];
  long long N = P + R;
  long long *slots = (long long *)malloc(sizeof(long long) * (size_t)N);
  double *l = (double *)malloc(sizeof(double) * (size_t)N);
  double *qv = (double *)malloc(sizeof(double) * (size_t)D);
  void *bad = NULL;
  if (!slots || !l || !qv) { bad = (void *)1; goto done; }
  for (long long j = 0; j < N; ++j) slots[j] = slot_of(c->page_table, c->max_pages, c->ps, b, j);
  for (int r = 0; r < R; ++r) {
    for (int d = 0; d < D; ++d)
      qv[d] = load_elem(c->q, c->dtype, (((size_t)b * R + r) * c->Hq + h) * (size_t)D + d);
    /* Verification is standard full attention (Vegas, section 2, core
     * mechanism, verification phase); causal among the new rows: row r sees
     * positions 0 .. P + r. */
    double *o = c->out + (((size_t)b * R + r) * c->Hq + h) * (size_t)D;
    if (attend(qv, D, c->dtype, c->scale, c->k_cache, c->v_cache, c->Hkv, g, slots, P + r + 1,
               l, o) != ORACLE_OK) {
      bad = (void *)1;
      goto done;
    }
    /* Collect-2-Query (section 2.B): only the first draft row and the bonus
     * row export their pre-softmax logits (section 3, kernel instrumentation),
     * over the prefix positions j < P. */
    if (c->logits) {
      if (r == 0)
        memcpy(c->logits + (((size_t)b * 2 + 0) * c->Hq + h) * (size_t)c->max_prefix, l,
               sizeof(double) * (size_t)P);
      if (r == c->gamma)
        memcpy(c->logits + (((size_t)b * 2 + 1) * c->Hq + h) * (size_t)c->max_prefix, l,
               sizeof(double) * (size_t)P);
    }
    /* Full collection: the selection objective as written sums every verify row. */
    if (c->logits_all)
      memcpy(c->logits_all + (((size_t)b * R + r) * c->Hq + h) * (size_t)c->max_prefix, l,
             sizeof(double) * (size_t)P);
  }
done:
  free(slots);
  free(l);
  free(qv);
  return bad;
}

/* One thread unit: the group export of KV head g of sequence b (after every
 * head's logits are written):  group[b][g][j] = sum over the G query heads of
 * KV head g of the two exported rows' logits. */
static void *group_unit(void *vctx, int unit) {
  verify_ctx *c = (verify_ctx *)vctx;
  int b = unit / c->Hkv, g = unit % c->Hkv;
  int G = c->Hq / c->Hkv;
  long long P = c->prefix_len[b];
  double *gs = c->group + ((size_t)b * c->Hkv + g) * (size_t)c->max_prefix;
  for (long long j = 0; j < P; ++j) {
    double s = 0.0;
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      s += c->logits[(((size_t)b * 2 + 0) * c->Hq + h) * (size_t)c->max_prefix + j];
      s += c->logits[(((size_t)b * 2 + 1) * c->Hq + h) * (size_t)c->max_prefix + j];
    }
    gs[j] = s;
  }
  return NULL;
}

/* Full causal attention of rows 0..gamma over keys [0, P_b + r] of each
 * sequence, with the Collect-2-Query export.
 *   out        [B][gamma+1][Hq][D]          (required)
 *   logits     [B][2][Hq][max_prefix]        rows 0 and gamma, j < P_b (nullable)
 *   group      [B][Hkv][max_prefix]          needs `logits`          (nullable)
 *   logits_all [B][gamma+1][Hq][max_prefix]  every row, j < P_b      (nullable)
 * Entries j >= P_b of the exports are left untouched. */
int oracle_verify(int B, int Hq, int Hkv, int D, int page_size, int max_pages, int dtype,
                  double scale, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *page_table, const int32_t *prefix_len, int gamma, int max_prefix,
                  double *out, double *logits, double *group, double *logits_all, int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || page_size < 1 || max_pages < 1 ||
      gamma < 0 || max_prefix < 0 || !q || !k_cache || !v_cache || !page_table || !prefix_len ||
      !out || (dtype != 0 && dtype != 1))
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    long long n = (long long)prefix_len[b] + gamma + 1;
    if (prefix_len[b] < 0 || prefix_len[b] > max_prefix ||
        (n + page_size - 1) / page_size > max_pages)
      return ORACLE_EINVAL;
  }
  if (group && !logits) return ORACLE_EINVAL;
  verify_ctx c = {B, Hq, Hkv, D, page_size, max_pages, dtype, gamma, max_prefix, scale,
                  q, k_cache, v_cache, page_table, prefix_len, out, logits, group, logits_all};
  int rc = run_units(B * Hq, verify_unit, &c, nthreads);
  if (rc == ORACLE_OK && group) rc = run_units(B * Hkv, group_unit, &c, nthreads);
  return rc;
}

/* --------------------------------------------------------------- aggregate */

/* Score of prefix position j: the selection objective (section 2.A) summed
 * over the exported rows `src_rows` (2 for Collect-2-Query, gamma+1 for full
 * collection) and every query head:  s[b][j] = sum_t sum_h l[b][t][h][j].
 * src [B][src_rows][Hq][max_prefix]; scores [B][max_prefix], j < P_b written. */
int oracle_aggregate(int B, int Hq, int src_rows, int max_prefix, const int32_t *prefix_len,
                     const double *src, double *scores) {
  if (B < 1 || Hq < 1 || src_rows < 1 || max_prefix < 0 || !prefix_len || !src || !scores)
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    if (prefix_len[b] < 0 || prefix_len[b] > max_prefix) return ORACLE_EINVAL;
    for (long long j = 0; j < prefix_len[b]; ++j) {
      double s = 0.0;
      for (int t = 0; t < src_rows; ++t)
        for (int h = 0; h < Hq; ++h)
          s += src[(((size_t)b * src_rows + t) * Hq + h) * (size_t)max_prefix + j];
      scores[(size_t)b * max_prefix + j] = s;
    }
  }
  return ORACLE_OK;
}

/* -------------------------------------------------------------------- topk */

typedef struct {
  double neg;
  long long pos;
} keyed;

static int cmp_keyed(const void *a, const void *b) {
  const keyed *x = (const keyed *)a, *y = (const keyed *)b;
  if (x->neg < y->neg) return -1;
  if (x->neg > y->neg) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_ll(const void *a, const void *b) {
  long long x = *(const long long *)a, y = *(const long long *)b;
  return (x > y) - (x < y);
}

/* The selected set maximises the summed score over all size-k subsets of the
 * prefix (section 2.A).  The objective is a sum of per-position terms, so the
 * maximisers are exactly the sets holding k largest scores.  Ties at the k-th
 * score are broken toward lower positions.  Steps: sort (-s_j, j) ascending,
 * keep the first min(k_b, P_b), re-sort them by position.  sel_pos/sel_slot
 * [B][max_k] (sel_slot nullable), sel_count [B]. */
int oracle_topk(int B, int max_prefix, const double *scores, const int32_t *prefix_len,
                const int32_t *k, int max_k, const int32_t *page_table, int page_size,
                int max_pages, int32_t *sel_pos, int32_t *sel_slot, int32_t *sel_count) {
  if (B < 1 || max_prefix < 0 || max_k < 0 || !scores || !prefix_len || !k || !sel_pos ||
      !sel_count || (sel_slot && (!page_table || page_size < 1 || max_pages < 1)))
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    long long P = prefix_len[b];
    if (P < 0 || P > max_prefix || k[b] < 0 || k[b] > max_k) return ORACLE_EINVAL;
    long long kk = k[b] < P ? k[b] : P;
    keyed *arr = (keyed *)malloc(sizeof(keyed) * (size_t)(P > 0 ? P : 1));
    long long *pick = (long long *)malloc(sizeof(long long) * (size_t)(kk > 0 ? kk : 1));
    if (!arr || !pick) { free(arr); free(pick); return ORACLE_ENOMEM; }
    for (long long j = 0; j < P; ++j) {
      arr[j].neg = -scores[(size_t)b * max_prefix + j];
      arr[j].pos = j;
    }
    qsort(arr, (size_t)P, sizeof(keyed), cmp_keyed);
    for (long long i = 0; i < kk; ++i) pick[i] = arr[i].pos;
    qsort(pick, (size_t)kk, sizeof(long long), cmp_ll);
    for (long long i = 0; i < kk; ++i) {
      sel_pos[(size_t)b * max_k + i] = (int32_t)pick[i];
      if (sel_slot)
        sel_slot[(size_t)b * max_k + i] =
            (int32_t)slot_of(page_table, max_pages, page_size, b, pick[i]);
    }
    sel_count[b] = (int32_t)kk;
    free(arr);
    free(pick);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ sparse */

typedef struct {
  int B, Hq, Hkv, D, ps, max_pages, dtype, n_q, max_k;
  double scale;
  const void *q, *k_cache, *v_cache;
  const int32_t *page_table, *sel_pos, *sel_count, *tail_start, *tail_len;
  double *out;
} sparse_ctx;

/* One thread unit: every draft row of query head h of sequence b. */
static void *sparse_unit(void *vctx, int unit) {
  sparse_ctx *c = (sparse_ctx *)vctx;
  int b = unit / c->Hq, h = unit % c->Hq;
  int G = c->Hq / c->Hkv, D = c->D, g = h / G;
  long long cnt = c->sel_count[b], t0 = c->tail_start[b], tl = c->tail_len[b];
  long long nmax = cnt + tl;
  long long *slots = (long long *)malloc(sizeof(long long) * (size_t)(nmax > 0 ? nmax : 1));
  double *l = (double *)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
  double *qv = (double *)malloc(sizeof(double) * (size_t)D);
  void *bad = NULL;
  if (!slots || !l || !qv) { bad = (void *)1; goto done; }
  /* Drafting attends only to the selected entries (section 2, core mechanism,
   * drafting phase), each passed as a page of one token (section 3, sparse
   * execution).  A draft row also sees the tokens after the prefix up to its
   * own position: row i of n_q sees tail positions t0 .. t0 + tl - n_q + i. */
  for (long long i = 0; i < cnt; ++i)
    slots[i] = slot_of(c->page_table, c->max_pages, c->ps, b,
                       c->sel_pos[(size_t)b * c->max_k + i]);
  for (long long i = 0; i < tl; ++i)
    slots[cnt + i] = slot_of(c->page_table, c->max_pages, c->ps, b, t0 + i);
  for (int row = 0; row < c->n_q; ++row) {
    for (int d = 0; d < D; ++d)
      qv[d] = load_elem(c->q, c->dtype, (((size_t)b * c->n_q + row) * c->Hq + h) * (size_t)D + d);
    long long n = cnt + tl - c->n_q + row + 1;
    double *o = c->out + (((size_t)b * c->n_q + row) * c->Hq + h) * (size_t)D;
    if (attend(qv, D, c->dtype, c->scale, c->k_cache, c->v_cache, c->Hkv, g, slots, n, l, o) !=
        ORACLE_OK) {
      bad = (void *)1;
      goto done;
    }
  }
done:
  free(slots);
  free(l);
  free(qv);
  return bad;
}

/* Sparse draft attention.  q [B][n_q][Hq][D]; sel_pos [B][max_k] logical
 * positions (first sel_count[b] used); tail_start/tail_len [B] with
 * tail_len >= n_q; out [B][n_q][Hq][D]. */
int oracle_sparse(int B, int Hq, int Hkv, int D, int page_size, int max_pages, int dtype,
                  double scale, const void *q, int n_q, const void *k_cache, const void *v_cache,
                  const int32_t *page_table, const int32_t *sel_pos, const int32_t *sel_count,
                  int max_k, const int32_t *tail_start, const int32_t *tail_len, double *out,
                  int nthreads) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || page_size < 1 || max_pages < 1 ||
      n_q < 1 || max_k < 0 || !q || !k_cache || !v_cache || !page_table || !sel_count ||
      !tail_start || !tail_len || !out || (max_k > 0 && !sel_pos) || (dtype != 0 && dtype != 1))
    return ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    if (sel_count[b] < 0 || sel_count[b] > max_k || tail_len[b] < n_q || tail_start[b] < 0 ||
        ((long long)tail_start[b] + tail_len[b] + page_size - 1) / page_size > max_pages)
      return ORACLE_EINVAL;
    for (int i = 0; i < sel_count[b]; ++i) {
      int32_t p = sel_pos[(size_t)b * max_k + i];
      if (p < 0 || (long long)p / page_size >= max_pages) return ORACLE_EINVAL;
    }
  }
  sparse_ctx c = {B, Hq, Hkv, D, page_size, max_pages, dtype, n_q, max_k, scale,
                  q, k_cache, v_cache, page_table, sel_pos, sel_count, tail_start, tail_len, out};
  return run_units(B * Hq, sparse_unit, &c, nthreads);
}

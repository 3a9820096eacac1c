/*
 * pisa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle of PISA's pyramid Top-K block selection.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library; the product path never does.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Sources (the method is described, not listed in code, on these pages):
 *  [A] "Block Sparse Attention with Log-Linear Complexity", paper summary on
 *      agihunt.info: paragraph on the key pyramid (levels, mean pooling,
 *      top-down walk, bounded candidate set), paragraph on LSE scoring and
 *      the forced first/previous/current leaf blocks, paragraph on the
 *      kernels and GQA sharing.
 *  [B] rcap.io explainer of the same paper: the tree paragraph (keys as
 *      leaves, pooling with g = 2), the top-down walk paragraph (at most g*K
 *      candidates per level), the scoring-rule paragraph (LSE over child
 *      summaries, Jensen), and the selection-walk sketch that follows it.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes):
 *  - levels: n_1 = ceil(N/C), n_l = ceil(n_{l-1}/g); the walk starts at the
 *    first level L with n_L <= g*K (every coarser level has <= K nodes, so a
 *    walk from a single root keeps all of them and reaches the same set);
 *  - mean pooling is the unweighted mean of the children that exist (a short
 *    last leaf block averages its present keys);
 *  - one pyramid per (batch, KV head), shared by that head's G query heads;
 *  - scale s (default 1/sqrt(d)) multiplies each dot product;
 *  - causality at levels >= 2 is node-granular: a node at level l with index
 *    j covers leaf blocks starting at j*g^(l-1) and is visible to a query in
 *    leaf block b iff j*g^(l-1) <= b; its full stored mean is used;
 *  - the leaf LSE runs over the block's raw keys t <= i (causal mask);
 *  - GQA: the group's score is the sum over its G query heads of the per-head
 *    LSE; Top-K orders by (score descending, block index ascending);
 *  - forced blocks F = {0, b-1, b} within [0, b] count inside K:
 *    Sel = F u TopK_{K-|F|}(X_1 \ F), reported ascending with their leaf
 *    scores, padded with (-1, -inf); K >= 3 is required;
 *  - the PISA-1 / PISA-2 ablations ([A] LSE paragraph: the first keeps only
 *    the mean, the second adds the variance term of the LSE's Taylor
 *    expansion; [B] scoring-rule paragraph: truncations at first and second
 *    order) replace the routing levels' per-head LSE over the m visible
 *    children's scaled dots x_c by log m + mean(x) (PISA-1) or
 *    log m + mean(x) + Var(x)/2 (PISA-2, population variance), the Taylor
 *    expansion of log sum exp(x_c) = log m + log mean exp(x_c) about the mean;
 *    leaf and forced scores stay the exact raw-key LSE;
 *  - the full-scan BSA selector the pages compare against has its own
 *    section and readings at the end of this file.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAXL 48

typedef struct {
  int32_t batch, seq_len, n_q_heads, n_kv_heads, head_dim, block, top_k, branch;
  double scale; /* > 0; the caller resolves the 1/sqrt(d) default */
  int32_t dtype; /* 0 = float32 values, 1 = bfloat16 bit patterns */
  int32_t scorer; /* routing-level score: 0 = LSE, 1 = PISA-1, 2 = PISA-2 */
} orc_problem;

typedef struct {
  int32_t levels_scored;  /* routing levels walked (L - 1), plus 1 for the leaf */
  int32_t max_candidates; /* largest candidate set scored at any level */
  int64_t dots;           /* per query head: routing + leaf + forced dot products */
  double min_margin;      /* smallest (K-th minus (K+1)-th) score gap met on the walk */
} orc_stats;

/* ---------------------------------------------------------------- levels */

/* n[0] = N raw keys, n[1] = ceil(N/C) leaf blocks, n[l] = ceil(n[l-1]/g);
 * returns L, the first level with n[L] <= g*K (L >= 1). */
int orc_levels(int64_t N, int32_t C, int32_t K, int32_t g, int64_t* n) {
  n[0] = N;
  n[1] = (N + C - 1) / C;
  int L = 1;
  while (n[L] > (int64_t)g * K && L < ORC_MAXL) {
    n[L + 1] = (n[L] + g - 1) / g;
    ++L;
  }
  return L;
}

typedef struct {
  const orc_problem* P;
  int64_t n[ORC_MAXL + 2];
  int64_t off[ORC_MAXL + 2]; /* node offset of level l inside one head's pyramid */
  int64_t span[ORC_MAXL + 2]; /* g^(l-1): leaf blocks per level-l node */
  int L, G, d, C, K, g, scorer;
  int64_t N, T;
  double s;
} geo_t;

static void geo_init(geo_t* q, const orc_problem* P) {
  memset(q, 0, sizeof(*q));
  q->P = P;
  q->N = P->seq_len;
  q->d = P->head_dim;
  q->C = P->block;
  q->K = P->top_k;
  q->g = P->branch;
  q->G = P->n_q_heads / P->n_kv_heads;
  q->s = P->scale;
  q->scorer = P->scorer;
  q->L = orc_levels(q->N, q->C, q->K, q->g, q->n);
  q->off[1] = 0;
  q->span[1] = 1;
  for (int l = 1; l <= q->L; ++l) {
    q->off[l + 1] = q->off[l] + q->n[l];
    q->span[l + 1] = q->span[l] * q->g;
  }
  q->T = q->off[q->L + 1];
}

int64_t orc_pyramid_nodes(const orc_problem* P) {
  geo_t q;
  geo_init(&q, P);
  return q.T;
}

/* ----------------------------------------------------------- basic math */

static inline double ld(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* log(sum_i exp(x_i)), computed after subtracting the maximum.
 * Entries equal to -inf contribute nothing; all -inf (or n == 0) gives -inf. */
double orc_lse(const double* x, int64_t n) {
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (x[i] > m) m = x[i];
  if (m == -INFINITY) return -INFINITY;
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += exp(x[i] - m);
  return m + log(acc);
}

static double dot(const double* a, const double* b, int d) {
  double acc = 0.0;
  for (int e = 0; e < d; ++e) acc += a[e] * b[e];
  return acc;
}

/* --------------------------------------------------------------- pyramid */

/* Pyramid of one (batch, KV head): levels 1..L, leaf level first, each node a
 * d-vector.  Level 1 node j = mean of keys [jC, min(jC+C, N)); level l node j
 * = mean of level l-1 nodes [jg, min(jg+g, n_{l-1})). */
static void pyramid_bh(const geo_t* q, const void* k, int64_t kbase, double* out) {
  const int d = q->d;
  for (int64_t j = 0; j < q->n[1]; ++j) {
    int64_t lo = j * q->C, hi = lo + q->C < q->N ? lo + q->C : q->N;
    double* o = out + (q->off[1] + j) * d;
    for (int e = 0; e < d; ++e) {
      double acc = 0.0;
      for (int64_t t = lo; t < hi; ++t) acc += ld(k, kbase + t * d + e, q->P->dtype);
      o[e] = acc / (double)(hi - lo);
    }
  }
  for (int l = 2; l <= q->L; ++l) {
    for (int64_t j = 0; j < q->n[l]; ++j) {
      int64_t c0 = j * q->g, c1 = c0 + q->g < q->n[l - 1] ? c0 + q->g : q->n[l - 1];
      double* o = out + (q->off[l] + j) * d;
      for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int64_t c = c0; c < c1; ++c) acc += out[(q->off[l - 1] + c) * d + e];
        o[e] = acc / (double)(c1 - c0);
      }
    }
  }
}

/* pyr: double [B, Hkv, T, d] */
int orc_build_pyramid(const orc_problem* P, const void* k, double* pyr) {
  geo_t q;
  geo_init(&q, P);
  int64_t nbh = (int64_t)P->batch * P->n_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nbh; ++bh) pyramid_bh(&q, k, bh * q.N * q.d, pyr + bh * q.T * q.d);
  return 0;
}

/* ----------------------------------------------------------- one query */

typedef struct {
  const geo_t* q;
  const double* qrows; /* G x d, the group's query rows at position i */
  const void* k;       /* keys, raw storage */
  int64_t kbase;       /* element offset of key row 0 of this (b, h) */
  const double* pyr;   /* this (b, h)'s pyramid, T x d */
  int64_t i, bq;       /* query position and its leaf block */
} row_t;

static int visible(const row_t* r, int l, int64_t j) { return j * r->q->span[l] <= r->bq; }

/* Routing score of m values: their LSE, or its first- / second-order Taylor
 * truncation about the mean (PISA-1 / PISA-2). */
static double routing_score(const double* x, int64_t m, int scorer) {
  if (scorer == 0) return orc_lse(x, m);
  double mean = 0.0;
  for (int64_t c = 0; c < m; ++c) mean += x[c];
  mean /= (double)m;
  double out = log((double)m) + mean;
  if (scorer == 2) {
    double var = 0.0;
    for (int64_t c = 0; c < m; ++c) var += (x[c] - mean) * (x[c] - mean);
    out += 0.5 * var / (double)m;
  }
  return out;
}

/* Score of node x at level l >= 2: sum over heads of the routing score (LSE,
 * or a truncation of it) over its visible children c (level l-1) of
 * s * <q_h, P_{l-1}[c]>.  per_head may be NULL. */
static double node_score(const row_t* r, int l, int64_t x, double* per_head) {
  const geo_t* q = r->q;
  int64_t c0 = x * q->g, c1 = c0 + q->g < q->n[l - 1] ? c0 + q->g : q->n[l - 1];
  double vals[64];
  double total = 0.0;
  for (int h = 0; h < q->G; ++h) {
    int64_t m = 0;
    for (int64_t c = c0; c < c1; ++c) {
      if (!visible(r, l - 1, c)) continue;
      vals[m++] = q->s * dot(r->qrows + (int64_t)h * q->d, r->pyr + (q->off[l - 1] + c) * q->d, q->d);
    }
    double v = routing_score(vals, m, q->scorer);
    if (per_head) per_head[h] = v;
    total += v;
  }
  return total;
}

/* Leaf score of block j for query i: sum over heads of LSE over keys t in
 * block j with t <= i of s * <q_h, k_t>. */
static double leaf_score(const row_t* r, int64_t j, double* per_head) {
  const geo_t* q = r->q;
  int64_t lo = j * q->C, hi = lo + q->C;
  if (hi > q->N) hi = q->N;
  if (hi > r->i + 1) hi = r->i + 1;
  double* vals = (double*)malloc(sizeof(double) * (size_t)q->C);
  double* key = (double*)malloc(sizeof(double) * (size_t)q->d);
  double total = 0.0;
  for (int h = 0; h < q->G; ++h) {
    int64_t m = 0;
    for (int64_t t = lo; t < hi; ++t) {
      for (int e = 0; e < q->d; ++e) key[e] = ld(r->k, r->kbase + t * q->d + e, q->P->dtype);
      vals[m++] = q->s * dot(r->qrows + (int64_t)h * q->d, key, q->d);
    }
    double v = orc_lse(vals, m);
    if (per_head) per_head[h] = v;
    total += v;
  }
  free(vals);
  free(key);
  return total;
}

typedef struct {
  double s;
  int64_t j;
} cand_t;

/* order: score descending, then index ascending */
static int by_score(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int by_index(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  return (x->j > y->j) - (x->j < y->j);
}

static int n_forced(int64_t bq, int64_t* F) {
  int m = 0;
  F[m++] = 0;
  if (bq - 1 > 0) F[m++] = bq - 1;
  if (bq > 0) F[m++] = bq;
  return m;
}

static int is_in(const int64_t* a, int n, int64_t v) {
  for (int t = 0; t < n; ++t)
    if (a[t] == v) return 1;
  return 0;
}

/* Visible children of the kept nodes (level l) at level l-1, in kept order. */
static int expand(const row_t* r, int l, const cand_t* kept, int nk, int64_t* X) {
  const geo_t* q = r->q;
  int m = 0;
  for (int t = 0; t < nk; ++t) {
    int64_t c0 = kept[t].j * q->g, c1 = c0 + q->g < q->n[l - 1] ? c0 + q->g : q->n[l - 1];
    for (int64_t c = c0; c < c1; ++c)
      if (visible(r, l - 1, c)) X[m++] = c;
  }
  return m;
}

static int64_t keys_seen(const row_t* r, int64_t j) {
  int64_t lo = j * r->q->C, hi = lo + r->q->C < r->q->N ? lo + r->q->C : r->q->N;
  if (hi > r->i + 1) hi = r->i + 1;
  return hi - lo;
}

/* Every candidate set holds at most g*K entries: the top level has
 * n_L <= g*K nodes, later levels hold the children of K kept nodes, and
 * with L = 1 there are n_1 <= g*K leaf blocks. */
static int cap_of(const geo_t* q) { return q->g * q->K + 4; }

/* The walk for one query group.  Writes K (index, score) pairs. */
static void walk(const row_t* r, int32_t* out_idx, double* out_score, orc_stats* st) {
  const geo_t* q = r->q;
  const int K = q->K, cap = cap_of(q);
  int64_t* X = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
  cand_t* S = (cand_t*)malloc(sizeof(cand_t) * (size_t)cap);
  cand_t* sel = (cand_t*)malloc(sizeof(cand_t) * (size_t)cap);
  int nx = 0, maxc = 0;
  int64_t dots = 0;
  double margin = INFINITY;

  if (q->L == 1) {
    for (int64_t j = 0; j <= r->bq; ++j) X[nx++] = j;
  } else {
    for (int64_t j = 0; j < q->n[q->L]; ++j)
      if (visible(r, q->L, j)) X[nx++] = j;
    for (int l = q->L; l >= 2; --l) {
      if (nx > maxc) maxc = nx;
      for (int t = 0; t < nx; ++t) {
        S[t].j = X[t];
        S[t].s = node_score(r, l, X[t], NULL);
        int64_t c0 = X[t] * q->g;
        for (int64_t c = c0; c < c0 + q->g && c < q->n[l - 1]; ++c) dots += visible(r, l - 1, c);
      }
      qsort(S, (size_t)nx, sizeof(cand_t), by_score);
      int nk = nx < K ? nx : K;
      if (nx > K && S[K - 1].s - S[K].s < margin) margin = S[K - 1].s - S[K].s;
      nx = expand(r, l, S, nk, X);
    }
  }
  if (nx > maxc) maxc = nx;
  /* leaf: forced blocks plus Top-(K-|F|) of the remaining candidates */
  int64_t F[3];
  int nf = n_forced(r->bq, F);
  int nr = 0;
  for (int t = 0; t < nx; ++t) {
    if (is_in(F, nf, X[t])) continue;
    S[nr].j = X[t];
    S[nr].s = leaf_score(r, X[t], NULL);
    dots += keys_seen(r, X[t]);
    ++nr;
  }
  qsort(S, (size_t)nr, sizeof(cand_t), by_score);
  int Kp = K - nf;
  int take = Kp < nr ? Kp : nr;
  if (nr > Kp && Kp > 0 && S[Kp - 1].s - S[Kp].s < margin) margin = S[Kp - 1].s - S[Kp].s;
  int ns = 0;
  for (int t = 0; t < take; ++t) sel[ns++] = S[t];
  for (int t = 0; t < nf; ++t) {
    sel[ns].j = F[t];
    sel[ns].s = leaf_score(r, F[t], NULL);
    dots += keys_seen(r, F[t]);
    ++ns;
  }
  qsort(sel, (size_t)ns, sizeof(cand_t), by_index);
  for (int t = 0; t < K; ++t) {
    out_idx[t] = t < ns ? (int32_t)sel[t].j : -1;
    out_score[t] = t < ns ? sel[t].s : -INFINITY;
  }
  if (st) {
    st->levels_scored = q->L;
    st->max_candidates = maxc;
    st->dots = dots;
    st->min_margin = margin;
  }
  free(X);
  free(S);
  free(sel);
}

/* Query rows of group (b, h) at position i, upcast to double.
 * decode == 0: q is [B, Hq, N, d]; decode != 0: q is [B, Hq, d]. */
static void load_qrows(const geo_t* q, const void* qp, int decode, int64_t b, int64_t h, int64_t i, double* out) {
  const orc_problem* P = q->P;
  for (int r = 0; r < q->G; ++r) {
    int64_t hq = h * q->G + r;
    int64_t base = decode ? (b * P->n_q_heads + hq) * q->d : ((b * P->n_q_heads + hq) * q->N + i) * q->d;
    for (int e = 0; e < q->d; ++e) out[(int64_t)r * q->d + e] = ld(qp, base + e, P->dtype);
  }
}

static void row_setup(const geo_t* q, const void* qp, const void* k, const double* pyr, int decode, int64_t rid,
                      double* qbuf, row_t* r) {
  int64_t bh = decode ? rid : rid / q->N;
  int64_t i = decode ? q->N - 1 : rid % q->N;
  int64_t b = bh / q->P->n_kv_heads, h = bh % q->P->n_kv_heads;
  load_qrows(q, qp, decode, b, h, i, qbuf);
  r->q = q;
  r->qrows = qbuf;
  r->k = k;
  r->kbase = bh * q->N * q->d;
  r->pyr = pyr ? pyr + bh * q->T * q->d : NULL;
  r->i = i;
  r->bq = i / q->C;
}

int orc_valid_problem(const orc_problem* P) {
  if (!P || P->batch < 1 || P->seq_len < 1 || P->n_kv_heads < 1 || P->n_q_heads < 1) return 0;
  if (P->n_q_heads % P->n_kv_heads) return 0;
  if (P->head_dim < 1 || P->block < 1 || P->branch < 2 || P->branch > 64 || P->top_k < 3) return 0;
  if ((int64_t)P->branch * P->top_k > 4096) return 0;
  if (!(P->scale > 0.0) || (P->dtype != 0 && P->dtype != 1)) return 0;
  if (P->scorer < 0 || P->scorer > 2) return 0;
  return 1;
}

/*
 * Selection for a list of query groups.  rows[t] = (b*Hkv + h)*N + i for
 * prefill, (b*Hkv + h) for decode (query at position N-1); rows == NULL
 * means every group in order.  idx/score: [n_rows, K].  st may be NULL.
 */
int orc_select_rows(const orc_problem* P, const void* qp, const void* k, const double* pyr, int32_t decode,
                    int64_t n_rows, const int64_t* rows, int32_t* idx, double* score, orc_stats* st) {
  if (!orc_valid_problem(P)) return 1;
  geo_t q;
  geo_init(&q, P);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n_rows; ++t) {
    double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
    row_t r;
    row_setup(&q, qp, k, pyr, decode, rows ? rows[t] : t, qbuf, &r);
    walk(&r, idx + t * q.K, score + t * q.K, st ? st + t : NULL);
    free(qbuf);
  }
  return 0;
}

/* Per-head pieces for the invariant tests. */
double orc_node_score(const orc_problem* P, const void* qp, const double* pyr, int32_t decode, int64_t rid,
                      int32_t level, int64_t j, double* per_head) {
  geo_t q;
  geo_init(&q, P);
  if (level < 2 || level > q.L) return NAN;
  double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
  row_t r;
  row_setup(&q, qp, NULL, pyr, decode, rid, qbuf, &r);
  double v = node_score(&r, level, j, per_head);
  free(qbuf);
  return v;
}

double orc_leaf_score(const orc_problem* P, const void* qp, const void* k, int32_t decode, int64_t rid, int64_t j,
                      double* per_head) {
  geo_t q;
  geo_init(&q, P);
  double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
  row_t r;
  row_setup(&q, qp, k, NULL, decode, rid, qbuf, &r);
  double v = leaf_score(&r, j, per_head);
  free(qbuf);
  return v;
}

/* ------------------------------------------------------- verification */

/*
 * Tie-tolerant check of a selection produced by another implementation.
 *
 * A kept set Y of candidate set X at some level is accepted when
 * |Y| = min(K', |X|) and every kept score >= every dropped score - tau
 * (K' = K at routing levels, K - |F| at the leaf).  With the oracle's scores
 * in fp64 this accepts exactly the sets that differ from the oracle's own
 * choice only by swaps among candidates whose scores lie within tau of the
 * K-th / (K+1)-th boundary.  The check searches the resolutions of those tie
 * bands level by level (each kept set defines the next candidate set) for
 * one that reproduces the given leaf selection; the non-forced selected
 * blocks must descend from the kept nodes, which prunes the search.
 *
 * status: 0 pass, 1 bad shape/padding/order, 2 forced block missing,
 *         3 score outside tolerance, 4 selection unreachable, 5 search
 *         capped (inconclusive).
 */
typedef struct {
  const row_t* r;
  const int64_t* R; /* non-forced selected blocks */
  int nR;
  const int64_t* F;
  int nf;
  double tau;
  int cap, used;
  int64_t tries, max_tries;
  int capped;
} vctx_t;

static int leaf_ok(vctx_t* v, const int64_t* X, int nx) {
  const row_t* r = v->r;
  const int Kp = r->q->K - v->nf;
  double mn = INFINITY, mx = -INFINITY;
  int nr = 0;
  for (int t = 0; t < nx; ++t)
    if (!is_in(v->F, v->nf, X[t])) ++nr;
  int want = Kp < nr ? Kp : nr;
  if (want != v->nR) return 0;
  for (int t = 0; t < v->nR; ++t)
    if (!is_in(X, nx, v->R[t])) return 0;
  for (int t = 0; t < nx; ++t) {
    if (is_in(v->F, v->nf, X[t])) continue;
    double s = leaf_score(r, X[t], NULL);
    if (is_in(v->R, v->nR, X[t])) {
      if (s < mn) mn = s;
    } else if (s > mx) {
      mx = s;
    }
  }
  return v->nR == 0 || mn >= mx - v->tau;
}

static int dfs(vctx_t* v, int l, const int64_t* X, int nx);

/* Descend with kept set Y (level l). */
static int descend(vctx_t* v, int l, const cand_t* Y, int ny) {
  if (++v->used > v->cap) {
    v->capped = 1;
    return 0;
  }
  int64_t* Xn = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap_of(v->r->q));
  int nn = expand(v->r, l, Y, ny, Xn);
  int ok = l == 2 ? leaf_ok(v, Xn, nn) : dfs(v, l - 1, Xn, nn);
  free(Xn);
  return ok;
}

/* in[t] marks the kept members of the sorted candidates S[0..nx). */
static int try_set(vctx_t* v, int l, const cand_t* S, int nx, const char* in) {
  const int K = v->r->q->K;
  double mn = INFINITY, mx = -INFINITY;
  int ny = 0;
  for (int t = 0; t < nx; ++t) {
    if (in[t]) {
      ++ny;
      if (S[t].s < mn) mn = S[t].s;
    } else if (S[t].s > mx) {
      mx = S[t].s;
    }
  }
  if (ny != K || !(mn >= mx - v->tau)) return 0;
  cand_t* Y = (cand_t*)malloc(sizeof(cand_t) * (size_t)K);
  int m = 0;
  for (int t = 0; t < nx; ++t)
    if (in[t]) Y[m++] = S[t];
  int ok = descend(v, l, Y, m);
  free(Y);
  return ok;
}

/* Choose `need` more members from the free band positions free_[start..). */
static int choose(vctx_t* v, int l, const cand_t* S, int nx, char* in, const int* free_, int nfree, int need,
                  int start) {
  if (v->capped) return 0;
  if (need == 0) {
    if (++v->tries > v->max_tries) {
      v->capped = 1;
      return 0;
    }
    return try_set(v, l, S, nx, in);
  }
  for (int t = start; t <= nfree - need; ++t) {
    in[free_[t]] = 1;
    int ok = choose(v, l, S, nx, in, free_, nfree, need - 1, t + 1);
    in[free_[t]] = 0;
    if (ok) return 1;
    if (v->capped) return 0;
  }
  return 0;
}

static int dfs(vctx_t* v, int l, const int64_t* X, int nx) {
  const row_t* r = v->r;
  const geo_t* q = r->q;
  const int K = q->K;
  cand_t* S = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nx > 0 ? nx : 1));
  for (int t = 0; t < nx; ++t) {
    S[t].j = X[t];
    S[t].s = node_score(r, l, X[t], NULL);
  }
  qsort(S, (size_t)nx, sizeof(cand_t), by_score);
  int ok = 0;
  if (nx <= K) {
    ok = descend(v, l, S, nx);
    free(S);
    return ok;
  }
  double sK = S[K - 1].s, sK1 = S[K].s;
  char* in = (char*)calloc((size_t)nx, 1);
  int* free_ = (int*)malloc(sizeof(int) * (size_t)nx);
  int nfree = 0, need = K;
  int dead = 0;
  for (int t = 0; t < nx; ++t) {
    /* ancestors (at level l) of the non-forced selected leaves must be kept */
    int required = 0;
    for (int u = 0; u < v->nR && !required; ++u) required = v->R[u] / q->span[l] == S[t].j;
    if (S[t].s > sK + v->tau || required) {
      if (S[t].s < sK1 - v->tau) dead = 1; /* required but certainly dropped */
      in[t] = 1;
      --need;
    } else if (S[t].s >= sK1 - v->tau) {
      free_[nfree++] = t;
    }
  }
  /* a required ancestor missing from X makes this branch impossible */
  for (int u = 0; u < v->nR && !dead; ++u) {
    int64_t a = v->R[u] / q->span[l];
    int found = 0;
    for (int t = 0; t < nx; ++t) found |= S[t].j == a;
    if (!found) dead = 1;
  }
  if (!dead && need >= 0) ok = choose(v, l, S, nx, in, free_, nfree, need, 0);
  free(in);
  free(free_);
  free(S);
  return ok;
}

int orc_check_rows(const orc_problem* P, const void* qp, const void* k, const double* pyr, int32_t decode,
                   int64_t n_rows, const int64_t* rows, const int32_t* gidx, const float* gscore, double tau,
                   double rtol, int32_t max_branches, int32_t* status, int32_t* branches) {
  if (!orc_valid_problem(P)) return 1;
  geo_t q;
  geo_init(&q, P);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < n_rows; ++t) {
    double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
    row_t r;
    row_setup(&q, qp, k, pyr, decode, rows ? rows[t] : t, qbuf, &r);
    const int32_t* gi = gidx + t * q.K;
    const float* gs = gscore + t * q.K;
    int st = 0;
    branches[t] = 0;
    /* shape: ascending distinct prefix inside [0, b], then (-1, -inf) */
    int64_t want = q.K < r.bq + 1 ? q.K : r.bq + 1;
    int ns = 0;
    while (ns < q.K && gi[ns] >= 0) ++ns;
    if (ns != want) st = 1;
    for (int u = 0; u < ns && !st; ++u)
      if (gi[u] > r.bq || (u > 0 && gi[u] <= gi[u - 1])) st = 1;
    for (int u = ns; u < q.K && !st; ++u)
      if (gi[u] != -1 || !(isinf(gs[u]) && gs[u] < 0)) st = 1;
    int64_t F[3];
    int nf = n_forced(r.bq, F);
    if (!st) {
      for (int u = 0; u < nf; ++u) {
        int found = 0;
        for (int w = 0; w < ns; ++w) found |= gi[w] == F[u];
        if (!found) st = 2;
      }
    }
    if (!st) {
      for (int u = 0; u < ns; ++u) {
        double ref = leaf_score(&r, gi[u], NULL);
        double tol = rtol * (fabs(ref) > 1.0 ? fabs(ref) : 1.0);
        if (!(fabs((double)gs[u] - ref) <= tol)) st = 3;
      }
    }
    if (!st) {
      int64_t* R = (int64_t*)malloc(sizeof(int64_t) * (size_t)q.K);
      int nR = 0;
      for (int u = 0; u < ns; ++u)
        if (!is_in(F, nf, gi[u])) R[nR++] = gi[u];
      vctx_t v = {&r, R, nR, F, nf, tau, max_branches, 0, 0, 200000, 0};
      int64_t* X = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap_of(&q));
      int nx = 0;
      int ok;
      if (q.L == 1) {
        for (int64_t j = 0; j <= r.bq; ++j) X[nx++] = j;
        ok = leaf_ok(&v, X, nx);
      } else {
        for (int64_t j = 0; j < q.n[q.L]; ++j)
          if (visible(&r, q.L, j)) X[nx++] = j;
        ok = dfs(&v, q.L, X, nx);
      }
      branches[t] = v.used;
      if (!ok) st = v.capped ? 5 : 4;
      free(X);
      free(R);
    }
    status[t] = st;
    free(qbuf);
  }
  return 0;
}

/* ------------------------------------------------------- BSA baseline */

/*
 * The full-scan selector the pages compare the pyramid against ([A] first
 * paragraphs and baselines paragraph; [B] picking-step paragraph and the
 * comparison-point paragraph: standard block-sparse
 * attention scores every query against every block summary, O(N^2/C); the
 * baseline is NSA's selected branch with mean-pooled block summaries).
 * Readings (also in the design notes):
 *  - the summary of leaf block j is its mean-pooled keys, i.e. pyramid
 *    level 1 (a short last block averages the keys it has);
 *  - block j's score for a query group is the sum over its G heads of the
 *    plain dot product s * <q_h, mean_j> (no LSE);
 *  - candidates are the blocks 0..b of the query's leaf block b, the forced
 *    blocks F = {0, b-1, b} are kept as in the pyramid selector, and
 *    Sel = F u TopK_{K-|F|}(candidates \ F) by (score descending, block
 *    index ascending);
 *  - output ascending by block index; the forced blocks are not ranked and
 *    report the score +inf (the current block's summary would average keys
 *    after the query); padding (-1, -inf).
 */
static double bsa_score(const row_t* r, int64_t j) {
  const geo_t* q = r->q;
  double total = 0.0;
  for (int h = 0; h < q->G; ++h)
    total += q->s * dot(r->qrows + (int64_t)h * q->d, r->pyr + (q->off[1] + j) * q->d, q->d);
  return total;
}

static void bsa_row(const row_t* r, int32_t* out_idx, double* out_score) {
  const geo_t* q = r->q;
  const int K = q->K;
  int64_t F[3];
  int nf = n_forced(r->bq, F);
  cand_t* S = (cand_t*)malloc(sizeof(cand_t) * (size_t)(r->bq + 1 + 3));
  int nr = 0;
  for (int64_t j = 0; j <= r->bq; ++j) {
    if (is_in(F, nf, j)) continue;
    S[nr].j = j;
    S[nr].s = bsa_score(r, j);
    ++nr;
  }
  qsort(S, (size_t)nr, sizeof(cand_t), by_score);
  int Kp = K - nf;
  int take = Kp < nr ? Kp : nr;
  for (int t = 0; t < nf; ++t) {
    S[take + t].j = F[t];
    S[take + t].s = INFINITY;
  }
  int ns = take + nf;
  qsort(S, (size_t)ns, sizeof(cand_t), by_index);
  for (int t = 0; t < K; ++t) {
    out_idx[t] = t < ns ? (int32_t)S[t].j : -1;
    out_score[t] = t < ns ? S[t].s : -INFINITY;
  }
  free(S);
}

/* Selection for a list of query groups (rows as for orc_select_rows). */
int orc_bsa_select_rows(const orc_problem* P, const void* qp, const double* pyr, int32_t decode, int64_t n_rows,
                        const int64_t* rows, int32_t* idx, double* score) {
  if (!orc_valid_problem(P)) return 1;
  geo_t q;
  geo_init(&q, P);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n_rows; ++t) {
    double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
    row_t r;
    row_setup(&q, qp, NULL, pyr, decode, rows ? rows[t] : t, qbuf, &r);
    bsa_row(&r, idx + t * q.K, score + t * q.K);
    free(qbuf);
  }
  return 0;
}

/* Scores of blocks 0..b for one row; returns b + 1 (out must hold n_1). */
int64_t orc_bsa_scores(const orc_problem* P, const void* qp, const double* pyr, int32_t decode, int64_t rid,
                       double* out) {
  geo_t q;
  geo_init(&q, P);
  double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
  row_t r;
  row_setup(&q, qp, NULL, pyr, decode, rid, qbuf, &r);
  for (int64_t j = 0; j <= r.bq; ++j) out[j] = bsa_score(&r, j);
  free(qbuf);
  return r.bq + 1;
}

/*
 * Tie-tolerant check of a BSA selection from another implementation: the
 * shape and padding as for orc_check_rows, every forced block present with
 * score +inf, every other reported score within rtol (floor 1) of the fp64
 * score, and the non-forced blocks a Top-(K-|F|) of the candidates up to
 * tau: min(K-|F|, |candidates|) of them, none scoring more than tau below
 * a candidate left out.  Status codes as for orc_check_rows.
 */
int orc_bsa_check_rows(const orc_problem* P, const void* qp, const double* pyr, int32_t decode, int64_t n_rows,
                       const int64_t* rows, const int32_t* gidx, const float* gscore, double tau, double rtol,
                       int32_t* status) {
  if (!orc_valid_problem(P)) return 1;
  geo_t q;
  geo_init(&q, P);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n_rows; ++t) {
    double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
    row_t r;
    row_setup(&q, qp, NULL, pyr, decode, rows ? rows[t] : t, qbuf, &r);
    const int32_t* gi = gidx + t * q.K;
    const float* gs = gscore + t * q.K;
    int st = 0;
    int64_t want = q.K < r.bq + 1 ? q.K : r.bq + 1;
    int ns = 0;
    while (ns < q.K && gi[ns] >= 0) ++ns;
    if (ns != want) st = 1;
    for (int u = 0; u < ns && !st; ++u)
      if (gi[u] > r.bq || (u > 0 && gi[u] <= gi[u - 1])) st = 1;
    for (int u = ns; u < q.K && !st; ++u)
      if (gi[u] != -1 || !(isinf(gs[u]) && gs[u] < 0)) st = 1;
    int64_t F[3];
    int nf = n_forced(r.bq, F);
    for (int u = 0; u < nf && !st; ++u) {
      int found = 0;
      for (int w = 0; w < ns; ++w)
        if (gi[w] == F[u]) found = isinf(gs[w]) && gs[w] > 0 ? 1 : -1;
      if (found == 0) st = 2;
      if (found < 0) st = 3;
    }
    double kept_min = INFINITY;
    for (int u = 0; u < ns && !st; ++u) {
      if (is_in(F, nf, gi[u])) continue;
      double ref = bsa_score(&r, gi[u]);
      double tol = rtol * (fabs(ref) > 1.0 ? fabs(ref) : 1.0);
      if (!(fabs((double)gs[u] - ref) <= tol)) st = 3;
      if (ref < kept_min) kept_min = ref;
    }
    if (!st) {
      for (int64_t j = 0; j <= r.bq && !st; ++j) {
        if (is_in(F, nf, j)) continue;
        int chosen = 0;
        for (int u = 0; u < ns; ++u) chosen |= gi[u] == j;
        if (!chosen && bsa_score(&r, j) > kept_min + tau) st = 4;
      }
    }
    status[t] = st;
    free(qbuf);
  }
  return 0;
}

/* ------------------------------------------- block-sparse attention */

/*
 * Attention of each query over the keys of its selected blocks, the
 * consumer of the selection ([A] opening paragraph: each query reads only
 * its Top-K tiles of C keys; [B] first paragraphs: attention then runs over
 * the original keys of the picked blocks).  Readings: one selection per
 * (batch, KV head, position), shared by the group's G query heads; the keys
 * are those of blocks idx[0..K) that lie in [0, b] (entries < 0 or > b are
 * skipped), each key t also causal (t <= i); per query head
 *   out = sum_t softmax_t(s * <q, k_t>) v_t,   lse = log sum_t exp(s * <q, k_t>)
 * (no key visible: out = 0, lse = -inf).  v has the shape of k.
 * rows as for orc_select_rows; idx [n_rows, K] (the selection of each
 * row); out [n_rows, G, d], lse [n_rows, G] (may be NULL).
 */
int orc_attention_rows(const orc_problem* P, const void* qp, const void* k, const void* v, int32_t decode,
                       int64_t n_rows, const int64_t* rows, const int32_t* idx, double* out, double* lse) {
  if (!orc_valid_problem(P)) return 1;
  geo_t q;
  geo_init(&q, P);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n_rows; ++t) {
    double* qbuf = (double*)malloc(sizeof(double) * (size_t)q.G * (size_t)q.d);
    double* x = (double*)malloc(sizeof(double) * (size_t)q.K * (size_t)q.C);
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)q.K * (size_t)q.C);
    row_t r;
    row_setup(&q, qp, k, NULL, decode, rows ? rows[t] : t, qbuf, &r);
    const int32_t* sel = idx + t * q.K;
    /* the attended keys: every position of a selected block in [0, b], causal */
    int64_t m = 0;
    for (int u = 0; u < q.K; ++u) {
      int64_t j = sel[u];
      if (j < 0 || j > r.bq) continue;
      int64_t lo = j * q.C, hi = lo + q.C < q.N ? lo + q.C : q.N;
      if (hi > r.i + 1) hi = r.i + 1;
      for (int64_t p = lo; p < hi; ++p) key[m++] = p;
    }
    for (int h = 0; h < q.G; ++h) {
      double* o = out + (t * q.G + h) * q.d;
      for (int e = 0; e < q.d; ++e) o[e] = 0.0;
      if (m == 0) {
        if (lse) lse[t * q.G + h] = -INFINITY;
        continue;
      }
      const double* qh = r.qrows + (int64_t)h * q.d;
      for (int64_t c = 0; c < m; ++c) {
        double acc = 0.0;
        for (int e = 0; e < q.d; ++e) acc += qh[e] * ld(k, r.kbase + key[c] * q.d + e, P->dtype);
        x[c] = q.s * acc;
      }
      double z = orc_lse(x, m);
      for (int64_t c = 0; c < m; ++c) {
        double w = exp(x[c] - z);
        for (int e = 0; e < q.d; ++e) o[e] += w * ld(v, r.kbase + key[c] * q.d + e, P->dtype);
      }
      if (lse) lse[t * q.G + h] = z;
    }
    free(key);
    free(x);
    free(qbuf);
  }
  return 0;
}

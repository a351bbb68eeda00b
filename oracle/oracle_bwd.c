/*
 * oracle_bwd.c -- fp64 CPU oracle for the gradients of exact attention
 * (TEST INFRASTRUCTURE ONLY; see oracle.h).
 *
 * For one head, with kept pairs (i, j) as in the forward (j <= i when causal),
 *   s_ij = scale * <q_i, k_j>,   P_ij = exp(s_ij - lse_i),   o_i = sum_j P_ij v_j,
 * and a given upstream gradient g_i = dL/do_i, the chain rule through
 * o = P v and through the row softmax gives
 *   dL/dv_j  = sum_i P_ij g_i
 *   dP_ij    = <g_i, v_j>
 *   D_i      = sum_j P_ij dP_ij  (= <g_i, o_i>)
 *   dS_ij    = P_ij (dP_ij - D_i)               (softmax Jacobian)
 *   dL/dq_i  = scale * sum_j dS_ij k_j
 *   dL/dk_j  = scale * sum_i dS_ij q_i
 * with masked pairs contributing nothing.  The forward statistics a
 * recomputing backward pass reuses are the per-row lse_i ("FlashAttention"
 * (ai360xpert), section "Recomputation in the backward pass"); here they are
 * computed afresh in fp64 by the same three passes as oracle.c.
 *
 * Plain code: a first sweep over every query row of each touched head
 * computes lse_i and D_i (three passes over the keys, then o_i); a second
 * sweep computes each requested dq row (a pass over its keys) and each
 * requested dk, dv row (a pass over the queries that keep that key).  Threads
 * only split lists of independent rows.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const void *q, *k, *v, *g;
  int dtype;
  long long H, Nq, Nk, d_qk, d_v; /* q, k rows have d_qk columns; v, o, g rows d_v */
  double scale;
  int causal;
  const long long* k_len; /* per-batch valid keys, or NULL (all Nk) */
  const long long* q_len; /* per-batch valid queries, or NULL (all Nq) */
  /* per touched head: lse and D of every query row, [n_heads][N] */
  const long long* heads; /* touched heads, ascending */
  long long n_heads;
  double *lse, *D;
  /* requested rows and outputs */
  const long long *q_rows, *k_rows;
  long long n_q, n_k;
  double *dq, *dk, *dv;
  /* work lists: phase 0 = statistics rows, 1 = dq rows, 2 = dk/dv rows */
  int phase;
  long long n_items;
  long long next;
} bjob_t;

static double ld(const bjob_t* jb, const void* base, long long idx) {
  return oracle_load(base, jb->dtype, idx);
}

/* index of `head` in the sorted list of touched heads */
static long long head_slot(const bjob_t* jb, long long head) {
  long long lo = 0, hi = jb->n_heads - 1;
  while (lo < hi) {
    long long mid = (lo + hi) / 2;
    if (jb->heads[mid] < head) lo = mid + 1; else hi = mid;
  }
  return lo;
}

/* valid keys L of the batch that head `head` (= b*H + h) belongs to */
static long long valid_keys(const bjob_t* jb, long long head) {
  long long L = jb->k_len ? jb->k_len[head / jb->H] : jb->Nk;
  if (L < 0) L = 0;
  if (L > jb->Nk) L = jb->Nk;
  return L;
}

/* valid queries Lq of the batch that head `head` belongs to */
static long long valid_queries(const bjob_t* jb, long long head) {
  long long L = jb->q_len ? jb->q_len[head / jb->H] : jb->Nq;
  if (L < 0) L = 0;
  if (L > jb->Nq) L = jb->Nq;
  return L;
}

/* |J_i|: query i keeps keys 0 .. nkeys-1 (i < Lq, j < L and, causal,
 * j <= i + L - Lq); a query at or past Lq keeps none */
static long long kept_keys(const bjob_t* jb, long long head, long long i) {
  const long long L = valid_keys(jb, head), Lq = valid_queries(jb, head);
  long long n = i < Lq ? L : 0;
  if (jb->causal && i + (L - Lq) + 1 < n) n = i + (L - Lq) + 1;
  return n < 0 ? 0 : n;
}

/* s_ij = scale * <q_i, k_j> of head `head` (over the d_qk columns) */
static double score(const bjob_t* jb, long long head, long long i, long long j) {
  const long long d = jb->d_qk, qb = head * jb->Nq * d, kb = head * jb->Nk * d;
  double dot = 0.0;
  for (long long c = 0; c < d; ++c)
    dot += ld(jb, jb->q, qb + i * d + c) * ld(jb, jb->k, kb + j * d + c);
  return jb->scale * dot;
}

/* phase 0: lse_i and D_i = <g_i, o_i> of query row i of touched head slot hs
 * (an empty row: lse = -inf, o = 0, D = 0) */
static void stats_row(const bjob_t* jb, long long hs, long long i, double* s, double* o) {
  const long long Nq = jb->Nq, d = jb->d_v, head = jb->heads[hs];
  const long long kb = head * jb->Nk * d;  /* value rows (d_v columns) */
  const long long nkeys = kept_keys(jb, head, i);
  double m = -INFINITY, l = 0.0;
  for (long long j = 0; j < nkeys; ++j) {
    s[j] = score(jb, head, i, j);
    if (s[j] > m) m = s[j];
  }
  for (long long j = 0; j < nkeys; ++j) l += exp(s[j] - m);
  for (long long c = 0; c < d; ++c) o[c] = 0.0;
  for (long long j = 0; j < nkeys; ++j) {
    const double w = exp(s[j] - m) / l;
    for (long long c = 0; c < d; ++c) o[c] += w * ld(jb, jb->v, kb + j * d + c);
  }
  double Di = 0.0;
  for (long long c = 0; c < d; ++c) Di += ld(jb, jb->g, head * Nq * d + i * d + c) * o[c];
  jb->lse[hs * Nq + i] = nkeys > 0 ? m + log(l) : -INFINITY;
  jb->D[hs * Nq + i] = Di;
}

/* dP_ij = <g_i, v_j> (over the d_v columns) */
static double dprob(const bjob_t* jb, long long head, long long i, long long j) {
  const long long d = jb->d_v, qb = head * jb->Nq * d, kb = head * jb->Nk * d;
  double dot = 0.0;
  for (long long c = 0; c < d; ++c)
    dot += ld(jb, jb->g, qb + i * d + c) * ld(jb, jb->v, kb + j * d + c);
  return dot;
}

/* phase 1: dq of flat query row r = head*Nq + i (d_qk columns) */
static void dq_row(const bjob_t* jb, long long t) {
  const long long Nq = jb->Nq, d = jb->d_qk, r = jb->q_rows[t];
  const long long head = r / Nq, i = r % Nq, hs = head_slot(jb, head);
  const long long kb = head * jb->Nk * d;
  const long long nkeys = kept_keys(jb, head, i);
  double* out = jb->dq + t * d;
  for (long long c = 0; c < d; ++c) out[c] = 0.0;
  for (long long j = 0; j < nkeys; ++j) {
    const double P = exp(score(jb, head, i, j) - jb->lse[hs * Nq + i]);
    const double dS = P * (dprob(jb, head, i, j) - jb->D[hs * Nq + i]);
    for (long long c = 0; c < d; ++c) out[c] += dS * ld(jb, jb->k, kb + j * d + c);
  }
  for (long long c = 0; c < d; ++c) out[c] *= jb->scale;
}

/* phase 2: dk and dv of flat key row r = head*Nk + j, summed over the query
 * rows that keep key j */
static void dkv_row(const bjob_t* jb, long long t) {
  const long long Nq = jb->Nq, Nk = jb->Nk, d_qk = jb->d_qk, d_v = jb->d_v, r = jb->k_rows[t];
  const long long head = r / Nk, j = r % Nk, hs = head_slot(jb, head);
  const long long qb = head * Nq * d_qk;  /* query rows */
  const long long gb = head * Nq * d_v;   /* upstream-gradient rows */
  double* dk = jb->dk + t * d_qk;
  double* dv = jb->dv + t * d_v;
  for (long long c = 0; c < d_qk; ++c) dk[c] = 0.0;
  for (long long c = 0; c < d_v; ++c) dv[c] = 0.0;
  for (long long i = 0; i < Nq; ++i) {
    if (j >= kept_keys(jb, head, i)) continue;
    const double P = exp(score(jb, head, i, j) - jb->lse[hs * Nq + i]);
    const double dS = P * (dprob(jb, head, i, j) - jb->D[hs * Nq + i]);
    for (long long c = 0; c < d_v; ++c) dv[c] += P * ld(jb, jb->g, gb + i * d_v + c);
    for (long long c = 0; c < d_qk; ++c) dk[c] += dS * ld(jb, jb->q, qb + i * d_qk + c);
  }
  for (long long c = 0; c < d_qk; ++c) dk[c] *= jb->scale;
}

static void* bworker(void* arg) {
  bjob_t* jb = (bjob_t*)arg;
  double* s = NULL;
  double* o = NULL;
  if (jb->phase == 0) {
    s = (double*)malloc((size_t)jb->Nk * sizeof(double));
    o = (double*)malloc((size_t)jb->d_v * sizeof(double));
    if (!s || !o) {
      free(s);
      free(o);
      return (void*)1;
    }
  }
  for (;;) {
    long long t = __atomic_fetch_add(&jb->next, 1, __ATOMIC_RELAXED);
    if (t >= jb->n_items) break;
    if (jb->phase == 0)
      stats_row(jb, t / jb->Nq, t % jb->Nq, s, o);
    else if (jb->phase == 1)
      dq_row(jb, t);
    else
      dkv_row(jb, t);
  }
  free(s);
  free(o);
  return NULL;
}

static int run_phase(bjob_t* jb, int phase, long long n_items, int threads) {
  jb->phase = phase;
  jb->n_items = n_items;
  jb->next = 0;
  if (n_items == 0) return 0;
  int nt = oracle_thread_count(threads);
  if (nt > n_items) nt = (int)n_items;
  pthread_t* tid = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  if (!tid) return -2;
  int started = 0, failed = 0;
  for (int t = 0; t < nt; ++t) {
    if (pthread_create(&tid[t], NULL, bworker, jb) != 0) break;
    ++started;
  }
  if (started == 0 && bworker(jb) != NULL) failed = 1;
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(tid[t], &ret);
    if (ret != NULL) failed = 1;
  }
  free(tid);
  return (failed && jb->next < n_items) ? -2 : 0;
}

static int cmp_ll(const void* a, const void* b) {
  const long long x = *(const long long*)a, y = *(const long long*)b;
  return (x > y) - (x < y);
}

int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    long long B, long long H, long long N, long long d,
                    double scale, int causal,
                    const long long* q_rows, long long n_q,
                    const long long* k_rows, long long n_k,
                    double* dq_out, double* dk_out, double* dv_out, int threads) {
  return oracle_attn_bwd_ex(q, k, v, dout, dtype, B, H, N, N, d, scale, causal, NULL, q_rows,
                            n_q, k_rows, n_k, dq_out, dk_out, dv_out, threads);
}

int oracle_attn_bwd_ex(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       long long B, long long H, long long Nq, long long Nk, long long d,
                       double scale, int causal, const long long* k_len,
                       const long long* q_rows, long long n_q,
                       const long long* k_rows, long long n_k,
                       double* dq_out, double* dk_out, double* dv_out, int threads) {
  return oracle_attn_bwd_gen(q, k, v, dout, dtype, B, H, Nq, Nk, d, d, scale, causal, k_len,
                             NULL, q_rows, n_q, k_rows, n_k, dq_out, dk_out, dv_out, threads);
}

int oracle_attn_bwd_gen(const void* q, const void* k, const void* v, const void* dout, int dtype,
                        long long B, long long H, long long Nq, long long Nk, long long d_qk,
                        long long d_v, double scale, int causal, const long long* k_len,
                        const long long* q_len, const long long* q_rows, long long n_q,
                        const long long* k_rows, long long n_k,
                        double* dq_out, double* dk_out, double* dv_out, int threads) {
  if (!q || !k || !v || !dout) return -1;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d_qk <= 0 || d_v <= 0 || n_q < 0 || n_k < 0)
    return -1;
  if ((n_q > 0 && (!q_rows || !dq_out)) || (n_k > 0 && (!k_rows || !dk_out || !dv_out)))
    return -1;
  if (causal != 0 && causal != 1) return -1;
  if (dtype < ORACLE_F32 || dtype > ORACLE_F64) return -1;
  for (long long t = 0; t < n_q; ++t)
    if (q_rows[t] < 0 || q_rows[t] >= B * H * Nq) return -1;
  for (long long t = 0; t < n_k; ++t)
    if (k_rows[t] < 0 || k_rows[t] >= B * H * Nk) return -1;
  if (n_q + n_k == 0) return 0;

  /* the heads the requested rows live in, sorted and unique */
  long long* heads = (long long*)malloc((size_t)(n_q + n_k) * sizeof(long long));
  if (!heads) return -2;
  long long nh = 0;
  for (long long t = 0; t < n_q; ++t) heads[nh++] = q_rows[t] / Nq;
  for (long long t = 0; t < n_k; ++t) heads[nh++] = k_rows[t] / Nk;
  qsort(heads, (size_t)nh, sizeof(long long), cmp_ll);
  long long u = 0;
  for (long long t = 0; t < nh; ++t)
    if (u == 0 || heads[t] != heads[u - 1]) heads[u++] = heads[t];
  double* lse = (double*)malloc((size_t)(u * Nq) * sizeof(double));
  double* D = (double*)malloc((size_t)(u * Nq) * sizeof(double));
  if (!lse || !D) {
    free(heads);
    free(lse);
    free(D);
    return -2;
  }
  bjob_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.g = dout; jb.dtype = dtype;
  jb.H = H; jb.Nq = Nq; jb.Nk = Nk; jb.d_qk = d_qk; jb.d_v = d_v;
  jb.scale = scale; jb.causal = causal;
  jb.k_len = k_len;
  jb.q_len = q_len;
  jb.heads = heads; jb.n_heads = u; jb.lse = lse; jb.D = D;
  jb.q_rows = q_rows; jb.k_rows = k_rows; jb.n_q = n_q; jb.n_k = n_k;
  jb.dq = dq_out; jb.dk = dk_out; jb.dv = dv_out;
  int rc = run_phase(&jb, 0, u * Nq, threads);
  if (rc == 0) rc = run_phase(&jb, 1, n_q, threads);
  if (rc == 0) rc = run_phase(&jb, 2, n_k, threads);
  free(heads);
  free(lse);
  free(D);
  return rc;
}

/*
 * oracle.c -- fp64 CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).
 *
 * The definition and its sources are stated in oracle.h.  This file is
 * deliberately plain: one row at a time, three passes over the keys, fp64
 * throughout, no blocking, no fused recurrence.  Threads only split the list
 * of independent rows.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* bf16 is the upper half of an IEEE binary32: widen by placing its 16 bits
 * above 16 zero bits. */
static double bf16_to_f64(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp_bits = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double mag;
  if (exp_bits == 0)
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-10 * 2^-14 */
  else if (exp_bits == 31)
    mag = frac ? NAN : INFINITY;
  else
    mag = ldexp((double)(frac | 0x400), exp_bits - 25); /* 1.frac * 2^(e-15) */
  return sign ? -mag : mag;
}

double oracle_load(const void* base, int dtype, long long idx) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float*)base)[idx];
    case ORACLE_F16: return f16_to_f64(((const uint16_t*)base)[idx]);
    case ORACLE_BF16: return bf16_to_f64(((const uint16_t*)base)[idx]);
    case ORACLE_F64: return ((const double*)base)[idx];
    default: return NAN;
  }
}

int oracle_thread_count(int threads) {
  if (threads > 0) return threads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

typedef struct {
  const void *q, *k, *v;
  int dtype;
  long long H, Nq, Nk, dk, dv; /* head dims: q and k rows dk, v and o rows dv */
  double scale;
  int causal;
  const long long* k_len; /* per-batch valid keys, or NULL (all Nk) */
  const long long* q_len; /* per-batch valid queries, or NULL (all Nq) */
  const long long* rows;
  long long n_rows;
  double *o_out, *lse_out;
  long long next; /* shared work counter, advanced atomically */
} job_t;

/* One query row r = (b*H + h)*Nq + i, three passes.  `qrow` (dk doubles) and
 * `s` (Nk doubles) are this thread's scratch: s holds the row's scaled scores,
 * so passes 2 and 3 reuse the dot products of the score step.  The scores
 * contract the dk columns of q and k; the output has the dv columns of v.
 * The kept keys J_i are a prefix 0 .. nkeys-1 of the head's keys: keys below
 * the batch's valid length L, and, when causal, at most i + (L - Lq), where Lq
 * is the batch's valid query count; a query row at or past Lq keeps none. */
static void one_row(const job_t* jb, long long r, double* qrow, double* s,
                    double* o, double* lse) {
  const long long Nq = jb->Nq, Nk = jb->Nk, dk = jb->dk, dv = jb->dv;
  const long long head = r / Nq;                 /* b*H + h */
  const long long i = r % Nq;                    /* query position */
  const long long b = head / jb->H;
  const long long qbase = head * Nq * dk;        /* this head's query rows */
  const long long kbase = head * Nk * dk;        /* this head's key rows */
  const long long vbase = head * Nk * dv;        /* this head's value rows */
  long long L = jb->k_len ? jb->k_len[b] : Nk;   /* valid keys of this batch */
  if (L < 0) L = 0;
  if (L > Nk) L = Nk;
  long long Lq = jb->q_len ? jb->q_len[b] : Nq;  /* valid queries of this batch */
  if (Lq < 0) Lq = 0;
  if (Lq > Nq) Lq = Nq;
  long long nkeys = i < Lq ? L : 0;              /* |J_i| */
  if (jb->causal && i + (L - Lq) + 1 < nkeys) nkeys = i + (L - Lq) + 1;
  if (nkeys < 0) nkeys = 0;

  for (long long c = 0; c < dv; ++c) o[c] = 0.0;
  if (nkeys == 0) { /* no kept key: the empty sum, o = 0 and lse = ln 0 */
    *lse = -INFINITY;
    return;
  }
  for (long long c = 0; c < dk; ++c)
    qrow[c] = oracle_load(jb->q, jb->dtype, qbase + i * dk + c);

  /* scores s_j = scale * <q_i, k_j> for j in J_i */
  for (long long j = 0; j < nkeys; ++j) {
    double dot = 0.0;
    for (long long c = 0; c < dk; ++c)
      dot += qrow[c] * oracle_load(jb->k, jb->dtype, kbase + j * dk + c);
    s[j] = jb->scale * dot;
  }

  /* pass 1: the row maximum m */
  double m = -INFINITY;
  for (long long j = 0; j < nkeys; ++j)
    if (s[j] > m) m = s[j];

  /* pass 2: the denominator l = sum exp(s_j - m) */
  double l = 0.0;
  for (long long j = 0; j < nkeys; ++j) l += exp(s[j] - m);

  /* pass 3: o = sum (exp(s_j - m) / l) v_j */
  for (long long j = 0; j < nkeys; ++j) {
    const double w = exp(s[j] - m) / l;
    for (long long c = 0; c < dv; ++c)
      o[c] += w * oracle_load(jb->v, jb->dtype, vbase + j * dv + c);
  }
  *lse = m + log(l);
}

static void* worker(void* arg) {
  job_t* jb = (job_t*)arg;
  double* qrow = (double*)malloc((size_t)jb->dk * sizeof(double));
  double* s = (double*)malloc((size_t)jb->Nk * sizeof(double));
  if (!qrow || !s) {
    free(qrow);
    free(s);
    return (void*)1;
  }
  for (;;) {
    long long t = __atomic_fetch_add(&jb->next, 1, __ATOMIC_RELAXED);
    if (t >= jb->n_rows) break;
    one_row(jb, jb->rows[t], qrow, s, jb->o_out + t * jb->dv, jb->lse_out + t);
  }
  free(qrow);
  free(s);
  return NULL;
}

int oracle_attn_rows(const void* q, const void* k, const void* v, int dtype,
                     long long B, long long H, long long N, long long d,
                     double scale, int causal,
                     const long long* rows, long long n_rows,
                     double* o_out, double* lse_out, int threads) {
  return oracle_attn_rows_ex(q, k, v, dtype, B, H, N, N, d, scale, causal, NULL, rows, n_rows,
                             o_out, lse_out, threads);
}

int oracle_attn_rows_ex(const void* q, const void* k, const void* v, int dtype,
                        long long B, long long H, long long Nq, long long Nk, long long d,
                        double scale, int causal, const long long* k_len,
                        const long long* rows, long long n_rows,
                        double* o_out, double* lse_out, int threads) {
  return oracle_attn_rows_gen(q, k, v, dtype, B, H, Nq, Nk, d, d, scale, causal, k_len, NULL,
                              rows, n_rows, o_out, lse_out, threads);
}

int oracle_attn_rows_gen(const void* q, const void* k, const void* v, int dtype,
                         long long B, long long H, long long Nq, long long Nk, long long dk,
                         long long dv, double scale, int causal, const long long* k_len,
                         const long long* q_len, const long long* rows, long long n_rows,
                         double* o_out, double* lse_out, int threads) {
  if (!q || !k || !v || !o_out || !lse_out || (n_rows > 0 && !rows)) return -1;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || dk <= 0 || dv <= 0 || n_rows < 0) return -1;
  if (causal != 0 && causal != 1) return -1;
  if (dtype < ORACLE_F32 || dtype > ORACLE_F64) return -1;
  const long long total = B * H * Nq;
  for (long long t = 0; t < n_rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return -1;
  if (n_rows == 0) return 0;

  job_t jb = {q, k, v, dtype, H, Nq, Nk, dk, dv, scale, causal, k_len, q_len, rows, n_rows,
              o_out, lse_out, 0};
  int nt = oracle_thread_count(threads);
  if (nt > n_rows) nt = (int)n_rows;
  pthread_t* tid = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  if (!tid) return -2;
  int started = 0, failed = 0;
  for (int t = 0; t < nt; ++t) {
    if (pthread_create(&tid[t], NULL, worker, &jb) != 0) break;
    ++started;
  }
  if (started == 0) { /* no thread could start: do the work here */
    if (worker(&jb) != NULL) failed = 1;
  }
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(tid[t], &ret);
    if (ret != NULL) failed = 1;
  }
  free(tid);
  /* A worker that could not get its scratch leaves its rows to the others;
   * only when every row was taken is the result complete. */
  if (failed && jb.next < n_rows) return -2;
  return 0;
}

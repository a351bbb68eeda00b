/*
 * oracle.h -- fp64 CPU oracle for exact scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker, not the product:
 * only the test suite, the package smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no source, header or build step with
 * the GPU library, and it never calls into it.
 *
 * What it computes (for each requested row r = (b, h, i) of a [B,H,N,d]
 * problem) is the definition of attention written out, in the order of the
 * three-pass safe softmax:
 *
 *   J_i  = {0..N-1}              (non-causal)
 *        = {0..i}                (causal: key j kept iff j <= i)
 *   s_j  = scale * sum_k q[b,h,i,k] * k[b,h,j,k]        for j in J_i
 *   m    = max_{j in J_i} s_j                            (pass 1)
 *   l    = sum_{j in J_i} exp(s_j - m)                   (pass 2)
 *   o    = sum_{j in J_i} (exp(s_j - m) / l) * v[b,h,j,:] (pass 3)
 *   lse  = m + ln(l)
 *
 * Sources: softmax(Q K^T / sqrt(d_k)) V -- "FlashAttention Engine" (the
 * attention equation) and "The Details of Flash Attention" (section "The
 * Attention Computation", eqs. 1-4); the three passes -- "The Details of
 * Flash Attention", section "Safe Softmax and the Three Passes"; the causal
 * mask as -inf fill of excluded scores -- "Transformer Attention: A
 * Mathematical Deep Dive" (the PyTorch ScaledDotProductAttention listing);
 * the per-row statistics kept for the backward pass (m and l) --
 * "FlashAttention" (ai360xpert), section "Recomputation in the backward pass".
 *
 * All arithmetic is IEEE fp64 with plain left-to-right summation.  Inputs of
 * lower precision are widened exactly (bf16 and fp16 by their bit-level
 * definitions, fp32 by a C cast).
 */
#ifndef ORACLE_ATTN_H
#define ORACLE_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes of the input arrays (this library's own numbering). */
enum {
  ORACLE_F32 = 0,
  ORACLE_F16 = 1,
  ORACLE_BF16 = 2,
  ORACLE_F64 = 3
};

/*
 * oracle_attn_rows
 *   q, k, v : host pointers to contiguous row-major [B][H][N][d] arrays, all of
 *             element type `dtype`.
 *   rows    : host array of n_rows flat row ids r = (b*H + h)*N + i, each in
 *             [0, B*H*N).  Rows are independent, so any subset is exact for the
 *             rows it names.
 *   o_out   : host [n_rows][d] fp64, written.
 *   lse_out : host [n_rows] fp64 (natural log, scaled-score units), written.
 *   threads : worker threads (<= 0 means one per online CPU).
 * Returns 0 on success, -1 on an invalid argument (nothing written), -2 when
 * memory for the per-thread scratch rows cannot be obtained.
 * The call is synchronous; the caller owns every buffer.
 */
int oracle_attn_rows(const void* q, const void* k, const void* v, int dtype,
                     long long B, long long H, long long N, long long d,
                     double scale, int causal,
                     const long long* rows, long long n_rows,
                     double* o_out, double* lse_out, int threads);

/*
 * oracle_attn_rows_ex -- the same definition for query and key sequences of
 * different lengths and per-batch padding of the keys (the n x m scores and
 * the "causal attention or padding" mask of the ScaledDotProductAttention
 * listing in "Transformer Attention: A Mathematical Deep Dive"):
 *   q : [B][H][Nq][d];  k, v : [B][H][Nk][d];  rows (b*H + h)*Nq + i.
 *   k_len : host array of B valid key counts (each clamped to [0, Nk]), or
 *           NULL for Nk.  With L = the batch's count,
 *           J_i = {j < L}                      (non-causal)
 *               = {j < L, j <= i + (L - Nq)}   (causal, bottom-right aligned:
 *                                               the last query sees every
 *                                               valid key; Nq = Nk = L gives
 *                                               the lower triangle)
 *   A row with J_i empty gets o = 0 and lse = -inf (the empty sum).
 * oracle_attn_rows is this with Nq = Nk = N and k_len = NULL.
 */
int oracle_attn_rows_ex(const void* q, const void* k, const void* v, int dtype,
                        long long B, long long H, long long Nq, long long Nk, long long d,
                        double scale, int causal, const long long* k_len,
                        const long long* rows, long long n_rows,
                        double* o_out, double* lse_out, int threads);

/*
 * oracle_attn_rows_gen -- oracle_attn_rows_ex with the value head dim apart
 * from the query/key one (Q of shape (n, d_k), K (m, d_k), V (m, d_v):
 * "Transformer Attention: A Mathematical Deep Dive", the scaled dot-product
 * attention definition) and per-batch padding of the queries too:
 * q [B][H][Nq][dk], k [B][H][Nk][dk], v [B][H][Nk][dv]; the scores contract
 * the dk columns, o_out is [n_rows][dv].
 *   q_len : host array of B valid query counts (each clamped to [0, Nq]), or
 *           NULL for Nq.  With Lq the batch's query count and L its key count,
 *           J_i = {}                            (i >= Lq: a padding row)
 *               = {j < L}                       (non-causal)
 *               = {j < L, j <= i + (L - Lq)}    (causal: the last valid query
 *                                                sees every valid key)
 * oracle_attn_rows_ex is this with dk = dv = d and q_len = NULL.
 */
int oracle_attn_rows_gen(const void* q, const void* k, const void* v, int dtype,
                         long long B, long long H, long long Nq, long long Nk, long long dk,
                         long long dv, double scale, int causal, const long long* k_len,
                         const long long* q_len, const long long* rows, long long n_rows,
                         double* o_out, double* lse_out, int threads);

/*
 * oracle_attn_bwd -- gradients of the same attention (oracle_bwd.c):
 * for an upstream gradient dout = dL/do ([B][H][N][d], type `dtype`), the
 * gradients dL/dq of the query rows q_rows (flat ids (b*H + h)*N + i) and
 * dL/dk, dL/dv of the key rows k_rows (flat ids (b*H + h)*N + j), fp64,
 * written to dq_out [n_q][d], dk_out [n_k][d], dv_out [n_k][d].  Rows of one
 * head need that head's per-row statistics, computed once per touched head.
 * Returns 0, -1 (invalid argument, nothing written) or -2 (no memory).
 */
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    long long B, long long H, long long N, long long d,
                    double scale, int causal,
                    const long long* q_rows, long long n_q,
                    const long long* k_rows, long long n_k,
                    double* dq_out, double* dk_out, double* dv_out, int threads);

/*
 * oracle_attn_bwd_ex -- the gradients of oracle_attn_rows_ex's attention
 * (query rows (b*H + h)*Nq + i, key rows (b*H + h)*Nk + j, k_len as there):
 * the same chain rule summed over the kept pairs only.  A query row that
 * keeps no key has dq = 0; a key that no query keeps has dk = dv = 0.
 * oracle_attn_bwd is this with Nq = Nk = N and k_len = NULL.
 */
int oracle_attn_bwd_ex(const void* q, const void* k, const void* v, const void* dout, int dtype,
                       long long B, long long H, long long Nq, long long Nk, long long d,
                       double scale, int causal, const long long* k_len,
                       const long long* q_rows, long long n_q,
                       const long long* k_rows, long long n_k,
                       double* dq_out, double* dk_out, double* dv_out, int threads);

/*
 * oracle_attn_bwd_gen -- the gradients of oracle_attn_rows_gen's attention:
 * q [B][H][Nq][dk], k [B][H][Nk][dk], v [B][H][Nk][dv], dout [B][H][Nq][dv];
 * dq_out [n_q][dk], dk_out [n_k][dk], dv_out [n_k][dv].  dP_ij = <g_i, v_j>
 * and D_i = <g_i, o_i> contract the dv columns, the scores and dq, dk the dk
 * columns; q_len as in oracle_attn_rows_gen (a padding query row has dq = 0
 * and adds nothing to dk, dv).  oracle_attn_bwd_ex is this with dk = dv = d
 * and q_len = NULL.
 */
int oracle_attn_bwd_gen(const void* q, const void* k, const void* v, const void* dout, int dtype,
                        long long B, long long H, long long Nq, long long Nk, long long dk,
                        long long dv, double scale, int causal, const long long* k_len,
                        const long long* q_len, const long long* q_rows, long long n_q,
                        const long long* k_rows, long long n_k,
                        double* dq_out, double* dk_out, double* dv_out, int threads);

/* Number of threads a call with `threads` would use. */
int oracle_thread_count(int threads);

/* Widen one element of type `dtype` at index `idx` of `base` to fp64. */
double oracle_load(const void* base, int dtype, long long idx);

#ifdef __cplusplus
}
#endif
#endif /* ORACLE_ATTN_H */

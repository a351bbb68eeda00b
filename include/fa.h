/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention library, libfa.so: the
 * forward pass and its gradients.
 *
 * The one operation is exact scaled dot-product attention,
 *     O = softmax(scale * Q K^T) V          (softmax over each query row),
 * as defined in "FlashAttention Engine" (the attention equation) and "The
 * Details of Flash Attention" (section "The Attention Computation", eqs. 1-4),
 * computed tile by tile with the online-softmax recurrence ("The Details of
 * Flash Attention", sections "Online Softmax" and "Tiling the Loop"; "Deep
 * Learning - Flash Attention", section "An Example", steps 4-6) so that the
 * N x N score matrix never exists in device memory.  Alongside O the library
 * writes the per-row log-sum-exp, the statistic a recomputing backward pass
 * needs ("FlashAttention" (ai360xpert), section "Recomputation in the backward
 * pass").
 *
 * No function here allocates or frees device memory or synchronizes.  The
 * only state kept between calls is a fixed table of work-counter slots in
 * the library's code object (see fa_fwd, "Scheduling").  No C++ exception
 * crosses this boundary.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
  FA_DTYPE_FP32 = 0,
  FA_DTYPE_FP16 = 1,
  FA_DTYPE_BF16 = 2
} fa_dtype_t;

/* Return codes. */
typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, causal not 0/1,
                             non-finite or non-positive scale, size overflow */
  FA_ERR_UNSUPPORTED = 2, /* head dim or dtype without a kernel, pointer not
                             16-byte aligned */
  FA_ERR_HIP = 3,         /* the kernel launch reported an error */
  FA_ERR_SCRATCH = 4      /* fa_fwd_gen_noalloc: the problem's key split needs
                             more than FA_NOALLOC_SCRATCH_BYTES of scratch */
} fa_status_t;

/*
 * fa_fwd -- attention forward pass on one GPU.
 *
 *   q, k, v : device pointers, contiguous row-major [B][H][N][d] arrays of
 *             element type `dtype` (the (batch, head, sequence, head-dim) order
 *             of "The Details of Flash Attention", section "The Attention
 *             Computation").  Batches and heads are independent problems.
 *   o       : device pointer, [B][H][N][d] of the same type, written: row i of
 *             head (b, h) is sum_j softmax_j(scale * q_i . k_j) v_j, rounded
 *             from fp32 to the element type (round to nearest even).
 *   lse     : device pointer, [B][H][N] fp32, written:
 *             lse_i = ln sum_{j kept} exp(scale * q_i . k_j)  (natural log,
 *             scaled-score units, masked keys excluded).
 *   B, H, N, d : batch, heads, sequence length (queries = keys = N), head dim.
 *   scale   : multiplies q_i . k_j before the softmax (callers normally pass
 *             1/sqrt(d)).  Applied to the fp32 scores, never folded into q.
 *   causal  : 0 = every key is kept; 1 = key j is kept for query i iff j <= i
 *             (lower-triangular mask with the diagonal; excluded scores behave
 *             as -inf, i.e. contribute exactly zero weight).
 *   dtype   : fa_dtype_t.  Supported head dims: bf16 and fp16 -- 64, 128;
 *             fp32 -- 64, 128, 256, 512, 1024.
 *   stream  : a hipStream_t passed as void*; NULL means the null stream.
 *
 * Ownership: the caller allocates and owns every buffer; q, k, v are only
 * read; o and lse must not overlap q, k, v or each other.  The call is
 * asynchronous on `stream` and returns once the kernel is enqueued; results
 * are valid after the stream is synchronized.
 *
 * Errors: every argument is checked before any HIP call.  On any error code
 * nothing is launched and o, lse are not written.  FA_ERR_HIP is returned when
 * hipGetLastError reports a failure right after the launch.
 *
 * Arithmetic: scores and all softmax statistics are fp32; bf16/fp16 products
 * accumulate in fp32 on the matrix cores; probabilities are rounded to the
 * input type before the product with V.  Results are bitwise reproducible run
 * to run (fixed reduction order, which depends only on the shape, the dtype
 * and the device's compute-unit count).
 *
 * Scheduling: at head dim 128 (bf16/fp16) one workgroup per compute unit
 * claims work items through atomic counters kept in the library's code
 * object: 64 counter slots per device, drawn round-robin per call.  A slot
 * belongs to one launch at a time, which the device identifies by a tag
 * derived from the launch's dispatch packet (its address and dispatch id);
 * the last workgroup of the owning launch clears the counters and frees the
 * slot.  A launch whose slot is held by another launch still in flight (a
 * captured call replayed beside a later call that drew the same slot, or
 * more than 64 calls in flight on one device) runs its items in a fixed
 * per-workgroup order instead, without the counters.  Which workgroup
 * computes an item never changes the result, so calls may overlap freely,
 * captured or not.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_workspace_size -- device workspace, in bytes, that fa_fwd_ws can use
 * for this problem on the current device; 0 when it would run exactly as
 * fa_fwd does.  Nonzero only for problems whose (query block, head, batch)
 * items are fewer than the device holds at once (fp32: 32-row blocks against
 * the compute units; 16-bit: 256-row blocks at d = 128, one per compute
 * unit, 128-row blocks at d = 64, three per compute unit): fa_fwd_ws then
 * splits each query block's keys into ranges, computes the softmax-weighted
 * output and log-sum-exp of every range in its own workgroup, and merges the
 * ranges with lse = ln sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s ("The
 * Details of Flash Attention", section "Online Softmax": partial softmax
 * results over disjoint key sets combine exactly; "FlashAttention Engine",
 * "Core FlashAttention Mechanics", item 3, the same merge of two blocks).
 * Returns 0 for invalid or unsupported arguments.
 */
size_t fa_fwd_workspace_size(int B, int H, int N, int d, int causal, int dtype);

/*
 * fa_fwd_ws -- fa_fwd with a caller-owned device workspace.  Same arguments,
 * outputs, errors and asynchrony as fa_fwd, plus:
 *   workspace       : device pointer, 16-byte aligned, used as scratch by the
 *                     call (contents on entry ignored, on return undefined);
 *                     it must stay allocated until the stream has run the
 *                     call, and must not overlap q, k, v, o or lse.
 *   workspace_bytes : its size.  NULL or 0 runs exactly as fa_fwd.  Otherwise
 *                     it must be >= fa_fwd_workspace_size(...) for the same
 *                     problem on the same device, else FA_ERR_INVALID_ARG
 *                     (a misaligned workspace gives FA_ERR_UNSUPPORTED).
 * The key-split result equals fa_fwd's up to rounding (the merge adds one
 * rounding per range, and 16-bit ranges keep their partial output in fp32);
 * it is bitwise reproducible run to run.
 */
int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_ex -- fa_fwd for query and key sequences of different lengths and
 * per-batch key padding: the n x m scores and the "causal attention or
 * padding" mask of the ScaledDotProductAttention listing in "Transformer
 * Attention: A Mathematical Deep Dive" (query (batch, n, d_k), key and value
 * (batch, m, d)).
 *   q, o    : device pointers, [B][H][Nq][d];  lse: [B][H][Nq] fp32.
 *   k, v    : device pointers, [B][H][Nk][d].
 *   k_len   : device pointer to B int32 valid key counts (4-byte aligned;
 *             each clamped to [0, Nk] when read), or NULL for Nk.  With L the
 *             batch's count, key j is kept for query i iff j < L and, when
 *             causal, j <= i + (L - Nq): the last query row is aligned with
 *             the last valid key (Nq = Nk = L gives the lower triangle).
 *             Keys at or past L are never read.
 *   workspace, workspace_bytes : as for fa_fwd_ws, sized by
 *             fa_fwd_ex_workspace_size for the same shapes.
 * A query row with no kept key (L = 0, or causal with i + L - Nq < 0) gets
 * O = 0 and lse = -inf: the empty sum.  Everything else -- arguments,
 * ownership, errors, asynchrony, arithmetic -- is as for fa_fwd; fa_fwd is
 * fa_fwd_ex with Nq = Nk = N, k_len = NULL and no workspace.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
              const int* k_len, void* workspace, size_t workspace_bytes, void* stream);

/* fa_fwd_workspace_size for fa_fwd_ex's shapes (0: none needed, or invalid). */
size_t fa_fwd_ex_workspace_size(int B, int H, int Nq, int Nk, int d, int causal, int dtype);

/*
 * fa_fwd_gen -- fa_fwd_ex with the value head dim apart from the query/key
 * one: Q of shape (n, d_k), K (m, d_k) and V (m, d_v), as the scaled
 * dot-product attention of "Transformer Attention: A Mathematical Deep Dive"
 * is defined.  The scores contract the d_qk columns; O has the d_v columns.
 *   q : [B][H][Nq][d_qk];  k : [B][H][Nk][d_qk];  v : [B][H][Nk][d_v];
 *   o : [B][H][Nq][d_v];   lse : [B][H][Nq] fp32.
 * Supported pairs: fa_fwd_gen_supported (d_qk = d_v as for fa_fwd; otherwise
 * d_qk, d_v in {64, 128} for bf16, fp16 and fp32).  The workspace is sized by
 * fa_fwd_gen_workspace_size.
 *   q_len : per-batch padding of the queries too (the same padding mask):
 *           device pointer to B int32 valid query counts (4-byte aligned; each
 *           clamped to [0, Nq] when read), or NULL for Nq.  With Lq the
 *           batch's count and L its key count, query row i < Lq keeps key j
 *           iff j < L and, when causal, j <= i + (L - Lq): the last valid
 *           query is aligned with the last valid key.  A row at or past Lq is
 *           padding: O = 0, lse = -inf, and its q row is never read.  NULL
 *           gives fa_fwd_ex's rule (Lq = Nq).
 * Everything else is as for fa_fwd_ex, which is fa_fwd_gen with
 * d_qk = d_v = d and q_len = NULL.  scale is the caller's (1/sqrt(d_qk) is
 * the usual choice).
 */
int fa_fwd_gen(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int d_qk, int d_v, float scale, int causal,
               int dtype, const int* k_len, const int* q_len, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * fa_fwd_gen_noalloc -- fa_fwd_gen for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It calls no allocating routine.  Where fa_fwd_gen would
 * split keys into a caller workspace (grids smaller than the device holds
 * at once), this call uses a scratch array of FA_NOALLOC_SCRATCH_BYTES that
 * the library's code object holds on every device it runs on, for the life
 * of the process.  Arguments, outputs, errors and asynchrony are those of
 * fa_fwd_gen without the workspace; the results equal fa_fwd_gen's with a
 * workspace of fa_fwd_gen_workspace_size bytes, bit for bit.
 *   Returns FA_ERR_SCRATCH (nothing launched) when that workspace size
 *   exceeds FA_NOALLOC_SCRATCH_BYTES.
 *   Every split call on one device uses the same scratch: calls that overlap
 *   in time on one device (other streams, concurrent graph replays) race on
 *   it and must be serialized by the caller.  Calls whose grids need no
 *   split do not touch the scratch.  Its contents are never read before the
 *   same call writes them.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_fwd_gen_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Nq, int Nk, int d_qk, int d_v, float scale,
                       int causal, int dtype, const int* k_len, const int* q_len,
                       void* stream);

/* fa_fwd_ex_workspace_size for fa_fwd_gen's shapes (0: none needed, or invalid). */
size_t fa_fwd_gen_workspace_size(int B, int H, int Nq, int Nk, int d_qk, int d_v, int causal,
                                 int dtype);

/* 1 when fa_fwd_gen has a kernel for (d_qk, d_v, dtype, causal), else 0. */
int fa_fwd_gen_supported(int d_qk, int d_v, int dtype, int causal);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs for this
 * problem: two fp32 row statistics per (batch, head, row), rows padded to a
 * multiple of 32; for problems with fewer query or key blocks than the
 * current device holds at once (fp32: 32-row blocks against its compute
 * units; 16-bit: 128-key blocks and 256-row query blocks, 128 at d = 64,
 * against the eight waves a compute unit holds, twelve at d = 64), also the
 * fp32 partial sums of the split that spreads each block's work over several
 * workgroups.  Depends on the current device.
 * 0 for invalid or unsupported arguments.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal, int dtype);

/*
 * fa_bwd -- gradients of the attention fa_fwd computes, on one GPU.
 *
 * Given the forward inputs q, k, v, its outputs o and lse, and dout = dL/dO,
 * writes for every (batch, head), with P_ij = exp(scale q_i.k_j - lse_i) over
 * the kept pairs (j <= i when causal) and delta_i = dout_i . o_i:
 *   dv_j = sum_i P_ij dout_i
 *   dq_i = scale sum_j P_ij (dout_i . v_j - delta_i) k_j
 *   dk_j = scale sum_i P_ij (dout_i . v_j - delta_i) q_i
 * -- the chain rule through O = P V and the row softmax, with P recomputed
 * tile by tile from the stored log-sum-exp instead of being kept ("FlashAttention"
 * (ai360xpert), section "Recomputation in the backward pass"; the softmax and
 * attention definitions of "The Details of Flash Attention", eqs. 1-4).
 *
 *   q, k, v, o, dout : device pointers, contiguous [B][H][N][d] of `dtype`;
 *                      o and lse as written by fa_fwd for the same q, k, v,
 *                      scale and causal (any o, lse are accepted; the
 *                      formulas above use them as given).
 *   lse             : device pointer, [B][H][N] fp32 (natural log).
 *   dq, dk, dv      : device pointers, [B][H][N][d] of `dtype`, written
 *                     (fp32, or rounded from fp32 to nearest even for the
 *                     16-bit types).  They must not
 *                     overlap the inputs or each other.
 *   B, H, N, d, scale, causal, dtype : as for fa_fwd.  Supported: bf16 and
 *                     fp16 with d = 64 or 128; fp32 with d = 64, 128, 256,
 *                     512 or 1024.
 *   workspace       : device pointer, 16-byte aligned, at least
 *                     fa_bwd_workspace_size(...) bytes (else
 *                     FA_ERR_INVALID_ARG); contents on entry ignored, on
 *                     return undefined; must stay allocated until the stream
 *                     has run the call.
 *   stream          : a hipStream_t passed as void*; NULL = the null stream.
 *
 * Asynchronous on `stream`; allocates nothing.  Every argument is checked
 * before any HIP call; on an error code nothing is launched and no output is
 * written.  Arithmetic: products of 16-bit operands accumulate in fp32; P and
 * dS are rounded to the element type before their products.  fp32 operands
 * take fp32 products throughout (no reduced-precision inputs).  No atomics: the
 * result is bitwise reproducible run to run (the order of every sum depends
 * only on the shape, the dtype and the device's compute-unit count).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * fa_bwd_ex -- fa_bwd for fa_fwd_ex's shapes: q, o, dout, dq are
 * [B][H][Nq][d], k, v, dk, dv [B][H][Nk][d], lse [B][H][Nq]; k_len as for
 * fa_fwd_ex (NULL: all Nk keys valid).  The sums run over the kept pairs of
 * fa_fwd_ex: a query row that keeps no key gets dq = 0, a key no query keeps
 * (padding, or past every row's causal limit) gets dk = dv = 0 -- every row of
 * dq, dk and dv is written.  The workspace must hold
 * fa_bwd_ex_workspace_size(...) bytes.  fa_bwd is fa_bwd_ex with Nq = Nk = N
 * and k_len = NULL; everything else is as for fa_bwd.
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d,
              float scale, int causal, int dtype, const int* k_len, void* workspace,
              size_t workspace_bytes, void* stream);

/* Workspace of fa_bwd_ex: two fp32 statistics per (batch, head, query row),
 * rows padded to a multiple of 32, plus the partial sums of fa_bwd_workspace_size
 * for small fp32 grids; 0 for invalid or unsupported arguments. */
size_t fa_bwd_ex_workspace_size(int B, int H, int Nq, int Nk, int d, int causal, int dtype);

/* 1 when fa_bwd has kernels for (d, dtype, causal), else 0. */
int fa_bwd_supported(int d, int dtype, int causal);

/*
 * fa_bwd_gen -- the gradients of fa_fwd_gen's attention (value head dim
 * apart from the query/key one): q, dq [B][H][Nq][d_qk]; k, dk
 * [B][H][Nk][d_qk]; v, dv [B][H][Nk][d_v]; o, dout [B][H][Nq][d_v]; lse
 * [B][H][Nq].  dP_ij = dout_i . v_j and delta_i = dout_i . o_i contract the
 * d_v columns; the scores, dq and dk the d_qk columns.  Supported pairs:
 * fa_bwd_gen_supported (d_qk = d_v as for fa_bwd; otherwise d_qk, d_v in
 * {64, 128} for bf16, fp16 and fp32).  The workspace must hold
 * fa_bwd_gen_workspace_size(...) bytes.  q_len as for fa_fwd_gen: a padding
 * query row (i >= Lq) gets dq = 0 and adds nothing to dk, dv; its q, o, dout
 * and lse entries are never read.  Everything else is as for fa_bwd_ex,
 * which is fa_bwd_gen with d_qk = d_v = d and q_len = NULL.
 */
int fa_bwd_gen(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
               int d_qk, int d_v, float scale, int causal, int dtype, const int* k_len,
               const int* q_len, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of fa_bwd_gen (as fa_bwd_ex_workspace_size, for both head dims). */
size_t fa_bwd_gen_workspace_size(int B, int H, int Nq, int Nk, int d_qk, int d_v, int causal,
                                 int dtype);

/* 1 when fa_bwd_gen has kernels for (d_qk, d_v, dtype, causal), else 0. */
int fa_bwd_gen_supported(int d_qk, int d_v, int dtype, int causal);

/* 1 when fa_fwd has a kernel for (d, dtype, causal), else 0. */
int fa_fwd_supported(int d, int dtype, int causal);

/* Static description of a status code ("ok", "invalid argument", ...). */
const char* fa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch (400: 0.4.0). */
int fa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_H */

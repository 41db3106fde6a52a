/*
 * pkm.h -- C ABI of the product-key memory (PKM) layer for AMD Instinct MI355X
 * (gfx950).  Forward and backward of one memory layer, as described in
 * "Large Memory Layers with Product Keys" (Lample et al., 2019); the pages
 * cited below are the summary on gptget.net (section "Methodology" and the
 * methodology list of its "Deep Analysis") and the companion page "Product
 * Keys Give Transformers Million-Slot Memory Layers" (sections "Implied keys
 * vs stored sub-keys", "Why top-k of each half is enough", "Search cost: flat
 * vs product keys").
 *
 * Notation: T tokens, H heads, n sub-keys per codebook (n*n memory slots),
 * k selected slots per head, d_k query width per head (half = d_k / 2),
 * d_v value width.  Slot f = i*n + j is the implied key made of left sub-key i
 * followed by right sub-key j.
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller, row-major
 *    and contiguous, 16-byte aligned, and must not alias one another.  The
 *    problem descriptor `p` is a HOST pointer, read during the call only.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  All work
 *    is enqueued on it; no call synchronises with the host.
 *  - The library allocates no memory and keeps no state between calls; it is
 *    re-entrant.  Scratch memory comes from the caller's `workspace`, sized by
 *    pkm_workspace_bytes() -- except for pkm_backward_noalloc, whose scratch is
 *    a static device array of the library (see there).
 *  - Arguments are validated completely before anything is enqueued.  On any
 *    error a non-zero status is returned and NOTHING has been enqueued.  A
 *    launch failure reported by the HIP runtime returns PKM_ERR_HIP (work
 *    enqueued before it may still run).
 *  - T == 0 is a successful no-op (pkm_backward and pkm_backward_queries still
 *    overwrite dkeys with zeros).  A pointer to an array with no elements may
 *    be NULL.
 *  - Supported shapes (else PKM_ERR_SHAPE): H in [1, 64]; n in [1, 1024];
 *    k in [1, min(n, 64)]; d_k in [16, 1024] and a multiple of 16; d_v >= 8
 *    and a multiple of 8; for pkm_backward additionally d_v <= 4096.
 *  - Inputs must be finite; the result for NaN or Inf inputs is unspecified.
 */
#ifndef PKM_H
#define PKM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, keys, values, y and dy.  Arithmetic is float32
 * (products of bfloat16 operands are exact in float32), except the sub-key
 * scores of float32 storage: float64 sums, each rounded once to float32. */
typedef enum { PKM_FP32 = 0, PKM_BF16 = 1 } pkm_dtype_t;

typedef enum {
    PKM_OK = 0,
    PKM_ERR_NULL = 1,      /* a required pointer is NULL                         */
    PKM_ERR_SHAPE = 2,     /* a size outside the supported range                 */
    PKM_ERR_DTYPE = 3,     /* unknown dtype                                      */
    PKM_ERR_WORKSPACE = 4, /* workspace smaller than pkm_workspace_bytes()       */
    PKM_ERR_HIP = 5,       /* the HIP runtime rejected a launch                  */
    PKM_ERR_ALIGN = 6,     /* an array pointer is not 16-byte aligned            */
    PKM_ERR_ARG = 7,       /* a scalar argument outside its domain (learning
                              rate, Adam constants, step)                        */
    PKM_ERR_TOO_LARGE = 8  /* pkm_backward_noalloc: the problem needs more than
                              its static scratch holds                           */
} pkm_status_t;

/* Or-ed into pkm_problem_t.dtype: ONE pair of codebooks serves every head
 * (gptget.net summary, "Technical Contribution": the heads differ in their
 * query mappings).  keys is then [2][n][d_k/2] instead of [H][2][n][d_k/2],
 * and dkeys [2][n][d_k/2] holds the sub-key gradient summed over the heads.
 * Every entry point that takes keys or dkeys accepts it; the others ignore it. */
#define PKM_KEYS_SHARED 0x100

/* Problem sizes.  32 bytes, no padding: T, then six int32 fields. */
typedef struct {
    int64_t T;      /* tokens (>= 0)                                          */
    int32_t H;      /* heads                                                  */
    int32_t n;      /* sub-keys per codebook; the memory has n*n slots        */
    int32_t k;      /* slots selected per head (also the per-half top-k)      */
    int32_t d_k;    /* query width per head; halves of d_k/2                  */
    int32_t d_v;    /* value row width                                        */
    int32_t dtype;  /* pkm_dtype_t, optionally | PKM_KEYS_SHARED              */
} pkm_problem_t;

/* Bytes of device workspace pkm_forward and pkm_forward_select (backward = 0),
 * pkm_backward and its stages (backward = 1) or pkm_backward_sgd
 * (backward = 2) need for this problem; 0 if none (the workspace may then be
 * NULL).  Returns (size_t)-1 for an invalid descriptor or another value of
 * `backward`.  The forward needs workspace only on its two-kernel selection
 * path (d_k = 512, k <= 32, and 128 <= n <= 1024 for bf16 storage,
 * 128 <= n <= 256 for float32): T*H*2*k*8 bytes rounded up to 256, for the
 * per-half top-k lists. */
size_t pkm_workspace_bytes(const pkm_problem_t *p, int backward);

/*
 * Forward pass (gptget.net summary, "Methodology"; companion page, "Why top-k
 * of each half is enough").  For every token t and head h:
 *   1. split q[t][h] into q1 = first half, q2 = second half;
 *   2. score q1 against the n left sub-keys and q2 against the n right
 *      sub-keys (inner products: float32 sums for bf16 storage; for float32
 *      storage float64 sums, each score rounded once to float32);
 *   3. keep the exact top-k of each half, ordered (score desc, index asc);
 *   4. combine: the score of slot (i, j) is left_i + right_j; keep the k best
 *      slots by (score desc, slot asc) -- the same set as a flat search over
 *      all n*n implied keys;
 *   5. weights = softmax of the k selected scores;
 * and y[t] = sum over heads and picks of weight * values[slot].
 *
 *   q        [T][H][d_k]        dtype   (q1 = first d_k/2 of each head)
 *   keys     [H][2][n][d_k/2]   dtype   ([h][0] left codebook, [h][1] right;
 *                                       [2][n][d_k/2] with PKM_KEYS_SHARED)
 *   values   [n*n][d_v]         dtype   (row f = i*n + j)
 *   y        [T][d_v]           dtype   OUT, overwritten (float32 sums,
 *                                       rounded to nearest-even for bf16)
 *   idx      [T][H][k]          int32   OUT, slots in (score desc, slot asc)
 *   weights  [T][H][k]          float32 OUT, softmax weights
 *   scores   [T][H][k]          float32 OUT, selected scores; may be NULL
 */
pkm_status_t pkm_forward(const pkm_problem_t *p, const void *q, const void *keys,
                         const void *values, void *y, int32_t *idx, float *weights,
                         float *scores, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Backward pass for an upstream gradient dy = dL/dy (gptget.net summary,
 * "Methodology": the whole layer is trained by backprop and only the selected
 * memory slots receive a value update).  The selection is held fixed; with
 * w = weights and picks (t, h, r) of slot f = idx[t][h][r] = i*n + j:
 *   dw     = <dy[t], values[f]>
 *   ds     = w_r * (dw_r - sum_r' w_r' dw_r')            (softmax backward)
 *   dvalues[f]         += w_r * dy[t]
 *   dq[t][h][left]      = sum_r ds_r * keys[h][0][i_r]
 *   dq[t][h][right]     = sum_r ds_r * keys[h][1][j_r]
 *   dkeys[h][0][i]      = sum over picks with left index i of ds * q1[t][h]
 *   dkeys[h][1][j]      = sum over picks with right index j of ds * q2[t][h]
 *
 *   q, keys, values   as for pkm_forward (same p)
 *   idx, weights      [T][H][k] as produced by pkm_forward for these inputs
 *   dy       [T][d_v]           dtype
 *   dq       [T][H][d_k]        float32 OUT, overwritten
 *   dkeys    [H][2][n][d_k/2]   float32 OUT, overwritten ([2][n][d_k/2], the
 *                               sum over heads, with PKM_KEYS_SHARED)
 *   dvalues  [n*n][d_v]         float32 IN/OUT, ACCUMULATED (+=): the caller
 *                               zeroes it (or keeps an earlier gradient to add
 *                               to); rows no pick selects are left untouched.
 *   workspace  pkm_workspace_bytes(p, 1) bytes (NULL allowed when that is 0)
 * Results are the same bits on every run: the picks of one slot meet in
 * ascending pick id (t*H*k + h*k + r), the pieces of a slot picked more
 * often than one wave's share are added in a fixed order, and no float
 * atomics are used anywhere in the backward.
 */
pkm_status_t pkm_backward(const pkm_problem_t *p, const void *q, const void *keys,
                          const void *values, const int32_t *idx, const float *weights,
                          const void *dy, float *dq, float *dkeys, float *dvalues, void *workspace,
                          size_t workspace_bytes, void *stream);

/* pkm_backward with dvalues OVERWRITTEN instead of accumulated: every row of
 * dvalues is written, rows no pick selects become 0, and the old contents are
 * never read (the mode of an optimizer that consumes a fresh gradient; it
 * spares reading the n*n x d_v float32 array).  Same arguments, same
 * workspace and the same run-to-run identical results as pkm_backward. */
pkm_status_t pkm_backward_overwrite(const pkm_problem_t *p, const void *q, const void *keys,
                                    const void *values, const int32_t *idx, const float *weights,
                                    const void *dy, float *dq, float *dkeys, float *dvalues,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * pkm_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same results bit for bit
 * (dvalues accumulated).  The scratch memory is a static array of 128 MiB
 * that the library holds on each GPU it runs on until the process ends (the
 * benchmark workload, T = 16384, H = 4, n = 512, k = 32, d_v = 1024, needs
 * 113 MiB); a problem whose pkm_workspace_bytes(p, 1) exceeds it returns
 * PKM_ERR_TOO_LARGE and enqueues nothing.  The call allocates nothing.
 * Every call on one GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must not be made;
 * calls in one stream's order are safe.  Nothing in the array needs to start
 * at zero, and it keeps whatever the last call left.
 */
pkm_status_t pkm_backward_noalloc(const pkm_problem_t *p, const void *q, const void *keys,
                                  const void *values, const int32_t *idx, const float *weights,
                                  const void *dy, float *dq, float *dkeys, float *dvalues,
                                  void *stream);

/*
 * The backward with the sparse SGD step fused in (gptget.net summary,
 * "Methodology": trained with sparse updates, only the selected memory slots
 * change): dq and dkeys exactly as pkm_backward, and instead of dvalues the
 * value rows themselves are updated in place -- every row f some pick
 * selected becomes values[f] = fmaf(-lr, g[f], values[f]) rounded once to the
 * storage type, g[f] being the float32 row pkm_backward would write to
 * dvalues; rows no pick selected are left as they are.  The same result as
 * pkm_backward (dvalues overwritten) followed by pkm_sparse_sgd, without the
 * n*n x d_v float32 gradient array: each row's sum is applied where it is
 * formed (rows picked more often than one wave's share -- 256 picks, fewer
 * on small batches -- go through a workspace buffer).
 *   values    [n*n][d_v]  dtype, IN/OUT
 *   lr        the learning rate; finite, else PKM_ERR_ARG
 *   workspace pkm_workspace_bytes(p, 2) bytes
 * Other arguments as pkm_backward.  dw is computed from the values as they
 * were on entry.
 */
pkm_status_t pkm_backward_sgd(const pkm_problem_t *p, const void *q, const void *keys,
                              void *values, const int32_t *idx, const float *weights,
                              const void *dy, float *dq, float *dkeys, float lr, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * The two passes above, stage by stage, for callers that keep the
 * intermediate results or time the stages: pkm_forward is
 * pkm_forward_select followed by pkm_forward_gather; pkm_backward is
 * pkm_slot_sort, pkm_backward_values and pkm_backward_queries (dvalues
 * accumulated, or overwritten for pkm_backward_overwrite).  Same
 * conventions, same array layouts as above.  A workspace of
 * pkm_workspace_bytes(p, 1) bytes serves pkm_slot_sort, pkm_backward_values
 * and pkm_backward_queries.
 */

/* Steps 1-5 of pkm_forward: the selection and its softmax weights
 * (companion page, "Why top-k of each half is enough").  The workspace
 * (pkm_workspace_bytes(p, 0) bytes) is the same as pkm_forward's. */
pkm_status_t pkm_forward_select(const pkm_problem_t *p, const void *q, const void *keys,
                                int32_t *idx, float *weights, float *scores, void *workspace,
                                size_t workspace_bytes, void *stream);

/* The flat-key search that product keys replace, as a workload of its own
 * (companion page, "Search cost: flat vs product keys": a flat memory
 * compares the query with every key): for every (t, h) all n*n implied keys
 * -- key f = i*n + j is left sub-key i followed by right sub-key j --
 * scored with one d_k-wide dot product each (float32 accumulation), the
 * exact top-k by (score desc, slot asc), and the softmax of the k scores.
 * Same outputs, layouts and PKM_KEYS_SHARED as pkm_forward_select; y follows
 * from pkm_forward_gather.  About n*n*d_k*2 flops per (token, head) against
 * the product keys' 2*n*d_k.  Supported: bf16 storage (else PKM_ERR_DTYPE),
 * d_k = 512, 32 <= n <= 1024, k <= 32 (else PKM_ERR_SHAPE).  No workspace. */
pkm_status_t pkm_flat_forward_select(const pkm_problem_t *p, const void *q, const void *keys,
                                     int32_t *idx, float *weights, float *scores, void *stream);

/* y[t] = sum over heads h and picks r of weights[t][h][r] * values[idx[t][h][r]]
 * (gptget.net summary, "Methodology": weighted sum of the selected values). */
pkm_status_t pkm_forward_gather(const pkm_problem_t *p, const void *values, const int32_t *idx,
                                const float *weights, void *y, void *stream);

/* Groups the T*H*k picks of idx by memory slot (a counting sort): the picks
 * that selected slot f are order[slot_start[f] .. slot_start[f+1]), as pick
 * ids t*H*k + h*k + r.  These are exactly the slots that receive a value
 * update (gptget.net summary, "Methodology": only a few memory slots are
 * updated).
 *   slot_start  [n*n + 1]  int32 OUT;  order  [T*H*k]  int32 OUT
 * The picks of one slot are in ascending pick id: the result is unique. */
pkm_status_t pkm_slot_sort(const pkm_problem_t *p, const int32_t *idx, int32_t *slot_start,
                           int32_t *order, void *workspace, size_t workspace_bytes, void *stream);

/* The value side of pkm_backward over the slot-sorted picks: dw [T][H][k]
 * float32 (OUT, overwritten), dw = <dy[t], values[f]>, and the sparse update
 * dvalues[f] += w * dy[t] (dvalues_accumulate != 0: accumulated, as in
 * pkm_backward; 0: overwritten, as in pkm_backward_overwrite).  Each value
 * row is read once per run of picks; the picks of a slot are summed in the
 * order of `order`, a slot picked more often than one wave's share in
 * pieces whose sums meet in a fixed order (through the workspace), so the
 * result is the same on every run.  slot_start and order come from
 * pkm_slot_sort on the same idx.  workspace: pkm_workspace_bytes(p, 1)
 * bytes. */
pkm_status_t pkm_backward_values(const pkm_problem_t *p, const void *values, const int32_t *idx,
                                 const float *weights, const void *dy, const int32_t *slot_start,
                                 const int32_t *order, float *dvalues, int dvalues_accumulate,
                                 float *dw, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* The query side of pkm_backward, from weights and dw: the softmax backward,
 * then dq and dkeys (both OUT, overwritten).  Each pick's ds reaches its left
 * sub-key i = f / n and its right sub-key j = f % n. */
pkm_status_t pkm_backward_queries(const pkm_problem_t *p, const void *q, const void *keys,
                                  const int32_t *idx, const float *weights, const float *dw,
                                  float *dq, float *dkeys, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * After the backward: the value table's sparse update and the slot-usage
 * counter.  Both read the slot sort of the batch (slot_start from
 * pkm_slot_sort, or the workspace of pkm_backward: its slot_start follows the
 * T*H*k floats of dw, rounded up to 256 bytes): slot f is TOUCHED iff
 * slot_start[f+1] > slot_start[f], i.e. some pick selected it.  Only T, H and
 * k of `p` may differ from the backward's problem; n, d_v and dtype must be
 * the same.
 */

/* Sparse update of the memory values (gptget.net summary, "Methodology": the
 * layer is trained with sparse updates, only the selected slots change),
 * plain SGD: for every touched slot f and every column c,
 *   values[f][c] = values[f][c] - lr * dvalues[f][c]
 * computed as one float32 fused multiply-add, rounded once to the storage
 * type (bf16: nearest, ties to even).  Rows of untouched slots are not read
 * or written.
 *   values   [n*n][d_v] dtype    IN/OUT
 *   dvalues  [n*n][d_v] float32  IN (pkm_backward's value gradient)
 *   lr       finite, else PKM_ERR_ARG */
pkm_status_t pkm_sparse_sgd(const pkm_problem_t *p, void *values, const float *dvalues,
                            const int32_t *slot_start, float lr, void *stream);

/* The same with Adam, moments kept and advanced only for touched rows (a
 * "lazy" Adam: a row's moments stand still while it is not selected):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   values -= lr * (m / c1) / (sqrt(v / c2) + eps),
 *   c1 = 1 - beta1^step, c2 = 1 - beta2^step (computed in double on the host,
 *   rounded to float32); float32 arithmetic, one rounding to the storage type.
 *   adam_m, adam_v  [n*n][d_v] float32 IN/OUT, caller-owned (zero at step 1)
 *   step >= 1, beta1, beta2 in [0, 1), eps > 0 and finite, lr finite, else
 *   PKM_ERR_ARG. */
pkm_status_t pkm_sparse_adam(const pkm_problem_t *p, void *values, const float *dvalues,
                             const int32_t *slot_start, float *adam_m, float *adam_v,
                             int64_t step, float lr, float beta1, float beta2, float eps,
                             void *stream);

/* Memory usage (gptget.net summary, "Key Results": the share of memory slots
 * in use, which batch-norm in the query network raises above 80%):
 *   counts[f] += slot_start[f+1] - slot_start[f]   (picks of slot f)
 *   *used      = number of slots f with counts[f] != 0 after the update
 *   counts  [n*n]  int64  IN/OUT, accumulates over calls (zero it to start)
 *   used    [1]    int64  OUT, device memory, 8-byte aligned; may be NULL
 * usage = *used / (n*n). */
pkm_status_t pkm_slot_usage(const pkm_problem_t *p, const int32_t *slot_start, int64_t *counts,
                            int64_t *used, void *stream);

/*
 * The query network in front of the layer (gptget.net summary, methodology
 * list of "Deep Analysis": the input x passes through the query network,
 * which gives q; "Key Results": batch normalization in the query network
 * raises memory utilization): one bias-free projection and batch
 * normalization of every output feature over the batch's T tokens,
 *   z = x W^T,   q = gamma (z - mean_t z) / sqrt(var_t z + eps) + beta,
 * with the batch's mean and biased variance (float32 sums, the variance from
 * a one-pass Welford merge; float64 for the final merge).  q has d_out =
 * H * d_k features and is the q of pkm_forward ([T][H][d_k] is [T][d_out]).
 */
typedef struct {
    int64_t T;        /* tokens (>= 0)                                        */
    int32_t d_model;  /* input width: a multiple of 8, in [8, 16384]          */
    int32_t d_out;    /* output width H * d_k: a multiple of 8, in [8, 65536] */
    int32_t dtype;    /* pkm_dtype_t of x, W and q                            */
    int32_t reserved; /* 0                                                    */
} pkm_query_problem_t;

/* Workspace bytes of pkm_query_forward (backward = 0) or pkm_query_backward
 * (backward = 1); (size_t)-1 for an invalid descriptor. */
size_t pkm_query_workspace_bytes(const pkm_query_problem_t *qp, int backward);

/*   x      [T][d_model]      dtype
 *   W      [d_out][d_model]  dtype
 *   gamma, beta [d_out]      float32, or NULL for gamma = 1, beta = 0
 *   eps    > 0 and finite, else PKM_ERR_ARG (PyTorch's default is 1e-5)
 *   q      [T][d_out]        dtype   OUT (nearest-even for bf16)
 *   z      [T][d_out]        float32 OUT, x W^T (kept for the backward)
 *   mean, rstd  [d_out]      float32 OUT, batch mean and 1/sqrt(var + eps)
 * T must be >= 2 for the statistics to mean anything; T == 0 is a no-op. */
pkm_status_t pkm_query_forward(const pkm_query_problem_t *qp, const void *x, const void *W,
                               const float *gamma, const float *beta, float eps, void *q,
                               float *z, float *mean, float *rstd, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Backward of pkm_query_forward for dq = dL/dq (float32, e.g. pkm_backward's
 * dq), with zhat = (z - mean) * rstd:
 *   dbeta = sum_t dq;  dgamma = sum_t dq * zhat;
 *   dz = gamma rstd (dq - mean_t dq - zhat mean_t(dq zhat));
 *   dx = dz W;  dW = dz^T x.
 *   x, W, gamma, z, mean, rstd   as given to / returned by the forward
 *   dq      [T][d_out]      float32
 *   dx      [T][d_model]    float32 OUT;  dW [d_out][d_model] float32 OUT
 *   dgamma, dbeta [d_out]   float32 OUT, each may be NULL
 * bf16 storage: dz enters the MFMA products split into two bfloat16 parts
 * (about 16 significant bits), float32 sums. */
pkm_status_t pkm_query_backward(const pkm_query_problem_t *qp, const void *x, const void *W,
                                const float *gamma, const float *z, const float *mean,
                                const float *rstd, const float *dq, float *dx, float *dW,
                                float *dgamma, float *dbeta, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *pkm_status_string(pkm_status_t s);

#ifdef __cplusplus
}
#endif
#endif /* PKM_H */

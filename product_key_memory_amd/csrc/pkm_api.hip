// pkm_api.hip -- the C ABI of libpkm.so (declared in include/pkm.h):
// argument validation, workspace carving, and kernel launches on the
// caller's stream.  Nothing here allocates memory or keeps state.
#include "pkm.h"
#include "pkm_kernels.hpp"
#include "pkm_query.hpp"
#include "pkm_scratch.hpp"
#include "pkm_update.hpp"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

namespace {

constexpr int kMaxH = 64;
constexpr int kMaxN = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxDk = 1024;
constexpr int kMaxDvBackward = 4096;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A pointer to an array with no elements (T == 0) may be NULL.
bool missing(const void *p, int64_t count) { return count > 0 && p == nullptr; }

// The storage type and the layout flag carried by pkm_problem_t.dtype.
int storage(const pkm_problem_t *p) { return p->dtype & 0xFF; }
bool keys_shared(const pkm_problem_t *p) { return (p->dtype & PKM_KEYS_SHARED) != 0; }
// elements from one head's codebooks to the next (0: every head reads the same pair)
int64_t key_hstride(const pkm_problem_t *p)
{
    return keys_shared(p) ? 0 : (int64_t)2 * p->n * (p->d_k / 2);
}

pkm_status_t check_problem(const pkm_problem_t *p, bool backward)
{
    if (!p)
        return PKM_ERR_NULL;
    if ((storage(p) != PKM_FP32 && storage(p) != PKM_BF16) ||
        (p->dtype & ~(0xFF | PKM_KEYS_SHARED)) != 0)
        return PKM_ERR_DTYPE;
    if (p->T < 0 || p->H < 1 || p->H > kMaxH || p->n < 1 || p->n > kMaxN || p->k < 1 ||
        p->k > p->n || p->k > kMaxK || p->d_k < 16 || p->d_k > kMaxDk || p->d_k % 16 != 0 ||
        p->d_v < 8 || p->d_v % 8 != 0)
        return PKM_ERR_SHAPE;
    if (backward && p->d_v > kMaxDvBackward)
        return PKM_ERR_SHAPE;
    // grid limits, and pick ids T*H*k held in int32 by the slot sort
    if (p->T > ((int64_t)1 << 32) || p->T * p->H > ((int64_t)1 << 32) ||
        p->T * p->H * p->k > (int64_t)INT32_MAX)
        return PKM_ERR_SHAPE;
    return PKM_OK;
}

size_t picks_bytes(const pkm_problem_t *p) { return pkm::align256((size_t)(p->T * p->H * p->k) * 4); }
size_t starts_bytes(const pkm_problem_t *p) { return pkm::align256(((size_t)p->n * p->n + 1) * 4); }

// What one stage of the backward needs beside its arrays: the slot sort's
// scratch, the value side's piece rows (the sums of the runs longer than one
// wave's share), the query side's scratch.  The stages run one after the
// other, so in pkm_backward they share one region.
size_t split_bytes(const pkm_problem_t *p)
{
    return pkm::split_rows_bytes(p->T * p->H * p->k, p->d_v);
}
size_t stage_scratch_bytes(const pkm_problem_t *p)
{
    const size_t v = pkm::slot_sort_scratch(p->T * p->H * p->k, p->n).total;
    const size_t q = pkm::bwd_query_scratch(p->T, p->H, p->n, p->k, p->d_k).total;
    const size_t s = split_bytes(p);
    return v > q ? (v > s ? v : s) : (q > s ? q : s);
}

// pkm_backward, pkm_backward_overwrite and pkm_backward_sgd: dw, slot_start,
// order, then the stages' scratch.
size_t backward_bytes(const pkm_problem_t *p)
{
    return picks_bytes(p) + starts_bytes(p) + picks_bytes(p) + stage_scratch_bytes(p);
}
size_t backward_sgd_bytes(const pkm_problem_t *p) { return backward_bytes(p); }

size_t forward_bytes(const pkm_problem_t *p)
{
    return pkm::select_workspace_bytes(p->T, p->H, p->n, p->k, storage(p), p->d_k);
}

pkm_status_t check_workspace(const pkm_problem_t *p, const void *ws, size_t have, size_t need)
{
    if (p->T == 0 || need == 0)
        return PKM_OK;
    if (!ws)
        return PKM_ERR_NULL;
    if (!aligned16(ws))
        return PKM_ERR_ALIGN;
    return have < need ? PKM_ERR_WORKSPACE : PKM_OK;
}

}  // namespace

extern "C" {

size_t pkm_workspace_bytes(const pkm_problem_t *p, int backward)
{
    if (backward < 0 || backward > 2 || check_problem(p, backward != 0) != PKM_OK)
        return (size_t)-1;
    return backward == 2 ? backward_sgd_bytes(p) : backward ? backward_bytes(p) : forward_bytes(p);
}

pkm_status_t pkm_forward_select(const pkm_problem_t *p, const void *q, const void *keys,
                                int32_t *idx, float *weights, float *scores, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || missing(idx, T) || missing(weights, T))
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(idx) || !aligned16(weights) ||
        (scores && !aligned16(scores)))
        return PKM_ERR_ALIGN;
    st = check_workspace(p, workspace, workspace_bytes, forward_bytes(p));
    if (st != PKM_OK)
        return st;
    if (T == 0)
        return PKM_OK;
    return pkm::launch_fwd_select(storage(p), q, keys, key_hstride(p), p->T, p->H, p->n, p->k,
                                  p->d_k, idx, weights,
                                  scores, workspace, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_flat_forward_select(const pkm_problem_t *p, const void *q, const void *keys,
                                     int32_t *idx, float *weights, float *scores, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    if (storage(p) != PKM_BF16)
        return PKM_ERR_DTYPE;
    if (p->d_k != 512 || p->n < 32 || p->k > 32)
        return PKM_ERR_SHAPE;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || missing(idx, T) || missing(weights, T))
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(idx) || !aligned16(weights) ||
        (scores && !aligned16(scores)))
        return PKM_ERR_ALIGN;
    if (T == 0)
        return PKM_OK;
    return pkm::launch_flat_select(q, keys, key_hstride(p), T, p->H, p->n, p->k, idx, weights,
                                   scores, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_forward_gather(const pkm_problem_t *p, const void *values, const int32_t *idx,
                                const float *weights, void *y, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (!values || missing(idx, T) || missing(weights, T) || missing(y, T))
        return PKM_ERR_NULL;
    if (!aligned16(values) || !aligned16(idx) || !aligned16(weights) || !aligned16(y))
        return PKM_ERR_ALIGN;
    if (T == 0)
        return PKM_OK;
    return pkm::launch_fwd_gather(storage(p), values, idx, weights, y, p->T, p->H * p->k, p->d_v,
                                  static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_forward(const pkm_problem_t *p, const void *q, const void *keys,
                         const void *values, void *y, int32_t *idx, float *weights,
                         float *scores, void *workspace, size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || !values || missing(y, T) || missing(idx, T) ||
        missing(weights, T))
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(values) || !aligned16(y) ||
        !aligned16(idx) || !aligned16(weights) || (scores && !aligned16(scores)))
        return PKM_ERR_ALIGN;
    st = pkm_forward_select(p, q, keys, idx, weights, scores, workspace, workspace_bytes, stream);
    if (st != PKM_OK)
        return st;
    return pkm_forward_gather(p, values, idx, weights, y, stream);
}

pkm_status_t pkm_slot_sort(const pkm_problem_t *p, const int32_t *idx, int32_t *slot_start,
                           int32_t *order, void *workspace, size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(idx, T) || !slot_start || missing(order, T))
        return PKM_ERR_NULL;
    if (!aligned16(idx) || !aligned16(slot_start) || !aligned16(order))
        return PKM_ERR_ALIGN;
    if (T == 0)      // no picks: every slot starts (and ends) at 0
        return pkm::launch_zero_f32(reinterpret_cast<float *>(slot_start),
                                    (int64_t)p->n * p->n + 1,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
                   ? PKM_OK
                   : PKM_ERR_HIP;
    if (!workspace)
        return PKM_ERR_NULL;
    if (!aligned16(workspace))
        return PKM_ERR_ALIGN;
    if (workspace_bytes < pkm::slot_sort_scratch(p->T * p->H * p->k, p->n).total)
        return PKM_ERR_WORKSPACE;
    return pkm::launch_slot_sort(idx, T * p->H * p->k, p->n, slot_start, order, workspace,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_backward_values(const pkm_problem_t *p, const void *values, const int32_t *idx,
                                 const float *weights, const void *dy, const int32_t *slot_start,
                                 const int32_t *order, float *dvalues, int dvalues_accumulate,
                                 float *dw, void *workspace, size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (!values || missing(idx, T) || missing(weights, T) || missing(dy, T) || !slot_start ||
        missing(order, T) || !dvalues || missing(dw, T))
        return PKM_ERR_NULL;
    if (!aligned16(values) || !aligned16(idx) || !aligned16(weights) || !aligned16(dy) ||
        !aligned16(slot_start) || !aligned16(order) || !aligned16(dvalues) || !aligned16(dw))
        return PKM_ERR_ALIGN;
    st = check_workspace(p, workspace, workspace_bytes, split_bytes(p));
    if (st != PKM_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0)      // no picks: overwrite leaves an all-zero gradient
        return dvalues_accumulate || pkm::launch_zero_f32(dvalues, (int64_t)p->n * p->n * p->d_v,
                                                          s) == hipSuccess
                   ? PKM_OK
                   : PKM_ERR_HIP;
    return pkm::launch_bwd_value(storage(p), values, idx, weights, dy, slot_start, order, dvalues,
                                 dvalues_accumulate, static_cast<float *>(workspace), dw, p->T,
                                 p->H, p->n, p->k, p->d_v, s) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_backward_queries(const pkm_problem_t *p, const void *q, const void *keys,
                                  const int32_t *idx, const float *weights, const float *dw,
                                  float *dq, float *dkeys, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || missing(idx, T) || missing(weights, T) || missing(dw, T) ||
        missing(dq, T) || !dkeys)
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(idx) || !aligned16(weights) ||
        !aligned16(dw) || !aligned16(dq) || !aligned16(dkeys))
        return PKM_ERR_ALIGN;
    st = check_workspace(p, workspace, workspace_bytes,
                         pkm::bwd_query_scratch(p->T, p->H, p->n, p->k, p->d_k).total);
    if (st != PKM_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int heads_of_dkeys = keys_shared(p) ? 1 : p->H;
    if (T == 0)
        return pkm::launch_zero_f32(dkeys, (int64_t)heads_of_dkeys * 2 * p->n * (p->d_k / 2),
                                    s) == hipSuccess
                   ? PKM_OK
                   : PKM_ERR_HIP;
    return pkm::launch_bwd_query(storage(p), q, keys, key_hstride(p), keys_shared(p), idx, weights,
                                 dw, dq, dkeys, p->T, p->H, p->n, p->k, p->d_k, workspace,
                                 s) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

}  // extern "C"

namespace {

// pkm_backward (accumulate != 0) and pkm_backward_overwrite (accumulate == 0)
pkm_status_t backward_impl(const pkm_problem_t *p, const void *q, const void *keys,
                           const void *values, const int32_t *idx, const float *weights,
                           const void *dy, float *dq, float *dkeys, float *dvalues,
                           int accumulate, void *workspace, size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || !values || missing(idx, T) || missing(weights, T) ||
        missing(dy, T) || missing(dq, T) || !dkeys || !dvalues)
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(values) || !aligned16(idx) ||
        !aligned16(weights) || !aligned16(dy) || !aligned16(dq) || !aligned16(dkeys) ||
        !aligned16(dvalues))
        return PKM_ERR_ALIGN;
    st = check_workspace(p, workspace, workspace_bytes, backward_bytes(p));
    if (st != PKM_OK)
        return st;
    char *base = static_cast<char *>(workspace);
    float *dw = reinterpret_cast<float *>(base);
    int32_t *slot_start = reinterpret_cast<int32_t *>(base + picks_bytes(p));
    int32_t *order = reinterpret_cast<int32_t *>(base + picks_bytes(p) + starts_bytes(p));
    const size_t head = 2 * picks_bytes(p) + starts_bytes(p);
    void *stage_ws = T > 0 ? base + head : nullptr;
    const size_t stage_ws_bytes = T > 0 ? workspace_bytes - head : 0;
    if (T > 0) {
        st = pkm_slot_sort(p, idx, slot_start, order, stage_ws, stage_ws_bytes, stream);
        if (st != PKM_OK)
            return st;
    }
    st = pkm_backward_values(p, values, idx, weights, dy, slot_start, order, dvalues, accumulate,
                             dw, stage_ws, stage_ws_bytes, stream);
    if (st != PKM_OK)
        return st;
    return pkm_backward_queries(p, q, keys, idx, weights, dw, dq, dkeys, stage_ws, stage_ws_bytes,
                                stream);
}

}  // namespace

extern "C" {

pkm_status_t pkm_backward(const pkm_problem_t *p, const void *q, const void *keys,
                          const void *values, const int32_t *idx, const float *weights,
                          const void *dy, float *dq, float *dkeys, float *dvalues, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    return backward_impl(p, q, keys, values, idx, weights, dy, dq, dkeys, dvalues, 1, workspace,
                         workspace_bytes, stream);
}

pkm_status_t pkm_backward_overwrite(const pkm_problem_t *p, const void *q, const void *keys,
                                    const void *values, const int32_t *idx, const float *weights,
                                    const void *dy, float *dq, float *dkeys, float *dvalues,
                                    void *workspace, size_t workspace_bytes, void *stream)
{
    return backward_impl(p, q, keys, values, idx, weights, dy, dq, dkeys, dvalues, 0, workspace,
                         workspace_bytes, stream);
}

pkm_status_t pkm_backward_sgd(const pkm_problem_t *p, const void *q, const void *keys,
                              void *values, const int32_t *idx, const float *weights,
                              const void *dy, float *dq, float *dkeys, float lr, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (missing(q, T) || !keys || !values || missing(idx, T) || missing(weights, T) ||
        missing(dy, T) || missing(dq, T) || !dkeys)
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(values) || !aligned16(idx) ||
        !aligned16(weights) || !aligned16(dy) || !aligned16(dq) || !aligned16(dkeys))
        return PKM_ERR_ALIGN;
    if (!std::isfinite(lr))
        return PKM_ERR_ARG;
    st = check_workspace(p, workspace, workspace_bytes, backward_sgd_bytes(p));
    if (st != PKM_OK)
        return st;
    char *base = static_cast<char *>(workspace);
    float *dw = reinterpret_cast<float *>(base);
    int32_t *slot_start = reinterpret_cast<int32_t *>(base + picks_bytes(p));
    int32_t *order = reinterpret_cast<int32_t *>(base + picks_bytes(p) + starts_bytes(p));
    const size_t head = 2 * picks_bytes(p) + starts_bytes(p);
    void *stage_ws = T > 0 ? base + head : nullptr;
    const size_t stage_ws_bytes = T > 0 ? workspace_bytes - head : 0;
    if (T > 0) {
        st = pkm_slot_sort(p, idx, slot_start, order, stage_ws, stage_ws_bytes, stream);
        if (st != PKM_OK)
            return st;
        if (pkm::launch_bwd_value_sgd(storage(p), values, idx, weights, dy, slot_start, order, lr,
                                      static_cast<float *>(stage_ws), dw, T, p->H, p->n, p->k,
                                      p->d_v, static_cast<hipStream_t>(stream)) != hipSuccess)
            return PKM_ERR_HIP;
    }
    return pkm_backward_queries(p, q, keys, idx, weights, dw, dq, dkeys, stage_ws, stage_ws_bytes,
                                stream);
}

pkm_status_t pkm_sparse_sgd(const pkm_problem_t *p, void *values, const float *dvalues,
                            const int32_t *slot_start, float lr, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    if (!values || !dvalues || !slot_start)
        return PKM_ERR_NULL;
    if (!aligned16(values) || !aligned16(dvalues) || !aligned16(slot_start))
        return PKM_ERR_ALIGN;
    if (!std::isfinite(lr))
        return PKM_ERR_ARG;
    pkm::UpdateParams prm{lr, 0.f, 0.f, 0.f, 1.f, 1.f};
    return pkm::launch_sparse_update(storage(p), values, dvalues, slot_start, nullptr, nullptr,
                                     (int64_t)p->n * p->n, p->d_v, false, prm,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_sparse_adam(const pkm_problem_t *p, void *values, const float *dvalues,
                             const int32_t *slot_start, float *adam_m, float *adam_v,
                             int64_t step, float lr, float beta1, float beta2, float eps,
                             void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    if (!values || !dvalues || !slot_start || !adam_m || !adam_v)
        return PKM_ERR_NULL;
    if (!aligned16(values) || !aligned16(dvalues) || !aligned16(slot_start) ||
        !aligned16(adam_m) || !aligned16(adam_v))
        return PKM_ERR_ALIGN;
    if (step < 1 || !std::isfinite(lr) || !(beta1 >= 0.f && beta1 < 1.f) ||
        !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f) || !std::isfinite(eps))
        return PKM_ERR_ARG;
    const double c1 = 1.0 - std::pow((double)beta1, (double)step);
    const double c2 = 1.0 - std::pow((double)beta2, (double)step);
    if (!(c1 > 0.0) || !(c2 > 0.0))
        return PKM_ERR_ARG;
    pkm::UpdateParams prm{lr, beta1, beta2, eps, (float)c1, (float)c2};
    return pkm::launch_sparse_update(storage(p), values, dvalues, slot_start, adam_m, adam_v,
                                     (int64_t)p->n * p->n, p->d_v, true, prm,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_slot_usage(const pkm_problem_t *p, const int32_t *slot_start, int64_t *counts,
                            int64_t *used, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    if (!slot_start || !counts)
        return PKM_ERR_NULL;
    if (!aligned16(slot_start) || !aligned16(counts) ||
        (used && (reinterpret_cast<uintptr_t>(used) & 7u)))
        return PKM_ERR_ALIGN;
    return pkm::launch_slot_usage(slot_start, counts, (int64_t)p->n * p->n, used,
                                  static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

}  // extern "C"

namespace {

pkm_status_t check_query(const pkm_query_problem_t *qp)
{
    if (!qp)
        return PKM_ERR_NULL;
    if (qp->dtype != PKM_FP32 && qp->dtype != PKM_BF16)
        return PKM_ERR_DTYPE;
    if (qp->T < 0 || qp->d_model < 8 || qp->d_model > 16384 || qp->d_model % 8 != 0 ||
        qp->d_out < 8 || qp->d_out > 65536 || qp->d_out % 8 != 0 || qp->reserved != 0)
        return PKM_ERR_SHAPE;
    // GEMM grids and int32 row counts
    if (qp->T > INT32_MAX / 2)
        return PKM_ERR_SHAPE;
    return PKM_OK;
}

}  // namespace

extern "C" {

size_t pkm_query_workspace_bytes(const pkm_query_problem_t *qp, int backward)
{
    if (check_query(qp) != PKM_OK)
        return (size_t)-1;
    return pkm::query_scratch(qp->T, qp->d_model, qp->d_out, backward != 0,
                              qp->dtype == PKM_BF16 ? 2 : 4).total;
}

pkm_status_t pkm_query_forward(const pkm_query_problem_t *qp, const void *x, const void *W,
                               const float *gamma, const float *beta, float eps, void *q,
                               float *z, float *mean, float *rstd, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_query(qp);
    if (st != PKM_OK)
        return st;
    const int64_t T = qp->T;
    if (missing(x, T) || !W || missing(q, T) || missing(z, T) || !mean || !rstd)
        return PKM_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(q) || !aligned16(z) || !aligned16(mean) ||
        !aligned16(rstd) || (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
        return PKM_ERR_ALIGN;
    if (!(eps > 0.f) || !std::isfinite(eps))
        return PKM_ERR_ARG;
    if (T == 0)
        return PKM_OK;
    const size_t need = pkm::query_scratch(T, qp->d_model, qp->d_out, 0,
                                           qp->dtype == PKM_BF16 ? 2 : 4).total;
    if (!workspace)
        return PKM_ERR_NULL;
    if (!aligned16(workspace))
        return PKM_ERR_ALIGN;
    if (workspace_bytes < need)
        return PKM_ERR_WORKSPACE;
    return pkm::launch_query_forward(qp->dtype, x, W, gamma, beta, eps, q, z, mean, rstd, T,
                                     qp->d_model, qp->d_out, workspace,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_query_backward(const pkm_query_problem_t *qp, const void *x, const void *W,
                                const float *gamma, const float *z, const float *mean,
                                const float *rstd, const float *dq, float *dx, float *dW,
                                float *dgamma, float *dbeta, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_query(qp);
    if (st != PKM_OK)
        return st;
    const int64_t T = qp->T;
    if (missing(x, T) || !W || missing(z, T) || !mean || !rstd || missing(dq, T) ||
        missing(dx, T) || !dW)
        return PKM_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(z) || !aligned16(mean) || !aligned16(rstd) ||
        !aligned16(dq) || !aligned16(dx) || !aligned16(dW) || (gamma && !aligned16(gamma)) ||
        (dgamma && !aligned16(dgamma)) || (dbeta && !aligned16(dbeta)))
        return PKM_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t D = qp->d_out;
    if (T == 0) {       // no tokens: every gradient is zero
        hipError_t e = pkm::launch_zero_f32(dW, D * qp->d_model, s);
        if (e == hipSuccess && dgamma)
            e = pkm::launch_zero_f32(dgamma, D, s);
        if (e == hipSuccess && dbeta)
            e = pkm::launch_zero_f32(dbeta, D, s);
        return e == hipSuccess ? PKM_OK : PKM_ERR_HIP;
    }
    const size_t need = pkm::query_scratch(T, qp->d_model, qp->d_out, 1,
                                           qp->dtype == PKM_BF16 ? 2 : 4).total;
    if (!workspace)
        return PKM_ERR_NULL;
    if (!aligned16(workspace))
        return PKM_ERR_ALIGN;
    if (workspace_bytes < need)
        return PKM_ERR_WORKSPACE;
    return pkm::launch_query_backward(qp->dtype, x, W, gamma, z, mean, rstd, dq, dx, dW, dgamma,
                                      dbeta, T, qp->d_model, qp->d_out, workspace,
                                      s) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

const char *pkm_status_string(pkm_status_t s)
{
    switch (s) {
    case PKM_OK: return "PKM_OK";
    case PKM_ERR_NULL: return "PKM_ERR_NULL: a required pointer is NULL";
    case PKM_ERR_SHAPE: return "PKM_ERR_SHAPE: a size is outside the supported range";
    case PKM_ERR_DTYPE: return "PKM_ERR_DTYPE: unknown dtype";
    case PKM_ERR_WORKSPACE: return "PKM_ERR_WORKSPACE: workspace smaller than pkm_workspace_bytes()";
    case PKM_ERR_HIP: return "PKM_ERR_HIP: the HIP runtime rejected a launch";
    case PKM_ERR_ALIGN: return "PKM_ERR_ALIGN: an array pointer is not 16-byte aligned";
    case PKM_ERR_ARG: return "PKM_ERR_ARG: a scalar argument is outside its domain";
    case PKM_ERR_TOO_LARGE:
        return "PKM_ERR_TOO_LARGE: the problem needs more scratch than pkm_backward_noalloc's "
               "static buffer (128 MiB per GPU) holds; call pkm_backward with a workspace";
    }
    return "PKM: unknown status";
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pkm_backward_noalloc: pkm_backward with its workspace in a static device
// array instead of the caller's memory, for callers that cannot allocate.
// Each GPU the library runs on holds its own copy of the array (module global
// memory, kept until the process ends).  In host code `scratch` names a host
// stand-in, not the device copy: the device address is looked up with
// hipGetSymbolAddress once per device, with that device current, and only
// that address is ever handed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_lookup;

// The device address of `scratch` on the current device.
pkm_status_t scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return PKM_ERR_HIP;
    void *ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_lookup);
        ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
                return PKM_ERR_HIP;
            g_scratch_addr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PKM_OK;
}

}  // namespace

extern "C" {

pkm_status_t pkm_backward_noalloc(const pkm_problem_t *p, const void *q, const void *keys,
                                  const void *values, const int32_t *idx, const float *weights,
                                  const void *dy, float *dq, float *dkeys, float *dvalues,
                                  void *stream)
{
    const pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    if (backward_bytes(p) > kNoAllocScratchBytes)
        return PKM_ERR_TOO_LARGE;
    void *ws = nullptr;
    if (p->T > 0) {
        const pkm_status_t sa = scratch_address(&ws);
        if (sa != PKM_OK)
            return sa;
    }
    return backward_impl(p, q, keys, values, idx, weights, dy, dq, dkeys, dvalues, 1, ws,
                         ws ? kNoAllocScratchBytes : 0, stream);
}

}  // extern "C"

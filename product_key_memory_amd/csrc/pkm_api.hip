// pkm_api.hip -- the C ABI of libpkm.so (declared in include/pkm.h):
// argument validation, workspace carving, and kernel launches on the
// caller's stream.  Nothing here allocates memory or keeps state.
#include "pkm.h"
#include "pkm_kernels.hpp"

#include <hip/hip_runtime.h>

namespace {

constexpr int kMaxH = 64;
constexpr int kMaxN = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxDk = 1024;
constexpr int kMaxDvBackward = 4096;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A pointer to an array with no elements (T == 0) may be NULL.
bool missing(const void *p, int64_t count) { return count > 0 && p == nullptr; }

pkm_status_t check_problem(const pkm_problem_t *p, bool backward)
{
    if (!p)
        return PKM_ERR_NULL;
    if (p->dtype != PKM_FP32 && p->dtype != PKM_BF16)
        return PKM_ERR_DTYPE;
    if (p->T < 0 || p->H < 1 || p->H > kMaxH || p->n < 1 || p->n > kMaxN || p->k < 1 ||
        p->k > p->n || p->k > kMaxK || p->d_k < 16 || p->d_k > kMaxDk || p->d_k % 16 != 0 ||
        p->d_v < 8 || p->d_v % 8 != 0)
        return PKM_ERR_SHAPE;
    if (backward && p->d_v > kMaxDvBackward)
        return PKM_ERR_SHAPE;
    // grid limits: every launch keeps its x dimension below 2^31 blocks
    if (p->T > ((int64_t)1 << 32) || p->T * p->H > ((int64_t)1 << 32))
        return PKM_ERR_SHAPE;
    return PKM_OK;
}

size_t backward_ws(const pkm_problem_t *p) { return (size_t)(p->T * p->H * p->k) * sizeof(float); }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

size_t pkm_workspace_bytes(const pkm_problem_t *p, int backward)
{
    if (check_problem(p, backward != 0) != PKM_OK)
        return (size_t)-1;
    return backward ? round256(backward_ws(p)) : 0;
}

pkm_status_t pkm_forward(const pkm_problem_t *p, const void *q, const void *keys,
                         const void *values, void *y, int32_t *idx, float *weights,
                         float *scores, void *workspace, size_t workspace_bytes, void *stream)
{
    pkm_status_t st = check_problem(p, false);
    if (st != PKM_OK)
        return st;
    (void)workspace;
    (void)workspace_bytes;      // the forward pass needs no workspace
    const int64_t T = p->T;
    if (missing(q, T) || !keys || !values || missing(y, T) || missing(idx, T) || missing(weights, T))
        return PKM_ERR_NULL;
    if (!aligned16(q) || !aligned16(keys) || !aligned16(values) || !aligned16(y) ||
        !aligned16(idx) || !aligned16(weights) || (scores && !aligned16(scores)))
        return PKM_ERR_ALIGN;
    if (p->T == 0)
        return PKM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pkm::launch_fwd_select(p->dtype, q, keys, p->T, p->H, p->n, p->k, p->d_k, idx, weights,
                               scores, s) != hipSuccess)
        return PKM_ERR_HIP;
    if (pkm::launch_fwd_gather(p->dtype, values, idx, weights, y, p->T, p->H * p->k, p->d_v, s) !=
        hipSuccess)
        return PKM_ERR_HIP;
    return PKM_OK;
}

pkm_status_t pkm_backward(const pkm_problem_t *p, const void *q, const void *keys,
                          const void *values, const int32_t *idx, const float *weights,
                          const void *dy, float *dq, float *dkeys, float *dvalues,
                          void *workspace, size_t workspace_bytes, void *stream)
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
        !aligned16(dvalues) || (workspace && !aligned16(workspace)))
        return PKM_ERR_ALIGN;
    const size_t need = round256(backward_ws(p));
    if (p->T > 0 && (!workspace || workspace_bytes < need))
        return workspace ? PKM_ERR_WORKSPACE : PKM_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t dkeys_count = (int64_t)p->H * 2 * p->n * (p->d_k / 2);
    if (pkm::launch_zero_f32(dkeys, dkeys_count, s) != hipSuccess)
        return PKM_ERR_HIP;
    if (p->T == 0)
        return PKM_OK;
    float *dw = static_cast<float *>(workspace);
    if (pkm::launch_bwd_value(p->dtype, values, idx, weights, dy, dvalues, dw, p->T, p->H, p->k,
                              p->d_v, s) != hipSuccess)
        return PKM_ERR_HIP;
    if (pkm::launch_bwd_query(p->dtype, q, keys, idx, weights, dw, dq, dkeys, p->T, p->H, p->n,
                              p->k, p->d_k, s) != hipSuccess)
        return PKM_ERR_HIP;
    return PKM_OK;
}

pkm_status_t pkm_forward_select(const pkm_problem_t *p, const void *q, const void *keys,
                                int32_t *idx, float *weights, float *scores, void *stream)
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
    if (p->T == 0)
        return PKM_OK;
    return pkm::launch_fwd_select(p->dtype, q, keys, p->T, p->H, p->n, p->k, p->d_k, idx, weights,
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
    if (p->T == 0)
        return PKM_OK;
    return pkm::launch_fwd_gather(p->dtype, values, idx, weights, y, p->T, p->H * p->k, p->d_v,
                                  static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_backward_values(const pkm_problem_t *p, const void *values, const int32_t *idx,
                                 const float *weights, const void *dy, float *dvalues,
                                 float *dw, void *stream)
{
    pkm_status_t st = check_problem(p, true);
    if (st != PKM_OK)
        return st;
    const int64_t T = p->T;
    if (!values || missing(idx, T) || missing(weights, T) || missing(dy, T) || !dvalues ||
        missing(dw, T))
        return PKM_ERR_NULL;
    if (!aligned16(values) || !aligned16(idx) || !aligned16(weights) || !aligned16(dy) ||
        !aligned16(dvalues) || !aligned16(dw))
        return PKM_ERR_ALIGN;
    if (p->T == 0)
        return PKM_OK;
    return pkm::launch_bwd_value(p->dtype, values, idx, weights, dy, dvalues, dw, p->T, p->H,
                                 p->k, p->d_v, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PKM_OK
               : PKM_ERR_HIP;
}

pkm_status_t pkm_backward_queries(const pkm_problem_t *p, const void *q, const void *keys,
                                  const int32_t *idx, const float *weights, const float *dw,
                                  float *dq, float *dkeys, void *stream)
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pkm::launch_zero_f32(dkeys, (int64_t)p->H * 2 * p->n * (p->d_k / 2), s) != hipSuccess)
        return PKM_ERR_HIP;
    if (p->T == 0)
        return PKM_OK;
    return pkm::launch_bwd_query(p->dtype, q, keys, idx, weights, dw, dq, dkeys, p->T, p->H, p->n,
                                 p->k, p->d_k, s) == hipSuccess
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
    }
    return "PKM: unknown status";
}

}  // extern "C"

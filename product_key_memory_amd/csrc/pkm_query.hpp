// pkm_query.hpp -- launchers of the query network (projection + batch
// normalization) and its scratch layout (internal to libpkm.so; the public
// interface is include/pkm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkm {

// Workspace: per-(row chunk, column) batch-norm partials, then (backward)
// two per-column coefficients, dz [T][D] and dz^T [D][Tp] (float32, or for
// bf16 storage two bf16 planes hi and lo of the same total size), W^T
// [d_model][D] and x^T [d_model][Tp] (storage type; Tp = T rounded up to 32,
// zero-padded), and the split-K partial sums of dW [dw_splits][D][d_model].
struct QueryScratch {
    int chunks;
    int64_t rows_per_chunk;
    int dw_splits;
    size_t off_part, off_coef, off_dz, off_dzt, off_wt, off_xt, off_dwp, total;
};
QueryScratch query_scratch(int64_t T, int d_model, int D, int backward, int elt);
int dw_splits(int64_t T, int d_model, int D, int elt);

// z = x W^T [T][D] (float32), mean/rstd per column, q = gamma (z - mean) rstd + beta.
hipError_t launch_query_forward(int dtype, const void *x, const void *W, const float *gamma,
                                const float *beta, float eps, void *q, float *z, float *mean,
                                float *rstd, int64_t T, int d_model, int D, void *ws,
                                hipStream_t stream);

// From dq: dgamma, dbeta (optional), dz, then dx = dz W and dW = dz^T x.
hipError_t launch_query_backward(int dtype, const void *x, const void *W, const float *gamma,
                                 const float *z, const float *mean, const float *rstd,
                                 const float *dq, float *dx, float *dW, float *dgamma,
                                 float *dbeta, int64_t T, int d_model, int D, void *ws,
                                 hipStream_t stream);

}  // namespace pkm

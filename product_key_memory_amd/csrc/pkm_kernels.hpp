// pkm_kernels.hpp -- host-side launchers of the PKM kernels (internal to
// libpkm.so; the public interface is include/pkm.h).  Every launcher assumes
// its arguments were validated by the C ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkm {

// Fused forward selection: sub-key scoring (MFMA), exact per-half top-k,
// pruned k x k combine, softmax.  Writes idx / weights / scores [T][H][k].
hipError_t launch_fwd_select(int dtype, const void *q, const void *keys, int64_t T, int H,
                             int n, int k, int d_k, int32_t *idx, float *weights,
                             float *scores, hipStream_t stream);

// y[t] = sum over the H*k picks of token t of weight * values[slot].
hipError_t launch_fwd_gather(int dtype, const void *values, const int32_t *idx,
                             const float *weights, void *y, int64_t T, int HK, int d_v,
                             hipStream_t stream);

// dw = <dy, values[slot]> written to `dw` [T][H][k]; dvalues[slot] += w * dy
// (atomics).
hipError_t launch_bwd_value(int dtype, const void *values, const int32_t *idx,
                            const float *weights, const void *dy, float *dvalues, float *dw,
                            int64_t T, int H, int k, int d_v, hipStream_t stream);

// Softmax backward, then dq (overwritten) and dkeys (accumulated; zero it
// first) from weights and dw.
hipError_t launch_bwd_query(int dtype, const void *q, const void *keys, const int32_t *idx,
                            const float *weights, const float *dw, float *dq, float *dkeys,
                            int64_t T, int H, int n, int k, int d_k, hipStream_t stream);

// Fill `count` floats with zero (a kernel, so it can sit inside a captured graph).
hipError_t launch_zero_f32(float *p, int64_t count, hipStream_t stream);

}  // namespace pkm

// pkm_kernels.hpp -- host-side launchers of the PKM kernels (internal to
// libpkm.so; the public interface is include/pkm.h).  Every launcher assumes
// its arguments were validated by the C ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkm {

constexpr int kSegChunk = 256;      // sorted picks per wave in the value segmented reduction

// Fused forward selection: sub-key scoring (MFMA), exact per-half top-k,
// pruned k x k combine, softmax.  Writes idx / weights / scores [T][H][k].
hipError_t launch_fwd_select(int dtype, const void *q, const void *keys, int64_t T, int H,
                             int n, int k, int d_k, int32_t *idx, float *weights,
                             float *scores, hipStream_t stream);

// y[t] = sum over the H*k picks of token t of weight * values[slot].
hipError_t launch_fwd_gather(int dtype, const void *values, const int32_t *idx,
                             const float *weights, void *y, int64_t T, int HK, int d_v,
                             hipStream_t stream);

// Counting sort of the T*H*k picks by slot: slot_start [n*n + 1] (the picks
// of slot f are order[slot_start[f] .. slot_start[f+1])), order [picks] (pick
// ids t*H*k + h*k + r).  `scratch` holds
// slot_sort_scratch(picks, n).total bytes.
hipError_t launch_slot_sort(const int32_t *idx, int64_t picks, int n, int32_t *slot_start,
                            int32_t *order, void *scratch, hipStream_t stream);

// Value side of the backward over the slot-sorted picks: dw = <dy, values[slot]>
// per pick and dvalues[slot] (+)= sum w * dy -- accumulated into dvalues when
// `accumulate`, else dvalues is overwritten (untouched rows become 0).
hipError_t launch_bwd_value(int dtype, const void *values, const int32_t *idx,
                            const float *weights, const void *dy, const int32_t *slot_start,
                            const int32_t *order, float *dvalues, int accumulate, float *dw,
                            int64_t T, int H, int n, int k, int d_v, hipStream_t stream);

// Query side: softmax backward per distinct sub-key, dq (overwritten) and
// dkeys (overwritten) from weights and dw.  `scratch` holds
// bwd_query_scratch(T, H, n, k, d_k).total bytes.
hipError_t launch_bwd_query(int dtype, const void *q, const void *keys, const int32_t *idx,
                            const float *weights, const float *dw, float *dq, float *dkeys,
                            int64_t T, int H, int n, int k, int d_k, void *scratch,
                            hipStream_t stream);

// Fill `count` floats with zero (a kernel, so it can sit inside a captured graph).
hipError_t launch_zero_f32(float *p, int64_t count, hipStream_t stream);

}  // namespace pkm

// pkm_kernels.hpp -- host-side launchers of the PKM kernels (internal to
// libpkm.so; the public interface is include/pkm.h).  Every launcher assumes
// its arguments were validated by the C ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkm {

constexpr int kSegChunk = 256;      // sorted picks per wave in the value segmented reduction, at most
constexpr int kSegShift = 8;        // log2(kSegChunk)
static_assert((1 << kSegShift) == kSegChunk, "kSegShift = log2(kSegChunk)");

// log2 of the picks per wave of the value side: 256, or fewer (down to 32) on
// small batches, so that about 2048 waves share the work.  Runs of more than
// that many sorted picks are "long" (cut between waves).
__host__ __device__ inline int seg_shift(int64_t picks)
{
    int s = kSegShift;
    while (s > 5 && (picks >> s) < 2048)
        --s;
    return s;
}

// Rank pairs (a, b) with (a + 1)(b + 1) <= k: the combine candidates.
inline int merge_candidates(int k)
{
    int c = 0;
    for (int a = 1; a <= k; ++a)
        c += k / a;
    return c;
}

// The two-kernel selection path: query halves of exactly 256, k <= 32, and
// 128 <= n <= 1024 for bf16 storage, 128 <= n <= 256 for float32.  Its
// per-half top-k lists pass through the workspace: [T][H][2][k] entries of
// (score bits, sub-key), 8 bytes each.
inline bool select_fast_ok(int dtype, int n, int k, int d_k)
{
    // bf16: 128 <= n <= 1024; float32 (scored on the fp64 MFMA, whose
    // 64 query registers leave room for blocks of 256 sub-keys): n <= 256
    const int n_max = dtype == 1 ? 1024 : dtype == 0 ? 256 : 0;
    return n >= 128 && n <= n_max && k <= 32 && d_k == 512;
}
inline size_t select_workspace_bytes(int64_t T, int H, int n, int k, int dtype, int d_k)
{
    if (!select_fast_ok(dtype, n, k, d_k))
        return 0;
    return (((size_t)T * H * 2 * k * 8) + 255) & ~(size_t)255;
}

// Forward selection: sub-key scoring (MFMA), exact per-half top-k, pruned
// k x k combine, softmax.  Writes idx / weights / scores [T][H][k].
// `workspace` holds select_workspace_bytes(...) bytes.
// keys of head h start key_hstride elements after those of head h - 1 (0:
// one codebook pair shared by every head).
hipError_t launch_fwd_select(int dtype, const void *q, const void *keys, int64_t key_hstride,
                             int64_t T, int H, int n, int k, int d_k, int32_t *idx,
                             float *weights, float *scores, void *workspace, hipStream_t stream);
hipError_t launch_select_fast(int dtype, const void *q, const void *keys, int64_t key_hstride,
                              int64_t T, int H, int n, int k, int d_k, int32_t *idx,
                              float *weights, float *scores, void *workspace, hipStream_t stream);

// The flat-key search: all n*n implied keys of each (token, head) scored
// with one d_k-wide dot product, exact top-k, softmax (bf16, d_k = 512,
// 32 <= n <= 1024, k <= 32).
hipError_t launch_flat_select(const void *q, const void *keys, int64_t key_hstride, int64_t T,
                              int H, int n, int k, int32_t *idx, float *weights, float *scores,
                              hipStream_t stream);

// y[t] = sum over the H*k picks of token t of weight * values[slot].
hipError_t launch_fwd_gather(int dtype, const void *values, const int32_t *idx,
                             const float *weights, void *y, int64_t T, int HK, int d_v,
                             hipStream_t stream);

// Counting sort of the T*H*k picks by slot: slot_start [n*n + 1] (the picks
// of slot f are order[slot_start[f] .. slot_start[f+1])), order [picks] (pick
// ids t*H*k + h*k + r, ascending within each slot: both levels place their
// picks stably).  `scratch` holds slot_sort_scratch(picks, n).total bytes.
hipError_t launch_slot_sort(const int32_t *idx, int64_t picks, int n, int32_t *slot_start,
                            int32_t *order, void *scratch, hipStream_t stream);

// Value side of the backward over the slot-sorted picks: dw = <dy, values[slot]>
// per pick and dvalues[slot] (+)= sum w * dy -- accumulated into dvalues when
// `accumulate`, else dvalues is overwritten (untouched rows become 0).  The
// runs longer than the reduction's chunk are summed through `split`
// (split_rows_bytes(...) bytes) in a fixed order: no float atomics, the same
// bits on every run.
hipError_t launch_bwd_value(int dtype, const void *values, const int32_t *idx,
                            const float *weights, const void *dy, const int32_t *slot_start,
                            const int32_t *order, float *dvalues, int accumulate, float *split,
                            float *dw, int64_t T, int H, int n, int k, int d_v, hipStream_t stream);

// The value side with the SGD step fused in: dw as launch_bwd_value, and every
// selected value row updated in place, w = fmaf(-lr, g, w) rounded once, with
// g the row's gradient; no dvalues.  `split` as for launch_bwd_value.
hipError_t launch_bwd_value_sgd(int dtype, void *values, const int32_t *idx, const float *weights,
                                const void *dy, const int32_t *slot_start, const int32_t *order,
                                float lr, float *split, float *dw, int64_t T, int H, int n,
                                int k, int d_v, hipStream_t stream);
// The value side's scratch: two piece rows of d_v floats per nominal chunk
// of 2^seg_shift sorted picks, then the list of long runs: a count, followed
// by at most picks / chunk + 1 slots (long_list points at the first slot,
// the count sits just before it).
__host__ __device__ inline size_t split_piece_bytes(int64_t picks, int d_v)
{
    return (size_t)(2 * ((picks >> seg_shift(picks)) + 1)) * (size_t)d_v * 4;
}
__host__ __device__ inline size_t split_rows_bytes(int64_t picks, int d_v)
{
    return split_piece_bytes(picks, d_v) + 256 + (size_t)((picks >> seg_shift(picks)) + 1) * 4;
}
__host__ __device__ inline int32_t *long_list(float *split, int64_t picks, int d_v)
{
    return reinterpret_cast<int32_t *>(reinterpret_cast<char *>(split) +
                                       split_piece_bytes(picks, d_v) + 256);
}

// Query side: softmax backward per distinct sub-key, dq (overwritten) and
// dkeys (overwritten) from weights and dw.  `scratch` holds
// bwd_query_scratch(T, H, n, k, d_k).total bytes.  keys_shared: every head
// reads one codebook pair (key_hstride 0) and dkeys [2][n][d_k/2] sums the
// heads' gradients.
hipError_t launch_bwd_query(int dtype, const void *q, const void *keys, int64_t key_hstride,
                            bool keys_shared, const int32_t *idx, const float *weights,
                            const float *dw, float *dq, float *dkeys, int64_t T, int H, int n,
                            int k, int d_k, void *scratch, hipStream_t stream);

// Fill `count` floats with zero (a kernel, so it can sit inside a captured graph).
hipError_t launch_zero_f32(float *p, int64_t count, hipStream_t stream);

}  // namespace pkm

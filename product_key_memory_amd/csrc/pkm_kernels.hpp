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

// ---- backward scratch layouts (byte offsets inside the caller's workspace) ----
constexpr int kSegChunk = 256;      // sorted picks per wave in the value segmented reduction

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Scratch of the slot sort: per-slot counts and cursors, scan block sums.
struct SlotSortScratch {
    size_t off_count, off_cursor, off_bsums, total;
};

inline SlotSortScratch slot_sort_scratch(int n)
{
    const size_t slots = (size_t)n * n;
    const size_t sblocks = (slots + 1023) / 1024;
    SlotSortScratch S;
    S.off_count = 0;
    S.off_cursor = align256(slots * 4);
    S.off_bsums = align256(S.off_cursor + slots * 4);
    S.total = align256(S.off_bsums + sblocks * 4);
    return S;
}

struct BwdQueryScratch {
    size_t off_gl_i, off_gl_g, off_partial, total;
    int blocks;             // token blocks (one partial sum each)
    int tokens_per_block;   // a multiple of 32
};

inline BwdQueryScratch bwd_query_scratch(int64_t T, int H, int n, int k, int d_k)
{
    BwdQueryScratch S;
    const int half = d_k / 2;
    // about one workgroup (16 waves, n x 32 LDS tile) per compute unit
    const int64_t groups = (int64_t)H * 2 * ((half + 63) / 64);
    int64_t blocks = (256 + groups - 1) / groups;
    const int64_t max_blocks = T > 128 ? (T + 127) / 128 : 1;
    if (blocks > max_blocks)
        blocks = max_blocks;
    if (blocks < 1)
        blocks = 1;
    int64_t tpb = T > 0 ? (T + blocks - 1) / blocks : 32;
    tpb = (tpb + 31) & ~(int64_t)31;
    S.tokens_per_block = (int)tpb;
    S.blocks = (int)(T > 0 ? (T + tpb - 1) / tpb : 1);
    const size_t lists = (size_t)T * H * 2 * k * 4;
    S.off_gl_i = 0;
    S.off_gl_g = align256(lists);
    S.off_partial = align256(S.off_gl_g + lists);
    S.total = align256(S.off_partial + (size_t)S.blocks * H * 2 * n * half * 4);
    return S;
}

// Counting sort of the T*H*k picks by slot: slot_start [n*n + 1] (the picks
// of slot f are order[slot_start[f] .. slot_start[f+1])), order [picks] (pick
// ids t*H*k + h*k + r).  `scratch` holds slot_sort_scratch(n).total bytes.
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

// pkm_scratch.hpp -- byte layouts of the backward stages' scratch inside the
// caller's workspace (internal to libpkm.so; shared by the C ABI layer, which
// sizes the workspace, and the backward launchers, which carve it up).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pkm {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Scratch of the two-level slot sort: level-1 block histograms [blocks][buckets],
// bucket totals and starts, the order in which level 2 takes the buckets, and
// the (pick, low slot bits) pairs grouped by bucket.
constexpr int kMaxBuckets = 4096;
constexpr int kMaxBucketSlots = 1024;
constexpr int kMinBucketShift = 7;    // buckets of at least 128 slots (measured: 2048
                                      // buckets of 128 at 512^2 slots, 4096 of 256 at
                                      // 1024^2 beat both finer and coarser ones)
constexpr int kMaxL1Blocks = 256;

struct SlotSortScratch {
    int shift;              // bucket = slot >> shift
    int buckets;            // ceil(slots / 2^shift) <= kMaxBuckets
    int blocks;             // level-1 workgroups, each over `chunk` consecutive picks
    int64_t chunk;
    size_t off_bhist, off_total, off_base, off_order, off_pairs, total;
};

inline SlotSortScratch slot_sort_scratch(int64_t picks, int n)
{
    const int64_t slots = (int64_t)n * n;
    SlotSortScratch S;
    S.shift = kMinBucketShift;
    while ((slots + ((int64_t)1 << S.shift) - 1) >> S.shift > kMaxBuckets)
        ++S.shift;
    S.buckets = (int)((slots + ((int64_t)1 << S.shift) - 1) >> S.shift);
    int64_t blocks = (picks + 4095) / 4096;
    if (blocks > kMaxL1Blocks)
        blocks = kMaxL1Blocks;
    if (blocks < 1)
        blocks = 1;
    int64_t chunk = (picks + blocks - 1) / blocks;
    chunk = (chunk + 255) & ~(int64_t)255;
    if (chunk < 256)
        chunk = 256;
    S.chunk = chunk;
    S.blocks = (int)((picks + chunk - 1) / chunk);
    if (S.blocks < 1)
        S.blocks = 1;
    S.off_bhist = 0;
    S.off_total = align256((size_t)S.blocks * S.buckets * 4);
    S.off_base = align256(S.off_total + (size_t)S.buckets * 4);
    S.off_order = align256(S.off_base + ((size_t)S.buckets + 1) * 4);
    S.off_pairs = align256(S.off_order + (size_t)S.buckets * 4);
    S.total = align256(S.off_pairs + (size_t)(picks > 0 ? picks : 0) * 8);
    return S;
}

// Sub-key gradient: codebook columns per workgroup (its MFMA accumulators
// are n/16 row tiles x cols/16 column tiles over 16 waves of <= 128 registers).
inline int dk_cols(int n) { return n > 512 ? 64 : 128; }

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
    const int cols = dk_cols(n);
    const int64_t groups = (int64_t)H * 2 * ((half + cols - 1) / cols);
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

}  // namespace pkm

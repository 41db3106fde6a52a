// pkm_backward.hip -- backward pass of the product-key memory layer
// (gptget.net summary of "Large Memory Layers with Product Keys",
// "Methodology": the layer is trained end to end by backprop, and only the
// selected memory slots are updated).  The selection is a constant of the
// backward pass; gradient reaches the k selected scores of each head, and from
// each score its left and right sub-key scores.
//
// Value side (no float atomics: the result is the same on every run):
//   1. the T*H*k picks are counting-sorted by slot into slot_start [n*n + 1]
//      and order [T*H*k], in two levels whose counters all sit in LDS, stably
//      (the picks of a slot in ascending pick id);
//   2. one wave per chunk of the sorted picks walks its slot segments: the
//      value row of a segment is read once, every pick p of it gives
//      dw_p = <dy[t_p], values[f]>, and sum_p w_p dy[t_p] goes to dvalues[f]
//      with a plain store (or read-modify-write) when the whole segment lies
//      in the chunk (no other wave touches that row); a segment longer than
//      the chunk (a Zipf-hot slot) is cut into pieces, each stored to a row
//      of its own, and the pieces are summed afterwards in position order.
// Query side:
//   3. one wave per (token, head), one lane per pick: the softmax backward
//      ds_r = w_r (dw_r - sum_r' w_r' dw_r') matters only summed over the
//      picks S sharing a sub-key i of one half, and that sum is taken as
//          g_i = A * (1 - W) - B * W,  A = sum_S w dw, W = sum_S w,
//                                      B = sum_notS w dw, 1 - W = sum_notS w,
//      both complements summed directly, so a sub-key shared by most picks
//      (a near-cancelling sum) keeps full relative accuracy;
//      dq = sum_i g_i * sub-key row i (the rows of the distinct sub-keys are
//      fetched in batches), and (i, g_i) goes to a compact list;
//   4. dkeys[h][s][i] = sum_t g * q_half[t]: each workgroup owns one token
//      block and 128 columns (64 for n > 512) of one codebook and accumulates
//      the product of the sparse g matrix (densified per 64- or 32-token step
//      in LDS) with q in MFMA registers; a last kernel sums the token blocks'
//      partials in block order.
#include <type_traits>

#include "pkm_device.hpp"
#include "pkm_kernels.hpp"
#include "pkm_scratch.hpp"

namespace pkm {

template <typename DT>
__device__ __forceinline__ float load_elem(const DT *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p, int64_t i)
{
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
}

// ---------------------------------------------------------------------------
// 1. counting sort of the picks by slot, in two levels so that every counter
//    lives in LDS: level 1 groups the picks by bucket = slot >> shift (at
//    most 4096 buckets of at least 128 slots) with per-block histograms;
//    level 2 sorts each bucket by the low bits of the slot inside one
//    workgroup.
// ---------------------------------------------------------------------------
constexpr int kL1Threads = 512;
constexpr int kColWaves = 16;
constexpr int kColRows = 16;          // block rows per wave in the column scan (blocks <= 256)
constexpr int kL2Threads = 512;
constexpr int kL2Unroll = 4;          // picks in flight per thread in the counting passes

__device__ __forceinline__ int64_t l1_begin(int64_t chunk, int64_t picks)
{
    const int64_t b = (int64_t)blockIdx.x * chunk;
    return b < picks ? b : picks;
}

// bhist[block][bucket] = number of picks of this block's chunk in the bucket.
__global__ __launch_bounds__(kL1Threads) void bucket_hist_kernel(
    const int32_t *__restrict__ idx, int64_t picks, int64_t chunk, int shift, int nb,
    int32_t *__restrict__ bhist)
{
    __shared__ int32_t h[kMaxBuckets];
    for (int b = threadIdx.x; b < nb; b += kL1Threads)
        h[b] = 0;
    __syncthreads();
    const int64_t p0 = l1_begin(chunk, picks);
    const int64_t p1 = p0 + chunk < picks ? p0 + chunk : picks;
    for (int64_t q = p0 + threadIdx.x; q < p1; q += kL1Threads * kL2Unroll) {
        int32_t f[kL2Unroll];
#pragma unroll
        for (int u = 0; u < kL2Unroll; ++u) {
            const int64_t p = q + (int64_t)u * kL1Threads;
            f[u] = p < p1 ? idx[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kL2Unroll; ++u)
            if (f[u] >= 0)
                atomicAdd(&h[f[u] >> shift], 1);
    }
    __syncthreads();
    int32_t *row = bhist + (int64_t)blockIdx.x * nb;
    for (int b = threadIdx.x; b < nb; b += kL1Threads)
        row[b] = h[b];
}

// Per bucket (a column of bhist), in place: bhist[block][i] becomes the number
// of picks of bucket i in the chunks before `block`; total[i] = all of them.
// One lane per bucket; the 16 waves of a workgroup split the block rows.
__global__ __launch_bounds__(kColWaves *kWave) void bucket_colscan_kernel(
    int32_t *__restrict__ bhist, int blocks, int nb, int32_t *__restrict__ total)
{
    __shared__ int32_t part[kColWaves][kWave];
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int i = blockIdx.x * kWave + lane;
    const int rows = (blocks + kColWaves - 1) / kColWaves;
    const int r0 = w * rows;
    int v[kColRows];
    int s = 0;
#pragma unroll
    for (int r = 0; r < kColRows; ++r) {
        const bool ok = r < rows && r0 + r < blocks && i < nb;
        v[r] = ok ? bhist[(int64_t)(r0 + r) * nb + i] : 0;
        s += v[r];
    }
    part[w][lane] = s;
    __syncthreads();
    int pre = 0;
    for (int u = 0; u < w; ++u)
        pre += part[u][lane];
    if (w == kColWaves - 1 && i < nb)
        total[i] = pre + s;
#pragma unroll
    for (int r = 0; r < kColRows; ++r) {
        if (r < rows && r0 + r < blocks && i < nb)
            bhist[(int64_t)(r0 + r) * nb + i] = pre;
        pre += v[r];
    }
}

// Both levels place their items stably: a workgroup's range is cut into one
// contiguous sub-range per wave; each wave counts its items per key in LDS,
// the counts become per-(wave, key) cursors (keys outer, waves inner), and
// each wave then walks its sub-range in order, 64 items at a time: an item's
// place is its wave's cursor for the key plus the lanes below it with the
// same key (wave_match).  Equal keys thus keep their order, and no barrier
// is needed while placing -- each wave owns its cursors.
constexpr int kSortWaves = kL1Threads / kWave;
static_assert(kL2Threads == kL1Threads, "the same wave count at both levels");
// items per lane in flight in the counting and placement loops of a wave's
// sub-range: a Zipf-hot bucket holds ~24k pairs, 3k per wave, and each trip
// waits for its loads
constexpr int kSortUnroll = 16;

__device__ __forceinline__ void sub_range(int64_t beg, int64_t end, int w, int64_t &sb,
                                          int64_t &se)
{
    const int64_t len = end - beg;
    sb = beg + len * w / kSortWaves;
    se = beg + len * (w + 1) / kSortWaves;
}

// One 64-item step of a wave's placement: the place of this lane's item
// (valid lanes only); the highest-ranked lane of each key advances the cursor.
__device__ __forceinline__ int place_step(uint32_t key, bool valid, int bits, int32_t *cursor)
{
    const uint64_t peers = wave_match(key, valid, bits);
    const int rank = __popcll(peers & lanes_below());
    int pos = 0;
    if (valid) {
        pos = cursor[key] + rank;
        if (rank == __popcll(peers) - 1)
            cursor[key] = pos + 1;
    }
    return pos;
}

// Level-1 scatter: bucket_base = exclusive scan of total (block 0 stores it,
// nb + 1 entries), then every pick of the chunk goes to
// pairs[base[bucket] + bhist[block][bucket] + rank in block] as
// (pick id, slot & (2^shift - 1)), in pick order within each bucket.
// Block 0 also writes bucket_order, the order in which level 2's workgroups
// take the buckets: the large ones (more than four times the mean, a
// Zipf-hot slot's) first, then the rest, each in bucket order, so that the
// longest workgroups start in the first round instead of finishing last.
__global__ __launch_bounds__(kL1Threads) void bucket_scatter_kernel(
    const int32_t *__restrict__ idx, int64_t picks, int64_t chunk, int shift, int nb, int nb_bits,
    const int32_t *__restrict__ bhist, const int32_t *__restrict__ total,
    int32_t *__restrict__ bucket_base, int32_t *__restrict__ bucket_order, int2 *__restrict__ pairs)
{
    constexpr int PER = kMaxBuckets / kL1Threads;
    constexpr int W = kL1Threads / kWave;
    __shared__ int32_t hw[kSortWaves][kMaxBuckets];   // per-wave counts, then cursors
    __shared__ int32_t wsum[W];
    __shared__ int32_t wbig[W];
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // only the nb buckets in use (the rows are kMaxBuckets long)
    for (int u = 0; u < kSortWaves; ++u)
        for (int b = threadIdx.x; b < nb; b += kL1Threads)
            hw[u][b] = 0;
    const int64_t p0 = l1_begin(chunk, picks);
    const int64_t p1 = p0 + chunk < picks ? p0 + chunk : picks;
    int64_t sb, se;
    sub_range(p0, p1, w, sb, se);
    __syncthreads();
    for (int64_t q = sb + lane; q < se; q += kWave * kSortUnroll) {
        int32_t f[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const int64_t p = q + (int64_t)u * kWave;
            f[u] = p < se ? idx[p] : -1;
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            if (q - lane + (int64_t)u * kWave >= se)
                break;              // (wave-uniform) the steps past the sub-range
            if (f[u] >= 0)
                atomicAdd(&hw[w][f[u] >> shift], 1);
        }
    }
    // thread t owns buckets [PER t, PER t + PER): their global starts (an
    // exclusive scan of total), this block's offset in each, then one cursor
    // per wave
    int c[PER];
    int local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int b = PER * threadIdx.x + j;
        c[j] = b < nb ? total[b] : 0;
        local += c[j];
    }
    if (blockIdx.x == 0) {
        const int64_t big = 4 * ((picks + nb - 1) / nb);
        int nbig = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            nbig += (PER * (int)threadIdx.x + j < nb && c[j] > big) ? 1 : 0;
        int tb;
        const int bexcl = wave_exclusive_scan(nbig, &tb);
        if (lane == 0)
            wbig[w] = tb;
        __syncthreads();
        int pos_big = bexcl, all_big = 0;
        for (int u = 0; u < W; ++u) {
            pos_big += u < w ? wbig[u] : 0;
            all_big += wbig[u];
        }
        // the buckets before this thread's first are all in use when it has one
        int pos_small = all_big + PER * (int)threadIdx.x - pos_big;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int b = PER * threadIdx.x + j;
            if (b < nb) {
                if (c[j] > big)
                    bucket_order[pos_big++] = b;
                else
                    bucket_order[pos_small++] = b;
            }
        }
    }
    int tw;
    const int excl = wave_exclusive_scan(local, &tw);
    if (lane == 0)
        wsum[w] = tw;
    __syncthreads();
    int run = excl;
    for (int u = 0; u < w; ++u)
        run += wsum[u];
    const int32_t *row = bhist + (int64_t)blockIdx.x * nb;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int b = PER * threadIdx.x + j;
        if (b < nb) {
            if (blockIdx.x == 0)
                bucket_base[b] = run;
            int cur = run + row[b];
#pragma unroll
            for (int u = 0; u < kSortWaves; ++u) {
                const int cnt = hw[u][b];
                hw[u][b] = cur;
                cur += cnt;
            }
        }
        run += c[j];
    }
    if (blockIdx.x == 0 && threadIdx.x == kL1Threads - 1)
        bucket_base[nb] = run;
    __syncthreads();
    const int32_t lowmask = (1 << shift) - 1;
    // kSortUnroll steps of 64 picks per trip: their loads are all in flight
    // before the first step is placed
    for (int64_t q = sb; q < se; q += kWave * kSortUnroll) {
        int32_t f[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const int64_t p = q + u * kWave + lane;
            f[u] = p < se ? idx[p] : 0;
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            if (q + (int64_t)u * kWave >= se)
                break;              // (wave-uniform) no item of this step or later ones
            const int64_t p = q + u * kWave + lane;
            const bool valid = p < se;
            const int pos = place_step((uint32_t)(f[u] >> shift), valid, nb_bits, hw[w]);
            if (valid)
                pairs[pos] = make_int2((int32_t)p, f[u] & lowmask);
        }
    }
}

// Level 2, one workgroup per bucket: per-wave histograms of the low slot bits
// in LDS, scan, slot_start of the bucket's 2^shift slots, then every pick's
// place (the bucket's pairs arrive in pick order, level 1 being stable, so
// each slot's picks end in ascending pick id).
__global__ __launch_bounds__(kL2Threads) void bucket_sort_kernel(
    const int2 *__restrict__ pairs, const int32_t *__restrict__ bucket_base,
    const int32_t *__restrict__ bucket_order, int shift, int64_t slots,
    int32_t *__restrict__ slot_start, int32_t *__restrict__ order)
{
    constexpr int W = kL2Threads / kWave;
    __shared__ int32_t hw[kSortWaves][kMaxBucketSlots];  // per-wave counts, then cursors
    __shared__ int32_t wsum[W];
    const int B = 1 << shift;
    const int bucket = bucket_order[blockIdx.x];
    const int64_t f0 = (int64_t)bucket << shift;
    const int nbins = (int)(slots - f0 < B ? slots - f0 : B);
    const int beg = bucket_base[bucket], end = bucket_base[bucket + 1];
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // only the B slots of a bucket (the rows are kMaxBucketSlots long)
    for (int u = 0; u < kSortWaves; ++u)
        for (int b = threadIdx.x; b < B; b += kL2Threads)
            hw[u][b] = 0;
    int64_t sb, se;
    sub_range(beg, end, w, sb, se);
    __syncthreads();
    // kSortUnroll pairs per lane in flight before their counters are bumped:
    // a large bucket (a Zipf-hot slot's) is this kernel's critical path
    for (int64_t q = sb + lane; q < se; q += kWave * kSortUnroll) {
        int key[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const int64_t p = q + (int64_t)u * kWave;
            key[u] = p < se ? pairs[p].y : -1;
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            if (q - lane + (int64_t)u * kWave >= se)
                break;              // (wave-uniform) the steps past the sub-range
            if (key[u] >= 0)
                atomicAdd(&hw[w][key[u]], 1);
        }
    }
    __syncthreads();
    // bin totals, their exclusive scan (thread t owns bins [BPT t, BPT t + BPT)),
    // then one cursor per (wave, bin)
    constexpr int BPT = kMaxBucketSlots / kL2Threads;
    int v[BPT], local = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
        const int bin = BPT * (int)threadIdx.x + e;
        int t = 0;
        if (bin < B) {
#pragma unroll
            for (int u = 0; u < kSortWaves; ++u)
                t += hw[u][bin];
        }
        v[e] = t;
        local += t;
    }
    int tw;
    const int excl = wave_exclusive_scan(local, &tw);
    if (lane == 0)
        wsum[w] = tw;
    __syncthreads();
    int run = beg + excl;
    for (int u = 0; u < w; ++u)
        run += wsum[u];
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
        const int bin = BPT * (int)threadIdx.x + e;
        if (bin < nbins) {
            slot_start[f0 + bin] = run;
            int cur = run;
#pragma unroll
            for (int u = 0; u < kSortWaves; ++u) {
                const int cnt = hw[u][bin];
                hw[u][bin] = cur;
                cur += cnt;
            }
        }
        run += v[e];
    }
    if (f0 + B >= slots && threadIdx.x == 0)
        slot_start[slots] = end;
    __syncthreads();
    for (int64_t q = sb; q < se; q += kWave * kSortUnroll) {
        int2 pr[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const int64_t p = q + u * kWave + lane;
            pr[u] = p < se ? pairs[p] : make_int2(0, 0);
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            if (q + (int64_t)u * kWave >= se)
                break;              // (wave-uniform) no item of this step or later ones
            const bool valid = q + u * kWave + lane < se;
            const int pos = place_step((uint32_t)pr[u].y, valid, shift, hw[w]);
            if (valid)
                order[pos] = pr[u].x;
        }
    }
}

// Pieces of the long runs.  A run of more than `chunk` sorted picks is cut at
// the nominal chunk bounds; the wave holding a piece stores the piece's sum
// (no atomics) in row 2 (a >> shift) + (a is not a chunk bound) of `split`,
// a = the piece's first position in the sorted order.  A run's first piece
// starts at its own start, every later one at a chunk bound, so no two
// pieces of one batch share a row (a chunk holds at most the last piece of
// one long run and the first piece of the next, told apart by the + 1).
__device__ __forceinline__ int64_t piece_row(int64_t a, int shift)
{
    return 2 * (a >> shift) + ((a & (((int64_t)1 << shift) - 1)) != 0 ? 1 : 0);
}

// After the segmented reduction, one pass over the slots (each wave checks
// 64 slots, one per lane): in overwrite mode (MODE 0) the rows no pick
// selected become 0, all lanes on one row at a time; every run longer than
// the chunk is appended to `longs` (its slot), counted in longs[-1], which
// seg_value_kernel reset.  The runs of the Zipf-hot queries' slots sit next
// to each other (slots i n + j of one hot left sub-key i), so they are summed
// by long_run_kernel, one workgroup each, rather than in turn by the wave
// that found them.
constexpr int kFinishWaves = 4;
template <int MODE>
__global__ __launch_bounds__(kFinishWaves *kWave) void slot_scan_kernel(
    const int32_t *__restrict__ start, int64_t slots, int d_v, int shift,
    float *__restrict__ dvalues, int32_t *__restrict__ longs)
{
    const int lane = lane_id();
    const int64_t chunk = (int64_t)1 << shift;
    const int64_t f0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * kWave;
    if (f0 >= slots)
        return;
    const int64_t f = f0 + lane;
    bool is_long = false, empty = false;
    if (f < slots) {
        const int64_t b = start[f], e = start[f + 1];
        is_long = e - b > chunk;
        empty = b == e;
    }
    const uint64_t lm = __ballot(is_long);
    if (lm) {
        int at = 0;
        if (lane == 0)
            at = atomicAdd(longs - 1, __popcll(lm));
        at = __shfl(at, 0);
        if (is_long)
            longs[at + __popcll(lm & lanes_below())] = (int32_t)f;
    }
    if constexpr (MODE == 0) {
        uint64_t todo = __ballot(empty);
        while (todo) {
            const int i = __builtin_ctzll(todo);
            todo &= todo - 1;
            float4 *row = reinterpret_cast<float4 *>(dvalues + (f0 + i) * d_v);
            for (int c = lane; c < d_v / 4; c += kWave)
                row[c] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// One wave per listed long run: its pieces summed in the order of their
// positions -- a fixed order, so the result does not depend on which wave
// ran first -- and the sum g stored (MODE 0), added to dvalues (MODE 1), or
// applied to the value row, w = fmaf(-lr, g, w) rounded once to the storage
// type (MODE 2, the fused SGD; the rows were only read until now).
template <typename DT, int MODE>
__global__ __launch_bounds__(kFinishWaves *kWave) void long_run_kernel(
    const int32_t *__restrict__ start, int d_v, int shift, const float *__restrict__ split,
    const int32_t *__restrict__ longs, float *__restrict__ dvalues, DT *__restrict__ values,
    float lr)
{
    constexpr int EPC = Elt<DT>::per16;
    const int lane = lane_id();
    // workgroup b takes the listed runs b, b + gridDim.x, ...; its waves
    // split a run's row into column parts, so each wave keeps more pieces
    // in flight (a Zipf-hot run has a few dozen)
    const int part = (int)(threadIdx.x / kWave);
    const int runs = longs[-1];
    for (int run = (int)blockIdx.x; run < runs; run += (int)gridDim.x) {
        const int64_t fr = longs[run];
        const int64_t b = start[fr], e = start[fr + 1];
        const int64_t cb = b >> shift, ce = (e - 1) >> shift;
        const int64_t r0 = piece_row(b, shift);
        auto row_of = [&](int64_t cc) { return cc == cb ? r0 : 2 * cc; };
        // one unit of EPC floats per lane per pass; the loads of PIECES pieces
        // are issued before any is added, then the pieces are added one after
        // the other in position order (the same order in every mode, so
        // overwrite + sparse SGD and the fused SGD agree bit for bit)
        constexpr int UPL = 1, PIECES = 128 / EPC;
        const int nunits = d_v / EPC;
        for (int u0 = part * UPL * kWave; u0 < nunits; u0 += kFinishWaves * UPL * kWave) {
            float g[UPL][EPC];
#pragma unroll
            for (int m = 0; m < UPL; ++m)
#pragma unroll
                for (int x = 0; x < EPC; ++x)
                    g[m][x] = 0.f;
            for (int64_t cc = cb; cc <= ce; cc += PIECES) {
                float4 ld[PIECES][UPL][EPC / 4];
#pragma unroll
                for (int pc = 0; pc < PIECES; ++pc) {
                    const int64_t rr = row_of(cc + pc <= ce ? cc + pc : cc);
#pragma unroll
                    for (int m = 0; m < UPL; ++m) {
                        const int u = u0 + lane + m * kWave;
                        const float *src = split + rr * d_v + (int64_t)(u < nunits ? u : 0) * EPC;
#pragma unroll
                        for (int x = 0; x < EPC / 4; ++x)
                            ld[pc][m][x] = *reinterpret_cast<const float4 *>(src + 4 * x);
                    }
                }
#pragma unroll
                for (int pc = 0; pc < PIECES; ++pc) {
                    if (cc + pc <= ce) {
#pragma unroll
                        for (int m = 0; m < UPL; ++m)
#pragma unroll
                            for (int x = 0; x < EPC / 4; ++x) {
                                g[m][4 * x] += ld[pc][m][x].x;
                                g[m][4 * x + 1] += ld[pc][m][x].y;
                                g[m][4 * x + 2] += ld[pc][m][x].z;
                                g[m][4 * x + 3] += ld[pc][m][x].w;
                            }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < UPL; ++m) {
                const int u = u0 + lane + m * kWave;
                if (u >= nunits)
                    continue;
                if constexpr (MODE == 2) {
                    DT *dst = values + fr * d_v + (int64_t)u * EPC;
                    float w[EPC];
                    unpack16(*reinterpret_cast<const uint4 *>(dst), w);
#pragma unroll
                    for (int x = 0; x < EPC; ++x)
                        w[x] = fmaf(-lr, g[m][x], w[x]);
                    if constexpr (sizeof(DT) == 2) {
                        uint4 r;
                        r.x = f32_to_bf16_bits(w[0]) | (f32_to_bf16_bits(w[1]) << 16);
                        r.y = f32_to_bf16_bits(w[2]) | (f32_to_bf16_bits(w[3]) << 16);
                        r.z = f32_to_bf16_bits(w[4]) | (f32_to_bf16_bits(w[5]) << 16);
                        r.w = f32_to_bf16_bits(w[6]) | (f32_to_bf16_bits(w[7]) << 16);
                        *reinterpret_cast<uint4 *>(dst) = r;
                    } else {
                        *reinterpret_cast<float4 *>(dst) = make_float4(w[0], w[1], w[2], w[3]);
                    }
                } else {
                    float *dst = dvalues + fr * d_v + (int64_t)u * EPC;
#pragma unroll
                    for (int x = 0; x < EPC; x += 4) {
                        float4 o = make_float4(g[m][x], g[m][x + 1], g[m][x + 2], g[m][x + 3]);
                        if (MODE == 1) {
                            const float4 old = *reinterpret_cast<const float4 *>(dst + x);
                            o.x += old.x;
                            o.y += old.y;
                            o.z += old.z;
                            o.w += old.w;
                        }
                        *reinterpret_cast<float4 *>(dst + x) = o;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 2. segmented reduction over the slot-sorted picks
// ---------------------------------------------------------------------------
constexpr int kSegWaves = 4;

// MCH: 16-byte chunks of a row per lane; U: picks per group.  Wave w takes
// the sorted picks of its nominal range [256 w, 256 w + 256), moved so that a
// slot's run of at most `chunk` picks is never cut: such a run belongs to
// the wave whose range holds its first pick (a range grows to < 2 chunk).
// chunk = 2^shift <= kSegChunk: 256, or less on small batches.
// Longer runs are cut at the nominal bounds.  The wave stages the (pick,
// token, slot, weight) of its picks in LDS and lists where each run starts,
// then streams the picks in groups of U with two groups of dy rows in flight;
// the value row of the next run is fetched while the current one is worked
// on.  A run's sum is stored (the row is this wave's alone) unless the run is
// longer than chunk: each wave holding a piece of such a run stores the
// piece's sum to the piece's own row of `split` (piece_row), and
// long_run_kernel adds the pieces in position order.
template <int MCH, int U>
struct DyGroup {
    uint4 r[U][MCH];
};

// dy rows of picks j .. j+U-1 of the chunk; picks past its end read as zeros.
// Exactly U * MCH loads whatever the data, so that the loop's waits stay
// partial (the other group remains in flight).
template <typename DT, int MCH, int U>
__device__ __forceinline__ void seg_load_group(DyGroup<MCH, U> &g, const DT *__restrict__ dy,
                                               const int32_t *s_tok, int j, int len, int d_v,
                                               int lane)
{
    const int row_bytes = d_v * (int)sizeof(DT);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool live = j + u < len;
        const int64_t t = __builtin_amdgcn_readfirstlane(s_tok[live ? j + u : len - 1]);
        const __amdgpu_buffer_rsrc_t r = buffer_over(dy + t * d_v, live ? row_bytes : 0);
#pragma unroll
        for (int m = 0; m < MCH; ++m)
            g.r[u][m] = buffer_load16(r, (lane + m * kWave) * 16, 0);
    }
}

template <typename DT, int MCH>
__device__ __forceinline__ void seg_load_row(uint4 (&v)[MCH], const DT *__restrict__ values,
                                             int64_t f, int d_v, int lane)
{
    const __amdgpu_buffer_rsrc_t r = buffer_over(values + f * d_v, d_v * (int)sizeof(DT));
#pragma unroll
    for (int m = 0; m < MCH; ++m)
        v[m] = buffer_load16(r, (lane + m * kWave) * 16, 0);
}

template <int MCH, int EPC>
__device__ __forceinline__ void seg_flush(float (&acc)[MCH][EPC], float *__restrict__ dvalues,
                                          float *__restrict__ piece, int64_t f, int d_v,
                                          int nchunks, int lane, bool exclusive, int accumulate)
{
    // a run this wave holds whole goes to its dvalues row; a piece of a long
    // run to its piece row (summed later, in order, by long_run_kernel)
    float *drow = exclusive ? dvalues + f * d_v : piece;
    const bool add = exclusive && accumulate;
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
        const int c = lane + m * kWave;
        if (c < nchunks) {
            float *dst = drow + (int64_t)c * EPC;
#pragma unroll
            for (int e = 0; e < EPC / 4; ++e) {
                float4 o = make_float4(acc[m][4 * e], acc[m][4 * e + 1], acc[m][4 * e + 2],
                                       acc[m][4 * e + 3]);
                if (add) {
                    const float4 old = *reinterpret_cast<const float4 *>(dst + 4 * e);
                    o.x += old.x;
                    o.y += old.y;
                    o.z += old.z;
                    o.w += old.w;
                }
                *reinterpret_cast<float4 *>(dst + 4 * e) = o;
            }
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[m][e] = 0.f;
    }
}

// The fused update: the run's sum g updates its value row in place,
// w = fmaf(-lr, g, w) rounded once to the storage type (vrow holds the row's
// old values), when the row is this wave's alone; a long run's piece goes to
// its piece row, applied after the kernel by long_run_kernel.
template <typename DT, int MCH, int EPC>
__device__ __forceinline__ void seg_flush_sgd(float (&acc)[MCH][EPC], const float (&vrow)[MCH][EPC],
                                              DT *values, float *__restrict__ piece, int64_t f,
                                              int d_v, int nchunks, int lane, bool exclusive,
                                              float lr)
{
    if (!exclusive) {
        seg_flush<MCH, EPC>(acc, nullptr, piece, f, d_v, nchunks, lane, false, 0);
        return;
    }
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
        const int c = lane + m * kWave;
        if (c < nchunks) {
            float w[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e)
                w[e] = fmaf(-lr, acc[m][e], vrow[m][e]);
            DT *dst = values + f * d_v + (int64_t)c * EPC;
            if constexpr (sizeof(DT) == 2) {
                uint4 r;
                r.x = f32_to_bf16_bits(w[0]) | (f32_to_bf16_bits(w[1]) << 16);
                r.y = f32_to_bf16_bits(w[2]) | (f32_to_bf16_bits(w[3]) << 16);
                r.z = f32_to_bf16_bits(w[4]) | (f32_to_bf16_bits(w[5]) << 16);
                r.w = f32_to_bf16_bits(w[6]) | (f32_to_bf16_bits(w[7]) << 16);
                *reinterpret_cast<uint4 *>(dst) = r;
            } else {
                *reinterpret_cast<float4 *>(dst) = make_float4(w[0], w[1], w[2], w[3]);
            }
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[m][e] = 0.f;
    }
}

// SGD: the value rows are updated in place (values is then written, and
// dvalues is unused, see seg_flush_sgd); dw is the same in every mode.
template <typename DT, bool SGD>
using ValuesPtr = typename std::conditional<SGD, DT *, const DT *>::type;

template <typename DT, int MCH, int U, bool SGD>
__global__ __launch_bounds__(kSegWaves *kWave) void seg_value_kernel(
    ValuesPtr<DT, SGD> values, const DT *__restrict__ dy, const int32_t *__restrict__ idx,
    const float *__restrict__ weights, const int32_t *__restrict__ order,
    const int32_t *__restrict__ start, float *__restrict__ dvalues, float *__restrict__ split,
    float *__restrict__ dw, int64_t picks, int HK, int d_v, int accumulate, float lr, int shift)
{
    const int chunk = 1 << shift;
    constexpr int EPC = Elt<DT>::per16;
    constexpr int kMaxLen = 2 * kSegChunk;
    __shared__ int32_t s_pk[kSegWaves][kMaxLen];
    __shared__ int32_t s_tok[kSegWaves][kMaxLen];
    __shared__ int32_t s_slot[kSegWaves][kMaxLen];
    __shared__ float s_w[kSegWaves][kMaxLen];
    __shared__ float s_dw[kSegWaves][kMaxLen];
    __shared__ int32_t s_seg[kSegWaves][kMaxLen + 1];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        long_list(split, picks, d_v)[-1] = 0;   // the count of the long-run list (slot_scan_kernel)
    // neighbouring chunks on one XCD: the slots i n + j of one left sub-key i
    // are picked by largely the same tokens, whose dy rows are then read
    // again from the same L2
    const int64_t nom = ((int64_t)xcd_contiguous_id() * kSegWaves + wv) * chunk;
    if (nom >= picks)
        return;
    // a bound inside a run of at most chunk picks moves to the run's end
    auto run_len = [&](int f) { return start[f + 1] - start[f]; };
    auto adjust = [&](int64_t p) -> int64_t {
        if (p == 0 || p >= picks)
            return p;
        const int f = idx[order[p]];
        const int64_t b = start[f], e = start[f + 1];
        return (p == b || e - b > chunk) ? p : e;
    };
    const int64_t p_begin = adjust(nom);
    const int64_t p_end = adjust(nom + chunk < picks ? nom + chunk : picks);
    if (p_end <= p_begin)
        return;
    const int len = (int)(p_end - p_begin);
    const int nchunks = d_v / EPC;
    const int32_t *tok = s_tok[wv];
    const int32_t *slot = s_slot[wv];
    int32_t *segs = s_seg[wv];

    for (int j = lane; j < len; j += kWave) {
        const int32_t pk = order[p_begin + j];
        s_pk[wv][j] = pk;
        s_tok[wv][j] = pk / HK;
        s_slot[wv][j] = idx[pk];
        s_w[wv][j] = weights[pk];
    }
    wave_lds_sync();
    // segment starts: positions whose slot differs from the previous one
    int nseg = 0;
    for (int b = 0; b < len; b += kWave) {
        const int j = b + lane;
        const bool head = j < len && (j == 0 || slot[j] != slot[j - 1]);
        const uint64_t mask = __ballot(head);
        if (head)
            segs[nseg + __builtin_popcountll(mask & ((1ull << lane) - 1))] = j;
        nseg += __builtin_popcountll(mask);
    }
    if (lane == 0)
        segs[nseg] = len;
    wave_lds_sync();

    // the value rows of segments 0 and 1, two groups of dy rows
    uint4 vcur[MCH], vnext[MCH];
    const int f_first = __builtin_amdgcn_readfirstlane(slot[0]);
    seg_load_row<DT, MCH>(vcur, values, f_first, d_v, lane);
    seg_load_row<DT, MCH>(vnext, values,
                          __builtin_amdgcn_readfirstlane(slot[segs[nseg > 1 ? 1 : 0]]), d_v, lane);
    DyGroup<MCH, U> ga, gb;
    seg_load_group<DT, MCH, U>(ga, dy, tok, 0, len, d_v, lane);
    seg_load_group<DT, MCH, U>(gb, dy, tok, U, len, d_v, lane);
    // only the first and the last run can be long ones, shared with other waves
    const int f_last = __builtin_amdgcn_readfirstlane(slot[len - 1]);
    const bool first_split = run_len(f_first) > chunk;
    const bool last_split = run_len(f_last) > chunk;

    float vrow[MCH][EPC], acc[MCH][EPC];
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
        unpack16(vcur[m], vrow[m]);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[m][e] = 0.f;
    }
    int seg = 0;
    int seg_end = __builtin_amdgcn_readfirstlane(segs[1]);
    int f_cur = f_first;
    // the current run's sum leaves: stored, added, or (SGD) applied to its
    // row; a piece of a long run goes to its piece row
    auto flush = [&](bool exclusive) {
        float *piece = nullptr;
        if (!exclusive)
            piece = split + piece_row(p_begin + __builtin_amdgcn_readfirstlane(segs[seg]), shift) *
                                (int64_t)d_v;
        if constexpr (SGD)
            seg_flush_sgd<DT, MCH, EPC>(acc, vrow, values, piece, f_cur, d_v, nchunks, lane,
                                        exclusive, lr);
        else
            seg_flush<MCH, EPC>(acc, dvalues, piece, f_cur, d_v, nchunks, lane, exclusive,
                                accumulate);
    };

    auto work = [&](DyGroup<MCH, U> &g, int j) {
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            part[u] = 0.f;
            if (j + u < len) {
                if (j + u == seg_end) {          // next run of slots
                    flush(!((seg == 0 && first_split) || (seg == nseg - 1 && last_split)));
                    ++seg;
                    seg_end = __builtin_amdgcn_readfirstlane(segs[seg + 1]);
                    f_cur = __builtin_amdgcn_readfirstlane(slot[j + u]);
#pragma unroll
                    for (int m = 0; m < MCH; ++m)
                        unpack16(vnext[m], vrow[m]);
                    const int nxt = seg + 1 < nseg ? seg + 1 : seg;
                    seg_load_row<DT, MCH>(vnext, values,
                                          __builtin_amdgcn_readfirstlane(slot[segs[nxt]]), d_v,
                                          lane);
                }
                const float w = s_w[wv][j + u];
#pragma unroll
                for (int m = 0; m < MCH; ++m) {
                    float x[EPC];
                    unpack16(g.r[u][m], x);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        part[u] = fmaf(vrow[m][e], x[e], part[u]);
                        acc[m][e] = fmaf(w, x[e], acc[m][e]);
                    }
                }
            }
        }
        // lane l ends with the dot of pick j + l / (64 / U)
        wave_multi_sum<U>(part);
        const int u_mine = lane / (kWave / U);
        if (lane % (kWave / U) == 0 && j + u_mine < len)
            s_dw[wv][j + u_mine] = part[0];
    };

    for (int j = 0; j < len; j += 2 * U) {
        work(ga, j);
        seg_load_group<DT, MCH, U>(ga, dy, tok, j + 2 * U, len, d_v, lane);
        work(gb, j + U);
        seg_load_group<DT, MCH, U>(gb, dy, tok, j + 3 * U, len, d_v, lane);
    }
    flush(!((seg == 0 && first_split) || (seg == nseg - 1 && last_split)));
    wave_lds_sync();
    for (int j = lane; j < len; j += kWave)
        dw[s_pk[wv][j]] = s_dw[wv][j];
}

// ---------------------------------------------------------------------------
// 3. softmax backward per distinct sub-key, dq, compact (i, g) lists
// ---------------------------------------------------------------------------
constexpr int kQryWaves = 4;
constexpr int kQryMaxK = 64;

// Four consecutive elements of a sub-key row through a buffer descriptor
// (offsets past the codebook read as zeros): raw load, then widening.
template <typename DT>
struct Row4;
template <>
struct Row4<float> {
    uint4 raw;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff)
    {
        raw = buffer_load16(r, voff, 0);
    }
    __device__ __forceinline__ float operator[](int e) const
    {
        return __uint_as_float(e == 0 ? raw.x : e == 1 ? raw.y : e == 2 ? raw.z : raw.w);
    }
};
template <>
struct Row4<bf16_t> {
    uint32_t lo, hi;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        lo = v[0];
        hi = v[1];
    }
    __device__ __forceinline__ float operator[](int e) const
    {
        const uint32_t w = e < 2 ? lo : hi;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// One wave per (token, head).  For k <= 32 one pass gives each lane one
// (half, pick): lanes 0-31 the left sub-keys, lanes 32-63 the right ones;
// for larger k two passes, one half each.  A lane's sums A, W, B, Wc run over
// its half's picks staged in LDS (one broadcast read per pick).  The distinct
// sub-keys then form a list in two segments of 32 positions (see below), and
// their rows are fetched in batches of kBatch before they are used: in the dq
// product each lane owns JPL groups of 4 consecutive elements of a half
// (half <= 256 JPL).
template <typename DT, int JPL>
__global__ __launch_bounds__(kQryWaves *kWave) void bwd_query_kernel(
    const DT *__restrict__ keys, int64_t key_hstride, const int32_t *__restrict__ idx,
    const float *__restrict__ weights, const float *__restrict__ dw, float *__restrict__ dq,
    int32_t *__restrict__ gl_i, float *__restrict__ gl_g, int64_t T, int H, int n, int k, int d_k)
{
    constexpr int kBatch = (sizeof(DT) == 2 ? 32 : 16) / JPL;     // sub-key rows in flight
    __shared__ int4 s_pick[kQryWaves][2][kQryMaxK];    // per half: sub-key, w, w dw, 0
    __shared__ int32_t s_sub[kQryWaves][kWave];      // distinct (half * n + sub), <= 64 a pass
    __shared__ float s_g[kQryWaves][kWave];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = (int64_t)blockIdx.x * kQryWaves + wv;
    if (row >= T * H)
        return;
    const int h = (int)(row % H);
    const int half = d_k / 2;
    const int groups = half / 4;
    const int64_t base = row * (int64_t)k;
    if (lane < k) {
        const int f = idx[base + lane];
        const float w = weights[base + lane];
        const int wi = __float_as_int(w), wdwi = __float_as_int(w * dw[base + lane]);
        s_pick[wv][0][lane] = make_int4(f / n, wi, wdwi, 0);
        s_pick[wv][1][lane] = make_int4(f % n, wi, wdwi, 0);
    } else if (lane < ((k + 3) & ~3)) {
        // padding up to a multiple of 4 picks: no sub-key, zero weights
        s_pick[wv][0][lane] = s_pick[wv][1][lane] = make_int4(-1, 0, 0, 0);
    }
    wave_lds_sync();

    const int passes = k <= kWave / 2 ? 1 : 2;
    const DT *kh = keys + h * key_hstride;
    const __amdgpu_buffer_rsrc_t rsrc = buffer_over(kh, 2 * n * half * (int)sizeof(DT));
    constexpr int kOut = 0x40000000;      // an offset past any codebook: reads zeros
    // byte offset of this lane's 4 elements in a sub-key row (kOut past the
    // half: kOut plus any row offset still reads zeros)
    int lane_off[JPL];
#pragma unroll
    for (int j = 0; j < JPL; ++j) {
        const int c = lane + j * kWave;
        lane_off[j] = c < groups ? 4 * c * (int)sizeof(DT) : kOut;
    }
    // one set of accumulators, for the half whose entries are being summed;
    // `flush` writes it to half `acc_half` of dq and clears it
    float acc[JPL][4];
#pragma unroll
    for (int j = 0; j < JPL; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[j][e] = 0.f;
    int acc_half = 0;
    float *dqr = dq + row * (int64_t)d_k;
    auto flush = [&]() {
#pragma unroll
        for (int j = 0; j < JPL; ++j) {
            const int c = lane + j * kWave;
            if (c < groups)
                *reinterpret_cast<float4 *>(dqr + acc_half * half + 4 * c) =
                    make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[j][e] = 0.f;
        }
    };

    for (int pass = 0; pass < passes; ++pass) {
        const int s = passes == 1 ? lane / (kWave / 2) : pass;
        const int r = passes == 1 ? lane % (kWave / 2) : lane;
        const bool valid = r < k;
        const int4 *picks = s_pick[wv][s];
        const int sub = picks[valid ? r : 0].x;
        // sums over the picks sharing this lane's sub-key (A, W) and over the
        // rest (B, Wc), as fmas with a 1 or 0 factor (the same roundings as
        // plain sums, and no exec-mask updates); the first pick of each
        // sub-key carries its g.  `earlier` collects, as a lane mask, the
        // lanes that an earlier pick with the same sub-key has already seen
        // (lane r is "later" than pick q iff r > q).
        float A = 0.f, W = 0.f, B = 0.f, Wc = 0.f;
        uint64_t earlier = 0;
        // lanes later than pick q: r > q, per 32-lane half with one pass
        const uint64_t keep = passes == 1 ? 0xFFFFFFFEFFFFFFFFull : ~0ull;
        uint64_t later = passes == 1 ? 0xFFFFFFFEFFFFFFFEull : ~1ull;
        for (int q0 = 0; q0 < k; q0 += 4) {
            int4 e[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                e[u] = picks[q0 + u];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w_q = __int_as_float(e[u].y), wdw_q = __int_as_float(e[u].z);
                const bool same = e[u].x == sub;
                const float in = same ? 1.f : 0.f, out = same ? 0.f : 1.f;
                A = fmaf(wdw_q, in, A);
                W = fmaf(w_q, in, W);
                B = fmaf(wdw_q, out, B);
                Wc = fmaf(w_q, out, Wc);
                earlier |= __ballot(same) & later;
                later = (later << 1) & keep;
            }
        }
        const bool first = valid && ((earlier >> lane) & 1ull) == 0;
        const float g = A * Wc - B * W;
        if (valid) {
            const int64_t at = (row * 2 + s) * (int64_t)k + r;
            gl_i[at] = sub;
            gl_g[at] = first ? g : 0.f;
        }
        // the distinct sub-keys of this pass, compacted into two segments of
        // 32 list positions: one pass (k <= 32) puts the left half's entries
        // in segment 0 and the right half's in segment 1; with two passes
        // (one half each) the pass's entries fill segment 0, then segment 1.
        // Position p is held by lane p (as codebook row s * n + sub, and g);
        // positions past a segment's count hold a row past the codebooks
        // (reads zeros) with g = 0.
        const uint64_t mask = __ballot(first);
        int seg_cnt[2];
        if (passes == 1) {
            seg_cnt[0] = __builtin_popcountll(mask & 0xFFFFFFFFull);
            seg_cnt[1] = __builtin_popcountll(mask >> 32);
        } else {
            const int cnt = __builtin_popcountll(mask);
            seg_cnt[0] = cnt < 32 ? cnt : 32;
            seg_cnt[1] = cnt - seg_cnt[0];
        }
        if (first) {
            const uint64_t below = mask & ((1ull << lane) - 1);
            const int pos = passes == 1
                                ? (lane & 32) + __builtin_popcountll(below & (lane < 32 ? 0xFFFFFFFFull : ~0xFFFFFFFFull))
                                : __builtin_popcountll(below);
            s_sub[wv][pos] = s * n + sub;
            s_g[wv][pos] = g;
        }
        wave_lds_sync();
        const bool in_list = (lane & 31) < seg_cnt[lane >> 5];
        const int l_row = in_list ? s_sub[wv][lane] : 2 * n;
        const float l_g = in_list ? s_g[wv][lane] : 0.f;

        // dq half += g * sub-key row, kBatch rows in flight, each entry 4 JPL
        // FMAs; a segment's unused tail is skipped 4 entries at a time
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
#pragma unroll
            for (int b = 0; b < 32 / kBatch; ++b) {
                const int first_e = b * kBatch;             // in the segment
                if (first_e >= seg_cnt[sg])
                    break;
                Row4<DT> x[kBatch][JPL];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int row_off = __builtin_amdgcn_readlane(l_row, 32 * sg + first_e + u) *
                                        half * (int)sizeof(DT);
#pragma unroll
                    for (int j = 0; j < JPL; ++j)
                        x[u][j].load(rsrc, lane_off[j] + row_off);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (u % 4 == 0 && first_e + u >= seg_cnt[sg])
                        break;
                    const float gv = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(l_g), 32 * sg + first_e + u));
#pragma unroll
                    for (int j = 0; j < JPL; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[j][e] = fmaf(gv, x[u][j][e], acc[j][e]);
                }
            }
            if (passes == 1) {
                acc_half = sg;
                flush();
            }
        }
        if (passes == 2) {
            acc_half = pass;
            flush();
        }
        wave_lds_sync();     // s_sub / s_g are rewritten by the next pass
    }
}

// ---------------------------------------------------------------------------
// 4. sub-key gradient as a dense MFMA product over token steps
// ---------------------------------------------------------------------------
// dkeys[h][s] = dS^T q_s, where dS [T][n] holds, per token, the g of each
// distinct sub-key of its k picks and zeros elsewhere.  A workgroup owns one
// token block and 16 CT columns of one codebook; per step of 32 tokens it
// scatters the (sub-key, g) entries into a zeroed LDS tile dS^T [n][32] (no
// two entries share a cell, so plain stores), stages q's columns transposed
// [16 CT][32], and accumulates [n][16 CT] in MFMA registers: wave w owns
// the 16-row tiles w, w + 16, ... and loads each of their A fragments once per
// step for all column tiles.  The global reads of step i + 1 are issued
// before the MFMAs of step i.  Tiles keep 16-byte chunks XOR-swizzled by row,
// so the 16 rows an MFMA operand read touches fall in distinct banks.  No
// atomics, so hot sub-keys cost nothing extra and the result does not depend
// on timing.
//   bf16 storage: g = hi + lo (two bfloat16, ~16 significant bits), q exact in
//     bfloat16, v_mfma_f32_16x16x32_bf16 twice per tile: exact products,
//     float32 sums;
//   float32 storage: v_mfma_f32_16x16x4_f32 on the float32 values.
constexpr int kDkWaves = 16;
constexpr int kDkTok = 32;          // tokens per step (the MFMA K extent), or 64 (see below)

template <typename DT> struct DkTile;
template <> struct DkTile<bf16_t> {
    typedef uint16_t elt;
    static constexpr int parts = 2;
};
template <> struct DkTile<float> {
    typedef float elt;
    static constexpr int parts = 1;
};

// Element offset of (row, token) in a [rows][TOK] tile of C 16-byte chunks
// per row, the chunks XOR-swizzled by row: the 16 rows of an operand read
// cover all banks.
template <int C, int TOK>
__device__ __forceinline__ int dk_cell(int row, int tl)
{
    constexpr int EPC = TOK / C;                    // elements per chunk
    const int c = (tl / EPC) ^ ((row / (16 / C)) % C);
    return row * TOK + c * EPC + tl % EPC;
}
template <typename E, int TOK>
__device__ __forceinline__ int dk_cell_of(int row, int tl)
{
    return dk_cell<TOK * (int)sizeof(E) / 16, TOK>(row, tl);
}

template <int TOK>
__device__ __forceinline__ uint4 dk_chunk(const uint16_t *tile, int row, int c)
{
    return *reinterpret_cast<const uint4 *>(tile + dk_cell<TOK / 8, TOK>(row, 8 * c));
}
template <int TOK>
__device__ __forceinline__ float4 dk_chunk(const float *tile, int row, int c)
{
    return *reinterpret_cast<const float4 *>(tile + dk_cell<TOK / 4, TOK>(row, 4 * c));
}

__device__ __forceinline__ void dk_store(uint16_t *hi, uint16_t *lo, int at, float g)
{
    const uint32_t h = f32_to_bf16_bits(g);
    hi[at] = (uint16_t)h;
    lo[at] = (uint16_t)f32_to_bf16_bits(g - bf16_to_f32(h));
}
__device__ __forceinline__ void dk_store(float *a, float *, int at, float g) { a[at] = g; }
__device__ __forceinline__ void dk_clear(uint16_t *hi, uint16_t *lo, int at)
{
    hi[at] = 0;
    lo[at] = 0;
}
__device__ __forceinline__ void dk_clear(float *a, float *, int at) { a[at] = 0.f; }

// q staging of one step.  bf16, 32-token steps: thread u < 256 takes the token pair
// (2 (u % 16), + 1) and 8 columns 8 (u / 16) ..: two 16-byte loads, eight
// packed 4-byte LDS stores.  float32: thread u takes token u % 32 and 4
// columns 4 (u / 32) ..: one 16-byte load, four LDS stores.
struct DkQBf16 {
    uint4 a, b;
};
struct DkQBf16One {
    uint4 a;
};
struct DkQF32 {
    float4 a;
};
template <typename DT, int TOK> struct DkQ;
template <> struct DkQ<bf16_t, 32> { typedef DkQBf16 type; };
template <> struct DkQ<bf16_t, 64> { typedef DkQBf16One type; };
template <> struct DkQ<float, 32> { typedef DkQF32 type; };

// bf16, 64-token steps: thread u takes token u % 64 and 8 columns 8 (u / 64)
// ..: one 16-byte load, eight 2-byte LDS stores.
template <int CT, int TOK>
__device__ __forceinline__ void dk_q_load(DkQBf16One &v, const bf16_t *q, int64_t t0, int64_t t_end,
                                          int H, int h, int d_k, int col0, int half, int tid)
{
    static_assert(TOK == 64, "one token per thread");
    v.a = make_uint4(0u, 0u, 0u, 0u);
    const int tl = tid % TOK, cg = tid / TOK;
    const int col = col0 + 8 * cg;
    const int64_t t = t0 + tl;
    if (cg < 16 * CT / 8 && col < half && t < t_end)
        v.a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(q) +
                                               (t * H + h) * (int64_t)d_k + col);
}
template <int CT, int TOK>
__device__ __forceinline__ void dk_q_store(const DkQBf16One &v, uint16_t *bt, int tid)
{
    const int tl = tid % TOK, cg = tid / TOK;
    if (cg >= 16 * CT / 8)
        return;
    const uint32_t a[4] = {v.a.x, v.a.y, v.a.z, v.a.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        bt[dk_cell<TOK / 8, TOK>(8 * cg + i, tl)] = (uint16_t)((i & 1) ? a[i / 2] >> 16 : a[i / 2]);
}

template <int CT, int TOK>
__device__ __forceinline__ void dk_q_load(DkQBf16 &v, const bf16_t *q, int64_t t0, int64_t t_end,
                                          int H, int h, int d_k, int col0, int half, int tid)
{
    constexpr int PAIRS = TOK / 2;
    v.a = v.b = make_uint4(0u, 0u, 0u, 0u);
    if (tid >= PAIRS * (16 * CT / 8))
        return;
    const int tp = tid % PAIRS, cg = tid / PAIRS;
    const int col = col0 + 8 * cg;
    if (col >= half)
        return;
    const int64_t ta = t0 + 2 * tp, tb = ta + 1;
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(q);
    if (ta < t_end)
        v.a = *reinterpret_cast<const uint4 *>(qb + (ta * H + h) * (int64_t)d_k + col);
    if (tb < t_end)
        v.b = *reinterpret_cast<const uint4 *>(qb + (tb * H + h) * (int64_t)d_k + col);
}
template <int CT, int TOK>
__device__ __forceinline__ void dk_q_store(const DkQBf16 &v, uint16_t *bt, int tid)
{
    constexpr int PAIRS = TOK / 2;
    if (tid >= PAIRS * (16 * CT / 8))
        return;
    const int tp = tid % PAIRS, cg = tid / PAIRS;
    const uint32_t a[4] = {v.a.x, v.a.y, v.a.z, v.a.w}, b[4] = {v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (i & 1) ? a[i / 2] >> 16 : a[i / 2] & 0xffffu;
        const uint32_t hi = (i & 1) ? b[i / 2] >> 16 : b[i / 2] & 0xffffu;
        *reinterpret_cast<uint32_t *>(bt + dk_cell<TOK / 8, TOK>(8 * cg + i, 2 * tp)) = lo | (hi << 16);
    }
}
template <int CT, int TOK>
__device__ __forceinline__ void dk_q_load(DkQF32 &v, const float *q, int64_t t0, int64_t t_end,
                                          int H, int h, int d_k, int col0, int half, int tid)
{
    static_assert(TOK == kDkTok, "float32 storage steps over 32 tokens");
    v.a = make_float4(0.f, 0.f, 0.f, 0.f);
    const int tl = tid % TOK, cg = tid / TOK;
    const int col = col0 + 4 * cg;
    const int64_t t = t0 + tl;
    if (cg < 16 * CT / 4 && col < half && t < t_end)
        v.a = *reinterpret_cast<const float4 *>(q + (t * H + h) * (int64_t)d_k + col);
}
template <int CT, int TOK>
__device__ __forceinline__ void dk_q_store(const DkQF32 &v, float *bt, int tid)
{
    const int tl = tid % TOK, cg = tid / TOK;
    if (cg >= 16 * CT / 4)
        return;
    const float a[4] = {v.a.x, v.a.y, v.a.z, v.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        bt[dk_cell<TOK / 4, TOK>(4 * cg + i, tl)] = a[i];
}

// One 16 x 16 x 32-token product on fragments read from the swizzled tiles.
__device__ __forceinline__ floatx4 dk_mfma(const uint4 &a, const uint4 &b, floatx4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <typename DT, int RT, int CT, int TOK>
__global__ __launch_bounds__(kDkWaves *kWave) void dkeys_mfma_kernel(
    const DT *__restrict__ q, const int32_t *__restrict__ gl_i, const float *__restrict__ gl_g,
    float *__restrict__ partial, int64_t T, int H, int n, int k, int d_k, int tokens_per_block)
{
    typedef typename DkTile<DT>::elt E;
    constexpr int PARTS = DkTile<DT>::parts;
    static_assert(TOK == 32 || (TOK == 64 && PARTS == 2), "steps of 32 tokens, or 64 for bf16");
    extern __shared__ __align__(16) unsigned char smem[];
    const int n_pad = (n + 15) & ~15;
    E *a_hi = reinterpret_cast<E *>(smem);                      // [n_pad][32]
    E *a_lo = a_hi + (PARTS == 2 ? (size_t)n_pad * TOK : 0);  // [n_pad][TOK] (bf16 only)
    E *bt = a_hi + (size_t)PARTS * n_pad * TOK;                // [16 CT][TOK]

    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tid = threadIdx.x;
    const int half = d_k / 2;
    constexpr int CW = 16 * CT;
    const int ncb = (half + CW - 1) / CW;
    const int hs = blockIdx.y / ncb;
    const int c0 = (blockIdx.y % ncb) * CW;
    const int width = half - c0 < CW ? half - c0 : CW;
    const int h = hs / 2, s = hs % 2;
    const int ntiles = n_pad / 16;
    const DT *qs = q + (int64_t)s * half;

    for (int e = tid; e < (PARTS * n_pad + CW) * TOK; e += kDkWaves * kWave)
        a_hi[e] = (E)0;

    floatx4 acc[RT][CT];
#pragma unroll
    for (int ti = 0; ti < RT; ++ti)
#pragma unroll
        for (int nb = 0; nb < CT; ++nb)
            acc[ti][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int64_t t_begin = (int64_t)blockIdx.x * tokens_per_block;
    const int64_t t_end = t_begin + tokens_per_block < T ? t_begin + tokens_per_block : T;
    // (token, pick) pairs per step, <= 2048 (64-token steps only with k <= 32)
    const int pairs = TOK * k;

    // this thread's entries of a step: g and the tile cell (or -1)
    auto load_entries = [&](int64_t t0, float (&g)[2], int (&cell)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pr = tid + j * kDkWaves * kWave;
            g[j] = 0.f;
            cell[j] = -1;
            if (pr < pairs) {
                const int tl = pr / k, r = pr % k;
                const int64_t t = t0 + tl;
                if (t < t_end) {
                    const int64_t at = ((t * H + h) * 2 + s) * (int64_t)k + r;
                    g[j] = gl_g[at];
                    cell[j] = gl_i[at] * 64 + tl;      // row * 64 + token, decoded below
                }
            }
        }
    };
    float g_next[2];
    int cell_next[2];
    typename DkQ<DT, TOK>::type q_next;
    load_entries(t_begin, g_next, cell_next);
    dk_q_load<CT, TOK>(q_next, qs, t_begin, t_end, H, h, d_k, c0, half, tid);
    int mine_at[2] = {-1, -1};                    // cells this thread wrote
    __syncthreads();

    const int r16 = lane & 15, kg = lane >> 4;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += TOK) {
        // scatter this step's entries into dS^T, stage q^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            mine_at[j] = -1;
            if (cell_next[j] >= 0 && g_next[j] != 0.f) {
                const int at = dk_cell_of<E, TOK>(cell_next[j] / 64, cell_next[j] % 64);
                dk_store(a_hi, a_lo, at, g_next[j]);
                mine_at[j] = at;
            }
        }
        dk_q_store<CT, TOK>(q_next, bt, tid);
        // the next step's global reads fly during this step's products
        if (t0 + TOK < t_end) {
            load_entries(t0 + TOK, g_next, cell_next);
            dk_q_load<CT, TOK>(q_next, qs, t0 + TOK, t_end, H, h, d_k, c0, half, tid);
        }
        __syncthreads();

#pragma unroll
        for (int ti = 0; ti < RT; ++ti) {
            const int tile = wave + ti * kDkWaves;
            if (tile < ntiles) {
                const int row = tile * 16 + r16;
                if constexpr (PARTS == 2) {
                    // K = TOK tokens in steps of 32: chunks 4 ks + kg of the rows
#pragma unroll
                    for (int ks = 0; ks < TOK / 32; ++ks) {
                        const uint4 ah = dk_chunk<TOK>(a_hi, row, 4 * ks + kg);
                        const uint4 al = dk_chunk<TOK>(a_lo, row, 4 * ks + kg);
#pragma unroll
                        for (int nb = 0; nb < CT; ++nb) {
                            const uint4 b = dk_chunk<TOK>(bt, nb * 16 + r16, 4 * ks + kg);
                            acc[ti][nb] = dk_mfma(ah, b, acc[ti][nb]);
                            acc[ti][nb] = dk_mfma(al, b, acc[ti][nb]);
                        }
                    }
                } else {
                    // K = 32 tokens as chunks kg and kg + 4 of the row (4 tokens each)
                    const float4 a0 = dk_chunk<TOK>(a_hi, row, kg), a1 = dk_chunk<TOK>(a_hi, row, kg + 4);
#pragma unroll
                    for (int nb = 0; nb < CT; ++nb) {
                        const float4 b0 = dk_chunk<TOK>(bt, nb * 16 + r16, kg);
                        const float4 b1 = dk_chunk<TOK>(bt, nb * 16 + r16, kg + 4);
                        floatx4 c = acc[ti][nb];
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.x, b0.x, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.y, b0.y, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.z, b0.z, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.w, b0.w, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.x, b1.x, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.y, b1.y, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.z, b1.z, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.w, b1.w, c, 0, 0, 0);
                        acc[ti][nb] = c;
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (mine_at[j] >= 0)
                dk_clear(a_hi, a_lo, mine_at[j]);
        __syncthreads();
    }

    // partial[block][h][s][row][c0 + col]; lane holds rows 4*(l/16)+i, column l%16
    float *dst = partial + ((int64_t)blockIdx.x * H * 2 + hs) * (int64_t)n * half + c0;
#pragma unroll
    for (int ti = 0; ti < RT; ++ti) {
        const int tile = wave + ti * kDkWaves;
        if (tile >= ntiles)
            continue;
#pragma unroll
        for (int nb = 0; nb < CT; ++nb) {
            const int col = nb * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = tile * 16 + 4 * (lane >> 4) + i;
                if (row < n && col < width)
                    dst[(int64_t)row * half + col] = acc[ti][nb][i];
            }
        }
    }
}

// dkeys = the token blocks' partials summed in block order; with shared
// codebooks (fold = H) also over the heads, head by head within each block:
// dkeys[s][i][c] = sum_b sum_h partial[b][h][s][i][c] (count = one block's
// partial, H * 2 * n * half).
// Four consecutive outputs per thread (16-byte loads; out is a multiple of 4,
// as half is), each summed in the same order as one at a time.
__global__ void dkeys_reduce_kernel(const float *__restrict__ partial, int blocks, int64_t count,
                                    int fold, float *__restrict__ dkeys)
{
    const int64_t out = count / fold;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * e4 < out; e4 += stride) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int b = 0; b < blocks; ++b)
            for (int h = 0; h < fold; ++h) {
                const float4 v =
                    *reinterpret_cast<const float4 *>(partial + (int64_t)b * count + h * out + 4 * e4);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
        *reinterpret_cast<float4 *>(dkeys + 4 * e4) = acc;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static unsigned grid1d(int64_t n, int per)
{
    return (unsigned)((n + per - 1) / per);
}

template <typename DT, int MCH, int U, bool SGD>
static hipError_t launch_seg_t(const void *values, const void *dy, const int32_t *idx,
                               const float *weights, const int32_t *order, const int32_t *start,
                               float *dvalues, float *split, float *dw, int64_t picks, int HK,
                               int d_v, int accumulate, float lr, hipStream_t stream)
{
    const int shift = seg_shift(picks);
    const int64_t waves = (picks + (1 << shift) - 1) >> shift;
    // SGD: the rows are written; launch_bwd_value_sgd's caller handed them over
    // as writable memory (void *), only the shared signature carries const
    const auto vptr = static_cast<ValuesPtr<DT, SGD>>(const_cast<void *>(values));
    hipLaunchKernelGGL((seg_value_kernel<DT, MCH, U, SGD>), dim3(grid1d(waves, kSegWaves)),
                       dim3(kSegWaves * kWave), 0, stream, vptr,
                       static_cast<const DT *>(dy), idx, weights, order, start, dvalues, split,
                       dw, picks, HK, d_v, accumulate, lr, shift);
    return hipGetLastError();
}

template <typename DT, bool SGD>
static hipError_t launch_seg_dt(const void *values, const void *dy, const int32_t *idx,
                                const float *weights, const int32_t *order, const int32_t *start,
                                float *dvalues, float *split, float *dw, int64_t picks, int HK,
                                int d_v, int accumulate, float lr, hipStream_t stream)
{
    const int per_lane = (d_v / Elt<DT>::per16 + kWave - 1) / kWave;
#define PKM_SEG(MCH, U)                                                                        \
    launch_seg_t<DT, MCH, U, SGD>(values, dy, idx, weights, order, start, dvalues, split, dw,   \
                                  picks, HK, d_v, accumulate, lr, stream)
    if (per_lane <= 1)
        return PKM_SEG(1, 8);
    if (per_lane <= 2)
        return PKM_SEG(2, 8);
    if (per_lane <= 4)
        return PKM_SEG(4, 2);
    if (per_lane <= 8 || sizeof(DT) == 2)       // bf16 rows of <= 4096 fit 8 chunks per lane
        return PKM_SEG(8, 1);
    if constexpr (sizeof(DT) == 4)
        return PKM_SEG(16, 1);
#undef PKM_SEG
    return hipErrorInvalidValue;
}

hipError_t launch_slot_sort(const int32_t *idx, int64_t picks, int n, int32_t *slot_start,
                            int32_t *order, void *scratch, hipStream_t stream)
{
    const SlotSortScratch S = slot_sort_scratch(picks, n);
    char *base = static_cast<char *>(scratch);
    int32_t *bhist = reinterpret_cast<int32_t *>(base + S.off_bhist);
    int32_t *total = reinterpret_cast<int32_t *>(base + S.off_total);
    int32_t *bucket_base = reinterpret_cast<int32_t *>(base + S.off_base);
    int32_t *bucket_order = reinterpret_cast<int32_t *>(base + S.off_order);
    int2 *pairs = reinterpret_cast<int2 *>(base + S.off_pairs);
    const int64_t slots = (int64_t)n * n;
    hipLaunchKernelGGL(bucket_hist_kernel, dim3(S.blocks), dim3(kL1Threads), 0, stream, idx,
                       picks, S.chunk, S.shift, S.buckets, bhist);
    hipLaunchKernelGGL(bucket_colscan_kernel, dim3(grid1d(S.buckets, kWave)),
                       dim3(kColWaves * kWave), 0, stream, bhist, S.blocks, S.buckets, total);
    int nb_bits = 0;
    while ((1 << nb_bits) < S.buckets)
        ++nb_bits;
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(S.blocks), dim3(kL1Threads), 0, stream, idx,
                       picks, S.chunk, S.shift, S.buckets, nb_bits, bhist, total, bucket_base,
                       bucket_order, pairs);
    hipLaunchKernelGGL(bucket_sort_kernel, dim3(S.buckets), dim3(kL2Threads), 0, stream, pairs,
                       bucket_base, bucket_order, S.shift, slots, slot_start, order);
    return hipGetLastError();
}

// slot_scan_kernel (untouched rows, the list of long runs) then
// long_run_kernel, up to 256 workgroups walking the listed runs (at most
// picks / chunk + 1), four waves to a run.  `longs` follows the piece rows in
// the split buffer (split_rows_bytes lays it out).
template <typename DT, int MODE>
static hipError_t launch_finish(const int32_t *slot_start, int64_t slots, int64_t picks, int d_v,
                                int shift, float *split, float *dvalues, void *values, float lr,
                                hipStream_t stream)
{
    int32_t *longs = long_list(split, picks, d_v);
    hipLaunchKernelGGL((slot_scan_kernel<MODE == 0 ? 0 : 1>),
                       dim3(grid1d(slots, kFinishWaves * kWave)), dim3(kFinishWaves * kWave), 0,
                       stream, slot_start, slots, d_v, shift, dvalues, longs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    // at most picks / chunk + 1 long runs, walked by at most 256 workgroups
    const int64_t max_long = (picks >> shift) + 1;
    hipLaunchKernelGGL((long_run_kernel<DT, MODE>), dim3((unsigned)(max_long < 256 ? max_long : 256)),
                       dim3(kFinishWaves * kWave), 0, stream, slot_start, d_v, shift, split, longs,
                       dvalues, static_cast<DT *>(values), lr);
    return hipGetLastError();
}

hipError_t launch_bwd_value(int dtype, const void *values, const int32_t *idx,
                            const float *weights, const void *dy, const int32_t *slot_start,
                            const int32_t *order, float *dvalues, int accumulate, float *split,
                            float *dw, int64_t T, int H, int n, int k, int d_v, hipStream_t stream)
{
    const int64_t picks = T * H * (int64_t)k;
    const int64_t slots = (int64_t)n * n;
    const int shift = seg_shift(picks);
    hipError_t err =
        dtype == 1 ? launch_seg_dt<bf16_t, false>(values, dy, idx, weights, order, slot_start,
                                                  dvalues, split, dw, picks, H * k, d_v,
                                                  accumulate, 0.f, stream)
                   : launch_seg_dt<float, false>(values, dy, idx, weights, order, slot_start,
                                                 dvalues, split, dw, picks, H * k, d_v,
                                                 accumulate, 0.f, stream);
    if (err != hipSuccess)
        return err;
    // the storage type does not enter modes 0 and 1 (dvalues is float32)
    return accumulate ? launch_finish<float, 1>(slot_start, slots, picks, d_v, shift, split,
                                                dvalues, nullptr, 0.f, stream)
                      : launch_finish<float, 0>(slot_start, slots, picks, d_v, shift, split,
                                                dvalues, nullptr, 0.f, stream);
}

hipError_t launch_bwd_value_sgd(int dtype, void *values, const int32_t *idx, const float *weights,
                                const void *dy, const int32_t *slot_start, const int32_t *order,
                                float lr, float *split, float *dw, int64_t T, int H, int n, int k,
                                int d_v, hipStream_t stream)
{
    const int64_t picks = T * H * (int64_t)k;
    const int64_t slots = (int64_t)n * n;
    const int shift = seg_shift(picks);
    hipError_t err =
        dtype == 1 ? launch_seg_dt<bf16_t, true>(values, dy, idx, weights, order, slot_start,
                                                 nullptr, split, dw, picks, H * k, d_v, 0, lr,
                                                 stream)
                   : launch_seg_dt<float, true>(values, dy, idx, weights, order, slot_start,
                                                nullptr, split, dw, picks, H * k, d_v, 0, lr,
                                                stream);
    if (err != hipSuccess)
        return err;
    return dtype == 1 ? launch_finish<bf16_t, 2>(slot_start, slots, picks, d_v, shift, split,
                                                 nullptr, values, lr, stream)
                      : launch_finish<float, 2>(slot_start, slots, picks, d_v, shift, split,
                                                nullptr, values, lr, stream);
}

template <typename DT>
static hipError_t launch_query_t(const void *q, const void *keys, int64_t key_hstride,
                                 bool keys_shared, const int32_t *idx, const float *weights,
                                 const float *dw, float *dq, float *dkeys, int64_t T, int H, int n,
                                 int k, int d_k, void *scratch, hipStream_t stream)
{
    const BwdQueryScratch S = bwd_query_scratch(T, H, n, k, d_k);
    char *base = static_cast<char *>(scratch);
    int32_t *gl_i = reinterpret_cast<int32_t *>(base + S.off_gl_i);
    float *gl_g = reinterpret_cast<float *>(base + S.off_gl_g);
    float *partial = reinterpret_cast<float *>(base + S.off_partial);
    const int64_t rows = T * H;
    if (d_k / 2 <= 4 * kWave)
        hipLaunchKernelGGL((bwd_query_kernel<DT, 1>), dim3(grid1d(rows, kQryWaves)),
                           dim3(kQryWaves * kWave), 0, stream, static_cast<const DT *>(keys), key_hstride, idx,
                           weights, dw, dq, gl_i, gl_g, T, H, n, k, d_k);
    else
        hipLaunchKernelGGL((bwd_query_kernel<DT, 2>), dim3(grid1d(rows, kQryWaves)),
                           dim3(kQryWaves * kWave), 0, stream, static_cast<const DT *>(keys), key_hstride, idx,
                           weights, dw, dq, gl_i, gl_g, T, H, n, k, d_k);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int n_pad = (n + 15) & ~15;
    const int cols = dk_cols(n);
    // bf16 with n <= 512 and k <= 32 steps over 64 tokens (twice the products
    // per barrier; the tiles fit in 147 KB of LDS), every other case over 32
    const int tok = (sizeof(DT) == 2 && n_pad <= 512 && k <= 32) ? 64 : kDkTok;
    const size_t lds = ((size_t)DkTile<DT>::parts * n_pad + cols) * tok * sizeof(typename DkTile<DT>::elt);
    const int half = d_k / 2;
    const int ncb = (half + cols - 1) / cols;
    const dim3 grid((unsigned)S.blocks, (unsigned)(H * 2 * ncb));
    const int rt = (n_pad / 16 + kDkWaves - 1) / kDkWaves;
    auto go = [&](auto kern) -> hipError_t {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, grid, dim3(kDkWaves * kWave), lds, stream,
                           static_cast<const DT *>(q), gl_i, gl_g, partial, T, H, n, k, d_k,
                           S.tokens_per_block);
        return hipGetLastError();
    };
    // accumulators: rt row tiles x cols / 16 column tiles of 4 registers
    if constexpr (sizeof(DT) == 2)
        if (tok == 64)
            err = rt <= 1 ? go(dkeys_mfma_kernel<DT, 1, 8, 64>) : go(dkeys_mfma_kernel<DT, 2, 8, 64>);
    if (tok == kDkTok)
        err = rt <= 1 ? go(dkeys_mfma_kernel<DT, 1, 8, kDkTok>)
            : rt <= 2 ? go(dkeys_mfma_kernel<DT, 2, 8, kDkTok>)
                      : go(dkeys_mfma_kernel<DT, 4, 4, kDkTok>);
    if (err != hipSuccess)
        return err;
    const int64_t count = (int64_t)H * 2 * n * half;
    const int fold = keys_shared ? H : 1;
    const int64_t rblocks = grid1d(count / fold / 4, 256);
    hipLaunchKernelGGL(dkeys_reduce_kernel, dim3((unsigned)(rblocks < 8192 ? rblocks : 8192)),
                       dim3(256), 0, stream, partial, S.blocks, count, fold, dkeys);
    return hipGetLastError();
}

hipError_t launch_bwd_query(int dtype, const void *q, const void *keys, int64_t key_hstride,
                            bool keys_shared, const int32_t *idx, const float *weights,
                            const float *dw, float *dq, float *dkeys, int64_t T, int H, int n,
                            int k, int d_k, void *scratch, hipStream_t stream)
{
    if (dtype == 1)
        return launch_query_t<bf16_t>(q, keys, key_hstride, keys_shared, idx, weights, dw, dq,
                                      dkeys, T, H, n, k, d_k, scratch, stream);
    return launch_query_t<float>(q, keys, key_hstride, keys_shared, idx, weights, dw, dq, dkeys,
                                 T, H, n, k, d_k, scratch, stream);
}

// ---------------------------------------------------------------------------
__global__ void zero_f32_kernel(float *__restrict__ p, int64_t count)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        p[i] = 0.f;
}

hipError_t launch_zero_f32(float *p, int64_t count, hipStream_t stream)
{
    if (count <= 0)
        return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid), dim3(256), 0, stream, p, count);
    return hipGetLastError();
}

}  // namespace pkm

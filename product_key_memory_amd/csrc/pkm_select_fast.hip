// pkm_select_fast.hip -- forward selection for bf16 storage, query halves of
// 256, 256 < n <= 1024, k <= 32, as two kernels (gptget.net summary of "Large
// Memory Layers with Product Keys", "Methodology": split q into q1, q2, search
// each against its own sub-key set, combine the best sub-keys; companion page
// "Why top-k of each half is enough").
//
// 1. fwd_topk_half_kernel: one wave per (16 tokens, head, half).  The
//    codebook is scored in blocks of 512 sub-keys (one block for n <= 512,
//    two for n <= 1024).  The wave computes its tokens' scores of a block
//    straight into registers with v_mfma_f32_16x16x32_bf16 (sub-keys as M,
//    tokens as N): lane l holds, for token l % 16, the scores of sub-keys
//    16 j + 4 (l / 16) + i of the block (tile j < 32, i < 4).  All selection
//    work then runs on the 4 lanes that share a token, so every instruction
//    serves the wave's 16 tokens at once:
//      - tau = k-th largest of the token's 64 group maxima (groups of 8
//        scores), by a bitonic sort inside the 4-lane group: the k groups
//        above it each hold a score >= tau, so at least k scores survive;
//      - survivors (score >= tau) are compacted into LDS and sorted as 64-bit
//        keys (score, then lower index first) inside the 4-lane group; when a
//        token has more than 64 survivors (heavy ties) its exact k-th largest
//        key is found by bisection on the score bits, then on the index among
//        exact ties, and exactly k survive;
//      - a second block's survivors must also reach the first block's k-th
//        key; its sorted list and the first block's (kept in LDS) are merged
//        (the top k of two sorted lists A, B are the larger of A[e] and
//        B[k - 1 - e], a bitonic sequence, which a bitonic merge orders);
//      - the top k (score, sub-key) of the half go to the workspace.
// 2. fwd_merge_kernel: one wave per 16 (token, head) rows, 4 lanes per row.
//    A pair of ranks (a, b) can only make the final top-k if
//    (a + 1)(b + 1) <= k: every pair (a', b') <= (a, b) componentwise scores at
//    least as high and, on a tie, has the lower slot f = i n + j.  The
//    sum_a floor(k / a) candidates (119 for k = 32) are sorted inside the
//    4-lane group by (score desc, slot asc), the first k kept, and a softmax
//    over them gives the weights.
// Splitting the two phases keeps each kernel's registers low enough for two
// or more waves per SIMD, which hides the latency a single wave exposes.
#include <type_traits>

#include "pkm_device.hpp"
#include "pkm_kernels.hpp"

namespace pkm {

constexpr int kFastWaves = 4;
constexpr int kFastTok = 16;                         // tokens per wave
constexpr int kFastTokWG = kFastWaves * kFastTok;    // tokens per workgroup
constexpr int kFastTiles = 32;                       // 16-sub-key tiles per block
constexpr int kFastBlock = 16 * kFastTiles;          // 512 sub-keys per block
constexpr int kFastKSteps = 8;                       // 32-wide K steps: half = 256
constexpr int kFastSurv = 64;                        // survivors per token at most
constexpr int kSurvStride = kFastSurv + 4;           // + one spare slot per lane group
constexpr int kMergeWaves = 4;
constexpr int kMergeRows = 16;                       // (token, head) rows per wave
constexpr int kMaxPairs = 128;                       // merge_candidates(32) = 119
// LDS row pitch of the merge, in 8-byte entries: a row's two lists (2 k <= 64)
// or its survivors (<= 64), plus one: an odd pitch puts the 16 rows a read
// instruction touches (same entry, rows tok = 0..15) in distinct banks
constexpr int kMergePitch = 2 * 32 + 1;

// Scores of the wave's 16 tokens against the sub-keys 0..n_loc-1 of one block
// (kb = its first row), as order-preserving integers: so[j][i] = ord(score of
// sub-key 16 j + 4 g + i) for token `tok` (rows past n_loc score 0; the caller
// masks them).  The workgroup's 4 waves (64 tokens)
// share the codebook through LDS: per step p it holds rows 32 p .. 32 p + 31
// (16 KB, double-buffered), each thread loading 4 of its 16-byte chunks, so
// the L2 serves each codebook once per 64 tokens instead of once per 16.
// Chunk c of local row r sits at position c ^ (r % 16) of the row: the 16
// rows an MFMA operand read touches (same chunk, rows r16 = 0..15) then fall
// in distinct banks.  Within a step the two tiles' accumulation chains
// alternate, so consecutive MFMAs do not wait on each other.
__device__ __forceinline__ void fast_scores(uint32_t (&so)[kFastTiles][4], const uint16_t *kb,
                                            const uint4 (&qf)[kFastKSteps], int n_loc, int r16,
                                            int g, uint4 *kbuf, int tid)
{
    constexpr int half = kFastKSteps * 32;
    constexpr int chunks = half * 2 / 16;            // 32 chunks of 16 bytes per row
    constexpr int step_units = 32 * chunks;          // 1024 chunks per 32-row step
    constexpr int per_thread = step_units / (kFastWaves * kWave);
    constexpr int steps = kFastTiles / 2;
    // rows past n_loc read as zeros
    const __amdgpu_buffer_rsrc_t rsrc = buffer_over(kb, n_loc * half * 2);
    uint4 pre[per_thread];
    auto gload = [&](int p) {
#pragma unroll
        for (int m = 0; m < per_thread; ++m) {
            const int u = tid + m * kFastWaves * kWave;
            const int rl = u / chunks, c = (u % chunks) ^ (rl & 15);
            pre[m] = buffer_load16(rsrc, ((32 * p + rl) * chunks + c) * 16, 0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int m = 0; m < per_thread; ++m)
            kbuf[buf * step_units + tid + m * kFastWaves * kWave] = pre[m];
    };
    gload(0);
    lstore(0);
    gload(1);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < steps; ++p) {
        const uint4 *cur = kbuf + (p & 1) * step_units;
        floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < kFastKSteps; ++kk) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const int rl = 16 * w + r16;
                const uint4 a = cur[rl * chunks + ((4 * kk + g) ^ r16)];
                acc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[kk]), acc[w],
                    0, 0, 0);
            }
        }
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[2 * p + w][i] = ord_f32(acc[w][i]);
        // step p + 1 goes to the other buffer (its readers finished at the
        // last barrier); step p + 2 is fetched while step p + 1 is worked on
        if (p + 1 < steps)
            lstore((p + 1) & 1);
        if (p + 2 < steps)
            gload(p + 2);
        __syncthreads();
    }
}

// lists[((t H + h) 2 + s) k + e] = (ord score, sub-key) of the e-th best
// sub-key of half s, e < k.  BLOCKS = number of 512-sub-key blocks (1: n <= 512,
// 2: n <= 1024), a template argument so that each case gets its own register
// allocation.
template <int BLOCKS>
// Three waves per SIMD: the register budget (168) makes the compiler spill a
// few dozen registers to scratch, which costs less than the latency a third
// wave hides (measured: 0.186 -> 0.177 ms for the selection at n = 512, and
// 0.61 -> 0.58 ms at n = 1024).
__global__ __launch_bounds__(kFastWaves *kWave) __attribute__((amdgpu_waves_per_eu(3, 3))) void fwd_topk_half_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ keys, int64_t T, int H, int n,
    int k, uint2 *__restrict__ lists)
{
    // the codebook steps during the scoring, the survivors afterwards
    constexpr int kSurvUnits = 2 * kFastWaves * kFastTok * kSurvStride * 4 / 16;
    __shared__ uint4 lds[kSurvUnits > 2 * 32 * 32 ? kSurvUnits : 2 * 32 * 32];
    // the first block's top k per token while the second block is scored
    // (row stride 33 keys: the 16 tokens' rows start in distinct banks)
    __shared__ uint64_t s_prev[kFastWaves][kFastTok][33];
    uint32_t(*surv_s_all)[kFastTok * kSurvStride] =
        reinterpret_cast<uint32_t(*)[kFastTok * kSurvStride]>(lds);
    uint32_t(*surv_i_all)[kFastTok * kSurvStride] = surv_s_all + kFastWaves;

    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tok = lane & 15, g_lane = lane >> 4;
    constexpr int half = kFastKSteps * 32;
    constexpr int d_k = 2 * half;
    const int h = blockIdx.y, s = blockIdx.z;
    const int64_t t = (int64_t)blockIdx.x * kFastTokWG + wave * kFastTok + tok;
    const bool live = t < T;
    uint32_t *surv_s = surv_s_all[wave] + tok * kSurvStride;
    uint32_t *surv_i = surv_i_all[wave] + tok * kSurvStride;
    uint64_t *prev = s_prev[wave][tok];

    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(q) +
                           ((live ? t : 0) * H + h) * (int64_t)d_k + (int64_t)s * half;
    const int tid0 = threadIdx.x;
    const uint16_t *kb = reinterpret_cast<const uint16_t *>(keys) + ((int64_t)h * 2 + s) * (int64_t)n * half;

    // one block of sub-keys; straight-line code for each block (a loop over
    // the blocks kept values alive across its back edge and cost a wave per
    // SIMD)
    auto block = [&](auto first_c, auto last_c) {
        constexpr bool kFirst = decltype(first_c)::value, kLast = decltype(last_c)::value;
        // opaque copies of the lane group and the thread id, so values derived
        // from them (the 128 sub-key indices, the LDS and codebook offsets) are
        // formed where used instead of being held in registers, also from one
        // block to the next
        int g = g_lane, tid = tid0;
        asm volatile("" : "+v"(g), "+v"(tid));
        const int base = kFirst ? 0 : kFastBlock;
        const int n_loc = n - base < kFastBlock ? n - base : kFastBlock;
        // B fragments: token `tok`, K slice 32 kk + 8 g .. + 7 (loaded per
        // block, so they are not held through the selection)
        uint4 qf[kFastKSteps];
#pragma unroll
        for (int kk = 0; kk < kFastKSteps; ++kk)
            qf[kk] = *reinterpret_cast<const uint4 *>(qrow + 32 * kk + 8 * g);
        uint32_t so[kFastTiles][4];
        fast_scores(so, kb + (int64_t)base * half, qf, n_loc, tok, g, lds, tid);
        if (n_loc < kFastBlock) {
            // sub-key 16 j + 4 g + i of the block exists iff 16 j + i < lim
            const int lim = n_loc - 4 * g;
            const uint32_t neg = ord_f32(-INFINITY);
#pragma unroll
            for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[j][i] = 16 * j + i < lim ? so[j][i] : neg;
        }

        // tau: k-th largest of the token's 64 group maxima (groups of 8 scores)
        uint32_t gm[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            uint32_t x = so[2 * m][0];
#pragma unroll
            for (int i = 1; i < 4; ++i)
                x = max(x, so[2 * m][i]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x = max(x, so[2 * m + 1][i]);
            gm[m] = x;
        }
        group4_sort_desc<16>(gm);
        uint32_t tau_src = gm[0];
#pragma unroll
        for (int r = 1; r < 16; ++r)
            if (r == ((k - 1) & 15))
                tau_src = gm[r];
        uint32_t tau = (uint32_t)__shfl((int)tau_src, tok + 16 * ((k - 1) >> 4));
        // A single block has n > 256 valid sub-keys, >= 33 groups of real
        // scores, so tau is a real score and the sub-keys past n never
        // survive.  A second block may hold fewer than k sub-keys: there the
        // first block's k-th key (a real score) raises the bar, and keys
        // below it cannot reach the top k anyway.
        if constexpr (!kFirst)
            tau = max(tau, (uint32_t)(prev[k - 1] >> 32));

        // survivors: ord >= tau
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cnt += so[j][i] >= tau ? 1 : 0;
        int total = group4_sum(cnt);
        bool fits = total <= kFastSurv;

        // heavy ties: the exact k-th largest key of the block instead of tau,
        // by bisection on the score bits and then on the index among exactly
        // tied scores (more than 64 survivors are real scores, so is the
        // k-th largest)
        uint32_t kth = tau, tie_idx = 0xFFFFFFFFu;
        if (__ballot(!fits && live) != 0) {
            uint32_t K = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = K | (1u << bit);
                int c = 0;
#pragma unroll
                for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        c += so[j][i] >= cand ? 1 : 0;
                if (group4_sum(c) >= k)
                    K = cand;
            }
            int above = 0;
#pragma unroll
            for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    above += so[j][i] > K ? 1 : 0;
            const int need = k - group4_sum(above);     // tied picks to take, lowest index first
            uint32_t I = 0;                              // largest bound with < need tied indices below it
            for (int bit = 9; bit >= 0; --bit) {
                const uint32_t cand = I | (1u << bit);
                // sub-key 16 j + 4 g + i < cand  <=>  16 j + i < cand - 4 g
                const int lim_c = (int)cand - 4 * g;
                int c = 0;
#pragma unroll
                for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        c += (so[j][i] == K && 16 * j + i < lim_c) ? 1 : 0;
                if (group4_sum(c) < need)
                    I = cand;
            }
            if (!fits) {
                kth = K;
                tie_idx = I;             // exactly k keys of the block are >= (K, I)
                total = k;
                fits = true;
            }
        }

        // compact the survivors per token as two 32-bit arrays (scores, and
        // the part 16 j + i of the sub-key known at compile time: 64-bit keys
        // built here would pin register pairs for all 128 candidates), then
        // sort them as keys in the 4-lane group.  The reader adds 4 x (the
        // writing lane group), which it knows from the survivor's position,
        // and the block's first sub-key.
        const bool exact = tie_idx != 0xFFFFFFFFu;
        const int lim_t = exact ? (int)tie_idx - 4 * g : 0;   // 16 j + i <= lim_t among ties
        int mine = cnt;
        if (exact) {
            // recount this lane's share under the exact bound
            int c = 0;
#pragma unroll
            for (int j = 0; j < kFastTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t o = so[j][i];
                    c += (o > kth || (o == kth && 16 * j + i <= lim_t)) ? 1 : 0;
                }
            mine = c;
        }
        // Lane group g writes its survivors from position g + (the counts of
        // the groups before it): every candidate is stored at the next free
        // position, which only a kept one claims, so the writes need no
        // branches; the last unclaimed store lands in the spare slot that
        // ends the group's range.
        const int c0 = __shfl(mine, tok), c1 = __shfl(mine, tok + 16), c2 = __shfl(mine, tok + 32);
        int off = g + (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
#pragma unroll
        for (int j = 0; j < kFastTiles; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t o = so[j][i];
                const bool keep = exact ? (o > kth || (o == kth && 16 * j + i <= lim_t)) : o >= kth;
                surv_s[off] = o;
                surv_i[off] = (uint32_t)(16 * j + i);
                off += keep ? 1 : 0;
            }
            __builtin_amdgcn_sched_barrier(0);     // one tile's keys at a time
        }
        wave_lds_sync();
        const int b1 = c0, b2 = c0 + c1, b3 = c0 + c1 + c2;
        uint64_t v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // survivor e was written by lane group src_g, at position e + src_g
            const int e = 16 * g + r;
            const int src_g = (e >= b1 ? 1 : 0) + (e >= b2 ? 1 : 0) + (e >= b3 ? 1 : 0);
            v[r] = e < total ? ((uint64_t)surv_s[e + src_g] << 32) |
                                   (uint64_t)~(surv_i[e + src_g] + 4u * (uint32_t)src_g + (uint32_t)base)
                             : 0ull;
        }
        group4_sort_desc<16>(v);
        // lane group g holds ranks 16 g .. 16 g + 15 of the block
        if constexpr (!kFirst) {
            // top k of the two sorted lists A (first block) and B (this one):
            // C[e] = max(A[e], B[31 - e]) for e < 32 (both padded with zero
            // keys past their ends), then a bitonic merge.  Lane groups 0 and
            // 1 hold C; B[31 - e] is register 15 - r of the other group.
            const int ga = g & 1;
            uint64_t c[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = 16 * ga + r;
                const uint64_t a = e < k ? prev[e] : 0ull;
                const uint64_t b = shfl_xor_u64(v[15 - r], 16);
                c[r] = a > b ? a : b;
            }
            // stride 16: across the two lane groups, group 0 keeps the larger
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint64_t o = shfl_xor_u64(c[r], 16);
                c[r] = ((c[r] > o) == (ga == 0)) ? c[r] : o;
            }
#pragma unroll
            for (int stride = 8; stride > 0; stride >>= 1)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((r & stride) == 0) {
                        const uint64_t x = c[r], y = c[r | stride];
                        c[r] = x > y ? x : y;
                        c[r | stride] = x > y ? y : x;
                    }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                v[r] = c[r];
        } else if constexpr (!kLast) {
            if (g < 2) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (16 * g + r < k)
                        prev[16 * g + r] = v[r];
            }
            wave_lds_sync();
            // the next block's codebook steps overwrite every wave's survivors
            __syncthreads();
            return;
        }

        // last block: lane groups 0 and 1 hold ranks 0 .. 31
        if (live && g < 2) {
            uint2 *out = lists + ((t * H + h) * 2 + s) * (int64_t)k;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = 16 * g + r;
                if (e < k)
                    out[e] = make_uint2((uint32_t)(v[r] >> 32), ~(uint32_t)v[r]);
            }
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    if constexpr (BLOCKS == 1) {
        block(yes{}, yes{});
    } else {
        block(yes{}, no{});
        block(no{}, yes{});
    }
}

// The combine and the softmax per (token, head) row from the two lists.
// First a lower bound on the k-th best combined score prunes the candidates:
// the set S = {(a, b) : (a + 1)(b + 1) <= m}, m the least value with |S| >= k,
// holds at least k candidates, so the k-th best score is at least the least
// score in S -- the least of its corner scores s(a, m / (a + 1) - 1), as the
// lists are sorted and rounding is monotone.  When no row of the wave keeps
// more than kMergeSurv candidates, the survivors are compacted into LDS and
// sorted 64 per row; otherwise every candidate is sorted, 128 per row.
constexpr int kMaxCorners = 16;
constexpr int kMergeSurv = 60;      // + a spare slot per lane group: < 64 per row

__device__ __forceinline__ float merge_score(uint2 l, uint2 r)
{
    return unord_f32(l.x) + unord_f32(r.x);
}

__global__ __launch_bounds__(kMergeWaves *kWave) void fwd_merge_kernel(
    const uint2 *__restrict__ lists, int64_t rows, int n, int k, int n_pairs, int m,
    int32_t *__restrict__ idx, float *__restrict__ weights, float *__restrict__ scores)
{
    __shared__ uint2 s_list[kMergeWaves][kMergeRows * kMergePitch];
    __shared__ uint16_t s_pairs[kMaxPairs];
    __shared__ uint16_t s_corner[kMaxCorners];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tok = lane & 15, g = lane >> 4;
    if (wave == 0) {
        const int cnt = lane < k ? k / (lane + 1) : 0;
        int total;
        const int start = wave_exclusive_scan(cnt, &total);
        for (int b = 0; b < cnt; ++b)
            s_pairs[start + b] = (uint16_t)(lane | (b << 8));
        if (lane < m)
            s_corner[lane] = (uint16_t)(lane | ((m / (lane + 1) - 1) << 8));
    }
    // the wave's rows are contiguous in the lists: stage them in LDS (row
    // pitch kMergePitch entries), all 16-byte loads in flight before the
    // first store
    const int64_t row0 = ((int64_t)blockIdx.x * kMergeWaves + wave) * kMergeRows;
    const int64_t nrows = rows - row0 < kMergeRows ? rows - row0 : kMergeRows;
    uint2 *sl = s_list[wave];
    if (nrows > 0) {
        constexpr int kPerLane = kMergeRows * 2 * 32 / 2 / kWave;     // uint4 per lane
        const int units = (int)nrows * k;                               // 2 entries each
        const uint4 *src = reinterpret_cast<const uint4 *>(lists + row0 * 2 * k);
        uint4 buf[kPerLane];
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            const int e = lane + u * kWave;
            buf[u] = e < units ? src[e] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kPerLane; ++u) {
            const int e = lane + u * kWave;
            if (e < units) {
                // entries 2 e, 2 e + 1 lie in one row (a row has 2 k entries)
                uint2 *d = sl + (e / k) * kMergePitch + 2 * (e % k);
                d[0] = make_uint2(buf[u].x, buf[u].y);
                d[1] = make_uint2(buf[u].z, buf[u].w);
            }
        }
    }
    __syncthreads();
    if (nrows <= 0)
        return;
    const bool live = tok < nrows;
    const uint2 *l = sl + tok * kMergePitch;
    const uint2 *r = l + k;

    // the bound: least corner score of the row (lane group g takes corners
    // g, g + 4, ...), as an order-preserving key
    float tau = INFINITY;
#pragma unroll
    for (int c0 = 0; c0 < kMaxCorners; c0 += 4) {
        const int c = c0 + g;
        if (c < m) {
            const int a = s_corner[c] & 0xFF, b = s_corner[c] >> 8;
            tau = fminf(tau, merge_score(l[a], r[b]));
        }
    }
    tau = fminf(tau, __shfl_xor(tau, 16));
    tau = fminf(tau, __shfl_xor(tau, 32));
    uint32_t otau = ord_f32(tau);

    uint64_t v[32];
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const int pc = 32 * g + c;
        if (live && pc < n_pairs) {
            const int a = s_pairs[pc] & 0xFF, b = s_pairs[pc] >> 8;
            const uint2 la = l[a], rb = r[b];
            v[c] = make_key(merge_score(la, rb), la.y * (uint32_t)n + rb.y);
        } else {
            v[c] = 0ull;
        }
        cnt += (uint32_t)(v[c] >> 32) >= otau ? 1 : 0;
    }
    if (!live)
        cnt = 0;        // rows past the end keep nothing
    int total = group4_sum(cnt);
    auto count_ge = [&](uint32_t o) {
        int c = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            c += (uint32_t)(v[e] >> 32) >= o ? 1 : 0;
        return c;
    };
    // Raise the bound while more than kMergeSurv survive: bisection on the
    // score between the bound (>= k survive) and the best pair (0, 0).
    {
        float lo = tau, hi = merge_score(l[0], r[0]);
        for (int it = 0; it < 8; ++it) {
            const bool more = live && total > kMergeSurv;
            if (__ballot(more) == 0)
                break;
            const float mid = lo + 0.5f * (hi - lo);
            const uint32_t om = ord_f32(mid);
            const int c_mid = count_ge(om);
            const int t_mid = group4_sum(c_mid);
            if (more && t_mid >= k) {
                lo = mid;
                otau = om;
                cnt = c_mid;
                total = t_mid;
            } else if (more) {
                hi = mid;
            }
        }
    }
    // Rows still above (heavy ties): the exact k-th largest key by bisection
    // on the 64-bit keys, which are distinct (the slot is part of the key);
    // exactly k keys are >= it.
    uint64_t kth = live ? (uint64_t)otau << 32 : ~0ull;
    if (__ballot(live && total > kMergeSurv) != 0) {
        const bool more = live && total > kMergeSurv;
        uint64_t K = 0;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t cand = K | (1ull << bit);
            int c = 0;
#pragma unroll
            for (int e = 0; e < 32; ++e)
                c += v[e] >= cand ? 1 : 0;
            if (group4_sum(c) >= k)
                K = cand;
        }
        if (more) {
            kth = K;
            int c = 0;
#pragma unroll
            for (int e = 0; e < 32; ++e)
                c += v[e] >= K ? 1 : 0;
            cnt = c;
            total = k;
        }
    }

    // The survivors (key >= kth) go to this wave's list area, free once every
    // lane has its candidates: 64 slots per row.  Lane group g writes from
    // position g + (the counts of the groups before it), every candidate at
    // the next free slot, which only a kept one claims.
    wave_lds_sync();
    uint64_t *surv = reinterpret_cast<uint64_t *>(sl) + tok * kMergePitch;
    const int c0 = __shfl(cnt, tok), c1 = __shfl(cnt, tok + 16), c2 = __shfl(cnt, tok + 32);
    int off = g + (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        surv[off] = v[c];
        off += live && v[c] >= kth ? 1 : 0;
    }
    wave_lds_sync();
    const int b1 = c0, b2 = c0 + c1, b3 = c0 + c1 + c2;
    uint64_t w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int e = 16 * g + q;
        const int src_g = (e >= b1 ? 1 : 0) + (e >= b2 ? 1 : 0) + (e >= b3 ? 1 : 0);
        w[q] = live && e < total ? surv[e + src_g] : 0ull;
    }
    group4_sort_desc<16>(w);

    // ranks 16 g + q sit in lane groups 0 and 1; the softmax sums both
    const int64_t out = (row0 + tok) * (int64_t)k;
    const float top = __shfl(key_score(w[0]), tok);
    float ex[16], z = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        ex[q] = 16 * g + q < k ? expf(key_score(w[q]) - top) : 0.f;
        z += ex[q];
    }
    z += __shfl_xor(z, 16);
    if (live && g < 2) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int e = 16 * g + q;
            if (e < k) {
                idx[out + e] = (int32_t)key_index(w[q]);
                weights[out + e] = ex[q] / z;
                if (scores)
                    scores[out + e] = key_score(w[q]);
            }
        }
    }
}

// The least m with |{(a, b) : (a + 1)(b + 1) <= m}| = sum_a floor(m / a) >= k.
static int merge_bound_size(int k)
{
    for (int m = 1;; ++m)
        if (merge_candidates(m) >= k)
            return m;
}

hipError_t launch_select_fast(const void *q, const void *keys, int64_t T, int H, int n, int k,
                              int d_k, int32_t *idx, float *weights, float *scores,
                              void *workspace, hipStream_t stream)
{
    (void)d_k;      // 512 on this path
    uint2 *lists = static_cast<uint2 *>(workspace);
    const dim3 grid((unsigned)((T + kFastTokWG - 1) / kFastTokWG), (unsigned)H, 2);
    if (n <= kFastBlock)
        hipLaunchKernelGGL(fwd_topk_half_kernel<1>, grid, dim3(kFastWaves * kWave), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(keys), T, H,
                           n, k, lists);
    else
        hipLaunchKernelGGL(fwd_topk_half_kernel<2>, grid, dim3(kFastWaves * kWave), 0, stream,
                           static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(keys), T, H,
                           n, k, lists);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t rows = T * H;
    const int64_t per_block = (int64_t)kMergeWaves * kMergeRows;
    hipLaunchKernelGGL(fwd_merge_kernel, dim3((unsigned)((rows + per_block - 1) / per_block)),
                       dim3(kMergeWaves * kWave), 0, stream, lists, rows, n, k,
                       merge_candidates(k), merge_bound_size(k), idx, weights, scores);
    return hipGetLastError();
}

}  // namespace pkm

// pkm_select_fast.hip -- forward selection for query halves of 256, k <= 32,
// 128 <= n <= 1024 for bf16 storage and 128 <= n <= 256 for float32, as two
// kernels (gptget.net summary of "Large
// Memory Layers with Product Keys", "Methodology": split q into q1, q2, search
// each against its own sub-key set, combine the best sub-keys; companion page
// "Why top-k of each half is enough").
//
// 1. fwd_topk_half_kernel: one wave per (16 tokens, head, half).  The
//    codebook is scored in one or two blocks of 128, 256 or 512 sub-keys
//    (the launcher picks the shape so that the first block is more than 3/4
//    full).  The wave computes its tokens' scores of a block straight into
//    registers with v_mfma_f32_16x16x32_bf16 (sub-keys as M, tokens as N):
//    lane l holds, for token l % 16, the scores of sub-keys
//    16 j + 4 (l / 16) + i of the block (tile j, i < 4).  All selection work
//    then runs on the 4 lanes that share a token, so every instruction serves
//    the wave's 16 tokens at once:
//      - tau = k-th largest of the token's 64 group maxima (groups of
//        TILES / 4 scores), by a bitonic network inside the 4-lane group:
//        the k groups above it each hold a score >= tau, so at least k
//        scores survive;
//      - survivors (score >= tau) are compacted into LDS and sorted as 64-bit
//        keys (score, then lower index first) inside the 4-lane group -- keys
//        whose bit patterns are normal float64 numbers of the same order, so
//        each exchange is one float64 max and one min; when a
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
constexpr int kFastTiles = 32;                       // 16-sub-key tiles per block (at most)
constexpr int kFastBlock = 16 * kFastTiles;          // 512 sub-keys per block (at most)
constexpr int kFastKSteps = 8;                       // 32-wide K steps: half = 256
constexpr int kFastSurv = 64;                        // survivors per token at most
constexpr int kSurvStride = kFastSurv + 4;           // row pitch of a token's survivors (words)
constexpr int kSubBits = 10;                         // sub-key index < n <= 1024
constexpr int kSlotBits = 20;                        // slot i n + j < n^2 <= 2^20
constexpr int kMergeWaves = 4;
constexpr int kMergeRows = 16;                       // (token, head) rows per wave
constexpr int kMaxPairs = 128;                       // merge_candidates(32) = 119
// LDS row pitch of the merge, in 8-byte entries: a row's two lists (2 k <= 64)
// or its survivors (<= 64), plus one: an odd pitch puts the 16 rows a read
// instruction touches (same entry, rows tok = 0..15) in distinct banks
constexpr int kMergePitch = 2 * 32 + 1;

// One 32-row step of the scoring: this wave's share of the next step's rows
// goes from the codebook straight into `fill` (buffer loads into LDS) while
// the MFMAs read the current step from `cur`.  The two are restrict
// pointers, so the compiler does not wait on the copy before the reads; each
// A fragment is read one MFMA pair ahead of its use.  Chunk c of local row r
// sits at position c ^ (r % 16) of the row: the 16 rows an MFMA operand read
// touches (same chunk, rows r16 = 0..15) then fall in distinct banks; thread
// u of the workgroup fills position u + 256 m (1 KB per wave and m, the
// layout a wave's LDS load writes).  The two tiles' accumulation chains
// alternate, so consecutive MFMAs do not wait on each other.
__device__ __forceinline__ void fast_step(uint4 *__restrict__ fill, const uint4 *__restrict__ cur,
                                          __amdgpu_buffer_rsrc_t rsrc, int p_next, int tid,
                                          const uint4 (&qf)[kFastKSteps], int r16, int g,
                                          floatx4 (&acc)[2])
{
    constexpr int chunks = kFastKSteps * 32 * 2 / 16;       // 32 chunks of 16 bytes per row
    constexpr int per_thread = 32 * chunks / (kFastWaves * kWave);
    if (fill) {
        const int wave = tid / kWave;
#pragma unroll
        for (int m = 0; m < per_thread; ++m) {
            const int u = tid + m * kFastWaves * kWave;
            const int rl = u / chunks, c = (u % chunks) ^ (rl & 15);
            buffer_load_lds16(rsrc, fill + m * kFastWaves * kWave + wave * kWave,
                              ((32 * p_next + rl) * chunks + c) * 16);
        }
    }
    uint4 a[2], b[2];
#pragma unroll
    for (int w = 0; w < 2; ++w)
        a[w] = cur[(16 * w + r16) * chunks + (g ^ r16)];
#pragma unroll
    for (int kk = 0; kk < kFastKSteps; ++kk) {
        if (kk + 1 < kFastKSteps) {
#pragma unroll
            for (int w = 0; w < 2; ++w)
                b[w] = cur[(16 * w + r16) * chunks + ((4 * (kk + 1) + g) ^ r16)];
        }
#pragma unroll
        for (int w = 0; w < 2; ++w)
            acc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[w]), __builtin_bit_cast(bf16x8, qf[kk]), acc[w], 0, 0, 0);
#pragma unroll
        for (int w = 0; w < 2; ++w)
            a[w] = b[w];
    }
}

// Scores of the wave's 16 tokens against the sub-keys 0..n_loc-1 of one block
// (kb = its first row), as float32 bit patterns: so[j][i] = the score of
// sub-key 16 j + 4 g + i for token `tok` (rows past n_loc read as zeros or
// stale data; the caller masks them).  The workgroup's 4 waves (64 tokens)
// share the codebook through LDS: per step p it holds rows 32 p .. 32 p + 31
// (16 KB, double-buffered), so the L2 serves each codebook once per 64
// tokens instead of once per 16.  A step's rows are complete once this
// wave's own copies have retired and every wave has passed the barrier that
// follows, which also frees the other buffer for the next step's copy.
template <int TILES>
__device__ __forceinline__ void fast_scores(uint32_t (&so)[TILES][4], const uint16_t *kb,
                                            const uint4 (&qf)[kFastKSteps], int n_loc, int r16,
                                            int g, uint4 *kbuf, int tid)
{
    constexpr int half = kFastKSteps * 32;
    constexpr int chunks = half * 2 / 16;
    constexpr int step_units = 32 * chunks;          // 1024 chunks per 32-row step
    constexpr int steps = TILES / 2;
    const __amdgpu_buffer_rsrc_t rsrc = buffer_over(kb, n_loc * half * 2);
    {
        const int wave = tid / kWave;
#pragma unroll
        for (int m = 0; m < step_units / (kFastWaves * kWave); ++m) {
            const int u = tid + m * kFastWaves * kWave;
            const int rl = u / chunks, c = (u % chunks) ^ (rl & 15);
            buffer_load_lds16(rsrc, kbuf + m * kFastWaves * kWave + wave * kWave,
                              (rl * chunks + c) * 16);
        }
    }
#pragma unroll
    for (int p = 0; p < steps; ++p) {
        wait_vmcnt<0>();
        __syncthreads();
        floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        fast_step(p + 1 < steps ? kbuf + ((p + 1) & 1) * step_units : nullptr,
                  kbuf + (p & 1) * step_units, rsrc, p + 1, tid, qf, r16, g, acc);
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[2 * p + w][i] = __float_as_uint(acc[w][i]);
    }
    // every wave is done with the last step's buffer before LDS is reused
    __syncthreads();
}

// float32 storage: a codebook row is 256 floats (1 KB, 64 chunks of 16
// bytes) and a step one tile of 16 rows (16 KB, double-buffered like the
// bf16 steps, chunk c of row r at position c ^ (r % 16)).  The operands widen
// exactly to float64 and v_mfma_f64_16x16x4_f64 accumulates in float64, so
// each score is the exact dot product rounded once to float32.  A lane's K
// slice of an MFMA is the same for A and B (element e of its float4 of K step
// ks), so the 64 MFMAs of a tile sum every product once.  The f64 MFMA leaves
// row 4 i + l / 16 of the tile in register i of lane l (the bf16 one: row
// 4 (l / 16) + i); A row m is therefore read from local row 4 (m % 4) + m / 4,
// which puts sub-key 4 g + i of the tile in register i of lane group g, the
// layout the selection reads.
constexpr int kF32Chunks = 64;                       // chunks of a 256-float row
constexpr int kF32KSteps = 16;                       // float4 K steps: half = 256
__device__ __forceinline__ void fast_step_f32(uint4 *__restrict__ fill, const uint4 *__restrict__ cur,
                                              __amdgpu_buffer_rsrc_t rsrc, int p_next, int tid,
                                              const float4 (&qf)[kF32KSteps], int r16, int g,
                                              doublex4 &acc)
{
    constexpr int per_thread = 16 * kF32Chunks / (kFastWaves * kWave);
    if (fill) {
        const int wave = tid / kWave;
#pragma unroll
        for (int m = 0; m < per_thread; ++m) {
            const int u = tid + m * kFastWaves * kWave;
            const int rl = u / kF32Chunks, c = (u % kF32Chunks) ^ (rl & 15);
            buffer_load_lds16(rsrc, fill + m * kFastWaves * kWave + wave * kWave,
                              ((16 * p_next + rl) * kF32Chunks + c) * 16);
        }
    }
    const int rr = (r16 & 3) << 2 | r16 >> 2;      // a permutation of 0..15
    float4 a = __builtin_bit_cast(float4, cur[rr * kF32Chunks + (g ^ rr)]), b;
#pragma unroll
    for (int ks = 0; ks < kF32KSteps; ++ks) {
        if (ks + 1 < kF32KSteps)
            b = __builtin_bit_cast(float4, cur[rr * kF32Chunks + ((4 * (ks + 1) + g) ^ rr)]);
        // an opaque copy of the query fragment: its widening to float64 stays
        // here (hoisted out of the step loop, all 64 would need 128 registers)
        float4 qv = qf[ks];
        asm volatile("" : "+v"(qv.x), "+v"(qv.y), "+v"(qv.z), "+v"(qv.w));
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.x, (double)qv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.y, (double)qv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.z, (double)qv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.w, (double)qv.w, acc, 0, 0, 0);
        a = b;
    }
}

template <int TILES>
__device__ __forceinline__ void fast_scores_f32(uint32_t (&so)[TILES][4], const float *kb,
                                                const float *qrow, int n_loc, int r16, int g,
                                                uint4 *kbuf, int tid)
{
    constexpr int half = 16 * kF32KSteps;            // 256 floats per row
    constexpr int step_units = 16 * kF32Chunks;      // 1024 chunks per 16-row step
    const __amdgpu_buffer_rsrc_t rsrc = buffer_over(kb, n_loc * half * 4);
    // B fragments: token `tok` (= r16), floats 16 ks + 4 g .. + 3
    float4 qf[kF32KSteps];
#pragma unroll
    for (int ks = 0; ks < kF32KSteps; ++ks)
        qf[ks] = *reinterpret_cast<const float4 *>(qrow + 16 * ks + 4 * g);
    {
        const int wave = tid / kWave;
#pragma unroll
        for (int m = 0; m < step_units / (kFastWaves * kWave); ++m) {
            const int u = tid + m * kFastWaves * kWave;
            const int rl = u / kF32Chunks, c = (u % kF32Chunks) ^ (rl & 15);
            buffer_load_lds16(rsrc, kbuf + m * kFastWaves * kWave + wave * kWave,
                              (rl * kF32Chunks + c) * 16);
        }
    }
#pragma unroll
    for (int p = 0; p < TILES; ++p) {
        wait_vmcnt<0>();
        __syncthreads();
        doublex4 acc = {0.0, 0.0, 0.0, 0.0};
        fast_step_f32(p + 1 < TILES ? kbuf + ((p + 1) & 1) * step_units : nullptr,
                      kbuf + (p & 1) * step_units, rsrc, p + 1, tid, qf, r16, g, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            so[p][i] = __float_as_uint((float)acc[i]);
    }
    // every wave is done with the last step's buffer before LDS is reused
    __syncthreads();
}

// lists[((t H + h) 2 + s) k + e] = (ord score, sub-key) of the e-th best
// sub-key of half s, e < k.  BLOCKS (1 or 2) blocks of TILES x 16 sub-keys
// (TILES = 8, 16, 32: 128, 256, 512 sub-keys); the group maxima are over
// groups of TILES / 4 scores, 64 groups per token.  The launcher picks the
// shape so that the first block is more than 3/4 full (at least 48 real
// groups, so tau is a real score and about k + 10 survive), the second
// block, if any, holding the rest: template arguments so that each case
// gets its own register allocation.
template <typename DT, int BLOCKS, int TILES>
// Three waves per SIMD: the register budget (168) makes the compiler spill a
// few dozen registers to scratch, which costs less than the latency a third
// wave hides (measured: 0.186 -> 0.177 ms for the selection at n = 512, and
// 0.61 -> 0.58 ms at n = 1024).
__global__ __launch_bounds__(kFastWaves *kWave) __attribute__((amdgpu_waves_per_eu(3, 3))) void fwd_topk_half_kernel(
    const DT *__restrict__ q, const DT *__restrict__ keys, int64_t key_hstride, int64_t T,
    int H, int n, int k, uint2 *__restrict__ lists)
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

    const DT *qrow = q + ((live ? t : 0) * H + h) * (int64_t)d_k + (int64_t)s * half;
    const int tid0 = threadIdx.x;
    const DT *kb = keys + h * key_hstride + (int64_t)s * n * half;

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
        const int base = kFirst ? 0 : (16 * TILES);
        const int n_loc = n - base < (16 * TILES) ? n - base : (16 * TILES);
        uint32_t so[TILES][4];
        if constexpr (std::is_same<DT, float>::value) {
            fast_scores_f32(so, kb + (int64_t)base * half, qrow, n_loc, tok, g, lds, tid);
        } else {
            // B fragments: token `tok`, K slice 32 kk + 8 g .. + 7 (loaded per
            // block, so they are not held through the selection)
            const uint16_t *qr = reinterpret_cast<const uint16_t *>(qrow);
            uint4 qf[kFastKSteps];
#pragma unroll
            for (int kk = 0; kk < kFastKSteps; ++kk)
                qf[kk] = *reinterpret_cast<const uint4 *>(qr + 32 * kk + 8 * g);
            fast_scores(so, reinterpret_cast<const uint16_t *>(kb + (int64_t)base * half), qf, n_loc,
                        tok, g, lds, tid);
        }
        if (n_loc < (16 * TILES)) {
            // (an asm statement keeps this a branch: a whole block skips the
            // selects)
            asm volatile("" ::: "memory");
            // sub-key 16 j + 4 g + i of the block exists iff 16 j + i < lim
            const int lim = n_loc - 4 * g;
            const uint32_t neg = __float_as_uint(-INFINITY);
#pragma unroll
            for (int j = 0; j < TILES; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[j][i] = 16 * j + i < lim ? so[j][i] : neg;
        }

        // The filter works on the float scores (compares, maxima); only the
        // survivors become order-preserving keys, when they are read back.
        auto sf = [&](int j, int i) { return __uint_as_float(so[j][i]); };
        // tau: k-th largest of the token's 64 group maxima (a lane's scores
        // 4 j + i in groups of SPG = TILES / 4 consecutive ones)
        constexpr int SPG = TILES / 4;
        float gm[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            float x = sf((SPG * m) / 4, (SPG * m) % 4);
#pragma unroll
            for (int e = SPG * m + 1; e < SPG * (m + 1); ++e)
                x = fmaxf(x, sf(e / 4, e % 4));
            gm[m] = x;
        }
        float tau = group4_kth(gm, k);
        // A first block is more than 3/4 full, >= 48 groups of real scores,
        // so tau is a real score and the sub-keys past n never survive.  A second block may hold fewer than k sub-keys: there the
        // first block's k-th key (a real score) raises the bar, and keys
        // below it cannot reach the top k anyway.
        if constexpr (!kFirst)
            tau = fmaxf(tau, unord_f32(dkey_ord<kSubBits>(prev[k - 1])));
        // a token past T (it scored token 0's query) keeps nothing: no score
        // compares >= NaN, so it counts no survivor, takes no bisection and
        // claims no position in the compaction (its 4 lanes share `live`)
        if (!live)
            tau = __uint_as_float(0x7fc00000u);

        // survivors: score >= tau
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < TILES; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cnt += sf(j, i) >= tau ? 1 : 0;
        int total = group4_sum(cnt);
        bool fits = total <= kFastSurv;

        // heavy ties: the exact k-th largest key of the block instead of tau,
        // by bisection on the score bits and then on the index among exactly
        // tied scores (more than 64 survivors are real scores, so is the
        // k-th largest)
        // (the whole wave then works on order-preserving keys: `ordm`)
        const bool ordm = __ballot(!fits) != 0;
        uint32_t kth = 0, tie_idx = 0xFFFFFFFFu;
        if (ordm) {
#pragma unroll
            for (int j = 0; j < TILES; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[j][i] = ord_f32(sf(j, i));
            kth = ord_f32(tau);
            uint32_t K = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = K | (1u << bit);
                int c = 0;
#pragma unroll
                for (int j = 0; j < TILES; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        c += so[j][i] >= cand ? 1 : 0;
                if (group4_sum(c) >= k)
                    K = cand;
            }
            int above = 0;
#pragma unroll
            for (int j = 0; j < TILES; ++j)
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
                for (int j = 0; j < TILES; ++j)
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

        // compact the survivors per token as two 32-bit arrays (scores and
        // sub-keys: 64-bit keys built here would pin register pairs for all
        // 128 candidates), then sort them as keys in the 4-lane group.
        const bool exact = tie_idx != 0xFFFFFFFFu;
        const int lim_t = exact ? (int)tie_idx - 4 * g : 0;   // 16 j + i <= lim_t among ties
        int mine = cnt;
        if (ordm && exact) {
            // recount this lane's share under the exact bound
            int c = 0;
#pragma unroll
            for (int j = 0; j < TILES; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t o = so[j][i];
                    c += (o > kth || (o == kth && 16 * j + i <= lim_t)) ? 1 : 0;
                }
            mine = c;
        }
        // Lane group g writes its survivors from position (the counts of the
        // groups before it), each at the next free position; the stores are
        // predicated (exec-masked), so only the lanes keeping a candidate
        // touch LDS, and survivor e ends at position e.  Sub-key 16 j + i +
        // gb: the constant part and the lane's own part, one add per store.
        const int c0 = __shfl(mine, tok), c1 = __shfl(mine, tok + 16), c2 = __shfl(mine, tok + 32);
        int off = (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
        const uint32_t gb = 4u * (uint32_t)g + (uint32_t)base;
        if (ordm) {
#pragma unroll
            for (int j = 0; j < TILES; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t o = so[j][i];
                    const bool keep =
                        live && (exact ? (o > kth || (o == kth && 16 * j + i <= lim_t)) : o >= kth);
                    if (keep) {
                        surv_s[off] = o;
                        surv_i[off] = (uint32_t)(16 * j + i) + gb;
                    }
                    off += keep ? 1 : 0;
                }
                __builtin_amdgcn_sched_barrier(0);     // one tile's keys at a time
            }
        } else {
#pragma unroll
            for (int j = 0; j < TILES; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool keep = sf(j, i) >= tau;
                    if (keep) {
                        surv_s[off] = so[j][i];
                        surv_i[off] = (uint32_t)(16 * j + i) + gb;
                    }
                    off += keep ? 1 : 0;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wave_lds_sync();
        uint64_t v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = 16 * g + r;
            const uint32_t sv = surv_s[e];
            const uint32_t hi = ordm ? sv : ord_f32(__uint_as_float(sv));
            v[r] = e < total ? dkey<kSubBits>(hi, surv_i[e]) : 0ull;
        }
        group4_sort_desc_dkey(v);
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
                    out[e] = make_uint2(dkey_ord<kSubBits>(v[r]), dkey_index<kSubBits>(v[r]));
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
// lists are sorted and rounding is monotone.  A row keeping more than
// kMergeSurv candidates raises the bound by bisection on the score (under
// heavy ties: the exact k-th key, by bisection on the 64-bit keys); the at
// most kMergeSurv survivors are then compacted into LDS and sorted per row.
constexpr int kMaxCorners = 16;
constexpr int kMergeSurv = 64;      // survivors per row at most: the sort's width

// list entries as staged in LDS: (score as float bits, sub-key)
__device__ __forceinline__ float merge_score(uint2 l, uint2 r)
{
    return __uint_as_float(l.x) + __uint_as_float(r.x);
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
                // entries 2 e, 2 e + 1 lie in one row (a row has 2 k entries);
                // the scores go back to floats once here, not per candidate
                uint2 *d = sl + (e / k) * kMergePitch + 2 * (e % k);
                d[0] = make_uint2(__float_as_uint(unord_f32(buf[u].x)), buf[u].y);
                d[1] = make_uint2(__float_as_uint(unord_f32(buf[u].z)), buf[u].w);
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
            v[c] = dkey<kSlotBits>(ord_f32(merge_score(la, rb)), la.y * (uint32_t)n + rb.y);
        } else {
            v[c] = 0ull;
        }
        cnt += dkey_ord<kSlotBits>(v[c]) >= otau ? 1 : 0;
    }
    if (!live)
        cnt = 0;        // rows past the end keep nothing
    int total = group4_sum(cnt);
    auto count_ge = [&](uint32_t o) {
        int c = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            c += dkey_ord<kSlotBits>(v[e]) >= o ? 1 : 0;
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
    uint64_t kth = live ? dkey<kSlotBits>(otau, (1u << kSlotBits) - 1u) : ~0ull;
    if (__ballot(live && total > kMergeSurv) != 0) {
        const bool more = live && total > kMergeSurv;
        uint64_t K = 0;
        for (int bit = 52; bit >= 0; --bit) {     // every key is below 2^53
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
    // position (the counts of the groups before it), each survivor at the
    // next free slot, by predicated stores (only lanes keeping a candidate
    // touch LDS): survivor e ends at position e.
    wave_lds_sync();
    uint64_t *surv = reinterpret_cast<uint64_t *>(sl) + tok * kMergePitch;
    const int c0 = __shfl(cnt, tok), c1 = __shfl(cnt, tok + 16), c2 = __shfl(cnt, tok + 32);
    int off = (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const bool keep = live && v[c] >= kth;
        if (keep)
            surv[off] = v[c];
        off += keep ? 1 : 0;
    }
    wave_lds_sync();
    uint64_t w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int e = 16 * g + q;
        w[q] = live && e < total ? surv[e] : 0ull;
    }
    group4_sort_desc_dkey(w);

    // ranks 16 g + q sit in lane groups 0 and 1 (k <= 32); lane group g'
    // takes ranks 8 g' .. 8 g' + 7, registers 8 (g' % 2) + r of lane group
    // g' / 2, so the softmax and the stores are spread over all four lanes
    const int src = tok + 16 * (g >> 1);
    uint64_t x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const uint64_t a = shfl_u64(w[r], src), b = shfl_u64(w[8 + r], src);
        x[r] = (g & 1) ? b : a;
    }
    const int64_t out = (row0 + tok) * (int64_t)k;
    const float top = __shfl(unord_f32(dkey_ord<kSlotBits>(w[0])), tok);
    const int e0 = 8 * g;
    float ex[8], z = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        ex[r] = e0 + r < k ? expf(unord_f32(dkey_ord<kSlotBits>(x[r])) - top) : 0.f;
        z += ex[r];
    }
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    if (live && e0 < k) {
        int32_t oi[8];
        float ow[8], os[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            oi[r] = (int32_t)dkey_index<kSlotBits>(x[r]);
            ow[r] = ex[r] / z;
            os[r] = unord_f32(dkey_ord<kSlotBits>(x[r]));
        }
        if ((k & 3) == 0) {
            // 16-byte stores: out + e0 is a multiple of 4 and so is k - e0
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                if (e0 + 4 * h4 < k) {
                    const int at = e0 + 4 * h4;
                    *reinterpret_cast<int4 *>(idx + out + at) =
                        make_int4(oi[4 * h4], oi[4 * h4 + 1], oi[4 * h4 + 2], oi[4 * h4 + 3]);
                    *reinterpret_cast<float4 *>(weights + out + at) =
                        make_float4(ow[4 * h4], ow[4 * h4 + 1], ow[4 * h4 + 2], ow[4 * h4 + 3]);
                    if (scores)
                        *reinterpret_cast<float4 *>(scores + out + at) =
                            make_float4(os[4 * h4], os[4 * h4 + 1], os[4 * h4 + 2], os[4 * h4 + 3]);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (e0 + r < k) {
                    idx[out + e0 + r] = oi[r];
                    weights[out + e0 + r] = ow[r];
                    if (scores)
                        scores[out + e0 + r] = os[r];
                }
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

hipError_t launch_select_fast(int dtype, const void *q, const void *keys, int64_t key_hstride,
                              int64_t T, int H, int n, int k, int d_k, int32_t *idx,
                              float *weights, float *scores, void *workspace, hipStream_t stream)
{
    (void)d_k;      // 512 on this path
    uint2 *lists = static_cast<uint2 *>(workspace);
    const dim3 grid((unsigned)((T + kFastTokWG - 1) / kFastTokWG), (unsigned)H, 2);
    // block shapes: the first block more than 3/4 full
    auto go = [&](auto kern, auto dt) {
        typedef decltype(dt) DT;
        hipLaunchKernelGGL(kern, grid, dim3(kFastWaves * kWave), 0, stream,
                           static_cast<const DT *>(q), static_cast<const DT *>(keys), key_hstride,
                           T, H, n, k, lists);
    };
    if (dtype == 0) {
        // float32 storage, n <= 256 (select_fast_ok): blocks of 128 sub-keys
        // (a block of 256 with the float32 query fragments spills)
        if (n <= 128)
            go(fwd_topk_half_kernel<float, 1, 8>, float{});
        else
            go(fwd_topk_half_kernel<float, 2, 8>, float{});
    } else if (n <= 128)
        go(fwd_topk_half_kernel<bf16_t, 1, 8>, bf16_t{});
    else if (n <= 192)
        go(fwd_topk_half_kernel<bf16_t, 2, 8>, bf16_t{});
    else if (n <= 256)
        go(fwd_topk_half_kernel<bf16_t, 1, 16>, bf16_t{});
    else if (n <= 384)
        go(fwd_topk_half_kernel<bf16_t, 2, 16>, bf16_t{});
    else if (n <= 512)
        go(fwd_topk_half_kernel<bf16_t, 1, 32>, bf16_t{});
    else
        go(fwd_topk_half_kernel<bf16_t, 2, 32>, bf16_t{});
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

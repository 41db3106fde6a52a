// pkm_flat.hip -- the flat-key search the product keys replace, as a GPU
// workload of its own (companion page "Product Keys Give Transformers
// Million-Slot Memory Layers", section "Search cost: flat vs product keys": a
// flat memory compares the query with every one of its N keys, the product
// keys with about 2 sqrt(N) half keys plus k^2 pairs).  Every (token, head)
// scores all n*n implied keys -- key f = i n + j is left sub-key i followed
// by right sub-key j (section "Implied keys vs stored sub-keys") -- with one
// d_k-wide dot product each, float32 accumulation, and keeps the exact top-k
// by (score desc, slot asc), then the softmax of the k scores.  Its result
// is the flat search's own; the product-key path reaches the same set by
// the argument of section "Why top-k of each half is enough".
//
// bf16 storage, d_k = 512, 32 <= n <= 1024, k <= 32.  One wave per (16
// tokens, head), 4 waves per workgroup sharing the key tiles through LDS.
// The N keys are scored in blocks of 256 straight into registers with
// v_mfma_f32_16x16x32_bf16 (keys as M, tokens as N): the left 256 dims of a
// key come from C[i], the right 256 from C'[j], accumulated into the same
// registers by a second pass.  A running top-k per token (64-bit keys:
// order-preserving score, then the complemented slot) stays in LDS, and so
// does a buffer of up to 48 candidates: a block's survivors -- the keys
// reaching the running k-th score (the first block: the k-th of its 64
// group maxima, groups of 4 keys) -- are appended to the buffer, and only
// when it would overflow (or at the end) is it sorted inside the token's 4
// lanes and merged into the running list by a bitonic merge.  Block b keeps
// about k / b keys on random data, so the sorts number about log(N / 256)
// instead of one per block, and the scoring's MFMAs dominate.
#include <type_traits>

#include "pkm_device.hpp"
#include "pkm_kernels.hpp"

namespace pkm {

constexpr int kFlatWaves = 4;
constexpr int kFlatTok = 16;                        // tokens per wave
constexpr int kFlatTokWG = kFlatWaves * kFlatTok;   // tokens per workgroup
constexpr int kFlatTiles = 16;                      // 16-key tiles per block
constexpr int kFlatBlock = 16 * kFlatTiles;         // 256 keys per block
constexpr int kFlatKSteps = 8;                      // 32-wide K steps per 256-dim half
constexpr int kFlatHalf = 32 * kFlatKSteps;         // 256
constexpr int kFlatBuf = 48;                        // buffered candidates per token at most
constexpr int kFlatBufStride = kFlatBuf + 4;        // + one dump slot per lane group

// Scores of the wave's 16 tokens against implied keys base .. base + 255,
// as order-preserving integers: so[j][i] = ord(score of key base + 16 j +
// 4 g + i) for token `tok`.  Two passes over the key tiles: the left halves
// C[f / n] against q1, then the right halves C'[f % n] against q2 added to
// the same accumulators (one float32 sum per key over all d_k products).
// The tile of step p (32 keys, 16 KB per half) is staged in LDS,
// double-buffered, its 16-byte chunks XOR-swizzled by row; rows past N read
// as zeros (their scores are masked by the caller).
__device__ __forceinline__ void flat_scores(uint32_t (&so)[kFlatTiles][4], const uint16_t *cl,
                                            const uint16_t *cr, int n, int64_t N, int64_t base,
                                            const uint16_t *qrow, int r16, int g, uint4 *kbuf,
                                            int tid)
{
    constexpr int chunks = kFlatHalf * 2 / 16;        // 32 chunks of 16 bytes per half row
    constexpr int step_units = 32 * chunks;           // 1024 chunks per 32-row step
    constexpr int per_thread = step_units / (kFlatWaves * kWave);
    constexpr int steps = kFlatTiles / 2;
    constexpr int kOut = 0x40000000;                  // an offset past any codebook: zeros
    const int row_bytes = kFlatHalf * 2;
    const __amdgpu_buffer_rsrc_t rl_rsrc = buffer_over(cl, n * row_bytes);
    const __amdgpu_buffer_rsrc_t rr_rsrc = buffer_over(cr, n * row_bytes);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const __amdgpu_buffer_rsrc_t rsrc = pass == 0 ? rl_rsrc : rr_rsrc;
        uint4 qf[kFlatKSteps];
#pragma unroll
        for (int kk = 0; kk < kFlatKSteps; ++kk)
            qf[kk] = *reinterpret_cast<const uint4 *>(qrow + pass * kFlatHalf + 32 * kk + 8 * g);
        // (i, j) of the key whose row each of this thread's chunks loads next
        int ii[per_thread], jj[per_thread];
#pragma unroll
        for (int m = 0; m < per_thread; ++m) {
            const int64_t f = base + (tid + m * kFlatWaves * kWave) / chunks;
            ii[m] = (int)(f / n);
            jj[m] = (int)(f % n);
        }
        uint4 pre[per_thread];
        auto gload = [&]() {
#pragma unroll
            for (int m = 0; m < per_thread; ++m) {
                const int u = tid + m * kFlatWaves * kWave;
                const int rl = u / chunks, c = (u % chunks) ^ (rl & 15);
                const int sub = pass == 0 ? ii[m] : jj[m];
                const int off = ii[m] < n ? sub * row_bytes + c * 16 : kOut;
                pre[m] = buffer_load16(rsrc, off, 0);
                // the next step's row is 32 keys further on (n >= 32: one wrap at most)
                jj[m] += 32;
                if (jj[m] >= n) {
                    jj[m] -= n;
                    ++ii[m];
                }
            }
        };
        auto lstore = [&](int buf) {
#pragma unroll
            for (int m = 0; m < per_thread; ++m)
                kbuf[buf * step_units + tid + m * kFlatWaves * kWave] = pre[m];
        };
        gload();
        lstore(0);
        gload();
        __syncthreads();
#pragma unroll
        for (int p = 0; p < steps; ++p) {
            const uint4 *cur = kbuf + (p & 1) * step_units;
            floatx4 acc[2];
#pragma unroll
            for (int w = 0; w < 2; ++w)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[w][i] = pass == 0 ? 0.f : __uint_as_float(so[2 * p + w][i]);
#pragma unroll
            for (int kk = 0; kk < kFlatKSteps; ++kk) {
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const int rl = 16 * w + r16;
                    const uint4 a = cur[rl * chunks + ((4 * kk + g) ^ r16)];
                    acc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[kk]),
                        acc[w], 0, 0, 0);
                }
            }
#pragma unroll
            for (int w = 0; w < 2; ++w)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[2 * p + w][i] = pass == 0 ? __float_as_uint(acc[w][i]) : ord_f32(acc[w][i]);
            if (p + 1 < steps)
                lstore((p + 1) & 1);
            if (p + 2 < steps)
                gload();
            __syncthreads();
        }
    }
}

// A token's buffered candidates (fill <= 48 entries of score and slot) merged
// into its running top k: they become 64-bit keys that order as float64
// values (order-preserving score, then the lower slot first; slots < 2^20),
// are sorted inside the token's 4 lanes, and the top k of the sorted list A
// (the running one) and B (the candidates) are max(A[e], B[31 - e]) for
// e < 32 -- a bitonic sequence -- put in order by a bitonic merge, every
// exchange one float64 max and one min.  Wave-wide: every lane takes part
// (tokens with an empty buffer merge zero keys, which changes nothing).
constexpr int kFlatSlotBits = 20;
__device__ __forceinline__ void merge_buffer(int g, int tok, int fill, const uint32_t *buf_s,
                                             const uint32_t *buf_f, uint64_t *best)
{
    uint64_t v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int e = 16 * g + r;
        v[r] = e < fill ? dkey<kFlatSlotBits>(buf_s[e], buf_f[e]) : 0ull;
    }
    group4_sort_desc_dkey(v);
    // lane groups 0 and 1 hold C; B[31 - e] is register 15 - r of the other group
    const int ga = g & 1;
    uint64_t c[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint64_t a = best[16 * ga + r];
        const uint64_t b = shfl_xor_u64(v[15 - r], 16);
        c[r] = dkey_max(a, b);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint64_t o = shfl_xor_u64(c[r], 16);
        c[r] = ga == 0 ? dkey_max(c[r], o) : dkey_min(c[r], o);
    }
#pragma unroll
    for (int stride = 8; stride > 0; stride >>= 1)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r & stride) == 0) {
                const uint64_t x = c[r], y = c[r | stride];
                c[r] = dkey_max(x, y);
                c[r | stride] = dkey_min(x, y);
            }
    wave_lds_sync();
    if (g < 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            best[16 * g + r] = c[r];
    }
    wave_lds_sync();
}

// idx, weights, scores [T][H][k]: the k best implied keys of (t, h) in
// (score desc, slot asc) order, their softmax weights and scores.
// two waves per SIMD: 251 registers, no spills (one wave per SIMD without the bound)
__global__ __launch_bounds__(kFlatWaves *kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_flat_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ keys, int64_t key_hstride,
    int64_t T, int H, int n, int k, int32_t *__restrict__ idx, float *__restrict__ weights,
    float *__restrict__ scores)
{
    // the key tiles of the scoring (two 32-row steps of 16 KB)
    __shared__ uint4 kbuf[2 * 32 * 32];
    // per wave and token: the candidate buffer (score, slot) and the running
    // top k (row stride 33: the 16 tokens' rows start in distinct banks)
    __shared__ uint32_t s_buf_s[kFlatWaves][kFlatTok][kFlatBufStride];
    __shared__ uint32_t s_buf_f[kFlatWaves][kFlatTok][kFlatBufStride];
    __shared__ uint64_t s_best[kFlatWaves][kFlatTok][33];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int tok_lane = lane & 15, g_lane = lane >> 4;
    constexpr int d_k = 2 * kFlatHalf;
    const int h = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * kFlatTokWG + wave * kFlatTok + tok_lane;
    const bool live = t < T;
    const uint16_t *qrow =
        reinterpret_cast<const uint16_t *>(q) + ((live ? t : 0) * H + h) * (int64_t)d_k;
    const uint16_t *cl = reinterpret_cast<const uint16_t *>(keys) + h * key_hstride;
    const uint16_t *cr = cl + (int64_t)n * kFlatHalf;
    const int64_t N = (int64_t)n * n;
    const int nblocks = (int)((N + kFlatBlock - 1) / kFlatBlock);
    const int tid0 = threadIdx.x;
    // the running lists start as zero keys (below every real key): until the
    // first merge, the k-th key lets everything through
    if (g_lane < 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s_best[wave][tok_lane][16 * g_lane + r] = 0ull;
    }
    wave_lds_sync();
    int fill = 0;                   // candidates in this token's buffer (same in its 4 lanes)

    for (int b = 0; b < nblocks; ++b) {
        // opaque copies of the lane's coordinates: values derived from them
        // (LDS offsets, the 64 key indices, masks) are formed where used
        // instead of being hoisted out of the loop and held in registers
        int g = g_lane, tok = tok_lane, tid = tid0;
        asm volatile("" : "+v"(g), "+v"(tok), "+v"(tid));
        uint32_t *buf_s = s_buf_s[wave][tok];
        uint32_t *buf_f = s_buf_f[wave][tok];
        uint64_t *best = s_best[wave][tok];
        const bool first = b == 0;
        const int64_t base = (int64_t)b * kFlatBlock;
        const int n_loc = N - base < kFlatBlock ? (int)(N - base) : kFlatBlock;
        uint32_t so[kFlatTiles][4];
        flat_scores(so, cl, cr, n, N, base, qrow, tok, g, kbuf, tid);
        if (n_loc < kFlatBlock) {
            // key 16 j + 4 g + i of the block exists iff 16 j + i < lim
            const int lim = n_loc - 4 * g;
            const uint32_t neg = ord_f32(-INFINITY);
#pragma unroll
            for (int j = 0; j < kFlatTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    so[j][i] = 16 * j + i < lim ? so[j][i] : neg;
        }

        uint32_t tau;
        if (first) {
            // the k-th largest of the token's 64 group maxima (groups of 4
            // keys, one tile's 4 scores of a lane): the k groups above it each
            // hold a score >= tau (about 40 survive, at most 64 in practice).
            // The first block is whole (N >= 1024), so tau is a real score.
            uint32_t gm[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                gm[m] = max(max(so[m][0], so[m][1]), max(so[m][2], so[m][3]));
            tau = group4_kth(gm, k);
        } else {
            // the running k-th best score: keys below it cannot enter
            tau = dkey_ord<kFlatSlotBits>(best[k - 1]);
        }

        // survivors: ord >= tau (a token past T keeps nothing)
        auto count_ge = [&](uint32_t th) {
            int c = 0;
#pragma unroll
            for (int j = 0; j < kFlatTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    c += so[j][i] >= th ? 1 : 0;
            return live ? c : 0;
        };
        int cnt = count_ge(tau);
        int total = group4_sum(cnt);
        // a token whose buffer would overflow: every buffer of the wave goes
        // into its running list first, whose (higher) k-th score then filters
        // this block again
        if (__ballot(fill + total > kFlatBuf) != 0) {
            merge_buffer(g, tok, fill, buf_s, buf_f, best);
            fill = 0;
            if (!first) {
                tau = dkey_ord<kFlatSlotBits>(best[k - 1]);
                cnt = count_ge(tau);
                total = group4_sum(cnt);
            }
        }
        bool fits = total <= kFlatBuf;

        // heavy ties: the exact k-th largest key of the block (bisection on
        // the score bits, then on the index among exactly tied scores); more
        // survivors than the buffer holds are real keys, and so is the k-th
        uint32_t kth = tau, tie_idx = 0xFFFFFFFFu;
        if (__ballot(!fits) != 0) {
            uint32_t K = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = K | (1u << bit);
                if (group4_sum(count_ge(cand)) >= k)
                    K = cand;
            }
            int above = 0;
#pragma unroll
            for (int j = 0; j < kFlatTiles; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    above += so[j][i] > K ? 1 : 0;
            const int need = k - group4_sum(above);
            uint32_t I = 0;
            for (int bit = 9; bit >= 0; --bit) {
                const uint32_t cand = I | (1u << bit);
                const int lim_c = (int)cand - 4 * g;
                int c = 0;
#pragma unroll
                for (int j = 0; j < kFlatTiles; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        c += (so[j][i] == K && 16 * j + i < lim_c) ? 1 : 0;
                if (group4_sum(c) < need)
                    I = cand;
            }
            if (!fits) {
                kth = K;
                tie_idx = I;
                total = k;
                fits = true;
            }
        }

        // append the survivors to the buffer, densely: lane group g writes
        // from fill + (the counts of the groups before it); a candidate that
        // is not kept goes to the group's dump slot past the buffer
        if (__ballot(total > 0) != 0) {
            const bool exact = tie_idx != 0xFFFFFFFFu;
            const int lim_t = exact ? (int)tie_idx - 4 * g : 0;
            int mine = cnt;
            if (exact) {
                int c = 0;
#pragma unroll
                for (int j = 0; j < kFlatTiles; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t o = so[j][i];
                        c += (o > kth || (o == kth && 16 * j + i <= lim_t)) ? 1 : 0;
                    }
                mine = live ? c : 0;
            }
            const int c0 = __shfl(mine, tok), c1 = __shfl(mine, tok + 16),
                      c2 = __shfl(mine, tok + 32);
            int off = fill + (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
            const int dump = kFlatBuf + g;
            const uint32_t fbase = (uint32_t)base + 4u * (uint32_t)g;
#pragma unroll
            for (int j = 0; j < kFlatTiles; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t o = so[j][i];
                    const bool keep =
                        live && (exact ? (o > kth || (o == kth && 16 * j + i <= lim_t)) : o >= kth);
                    const int at = keep ? off : dump;
                    buf_s[at] = o;
                    buf_f[at] = fbase + (uint32_t)(16 * j + i);
                    off += keep ? 1 : 0;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            fill += total;
            wave_lds_sync();
        }
    }
    // the last candidates
    {
        const int g = g_lane, tok = tok_lane;
        if (__ballot(fill > 0) != 0)
            merge_buffer(g, tok, fill, s_buf_s[wave][tok], s_buf_f[wave][tok], s_best[wave][tok]);
    }

    // softmax over the k best (ranks 16 g + r in lane groups 0 and 1)
    const int g = g_lane;
    const uint64_t *best = s_best[wave][tok_lane];
    uint64_t v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        v[r] = g < 2 && 16 * g + r < k ? best[16 * g + r] : 0ull;
    const float top = unord_f32(dkey_ord<kFlatSlotBits>(best[0]));
    float ex[16], z = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ex[r] = g < 2 && 16 * g + r < k ? expf(unord_f32(dkey_ord<kFlatSlotBits>(v[r])) - top) : 0.f;
        z += ex[r];
    }
    z += __shfl_xor(z, 16);
    if (live && g < 2) {
        const int64_t out = (t * H + h) * (int64_t)k;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int e = 16 * g + r;
            if (e < k) {
                idx[out + e] = (int32_t)dkey_index<kFlatSlotBits>(v[r]);
                weights[out + e] = ex[r] / z;
                if (scores)
                    scores[out + e] = unord_f32(dkey_ord<kFlatSlotBits>(v[r]));
            }
        }
    }
}

hipError_t launch_flat_select(const void *q, const void *keys, int64_t key_hstride, int64_t T,
                              int H, int n, int k, int32_t *idx, float *weights, float *scores,
                              hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kFlatTokWG - 1) / kFlatTokWG), (unsigned)H);
    hipLaunchKernelGGL(fwd_flat_kernel, grid, dim3(kFlatWaves * kWave), 0, stream,
                       static_cast<const bf16_t *>(q), static_cast<const bf16_t *>(keys),
                       key_hstride, T, H, n, k, idx, weights, scores);
    return hipGetLastError();
}

}  // namespace pkm

// pkm_select.hip -- fused forward selection of the product-key memory layer.
//
// One workgroup (4 waves) owns 16 tokens of one head.  For each half s of the
// query (gptget.net summary of "Large Memory Layers with Product Keys",
// "Methodology": split q into q1, q2 and search each against its own sub-key
// set):
//   1. the 16 query halves are staged in LDS, and the 16 x n score tile
//      <q_s[t], C_s[i]> is computed with MFMA (bf16 storage:
//      v_mfma_f32_16x16x32_bf16, exact products, float32 accumulation; float32
//      storage: v_mfma_f64_16x16x4_f64, exact products and float64
//      accumulation, rounded once), sub-keys as the M dimension, tokens as N,
//      straight into LDS -- scores never reach HBM;
//   2. every row's exact top-k, ordered (score desc, index asc), is found by a
//      threshold filter: tau = k-th largest of the 64 per-lane maxima is a
//      lower bound of the k-th largest score (the k lanes above it each hold
//      one score >= tau), so every score >= tau survives, and only the
//      survivors are bitonic-sorted.
// Then each row's two lists are combined (companion page "Why top-k of each
// half is enough"): a pair of ranks (a, b) can only make the final top-k if
// (a+1)(b+1) <= k, because every pair (a', b') <= (a, b) componentwise scores
// at least as high and, on a tie, has the lower slot.  That leaves
// sum_a floor(k/a) candidates (119 for k = 32) instead of k^2.  Their scores
// left_a + right_b are sorted with the slot f = i*n + j as tie-break, the
// first k are kept, and a softmax over them gives the weights.
#include "pkm_device.hpp"
#include "pkm_kernels.hpp"

namespace pkm {

constexpr int kSelTokens = 16;   // tokens per workgroup (the MFMA N dimension)
constexpr int kSelWaves = 4;
constexpr int kSelThreads = kSelWaves * kWave;

struct SelLayout {
    int n_pad;          // score row stride (floats)
    int q_stride;       // query tile row stride (elements)
    int n_pairs;        // merge candidates for this k
    unsigned off_q, off_ls, off_li, off_surv, off_pairs, total;  // byte offsets in LDS
};

static inline unsigned align16(unsigned x) { return (x + 15u) & ~15u; }

static SelLayout sel_layout(int n, int k, int half, int elt_bytes)
{
    SelLayout L;
    L.n_pad = ((n + 15) / 16) * 16 + 4;
    L.q_stride = half + 16 / elt_bytes;          // +16 bytes: spreads rows over LDS banks
    L.n_pairs = merge_candidates(k);
    unsigned off = align16((unsigned)(kSelTokens * L.n_pad * 4));
    L.off_q = off;
    off = align16(off + (unsigned)(kSelTokens * L.q_stride * elt_bytes));
    L.off_ls = off;
    off = align16(off + (unsigned)(kSelTokens * 2 * k * 4));
    L.off_li = off;
    off = align16(off + (unsigned)(kSelTokens * 2 * k * 4));
    L.off_surv = off;
    off = align16(off + (unsigned)(kSelWaves * n * 8));
    L.off_pairs = off;
    off = align16(off + (unsigned)(L.n_pairs * 2));
    L.total = off;
    return L;
}

// ---- step 1: score tile --------------------------------------------------
// Scores of sub-keys [tile*16, tile*16+16) against the 16 staged queries.
// Lane l supplies A row (sub-key) l%16 and B column (token) l%16; the K slice
// of a lane is the same for A and B, so the dot products are exact sums.
__device__ __forceinline__ floatx4 score_tile(const bf16_t *krow_base, int n, int half,
                                              const bf16_t *qt, int q_stride, int tile)
{
    const int lane = lane_id();
    const int r16 = lane & 15, kg = lane >> 4;
    const int sub = tile * 16 + r16;
    const bool valid = sub < n;
    const uint16_t *arow = reinterpret_cast<const uint16_t *>(krow_base) + (int64_t)(valid ? sub : 0) * half;
    const uint16_t *brow = reinterpret_cast<const uint16_t *>(qt) + r16 * q_stride;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < half; kk += 32) {
        const int c = kk + kg * 8;
        uint4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (c < half) {
            if (valid)
                a = *reinterpret_cast<const uint4 *>(arow + c);
            b = *reinterpret_cast<const uint4 *>(brow + c);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    return acc;
}

// float32 storage: the operands widen exactly to float64 and v_mfma_f64_16x16x4_f64
// accumulates in float64, so each score is the exact dot product rounded once
// to float32 (scores of any magnitude keep full float32 accuracy, which the
// softmax weights inherit).
__device__ __forceinline__ floatx4 score_tile(const float *krow_base, int n, int half,
                                              const float *qt, int q_stride, int tile)
{
    const int lane = lane_id();
    const int r16 = lane & 15, kg = lane >> 4;
    const int sub = tile * 16 + r16;
    const bool valid = sub < n;
    const float *arow = krow_base + (int64_t)(valid ? sub : 0) * half;
    const float *brow = qt + r16 * q_stride;
    doublex4 acc = {0.0, 0.0, 0.0, 0.0};
    for (int kk = 0; kk < half; kk += 16) {
        const int c = kk + kg * 4;
        float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (c < half) {
            if (valid)
                a = *reinterpret_cast<const float4 *>(arow + c);
            b = *reinterpret_cast<const float4 *>(brow + c);
        }
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.x, (double)b.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.y, (double)b.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.z, (double)b.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.w, (double)b.w, acc, 0, 0, 0);
    }
    floatx4 out = {(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
    return out;
}

// ---- step 2: exact top-k of one score row --------------------------------
template <int R>
__device__ __forceinline__ void sort_survivors(const uint64_t *surv, int total, int k,
                                               float *out_s, int *out_i)
{
    const int lane = lane_id();
    uint64_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kWave + lane;
        v[r] = i < total ? surv[i] : 0ull;
    }
    wave_sort_desc<R>(v);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kWave + lane;
        if (i < k) {
            out_s[i] = key_score(v[r]);
            out_i[i] = (int)key_index(v[r]);
        }
    }
}

__device__ void select_row(const float *srow, int n, int k, uint64_t *surv, float *out_s,
                           int *out_i)
{
    const int lane = lane_id();
    float m = -INFINITY;
    for (int e = lane; e < n; e += kWave)
        m = fmaxf(m, srow[e]);
    const float tau = __shfl(wave_sort64_desc(m), k - 1);
    int cnt = 0;
    for (int e = lane; e < n; e += kWave)
        cnt += srow[e] >= tau ? 1 : 0;
    int total;
    int off = wave_exclusive_scan(cnt, &total);
    for (int e = lane; e < n; e += kWave) {
        const float s = srow[e];
        if (s >= tau)
            surv[off++] = make_key(s, (uint32_t)e);
    }
    wave_lds_sync();
    if (total <= 64)
        sort_survivors<1>(surv, total, k, out_s, out_i);
    else if (total <= 128)
        sort_survivors<2>(surv, total, k, out_s, out_i);
    else if (total <= 256)
        sort_survivors<4>(surv, total, k, out_s, out_i);
    else if (total <= 512)
        sort_survivors<8>(surv, total, k, out_s, out_i);
    else
        sort_survivors<16>(surv, total, k, out_s, out_i);
    wave_lds_sync();
}

// ---- step 3: combine the two halves, softmax ------------------------------
template <int R>
__device__ __forceinline__ void merge_row(const float *ls, const int *li, const float *rs,
                                          const int *ri, const uint16_t *pairs, int n_pairs,
                                          int n, int k, int64_t out_off, int32_t *idx,
                                          float *weights, float *scores)
{
    const int lane = lane_id();
    uint64_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = r * kWave + lane;
        if (c < n_pairs) {
            const int a = pairs[c] & 0xFF, b = pairs[c] >> 8;
            const uint32_t f = (uint32_t)li[a] * (uint32_t)n + (uint32_t)ri[b];
            v[r] = make_key(ls[a] + rs[b], f);
        } else {
            v[r] = 0ull;
        }
    }
    wave_sort_desc<R>(v);
    // k <= 64: the winners are element r = 0 of lanes 0..k-1
    const float sc = key_score(v[0]);
    const float top = __shfl(sc, 0);
    const float e = lane < k ? expf(sc - top) : 0.f;
    const float z = wave_sum(e);
    if (lane < k) {
        idx[out_off + lane] = (int32_t)key_index(v[0]);
        weights[out_off + lane] = e / z;
        if (scores)
            scores[out_off + lane] = sc;
    }
}

template <typename DT>
__global__ __launch_bounds__(kSelThreads) void fwd_select_kernel(
    const DT *__restrict__ q, const DT *__restrict__ keys, int64_t key_hstride, int64_t T, int H,
    int n, int k, int d_k, SelLayout L, int32_t *__restrict__ idx, float *__restrict__ weights,
    float *__restrict__ scores)
{
    extern __shared__ __align__(16) unsigned char smem[];
    float *sc = reinterpret_cast<float *>(smem);
    DT *qt = reinterpret_cast<DT *>(smem + L.off_q);
    float *ls = reinterpret_cast<float *>(smem + L.off_ls);   // [tok][s][k]
    int *li = reinterpret_cast<int *>(smem + L.off_li);       // [tok][s][k]
    uint16_t *pairs = reinterpret_cast<uint16_t *>(smem + L.off_pairs);

    const int half = d_k / 2;
    const int64_t t0 = (int64_t)blockIdx.x * kSelTokens;
    const int h = blockIdx.y;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    uint64_t *surv = reinterpret_cast<uint64_t *>(smem + L.off_surv) + (size_t)wave * n;

    // candidate rank pairs (a, b) with (a+1)(b+1) <= k, row a holding floor(k/(a+1))
    if (wave == 0) {
        const int cnt = lane < k ? k / (lane + 1) : 0;
        int total;
        const int start = wave_exclusive_scan(cnt, &total);
        for (int b = 0; b < cnt; ++b)
            pairs[start + b] = (uint16_t)(lane | (b << 8));
    }

    constexpr int elt = (int)sizeof(DT);
    const int chunks_per_row = half * elt / 16;
    for (int s = 0; s < 2; ++s) {
        // stage the 16 query halves (zeros past the last token)
        for (int c = threadIdx.x; c < kSelTokens * chunks_per_row; c += kSelThreads) {
            const int row = c / chunks_per_row, cc = c % chunks_per_row;
            const int64_t t = t0 + row;
            uint4 v = {0u, 0u, 0u, 0u};
            if (t < T)
                v = *reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const unsigned char *>(q + (t * H + h) * (int64_t)d_k + (int64_t)s * half) + cc * 16);
            *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(qt) + (size_t)row * L.q_stride * elt + cc * 16) = v;
        }
        __syncthreads();

        const DT *kbase = keys + h * key_hstride + (int64_t)s * n * half;
        const int ntiles = (n + 15) / 16;
        for (int tile = wave; tile < ntiles; tile += kSelWaves) {
            const floatx4 acc = score_tile(kbase, n, half, qt, L.q_stride, tile);
            float *dst = sc + (lane & 15) * L.n_pad + tile * 16;
            if constexpr (sizeof(DT) == 2) {
                // f32 MFMA: lane l holds sub-keys 4*(l/16) + i of token l%16
                float4 out = {acc[0], acc[1], acc[2], acc[3]};
                *reinterpret_cast<float4 *>(dst + 4 * (lane >> 4)) = out;
            } else {
                // f64 MFMA: lane l holds sub-keys 4*i + l/16 of token l%16
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[4 * i + (lane >> 4)] = acc[i];
            }
        }
        __syncthreads();

        for (int row = wave; row < kSelTokens; row += kSelWaves) {
            if (t0 + row < T)
                select_row(sc + row * L.n_pad, n, k, surv, ls + (row * 2 + s) * k,
                           li + (row * 2 + s) * k);
        }
        __syncthreads();
    }

    for (int row = wave; row < kSelTokens; row += kSelWaves) {
        const int64_t t = t0 + row;
        if (t >= T)
            continue;
        const int64_t out_off = (t * H + h) * (int64_t)k;
        const float *l_s = ls + (row * 2 + 0) * k;
        const int *l_i = li + (row * 2 + 0) * k;
        const float *r_s = ls + (row * 2 + 1) * k;
        const int *r_i = li + (row * 2 + 1) * k;
        if (L.n_pairs <= 64)
            merge_row<1>(l_s, l_i, r_s, r_i, pairs, L.n_pairs, n, k, out_off, idx, weights, scores);
        else if (L.n_pairs <= 128)
            merge_row<2>(l_s, l_i, r_s, r_i, pairs, L.n_pairs, n, k, out_off, idx, weights, scores);
        else if (L.n_pairs <= 256)
            merge_row<4>(l_s, l_i, r_s, r_i, pairs, L.n_pairs, n, k, out_off, idx, weights, scores);
        else
            merge_row<8>(l_s, l_i, r_s, r_i, pairs, L.n_pairs, n, k, out_off, idx, weights, scores);
    }
}

template <typename DT>
static hipError_t launch_select_t(const void *q, const void *keys, int64_t key_hstride, int64_t T,
                                  int H, int n, int k, int d_k, int32_t *idx, float *weights,
                                  float *scores, hipStream_t stream)
{
    const SelLayout L = sel_layout(n, k, d_k / 2, (int)sizeof(DT));
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_select_kernel<DT>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.total);
    if (err != hipSuccess)
        return err;
    const dim3 grid((unsigned)((T + kSelTokens - 1) / kSelTokens), (unsigned)H);
    hipLaunchKernelGGL(fwd_select_kernel<DT>, grid, dim3(kSelThreads), L.total, stream,
                       static_cast<const DT *>(q), static_cast<const DT *>(keys), key_hstride, T,
                       H, n, k, d_k, L, idx, weights, scores);
    return hipGetLastError();
}

hipError_t launch_fwd_select(int dtype, const void *q, const void *keys, int64_t key_hstride,
                             int64_t T, int H, int n, int k, int d_k, int32_t *idx,
                             float *weights, float *scores, void *workspace, hipStream_t stream)
{
    if (select_fast_ok(dtype, n, k, d_k))
        return launch_select_fast(dtype, q, keys, key_hstride, T, H, n, k, d_k, idx, weights,
                                  scores, workspace, stream);
    if (dtype == 1)
        return launch_select_t<bf16_t>(q, keys, key_hstride, T, H, n, k, d_k, idx, weights,
                                       scores, stream);
    return launch_select_t<float>(q, keys, key_hstride, T, H, n, k, d_k, idx, weights, scores,
                                  stream);
}

}  // namespace pkm

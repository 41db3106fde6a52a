// pkm_backward.hip -- backward pass of the product-key memory layer
// (gptget.net summary of "Large Memory Layers with Product Keys",
// "Methodology": the layer is trained end to end by backprop, and only the
// selected memory slots are updated).  The selection is a constant of the
// backward pass; gradient reaches the k selected scores of each head, and from
// each score its left and right sub-key scores.
//
// bwd_value: one wave per token.  For each pick (h, r) the value row is
//   re-read once and serves both  dw = <dy[t], values[f]>  and the sparse
//   update  dvalues[f] += w * dy[t]  (float32 hardware atomics, lane-
//   contiguous 256-byte bursts).  dw goes to [T][H][k].
// bwd_query: one wave per (token, head), one lane per pick.  The softmax
//   backward ds_r = w_r (dw_r - sum_r' w_r' dw_r') only matters summed over the
//   picks S that share a sub-key i of one half; that sum is taken as
//       g_i = A * (1 - W) - B * W,  A = sum_S w dw, W = sum_S w,
//                                   B = sum_notS w dw, 1 - W = sum_notS w,
//   with both complements summed directly, so a sub-key shared by most picks
//   (its g is a near-cancelling sum) keeps full relative accuracy.  Then
//   dq = sum_i g_i * sub-key row i  and  dkeys[i] += g_i * q_half  (atomics).
#include "pkm_device.hpp"
#include "pkm_kernels.hpp"

namespace pkm {

constexpr int kBwdWaves = 4;

template <typename DT>
__device__ __forceinline__ float load_elem(const DT *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p, int64_t i)
{
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
}

// MCH: 16-byte chunks per lane covering the whole row; U: picks in flight.
template <typename DT, int MCH, int U>
__global__ __launch_bounds__(kBwdWaves *kWave) void bwd_value_kernel(
    const DT *__restrict__ values, const int32_t *__restrict__ idx,
    const float *__restrict__ weights, const DT *__restrict__ dy, float *__restrict__ dvalues,
    float *__restrict__ dw, int64_t T, int H, int k, int d_v)
{
    constexpr int EPC = Elt<DT>::per16;
    constexpr int NI = MCH * EPC;          // interleaved dy elements per lane (>= d_v / 64)
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * kBwdWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= T)
        return;
    const int nchunks = d_v / EPC;

    // dy[t] twice: 16-byte chunk layout for the dot products, and lane-interleaved
    // (element lane + 64*j) for contiguous atomics.
    float dyc[MCH][EPC];
    const uint4 *dyrow = reinterpret_cast<const uint4 *>(dy + t * d_v);
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
        const int c = lane + m * kWave;
        unpack16(c < nchunks ? dyrow[c] : make_uint4(0u, 0u, 0u, 0u), dyc[m]);
    }
    float dyi[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int x = lane + j * kWave;
        dyi[j] = x < d_v ? load_elem(dy, t * d_v + x) : 0.f;
    }

    for (int h = 0; h < H; ++h) {
        const int64_t base = (t * H + h) * (int64_t)k;
        float dw_mine = 0.f;                 // lane r keeps dw of pick r
        for (int r0 = 0; r0 < k; r0 += U) {
            uint4 buf[U][MCH];
            int64_t f[U];
            float w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool live = r0 + u < k;
                f[u] = live ? idx[base + r0 + u] : 0;
                w[u] = live ? weights[base + r0 + u] : 0.f;
                const uint4 *row = reinterpret_cast<const uint4 *>(values + f[u] * d_v);
#pragma unroll
                for (int m = 0; m < MCH; ++m) {
                    const int c = lane + m * kWave;
                    buf[u][m] = (live && c < nchunks) ? row[c] : make_uint4(0u, 0u, 0u, 0u);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < MCH; ++m) {
                    float v[EPC];
                    unpack16(buf[u][m], v);
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        part = fmaf(v[e], dyc[m][e], part);
                }
                const float dot = wave_sum(part);
                if (lane == r0 + u)
                    dw_mine = dot;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (r0 + u >= k)
                    break;
                float *drow = dvalues + f[u] * d_v;
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    const int x = lane + j * kWave;
                    if (x < d_v)
                        __hip_atomic_fetch_add(drow + x, w[u] * dyi[j], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (lane < k)
            dw[base + lane] = dw_mine;
    }
}

template <typename DT, int MCH, int U>
static hipError_t launch_bwd_value_t(const void *values, const int32_t *idx, const float *weights,
                                     const void *dy, float *dvalues, float *dw, int64_t T, int H,
                                     int k, int d_v, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kBwdWaves - 1) / kBwdWaves));
    hipLaunchKernelGGL((bwd_value_kernel<DT, MCH, U>), grid, dim3(kBwdWaves * kWave), 0, stream,
                       static_cast<const DT *>(values), idx, weights,
                       static_cast<const DT *>(dy), dvalues, dw, T, H, k, d_v);
    return hipGetLastError();
}

template <typename DT>
static hipError_t launch_bwd_value_dt(const void *values, const int32_t *idx, const float *weights,
                                      const void *dy, float *dvalues, float *dw, int64_t T, int H,
                                      int k, int d_v, hipStream_t stream)
{
    const int per_lane = (d_v / Elt<DT>::per16 + kWave - 1) / kWave;
    if (per_lane <= 1)
        return launch_bwd_value_t<DT, 1, 8>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
    if (per_lane <= 2)
        return launch_bwd_value_t<DT, 2, 4>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
    if (per_lane <= 4)
        return launch_bwd_value_t<DT, 4, 2>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
    if (per_lane <= 8)
        return launch_bwd_value_t<DT, 8, 1>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
    return launch_bwd_value_t<DT, 16, 1>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
}

hipError_t launch_bwd_value(int dtype, const void *values, const int32_t *idx,
                            const float *weights, const void *dy, float *dvalues, float *dw,
                            int64_t T, int H, int k, int d_v, hipStream_t stream)
{
    if (dtype == 1)
        return launch_bwd_value_dt<bf16_t>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
    return launch_bwd_value_dt<float>(values, idx, weights, dy, dvalues, dw, T, H, k, d_v, stream);
}

// ---------------------------------------------------------------------------
constexpr int kMaxHalfPerLane = 8;   // half <= 512

template <typename DT>
__global__ __launch_bounds__(kBwdWaves *kWave) void bwd_query_kernel(
    const DT *__restrict__ q, const DT *__restrict__ keys, const int32_t *__restrict__ idx,
    const float *__restrict__ weights, const float *__restrict__ dw, float *__restrict__ dq,
    float *__restrict__ dkeys, int64_t T, int H, int n, int k, int d_k)
{
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * kBwdWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (row >= T * H)
        return;
    const int64_t t = row / H;
    const int h = (int)(row % H);
    const int half = d_k / 2;
    const int64_t base = row * (int64_t)k;
    const int f = lane < k ? idx[base + lane] : 0;
    const float w_mine = lane < k ? weights[base + lane] : 0.f;
    const float wdw_mine = lane < k ? w_mine * dw[base + lane] : 0.f;

    for (int s = 0; s < 2; ++s) {
        const int sub = s == 0 ? f / n : f % n;
        // sums over the picks sharing this lane's sub-key (A, W) and over the
        // rest (B, Wc); the first pick of each sub-key carries its g
        float A = 0.f, W = 0.f, B = 0.f, Wc = 0.f;
        bool first = lane < k;
        for (int r = 0; r < k; ++r) {
            const int sub_r = __shfl(sub, r);
            const float w_r = __shfl(w_mine, r);
            const float wdw_r = __shfl(wdw_mine, r);
            if (sub_r == sub) {
                A += wdw_r;
                W += w_r;
                if (r < lane)
                    first = false;
            } else {
                B += wdw_r;
                Wc += w_r;
            }
        }
        const float g = A * Wc - B * W;
        const DT *qh = q + row * (int64_t)d_k + (int64_t)s * half;
        const DT *kb = keys + ((int64_t)h * 2 + s) * (int64_t)n * half;
        float *dkb = dkeys + ((int64_t)h * 2 + s) * (int64_t)n * half;
        float qv[kMaxHalfPerLane], acc[kMaxHalfPerLane];
#pragma unroll
        for (int j = 0; j < kMaxHalfPerLane; ++j) {
            const int c = lane + j * kWave;
            qv[j] = c < half ? load_elem(qh, c) : 0.f;
            acc[j] = 0.f;
        }
        uint64_t todo = __ballot(first);
        while (todo) {
            const int r = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int sub_r = __shfl(sub, r);
            const float g_r = __shfl(g, r);
            const DT *krow = kb + (int64_t)sub_r * half;
            float *dkrow = dkb + (int64_t)sub_r * half;
#pragma unroll
            for (int j = 0; j < kMaxHalfPerLane; ++j) {
                const int c = lane + j * kWave;
                if (c < half) {
                    acc[j] = fmaf(g_r, load_elem(krow, c), acc[j]);
                    __hip_atomic_fetch_add(dkrow + c, g_r * qv[j], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        float *dqh = dq + row * (int64_t)d_k + (int64_t)s * half;
#pragma unroll
        for (int j = 0; j < kMaxHalfPerLane; ++j) {
            const int c = lane + j * kWave;
            if (c < half)
                dqh[c] = acc[j];
        }
    }
}

template <typename DT>
static hipError_t launch_bwd_query_t(const void *q, const void *keys, const int32_t *idx,
                                     const float *weights, const float *dw, float *dq,
                                     float *dkeys, int64_t T, int H, int n, int k, int d_k,
                                     hipStream_t stream)
{
    const int64_t rows = T * H;
    const dim3 grid((unsigned)((rows + kBwdWaves - 1) / kBwdWaves));
    hipLaunchKernelGGL(bwd_query_kernel<DT>, grid, dim3(kBwdWaves * kWave), 0, stream,
                       static_cast<const DT *>(q), static_cast<const DT *>(keys), idx, weights,
                       dw, dq, dkeys, T, H, n, k, d_k);
    return hipGetLastError();
}

hipError_t launch_bwd_query(int dtype, const void *q, const void *keys, const int32_t *idx,
                            const float *weights, const float *dw, float *dq, float *dkeys,
                            int64_t T, int H, int n, int k, int d_k, hipStream_t stream)
{
    if (dtype == 1)
        return launch_bwd_query_t<bf16_t>(q, keys, idx, weights, dw, dq, dkeys, T, H, n, k, d_k, stream);
    return launch_bwd_query_t<float>(q, keys, idx, weights, dw, dq, dkeys, T, H, n, k, d_k, stream);
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

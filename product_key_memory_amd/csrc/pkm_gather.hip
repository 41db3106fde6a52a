// pkm_gather.hip -- forward read of the memory: y[t] = sum over the H*k picks
// of token t of weight * values[slot] (gptget.net summary of "Large Memory
// Layers with Product Keys", "Methodology": the output is the weighted sum of
// the selected value vectors, combined over the heads).
//
// HBM-bound row gather.  One wave per (token, slice of the row): each lane owns
// MCH 16-byte chunks of the slice, U picks are loaded before any is consumed
// so U*MCH 16-byte loads per lane are in flight, and the sum is kept in
// float32 registers; the result is rounded once on store.
#include "pkm_device.hpp"
#include "pkm_kernels.hpp"

namespace pkm {

constexpr int kGatherWaves = 4;

template <typename DT, int MCH, int U>
__global__ __launch_bounds__(kGatherWaves *kWave) void fwd_gather_kernel(
    const DT *__restrict__ values, const int32_t *__restrict__ idx,
    const float *__restrict__ weights, DT *__restrict__ y, int64_t T, int HK, int d_v)
{
    constexpr int EPC = Elt<DT>::per16;      // elements per 16-byte chunk
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * kGatherWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= T)
        return;
    const int nchunks = d_v / EPC;
    const int c_base = blockIdx.y * (kWave * MCH) + lane;

    float acc[MCH][EPC];
#pragma unroll
    for (int m = 0; m < MCH; ++m)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            acc[m][e] = 0.f;

    const int32_t *it = idx + t * HK;
    const float *wt = weights + t * HK;
    for (int p0 = 0; p0 < HK; p0 += U) {
        uint4 buf[U][MCH];
        float wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = p0 + u < HK;
            const int64_t f = live ? it[p0 + u] : 0;
            wv[u] = live ? wt[p0 + u] : 0.f;
            const uint4 *row = reinterpret_cast<const uint4 *>(values + f * d_v);
#pragma unroll
            for (int m = 0; m < MCH; ++m) {
                const int c = c_base + m * kWave;
                buf[u][m] = (live && c < nchunks) ? row[c] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MCH; ++m) {
                float v[EPC];
                unpack16(buf[u][m], v);
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    acc[m][e] = fmaf(wv[u], v[e], acc[m][e]);
            }
        }
    }

    uint4 *yrow = reinterpret_cast<uint4 *>(y + t * d_v);
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
        const int c = c_base + m * kWave;
        if (c >= nchunks)
            continue;
        uint4 o;
        if constexpr (EPC == 8) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = f32_to_bf16_bits(acc[m][2 * i]) | (f32_to_bf16_bits(acc[m][2 * i + 1]) << 16);
            o = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            o = make_uint4(__float_as_uint(acc[m][0]), __float_as_uint(acc[m][1]),
                           __float_as_uint(acc[m][2]), __float_as_uint(acc[m][3]));
        }
        yrow[c] = o;
    }
}

template <typename DT, int MCH, int U>
static hipError_t launch_gather_t(const void *values, const int32_t *idx, const float *weights,
                                  void *y, int64_t T, int HK, int d_v, hipStream_t stream)
{
    const int nchunks = d_v / Elt<DT>::per16;
    const int slices = (nchunks + kWave * MCH - 1) / (kWave * MCH);
    const dim3 grid((unsigned)((T + kGatherWaves - 1) / kGatherWaves), (unsigned)slices);
    hipLaunchKernelGGL((fwd_gather_kernel<DT, MCH, U>), grid, dim3(kGatherWaves * kWave), 0,
                       stream, static_cast<const DT *>(values), idx, weights,
                       static_cast<DT *>(y), T, HK, d_v);
    return hipGetLastError();
}

template <typename DT>
static hipError_t launch_gather_dt(const void *values, const int32_t *idx, const float *weights,
                                   void *y, int64_t T, int HK, int d_v, hipStream_t stream)
{
    const int per_lane = (d_v / Elt<DT>::per16 + kWave - 1) / kWave;
    if (per_lane <= 1)
        return launch_gather_t<DT, 1, 8>(values, idx, weights, y, T, HK, d_v, stream);
    if (per_lane <= 2)
        return launch_gather_t<DT, 2, 8>(values, idx, weights, y, T, HK, d_v, stream);
    return launch_gather_t<DT, 4, 4>(values, idx, weights, y, T, HK, d_v, stream);
}

hipError_t launch_fwd_gather(int dtype, const void *values, const int32_t *idx,
                             const float *weights, void *y, int64_t T, int HK, int d_v,
                             hipStream_t stream)
{
    if (dtype == 1)
        return launch_gather_dt<bf16_t>(values, idx, weights, y, T, HK, d_v, stream);
    return launch_gather_dt<float>(values, idx, weights, y, T, HK, d_v, stream);
}

}  // namespace pkm

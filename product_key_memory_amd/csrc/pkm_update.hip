// pkm_update.hip -- what follows the backward on the value table: the sparse
// update of the selected memory slots and the slot-usage counter (gptget.net
// summary of "Large Memory Layers with Product Keys": "Methodology", the
// layer is trained with sparse updates, only the selected slots change;
// "Key Results", the share of memory slots in use).  Both read the slot sort
// (slot_start, from pkm_slot_sort): a slot is touched in this batch iff its
// run slot_start[f] .. slot_start[f+1] is not empty.
#include "pkm_device.hpp"
#include "pkm_update.hpp"

namespace pkm {

constexpr int kUpdWaves = 4;

// Row access of the value table in 16-byte chunks (EPC elements each).
__device__ __forceinline__ void upd_unpack(const uint4 &raw, float (&x)[8])
{
    unpack16(raw, x);
}
__device__ __forceinline__ uint4 upd_pack(const float (&x)[8])
{
    uint4 r;
    r.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
    r.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
    r.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
    r.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
    return r;
}

// One wave per slot; rows no pick selected are left as they are.  SGD:
// w = fma(-lr, g, w).  Adam with moments kept only for touched rows ("lazy"):
// m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
// w = w - lr (m / c1) / (sqrt(v / c2) + eps), c1 = 1 - b1^t, c2 = 1 - b2^t.
// Each float32 result is rounded once to the storage type.
template <typename DT, bool ADAM>
__global__ __launch_bounds__(kUpdWaves *kWave) void sparse_update_kernel(
    DT *__restrict__ values, const float *__restrict__ dvalues, const int32_t *__restrict__ start,
    float *__restrict__ m1, float *__restrict__ m2, int64_t slots, int d_v, UpdateParams prm)
{
    const int lane = lane_id();
    const int64_t f = (int64_t)blockIdx.x * kUpdWaves + threadIdx.x / kWave;
    if (f >= slots || start[f + 1] == start[f])
        return;
    // 8 elements per step: one 16-byte chunk of a bf16 row, two of a float32
    // row; a lane's steps are all loaded before the first is updated
    const int64_t row = f * d_v;
    // d_v <= 2 * 8 * 64 = 1024 in one pass (wider rows take more passes);
    // four steps a pass held registers for d_v = 2048 and cut the occupancy
    constexpr int kMaxSteps = 2;
    for (int base = 0; base < d_v; base += kMaxSteps * 8 * kWave) {
        float w[kMaxSteps][8], g[kMaxSteps][8];
#pragma unroll
        for (int st = 0; st < kMaxSteps; ++st) {
            const int e0 = base + 8 * (lane + st * kWave);
            if (e0 >= d_v)
                continue;
            const float4 *gs = reinterpret_cast<const float4 *>(dvalues + row + e0);
            const float4 g0 = gs[0], g1 = gs[1];
            g[st][0] = g0.x; g[st][1] = g0.y; g[st][2] = g0.z; g[st][3] = g0.w;
            g[st][4] = g1.x; g[st][5] = g1.y; g[st][6] = g1.z; g[st][7] = g1.w;
            if constexpr (sizeof(DT) == 2) {
                upd_unpack(*reinterpret_cast<const uint4 *>(values + row + e0), w[st]);
            } else {
                const float4 *ws = reinterpret_cast<const float4 *>(values + row + e0);
                const float4 w0 = ws[0], w1 = ws[1];
                w[st][0] = w0.x; w[st][1] = w0.y; w[st][2] = w0.z; w[st][3] = w0.w;
                w[st][4] = w1.x; w[st][5] = w1.y; w[st][6] = w1.z; w[st][7] = w1.w;
            }
        }
#pragma unroll
        for (int st = 0; st < kMaxSteps; ++st) {
            const int e0 = base + 8 * (lane + st * kWave);
            if (e0 >= d_v)
                continue;
            if constexpr (ADAM) {
                float4 *ma = reinterpret_cast<float4 *>(m1 + row + e0);
                float4 *va = reinterpret_cast<float4 *>(m2 + row + e0);
                float m[8], v[8];
                const float4 ma0 = ma[0], ma1 = ma[1], va0 = va[0], va1 = va[1];
                m[0] = ma0.x; m[1] = ma0.y; m[2] = ma0.z; m[3] = ma0.w;
                m[4] = ma1.x; m[5] = ma1.y; m[6] = ma1.z; m[7] = ma1.w;
                v[0] = va0.x; v[1] = va0.y; v[2] = va0.z; v[3] = va0.w;
                v[4] = va1.x; v[5] = va1.y; v[6] = va1.z; v[7] = va1.w;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    m[i] = prm.b1 * m[i] + (1.f - prm.b1) * g[st][i];
                    v[i] = prm.b2 * v[i] + (1.f - prm.b2) * (g[st][i] * g[st][i]);
                    const float step = (m[i] / prm.c1) / (sqrtf(v[i] / prm.c2) + prm.eps);
                    w[st][i] = fmaf(-prm.lr, step, w[st][i]);
                }
                ma[0] = make_float4(m[0], m[1], m[2], m[3]);
                ma[1] = make_float4(m[4], m[5], m[6], m[7]);
                va[0] = make_float4(v[0], v[1], v[2], v[3]);
                va[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    w[st][i] = fmaf(-prm.lr, g[st][i], w[st][i]);
            }
            if constexpr (sizeof(DT) == 2) {
                *reinterpret_cast<uint4 *>(values + row + e0) = upd_pack(w[st]);
            } else {
                float4 *ws = reinterpret_cast<float4 *>(values + row + e0);
                ws[0] = make_float4(w[st][0], w[st][1], w[st][2], w[st][3]);
                ws[1] = make_float4(w[st][4], w[st][5], w[st][6], w[st][7]);
            }
        }
    }
}

// counts[f] += the run length of slot f; *used += slots with a non-zero count
// (one atomic per workgroup; *used is cleared first by a one-thread kernel).
constexpr int kUsageThreads = 256;
constexpr int kUsagePer = 4;        // slots per thread

__global__ void usage_clear_kernel(unsigned long long *used)
{
    if (threadIdx.x == 0)
        *used = 0ull;
}

__global__ __launch_bounds__(kUsageThreads) void usage_kernel(const int32_t *__restrict__ start,
                                                              int64_t *__restrict__ counts,
                                                              int64_t slots,
                                                              unsigned long long *__restrict__ used)
{
    __shared__ int part[kUsageThreads / kWave];
    const int64_t base = ((int64_t)blockIdx.x * kUsageThreads + threadIdx.x) * kUsagePer;
    int nz = 0;
#pragma unroll
    for (int i = 0; i < kUsagePer; ++i) {
        const int64_t f = base + i;
        if (f < slots) {
            const int64_t c = counts[f] + (start[f + 1] - start[f]);
            counts[f] = c;
            nz += c != 0 ? 1 : 0;
        }
    }
    if (!used)
        return;
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1)
        nz += __shfl_xor(nz, mask);
    if (lane_id() == 0)
        part[threadIdx.x / kWave] = nz;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
        for (int w = 0; w < kUsageThreads / kWave; ++w)
            total += part[w];
        atomicAdd(used, (unsigned long long)total);
    }
}

hipError_t launch_sparse_update(int dtype, void *values, const float *dvalues,
                                const int32_t *slot_start, float *m1, float *m2, int64_t slots,
                                int d_v, bool adam, const UpdateParams &prm, hipStream_t stream)
{
    const dim3 grid((unsigned)((slots + kUpdWaves - 1) / kUpdWaves)), block(kUpdWaves * kWave);
    if (dtype == 1) {
        bf16_t *v = static_cast<bf16_t *>(values);
        if (adam)
            hipLaunchKernelGGL((sparse_update_kernel<bf16_t, true>), grid, block, 0, stream, v,
                               dvalues, slot_start, m1, m2, slots, d_v, prm);
        else
            hipLaunchKernelGGL((sparse_update_kernel<bf16_t, false>), grid, block, 0, stream, v,
                               dvalues, slot_start, m1, m2, slots, d_v, prm);
    } else {
        float *v = static_cast<float *>(values);
        if (adam)
            hipLaunchKernelGGL((sparse_update_kernel<float, true>), grid, block, 0, stream, v,
                               dvalues, slot_start, m1, m2, slots, d_v, prm);
        else
            hipLaunchKernelGGL((sparse_update_kernel<float, false>), grid, block, 0, stream, v,
                               dvalues, slot_start, m1, m2, slots, d_v, prm);
    }
    return hipGetLastError();
}

hipError_t launch_slot_usage(const int32_t *slot_start, int64_t *counts, int64_t slots,
                             int64_t *used, hipStream_t stream)
{
    unsigned long long *u = reinterpret_cast<unsigned long long *>(used);
    if (u) {
        hipLaunchKernelGGL(usage_clear_kernel, dim3(1), dim3(64), 0, stream, u);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    const int64_t per_block = (int64_t)kUsageThreads * kUsagePer;
    hipLaunchKernelGGL(usage_kernel, dim3((unsigned)((slots + per_block - 1) / per_block)),
                       dim3(kUsageThreads), 0, stream, slot_start, counts, slots, u);
    return hipGetLastError();
}

}  // namespace pkm

// pkm_query.hip -- the query network in front of the memory layer (gptget.net
// summary of "Large Memory Layers with Product Keys", "Deep Analysis",
// methodology list: the input x goes through the query network, which gives
// q; "Key Results": batch normalization in the query network raises memory
// utilization): q = BN(x W^T), one bias-free projection followed by batch
// normalization of every output feature over the batch's tokens (batch
// statistics, biased variance, optional affine gamma, beta), and its backward.
//
// Kernels:
//   gemm_kernel        C[M][N] (fp32) = sum_k A(m, k) B(n, k) on MFMA, 128 x 128
//                      tiles, 32-wide K steps staged in double-buffered LDS
//                      tiles with XOR-swizzled 16-byte chunks; A and B may be
//                      stored K-contiguous or M/N-contiguous (transposed while
//                      staging).  bf16 operands use v_mfma_f32_16x16x32_bf16
//                      (a float32 A is split into bf16 hi + lo, two MFMAs);
//                      float32 storage uses v_mfma_f32_16x16x4_f32.
//   bn_partial_kernel  per (row chunk, column): count, mean, M2 (Welford over
//                      the chunk's rows, merged across waves by Chan's rule)
//   bn_finalize_kernel per column: merge the chunks -> mean, rstd
//   bn_apply_kernel    q = gamma (z - mean) rstd + beta, rounded once
//   bn_bwd_*           the batch-norm backward (column sums of dq and
//                      dq * zhat, then dz), followed by two GEMMs:
//                      dx = dz W and dW = dz^T x.
#include "pkm_device.hpp"
#include "pkm_query.hpp"

#include <type_traits>

namespace pkm {

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------
constexpr int kGBM = 128, kGBN = 128, kGBK = 32;
constexpr int kGThreads = 256;

enum GemmMode { kBf16 = 0, kBf16SplitA = 1, kF32 = 2 };

template <int MODE> struct GTile;
template <> struct GTile<kBf16> { typedef uint16_t E; static constexpr int C = 4; static constexpr int parts = 1; };
template <> struct GTile<kBf16SplitA> { typedef uint16_t E; static constexpr int C = 4; static constexpr int parts = 2; };
template <> struct GTile<kF32> { typedef float E; static constexpr int C = 8; static constexpr int parts = 1; };

// element offset of (row, k) in a [rows][32] tile whose 16-byte chunks are
// XOR-swizzled by row (the 16 rows an MFMA operand read touches hit distinct banks)
template <int C>
__device__ __forceinline__ int g_cell(int row, int k)
{
    constexpr int EPC = kGBK / C;
    return row * kGBK + (((k / EPC) ^ ((row / (16 / C)) % C)) * EPC) + k % EPC;
}

// One operand's staging: T elements, stored K-contiguous (KMAJ = false: [R][K])
// or R-contiguous (KMAJ = true: [K][R]); R = the operand's M or N.  Each
// thread moves 16-byte pieces (8 bf16 or 4 float32); K-contiguous pieces go
// to LDS whole (one 16- or 8-byte store), R-contiguous ones are transposed
// element by element.
template <typename T> struct GRaw;
template <> struct GRaw<bf16_t> { static constexpr int V = 8; };
template <> struct GRaw<float> { static constexpr int V = 4; };

template <typename T, bool KMAJ, int MODE, bool SPLIT>
struct GStage {
    static constexpr int V = GRaw<T>::V;                    // elements per 16-byte load
    static constexpr int loads = kGBM * kGBK / V / kGThreads;
    uint4 raw[loads];
    __device__ static void coords(int u, int &r, int &k)
    {
        if (!KMAJ) {        // V consecutive k of one row
            r = u / (kGBK / V);
            k = (u % (kGBK / V)) * V;
        } else {            // V consecutive rows of one k
            k = u / (kGBM / V);
            r = (u % (kGBM / V)) * V;
        }
    }
    __device__ void load(const T *__restrict__ src, int64_t ld, int r0, int R, int k0, int K, int tid)
    {
#pragma unroll
        for (int l = 0; l < loads; ++l) {
            int r, k;
            coords(tid + l * kGThreads, r, k);
            const int gr = r0 + r, gk = k0 + k;
            raw[l] = (gr < R && gk < K)
                         ? *reinterpret_cast<const uint4 *>(!KMAJ ? src + (int64_t)gr * ld + gk
                                                                  : src + (int64_t)gk * ld + gr)
                         : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ void store(typename GTile<MODE>::E *hi, typename GTile<MODE>::E *lo, int tid) const
    {
        constexpr int C = GTile<MODE>::C;
#pragma unroll
        for (int l = 0; l < loads; ++l) {
            int r, k;
            coords(tid + l * kGThreads, r, k);
            if constexpr (!KMAJ && (MODE == kF32 || (sizeof(T) == 2 && !SPLIT))) {
                // a whole chunk (8 bf16 / 4 float32) in place
                *reinterpret_cast<uint4 *>(hi + g_cell<C>(r, k)) = raw[l];
            } else if constexpr (!KMAJ && SPLIT) {
                // 4 float32 -> 4 bf16 hi + 4 bf16 lo, half a chunk each
                const uint32_t w[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
                uint32_t h[4], o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = __uint_as_float(w[e]);
                    h[e] = f32_to_bf16_bits(f);
                    o[e] = f32_to_bf16_bits(f - bf16_to_f32(h[e]));
                }
                *reinterpret_cast<uint2 *>(hi + g_cell<C>(r, k)) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                *reinterpret_cast<uint2 *>(lo + g_cell<C>(r, k)) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
            } else {
                float x[V];
                if constexpr (V == 8)
                    unpack16(raw[l], x);
                else {
                    x[0] = __uint_as_float(raw[l].x); x[1] = __uint_as_float(raw[l].y);
                    x[2] = __uint_as_float(raw[l].z); x[3] = __uint_as_float(raw[l].w);
                }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const int at = g_cell<C>(KMAJ ? r + e : r, KMAJ ? k : k + e);
                    if constexpr (MODE == kF32) {
                        hi[at] = x[e];
                    } else {
                        const uint32_t hb = f32_to_bf16_bits(x[e]);
                        hi[at] = (uint16_t)hb;
                        if constexpr (SPLIT)
                            lo[at] = (uint16_t)f32_to_bf16_bits(x[e] - bf16_to_f32(hb));
                    }
                }
            }
        }
    }
};

// blockIdx.z = a slice of K (split-K): slice z covers [z k_slice, (z+1) k_slice)
// and writes its own C at Cm + z M N.
template <typename TA, typename TB, bool A_KM, bool B_KN, int MODE>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(const TA *__restrict__ A,
                                                         const TB *__restrict__ B,
                                                         float *__restrict__ Cm, int M, int N,
                                                         int K, int64_t lda, int64_t ldb,
                                                         int k_slice)
{
    typedef typename GTile<MODE>::E E;
    constexpr int C = GTile<MODE>::C;
    constexpr int PA = GTile<MODE>::parts;
    constexpr int TILE = kGBM * kGBK;
    __shared__ __align__(16) E lds[2][(PA + 1) * TILE];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int m0 = blockIdx.y * kGBM, n0 = blockIdx.x * kGBN;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
    const int r16 = lane & 15, kg = lane >> 4;

    GStage<TA, A_KM, MODE, MODE == kBf16SplitA> sa;
    GStage<TB, B_KN, MODE, false> sb;
    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int kb = blockIdx.z * k_slice;
    const int ke = kb + k_slice < K ? kb + k_slice : K;
    Cm += (int64_t)blockIdx.z * M * N;
    const int nk = (ke - kb + kGBK - 1) / kGBK;
    sa.load(A, lda, m0, M, kb, ke, tid);
    sb.load(B, ldb, n0, N, kb, ke, tid);
    sa.store(lds[0], lds[0] + TILE, tid);
    sb.store(lds[0] + PA * TILE, nullptr, tid);
    __syncthreads();
    for (int c = 0; c < nk; ++c) {
        if (c + 1 < nk) {
            sa.load(A, lda, m0, M, kb + (c + 1) * kGBK, ke, tid);
            sb.load(B, ldb, n0, N, kb + (c + 1) * kGBK, ke, tid);
        }
        const E *ah = lds[c & 1], *al = lds[c & 1] + TILE, *bt = lds[c & 1] + PA * TILE;
        if constexpr (MODE == kF32) {
            float4 a[4][2], b[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm + 16 * i + r16;
                a[i][0] = *reinterpret_cast<const float4 *>(ah + g_cell<C>(row, 4 * kg));
                a[i][1] = *reinterpret_cast<const float4 *>(ah + g_cell<C>(row, 4 * kg + 16));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn + 16 * j + r16;
                b[j][0] = *reinterpret_cast<const float4 *>(bt + g_cell<C>(row, 4 * kg));
                b[j][1] = *reinterpret_cast<const float4 *>(bt + g_cell<C>(row, 4 * kg + 16));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][h].x, b[j][h].x, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][h].y, b[j][h].y, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][h].z, b[j][h].z, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][h].w, b[j][h].w, acc[i][j], 0, 0, 0);
                    }
        } else {
            uint4 a[4][PA], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm + 16 * i + r16;
                a[i][0] = *reinterpret_cast<const uint4 *>(ah + g_cell<C>(row, 8 * kg));
                if constexpr (PA == 2)
                    a[i][PA - 1] = *reinterpret_cast<const uint4 *>(al + g_cell<C>(row, 8 * kg));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const uint4 *>(bt + g_cell<C>(wn + 16 * j + r16, 8 * kg));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int pa = 0; pa < PA; ++pa)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[i][pa]), __builtin_bit_cast(bf16x8, b[j]),
                            acc[i][j], 0, 0, 0);
        }
        if (c + 1 < nk) {
            E *dst = lds[(c + 1) & 1];
            sa.store(dst, dst + TILE, tid);
            sb.store(dst + PA * TILE, nullptr, tid);
        }
        __syncthreads();
    }
    // lane holds D rows 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + 16 * j + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm + 16 * i + 4 * kg + e;
                if (row < M && col < N)
                    Cm[(int64_t)row * N + col] = acc[i][j][e];
            }
        }
}

// C = A B^T with both operands K-contiguous unless A_KM / B_KN.  With
// splits > 1 the K range is cut into `splits` slices whose partial products
// go to `parts` ([splits][M][N]) and are then summed into C.
__global__ void sum_slices_kernel(const float *__restrict__ parts, int splits, int64_t count,
                                  float *__restrict__ C)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float a = 0.f;
        for (int z = 0; z < splits; ++z)
            a += parts[(int64_t)z * count + i];
        C[i] = a;
    }
}

template <typename TA, typename TB, bool A_KM, bool B_KN, int MODE>
static hipError_t gemm(const TA *A, const TB *B, float *Cm, int M, int N, int K, int64_t lda,
                       int64_t ldb, hipStream_t stream, int splits = 1, float *parts = nullptr)
{
    int k_slice = K;
    if (splits > 1) {
        k_slice = (K + splits - 1) / splits;
        k_slice = (k_slice + kGBK - 1) / kGBK * kGBK;
        splits = (K + k_slice - 1) / k_slice;
    }
    const dim3 grid((unsigned)((N + kGBN - 1) / kGBN), (unsigned)((M + kGBM - 1) / kGBM),
                    (unsigned)splits);
    hipLaunchKernelGGL((gemm_kernel<TA, TB, A_KM, B_KN, MODE>), grid, dim3(kGThreads), 0, stream,
                       A, B, splits > 1 ? parts : Cm, M, N, K, lda, ldb, k_slice);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || splits <= 1)
        return err;
    const int64_t count = (int64_t)M * N;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256),
                       0, stream, parts, splits, count, Cm);
    return hipGetLastError();
}

// out[c][r] = in[r][c] for an R x C matrix of 2- or 4-byte elements, through
// 64 x 64 LDS tiles (both sides coalesced); out rows have pitch ldo >= R and
// their tail r in [R, ldo) is written with zeros.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ in, E *__restrict__ out,
                                                        int64_t R, int64_t C, int64_t ldo)
{
    __shared__ E tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        tile[i][tx] = (r < R && c < C) ? in[r * C + c] : (E)0;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (r < ldo && c < C)
            out[c * ldo + r] = tile[tx][i];
    }
}

// K of the GEMM that runs over the tokens (dW = dz^T x): the token count
// rounded up to 8, so that every 16-byte piece of a transposed row (8 bf16 or
// 4 float32 elements) lies inside the row and is 16-byte aligned; the padding
// holds zeros.
static int64_t token_pitch(int64_t T)
{
    return (T + 7) & ~(int64_t)7;
}

template <typename E>
static hipError_t transpose(const E *in, E *out, int64_t R, int64_t C, hipStream_t stream,
                            int64_t ldo = -1)
{
    if (ldo < 0)
        ldo = R;
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((ldo + 63) / 64));
    hipLaunchKernelGGL((transpose_kernel<E>), grid, dim3(256), 0, stream, in, out, R, C, ldo);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// batch normalization over the tokens, per output feature
// ---------------------------------------------------------------------------
constexpr int kBnCols = 64;         // columns per workgroup (one per lane)
constexpr int kBnWaves = 4;

// Welford over this thread's rows, then Chan's merge across the 4 waves.
__global__ __launch_bounds__(kBnWaves *kWave) void bn_partial_kernel(const float *__restrict__ z,
                                                                      int64_t T, int D,
                                                                      int64_t rows_per_chunk,
                                                                      float *__restrict__ part)
{
    __shared__ float sh[3][kBnWaves][kBnCols];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int col = blockIdx.x * kBnCols + lane;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < T ? r0 + rows_per_chunk : T;
    float n = 0.f, mean = 0.f, m2 = 0.f;
    if (col < D)
        for (int64_t r = r0 + wave; r < r1; r += kBnWaves) {
            const float x = z[r * D + col];
            n += 1.f;
            const float d = x - mean;
            mean += d / n;
            m2 += d * (x - mean);
        }
    sh[0][wave][lane] = n;
    sh[1][wave][lane] = mean;
    sh[2][wave][lane] = m2;
    __syncthreads();
    if (wave == 0 && col < D) {
        float N = sh[0][0][lane], M = sh[1][0][lane], S = sh[2][0][lane];
        for (int w = 1; w < kBnWaves; ++w) {
            const float nb = sh[0][w][lane];
            if (nb == 0.f)
                continue;
            const float nt = N + nb, d = sh[1][w][lane] - M;
            M += d * (nb / nt);
            S += sh[2][w][lane] + d * d * (N * nb / nt);
            N = nt;
        }
        float *p = part + ((int64_t)blockIdx.y * D + col) * 3;
        p[0] = N;
        p[1] = M;
        p[2] = S;
    }
}

// Chan's merge of (count, mean, M2) b into a, in double.
__device__ __forceinline__ void chan_merge(double &N, double &M, double &S, double nb, double mb,
                                           double sb)
{
    if (nb == 0.0)
        return;
    const double nt = N + nb, d = mb - M;
    M += d * (nb / nt);
    S += sb + d * d * (N * nb / nt);
    N = nt;
}

// One wave per column: lane l merges chunks l, l + 64, ..., then a butterfly
// merges the lanes.
__global__ void bn_finalize_kernel(const float *__restrict__ part, int chunks, int D, float eps,
                                   float *__restrict__ mean_out, float *__restrict__ rstd_out)
{
    const int lane = lane_id();
    const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (col >= D)
        return;
    double N = 0.0, M = 0.0, S = 0.0;
    for (int c = lane; c < chunks; c += kWave) {
        const float *p = part + ((int64_t)c * D + col) * 3;
        chan_merge(N, M, S, p[0], p[1], p[2]);
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const double nb = __shfl_xor(N, m), mb = __shfl_xor(M, m), sb = __shfl_xor(S, m);
        chan_merge(N, M, S, nb, mb, sb);
    }
    if (lane == 0) {
        const double var = N > 0.0 ? S / N : 0.0;
        mean_out[col] = (float)M;
        rstd_out[col] = (float)(1.0 / sqrt(var + (double)eps));
    }
}

// q = gamma (z - mean) rstd + beta, rounded once.  A thread owns 4 columns
// (blockIdx.x picks 1024 of them) and walks the rows blockIdx.y, + gridDim.y,
// ...: its columns' constants are loaded once.
constexpr int kBnApplyRows = 2048;      // gridDim.y at most

template <typename DT>
__global__ void bn_apply_kernel(const float *__restrict__ z, int64_t T, int D,
                                const float *__restrict__ mean, const float *__restrict__ rstd,
                                const float *__restrict__ gamma, const float *__restrict__ beta,
                                DT *__restrict__ q)
{
    const int c = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (c >= D)
        return;
    float a[4], o[4];        // y = a x + o with a = gamma rstd, o = beta - a mean
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float g = gamma ? gamma[c + e] : 1.f, b = beta ? beta[c + e] : 0.f;
        a[e] = g;
        o[e] = b;
    }
    float mu[4], rs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mu[e] = mean[c + e];
        rs[e] = rstd[c + e];
    }
    for (int64_t r = blockIdx.y; r < T; r += gridDim.y) {
        const float4 v = *reinterpret_cast<const float4 *>(z + r * D + c);
        const float x[4] = {v.x, v.y, v.z, v.w};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = fmaf(a[e], (x[e] - mu[e]) * rs[e], o[e]);
        if constexpr (sizeof(DT) == 2) {
            uint2 w;
            w.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
            w.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
            *reinterpret_cast<uint2 *>(q + r * D + c) = w;
        } else {
            *reinterpret_cast<float4 *>(q + r * D + c) = make_float4(y[0], y[1], y[2], y[3]);
        }
    }
}

// Backward sums per (row chunk, column): sum dq and sum dq * zhat.
__global__ __launch_bounds__(kBnWaves *kWave) void bn_bwd_partial_kernel(
    const float *__restrict__ z, const float *__restrict__ dq, int64_t T, int D,
    const float *__restrict__ mean, const float *__restrict__ rstd, int64_t rows_per_chunk,
    float *__restrict__ part)
{
    __shared__ float sh[2][kBnWaves][kBnCols];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int col = blockIdx.x * kBnCols + lane;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r1 = r0 + rows_per_chunk < T ? r0 + rows_per_chunk : T;
    float s1 = 0.f, s2 = 0.f;
    if (col < D) {
        const float mu = mean[col], rs = rstd[col];
        for (int64_t r = r0 + wave; r < r1; r += kBnWaves) {
            const float g = dq[r * D + col];
            s1 += g;
            s2 += g * ((z[r * D + col] - mu) * rs);
        }
    }
    sh[0][wave][lane] = s1;
    sh[1][wave][lane] = s2;
    __syncthreads();
    if (wave == 0 && col < D) {
        float a = 0.f, b = 0.f;
        for (int w = 0; w < kBnWaves; ++w) {
            a += sh[0][w][lane];
            b += sh[1][w][lane];
        }
        float *p = part + ((int64_t)blockIdx.y * D + col) * 2;
        p[0] = a;
        p[1] = b;
    }
}

// dbeta = sum dq, dgamma = sum dq * zhat; coef = (sum dq / T, sum dq zhat / T).
// One wave per column: lanes sum the chunks in double, then a butterfly.
__global__ void bn_bwd_finalize_kernel(const float *__restrict__ part, int chunks, int D,
                                       int64_t T, float *__restrict__ coef,
                                       float *__restrict__ dgamma, float *__restrict__ dbeta)
{
    const int lane = lane_id();
    const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (col >= D)
        return;
    double a = 0.0, b = 0.0;
    for (int c = lane; c < chunks; c += kWave) {
        a += part[((int64_t)c * D + col) * 2];
        b += part[((int64_t)c * D + col) * 2 + 1];
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        a += __shfl_xor(a, m);
        b += __shfl_xor(b, m);
    }
    if (lane == 0) {
        coef[2 * col] = (float)(a / (double)T);
        coef[2 * col + 1] = (float)(b / (double)T);
        if (dbeta)
            dbeta[col] = (float)a;
        if (dgamma)
            dgamma[col] = (float)b;
    }
}

// dz = gamma rstd (dq - mean(dq) - zhat mean(dq zhat)); laid out like
// bn_apply_kernel: 4 columns per thread, rows strided by gridDim.y.
__global__ void bn_bwd_apply_kernel(const float *__restrict__ z, const float *__restrict__ dq,
                                    int64_t T, int D, const float *__restrict__ mean,
                                    const float *__restrict__ rstd,
                                    const float *__restrict__ gamma,
                                    const float *__restrict__ coef, float *__restrict__ dz)
{
    const int c = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (c >= D)
        return;
    float mu[4], rs[4], gr[4], c0[4], c1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mu[e] = mean[c + e];
        rs[e] = rstd[c + e];
        gr[e] = (gamma ? gamma[c + e] : 1.f) * rs[e];
        c0[e] = coef[2 * (c + e)];
        c1[e] = coef[2 * (c + e) + 1];
    }
    for (int64_t r = blockIdx.y; r < T; r += gridDim.y) {
        const float4 zv = *reinterpret_cast<const float4 *>(z + r * D + c);
        const float4 gv = *reinterpret_cast<const float4 *>(dq + r * D + c);
        const float zz[4] = {zv.x, zv.y, zv.z, zv.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w};
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float zh = (zz[e] - mu[e]) * rs[e];
            o[e] = gr[e] * (gg[e] - c0[e] - zh * c1[e]);
        }
        *reinterpret_cast<float4 *>(dz + r * D + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
QueryScratch query_scratch(int64_t T, int d_model, int D, int backward, int elt)
{
    QueryScratch S;
    int64_t chunks = (T + 255) / 256;           // rows per chunk >= 256
    if (chunks > 256)
        chunks = 256;
    if (chunks < 1)
        chunks = 1;
    S.chunks = (int)chunks;
    S.rows_per_chunk = T > 0 ? (T + chunks - 1) / chunks : 1;
    auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
    S.off_part = 0;
    S.off_coef = a256((size_t)chunks * D * 3 * 4);
    const int64_t Tp = token_pitch(T);
    S.off_dz = a256(S.off_coef + (size_t)D * 2 * 4);
    S.off_dzt = a256(S.off_dz + (size_t)T * D * 4);
    S.off_wt = a256(S.off_dzt + (size_t)Tp * D * 4);
    S.off_xt = a256(S.off_wt + (size_t)D * d_model * elt);
    S.off_dwp = a256(S.off_xt + (size_t)Tp * d_model * elt);
    S.dw_splits = dw_splits(T, d_model, D);
    S.total = backward ? a256(S.off_dwp + (size_t)S.dw_splits * D * d_model * 4) : S.off_coef;
    return S;
}

// dW = dz^T x has only (D / 128) (d_model / 128) output tiles and a long K
// (the tokens): cut K so that about 1024 workgroups run.
int dw_splits(int64_t T, int d_model, int D)
{
    const int64_t tiles = (int64_t)((D + kGBM - 1) / kGBM) * ((d_model + kGBN - 1) / kGBN);
    int64_t s = (1024 + tiles - 1) / tiles;
    const int64_t max_s = (T + 8 * kGBK - 1) / (8 * kGBK);     // >= 8 K steps a slice
    if (s > max_s)
        s = max_s;
    return (int)(s < 1 ? 1 : s);
}

// bn_apply / bn_bwd_apply: 1024 columns per workgroup along x, row groups
// along y (T > 0)
static dim3 bn_rows_grid(int64_t T, int D)
{
    const int64_t rows = T < kBnApplyRows ? T : kBnApplyRows;
    return dim3((unsigned)((D + 1023) / 1024), (unsigned)rows);
}

template <typename DT>
static hipError_t query_forward_t(const DT *x, const DT *W, const float *gamma, const float *beta,
                                  float eps, DT *q, float *z, float *mean, float *rstd, int64_t T,
                                  int d_model, int D, void *ws, hipStream_t stream)
{
    const QueryScratch S = query_scratch(T, d_model, D, 0, (int)sizeof(DT));
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + S.off_part);
    constexpr int MODE = sizeof(DT) == 2 ? kBf16 : kF32;
    hipError_t err = gemm<DT, DT, false, false, MODE>(x, W, z, (int)T, D, d_model, d_model,
                                                      d_model, stream);
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(bn_partial_kernel, dim3((unsigned)((D + kBnCols - 1) / kBnCols), (unsigned)S.chunks),
                       dim3(kBnWaves * kWave), 0, stream, z, T, D, S.rows_per_chunk, part);
    hipLaunchKernelGGL(bn_finalize_kernel, dim3((unsigned)((D + 3) / 4)), dim3(4 * kWave), 0, stream,
                       part, S.chunks, D, eps, mean, rstd);
    hipLaunchKernelGGL((bn_apply_kernel<DT>), bn_rows_grid(T, D), dim3(256), 0, stream, z, T, D,
                       mean, rstd, gamma, beta, q);
    return hipGetLastError();
}

template <typename DT>
static hipError_t query_backward_t(const DT *x, const DT *W, const float *gamma, const float *z,
                                   const float *mean, const float *rstd, const float *dq,
                                   float *dx, float *dW, float *dgamma, float *dbeta, int64_t T,
                                   int d_model, int D, void *ws, hipStream_t stream)
{
    const QueryScratch S = query_scratch(T, d_model, D, 1, (int)sizeof(DT));
    char *base = static_cast<char *>(ws);
    float *part = reinterpret_cast<float *>(base + S.off_part);
    float *coef = reinterpret_cast<float *>(base + S.off_coef);
    float *dz = reinterpret_cast<float *>(base + S.off_dz);
    float *dzt = reinterpret_cast<float *>(base + S.off_dzt);
    DT *Wt = reinterpret_cast<DT *>(base + S.off_wt);
    DT *xt = reinterpret_cast<DT *>(base + S.off_xt);
    float *dwp = reinterpret_cast<float *>(base + S.off_dwp);
    const int64_t Tp = token_pitch(T);
    typedef typename std::conditional<sizeof(DT) == 2, uint16_t, float>::type E;
    hipLaunchKernelGGL(bn_bwd_partial_kernel, dim3((unsigned)((D + kBnCols - 1) / kBnCols), (unsigned)S.chunks),
                       dim3(kBnWaves * kWave), 0, stream, z, dq, T, D, mean, rstd,
                       S.rows_per_chunk, part);
    hipLaunchKernelGGL(bn_bwd_finalize_kernel, dim3((unsigned)((D + 3) / 4)), dim3(4 * kWave), 0,
                       stream, part, S.chunks, D, T, coef, dgamma, dbeta);
    hipLaunchKernelGGL(bn_bwd_apply_kernel, bn_rows_grid(T, D), dim3(256), 0, stream, z, dq, T, D,
                       mean, rstd, gamma, coef, dz);
    hipError_t err = hipGetLastError();
    // every GEMM operand K-contiguous: W^T [d_model][D], x^T [d_model][T], dz^T [D][T]
    if (err == hipSuccess)
        err = transpose<E>(reinterpret_cast<const E *>(W), reinterpret_cast<E *>(Wt), D, d_model, stream);
    if (err == hipSuccess)
        err = transpose<E>(reinterpret_cast<const E *>(x), reinterpret_cast<E *>(xt), T, d_model, stream,
                           Tp);
    if (err == hipSuccess)
        err = transpose<float>(dz, dzt, T, D, stream, Tp);
    if (err != hipSuccess)
        return err;
    constexpr int MODE = sizeof(DT) == 2 ? kBf16SplitA : kF32;
    // dx [T][d_model] = dz [T][D] . (W^T)^T
    err = gemm<float, DT, false, false, MODE>(dz, Wt, dx, (int)T, d_model, D, D, D, stream);
    if (err != hipSuccess)
        return err;
    // dW [D][d_model] = dz^T [D][Tp] . (x^T)^T, K = Tp (zero-padded tokens) cut
    // into slices
    return gemm<float, DT, false, false, MODE>(dzt, xt, dW, D, d_model, (int)Tp, Tp, Tp, stream,
                                               S.dw_splits, dwp);
}

hipError_t launch_query_forward(int dtype, const void *x, const void *W, const float *gamma,
                                const float *beta, float eps, void *q, float *z, float *mean,
                                float *rstd, int64_t T, int d_model, int D, void *ws,
                                hipStream_t stream)
{
    if (dtype == 1)
        return query_forward_t<bf16_t>(static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(W),
                                       gamma, beta, eps, static_cast<bf16_t *>(q), z, mean, rstd,
                                       T, d_model, D, ws, stream);
    return query_forward_t<float>(static_cast<const float *>(x), static_cast<const float *>(W),
                                  gamma, beta, eps, static_cast<float *>(q), z, mean, rstd, T,
                                  d_model, D, ws, stream);
}

hipError_t launch_query_backward(int dtype, const void *x, const void *W, const float *gamma,
                                 const float *z, const float *mean, const float *rstd,
                                 const float *dq, float *dx, float *dW, float *dgamma,
                                 float *dbeta, int64_t T, int d_model, int D, void *ws,
                                 hipStream_t stream)
{
    if (dtype == 1)
        return query_backward_t<bf16_t>(static_cast<const bf16_t *>(x),
                                        static_cast<const bf16_t *>(W), gamma, z, mean, rstd, dq,
                                        dx, dW, dgamma, dbeta, T, d_model, D, ws, stream);
    return query_backward_t<float>(static_cast<const float *>(x), static_cast<const float *>(W),
                                   gamma, z, mean, rstd, dq, dx, dW, dgamma, dbeta, T, d_model, D,
                                   ws, stream);
}

}  // namespace pkm

// pkm_query.hip -- the query network in front of the memory layer (gptget.net
// summary of "Large Memory Layers with Product Keys", "Deep Analysis",
// methodology list: the input x goes through the query network, which gives
// q; "Key Results": batch normalization in the query network raises memory
// utilization): q = BN(x W^T), one bias-free projection followed by batch
// normalization of every output feature over the batch's tokens (batch
// statistics, biased variance, optional affine gamma, beta), and its backward.
//
// Kernels:
//   gemm_lds_kernel    C[M][N] (fp32) = sum_k A[m][k] B[n][k] for bf16 operands
//                      (A optionally as two bf16 planes hi + lo, two MFMAs a
//                      product) on v_mfma_f32_16x16x32_bf16: 256 x 256 tiles of
//                      8 waves, operands copied from global memory straight
//                      into LDS (global_load_lds) through a ring of 64-wide K
//                      stages, one stage in flight while the other is used
//   gemm_kernel        the same product with register-staged tiles (256 x 128
//                      for bf16, 128 x 128 for float32), for float32 operands
//                      (v_mfma_f32_16x16x4_f32) and for bf16 shapes the direct
//                      kernel does not take (K not a multiple of 64, unaligned
//                      rows)
//   sum_slices_kernel  the split-K partial products summed
//   bn_partial_kernel  per (row chunk, column): count, mean, M2 (Welford over
//                      the chunk's rows, merged across waves by Chan's rule)
//   bn_finalize_kernel per column: merge the chunks -> mean, rstd
//   bn_apply_kernel    q = gamma (z - mean) rstd + beta, rounded once
//   bn_bwd_*           the batch-norm backward (column sums of dq and
//                      dq * zhat, then dz; for bf16 dz leaves as hi + lo
//                      planes, row-major and transposed), followed by two
//                      products: dx = dz W and dW = dz^T x
//   transpose*_kernel  W^T and x^T (K-contiguous operands for the products)
#include "pkm_device.hpp"
#include "pkm_query.hpp"

#include <type_traits>

namespace pkm {

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------
constexpr int kGBN = 128, kGBK = 32;
constexpr int kGThreads = 256;
constexpr int kGroupM = 8;        // tile rows walked together on one XCD

// kBf16: bf16 A and B.  kBf16SplitA: A given as two bf16 planes, hi + lo (a
// float32 operand split once by its producer), two MFMAs per product.
// kF32: float32 A and B on the float32 MFMA.
enum GemmMode { kBf16 = 0, kBf16SplitA = 1, kF32 = 2 };

// Per mode: LDS element type, 16-byte chunks per 32-wide K row (C), A planes,
// and the rows of C a wave owns (WM; a workgroup is 2 x 2 waves: 2 WM rows by
// 128 columns).
template <int MODE> struct GTile;
template <> struct GTile<kBf16> { typedef uint16_t E; static constexpr int C = 4, parts = 1, WM = 128; };
template <> struct GTile<kBf16SplitA> { typedef uint16_t E; static constexpr int C = 4, parts = 2, WM = 128; };
template <> struct GTile<kF32> { typedef float E; static constexpr int C = 8, parts = 1, WM = 64; };

// The 16-byte chunks of a [rows][32] tile are XOR-swizzled by row so that an
// MFMA operand read (rows r16 = 0..15 of the fragment, chunk kg = 0..3 by lane
// group) is free of bank conflicts.  bf16 (4 chunks, 64-byte rows): chunk kg
// of row r sits at position kg ^ swz4(r mod 16), which gives distinct banks to
// any 8 consecutive rows (32 banks, 8 lanes per cycle) and to any 4 rows of
// one residue mod 4 in 16 (64 banks, 16 lanes per cycle).  float32 (8 chunks,
// 128-byte rows): position kg ^ ((r / 2) mod 8).
__device__ __forceinline__ int swz4(int r)
{
    return ((r >> 1) ^ (r >> 3)) & 3;
}

// element offset of (row, k) in such a tile
template <int C>
__device__ __forceinline__ int g_cell(int row, int k)
{
    constexpr int EPC = kGBK / C;
    const int s = C == 4 ? swz4(row & 15) : (row / 2) % 8;
    return row * kGBK + (((k / EPC) ^ s) * EPC) + k % EPC;
}

// The output tile (tx, ty) and K slice tz of this workgroup; the grid is 1-D,
// gx x gy tiles times the K slices.  Workgroup ids are renumbered so that
// each XCD gets one contiguous range of tiles, walked kGroupM tile rows at a
// time: tiles that share A and B panels run on the same XCD at about the same
// time and meet in its L2.
__device__ __forceinline__ void gemm_tile(int gx, int gy, int &tx, int &ty, int &tz)
{
    const int id = xcd_contiguous_id();
    const int per_z = gx * gy;
    tz = id / per_z;
    const int l = id % per_z;
    const int span = kGroupM * gx;
    const int first = l / span * kGroupM;
    const int rows = gy - first < kGroupM ? gy - first : kGroupM;
    ty = first + l % span % rows;
    tx = l % span / rows;
}

// lane holds D rows 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
template <int FI>
__device__ __forceinline__ void gemm_store(const floatx4 (&acc)[FI][4], float *__restrict__ Cm, int M,
                                           int N, int m0, int n0, int lane)
{
    const int r16 = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + 16 * j + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * i + 4 * kg + e;
                if (row < M && col < N)
                    Cm[(int64_t)row * N + col] = acc[i][j][e];
            }
        }
}

// ---- register-staged kernel (any K, any alignment; float32 operands) -------
// One operand's staging, ROWS x 32 elements of a K-contiguous [R][K] array:
// each thread loads 16-byte pieces (8 bf16 or 4 float32) into registers, then
// stores them to LDS whole.  Pieces past R or K read as zeros.
template <typename T> struct GRaw;
template <> struct GRaw<bf16_t> { static constexpr int V = 8; };
template <> struct GRaw<float> { static constexpr int V = 4; };

template <int ROWS, typename T, typename E>
struct GStage {
    static constexpr int V = GRaw<T>::V;                    // elements per 16-byte load
    static constexpr int CPR = kGBK / V;                    // pieces per row
    static constexpr int C = 16 / sizeof(E) == 8 ? 4 : 8;   // chunks per LDS row
    static constexpr int loads = ROWS * CPR / kGThreads;
    uint4 raw[loads];
    __device__ void load(const T *__restrict__ src, int64_t ld, int r0, int R, int k0, int K, int tid)
    {
#pragma unroll
        for (int l = 0; l < loads; ++l) {
            const int u = tid + l * kGThreads;
            const int gr = r0 + u / CPR, gk = k0 + (u % CPR) * V;
            raw[l] = (gr < R && gk < K) ? *reinterpret_cast<const uint4 *>(src + (int64_t)gr * ld + gk)
                                        : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ void store(E *dst, int tid) const
    {
#pragma unroll
        for (int l = 0; l < loads; ++l) {
            const int u = tid + l * kGThreads;
            *reinterpret_cast<uint4 *>(dst + g_cell<C>(u / CPR, (u % CPR) * V)) = raw[l];
        }
    }
};

// C[M][N] (+ slice z of K) = sum_k A[m][k] B[n][k] (A = A + A2 for the split
// mode); slice z covers [z k_slice, (z+1) k_slice) and writes its own C at
// Cm + z M N.
template <typename TA, typename TB, int MODE>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(const TA *__restrict__ A,
                                                         const TA *__restrict__ A2,
                                                         const TB *__restrict__ B,
                                                         float *__restrict__ Cm, int M, int N,
                                                         int K, int64_t lda, int64_t ldb,
                                                         int k_slice, int gx, int gy)
{
    typedef typename GTile<MODE>::E E;
    constexpr int C = GTile<MODE>::C;
    constexpr int PA = GTile<MODE>::parts;
    constexpr int WM = GTile<MODE>::WM, BM = 2 * WM, FI = WM / 16;
    constexpr int TILE_A = BM * kGBK, TILE_B = kGBN * kGBK;
    __shared__ __align__(16) E lds[2][PA * TILE_A + TILE_B];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    int tx, ty, tz;
    gemm_tile(gx, gy, tx, ty, tz);
    const int m0 = ty * BM, n0 = tx * kGBN;
    const int wm = (wave & 1) * WM, wn = (wave >> 1) * 64;
    const int r16 = lane & 15, kg = lane >> 4;

    GStage<BM, TA, E> sa[PA];
    GStage<kGBN, TB, E> sb;
    floatx4 acc[FI][4];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int kb = tz * k_slice;
    const int ke = kb + k_slice < K ? kb + k_slice : K;
    Cm += (int64_t)tz * M * N;
    const int nk = (ke - kb + kGBK - 1) / kGBK;
    auto load = [&](int k0) {
        sa[0].load(A, lda, m0, M, k0, ke, tid);
        if constexpr (PA == 2)
            sa[1].load(A2, lda, m0, M, k0, ke, tid);
        sb.load(B, ldb, n0, N, k0, ke, tid);
    };
    auto store = [&](E *dst) {
#pragma unroll
        for (int pa = 0; pa < PA; ++pa)
            sa[pa].store(dst + pa * TILE_A, tid);
        sb.store(dst + PA * TILE_A, tid);
    };
    load(kb);
    store(lds[0]);
    __syncthreads();
    for (int c = 0; c < nk; ++c) {
        if (c + 1 < nk)
            load(kb + (c + 1) * kGBK);
        const E *at = lds[c & 1], *bt = lds[c & 1] + PA * TILE_A;
        if constexpr (MODE == kF32) {
            float4 a[FI][2], b[4][2];
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int row = wm + 16 * i + r16;
                a[i][0] = *reinterpret_cast<const float4 *>(at + g_cell<C>(row, 4 * kg));
                a[i][1] = *reinterpret_cast<const float4 *>(at + g_cell<C>(row, 4 * kg + 16));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn + 16 * j + r16;
                b[j][0] = *reinterpret_cast<const float4 *>(bt + g_cell<C>(row, 4 * kg));
                b[j][1] = *reinterpret_cast<const float4 *>(bt + g_cell<C>(row, 4 * kg + 16));
            }
#pragma unroll
            for (int i = 0; i < FI; ++i)
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
            // B fragments stay in registers; A fragments are read one row of
            // MFMA tiles at a time
            uint4 b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const uint4 *>(bt + g_cell<C>(wn + 16 * j + r16, 8 * kg));
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int row = wm + 16 * i + r16;
                uint4 a[PA];
#pragma unroll
                for (int pa = 0; pa < PA; ++pa)
                    a[pa] = *reinterpret_cast<const uint4 *>(at + pa * TILE_A + g_cell<C>(row, 8 * kg));
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int pa = 0; pa < PA; ++pa)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[pa]), __builtin_bit_cast(bf16x8, b[j]),
                            acc[i][j], 0, 0, 0);
            }
        }
        if (c + 1 < nk)
            store(lds[(c + 1) & 1]);
        __syncthreads();
    }
    gemm_store<FI>(acc, Cm, M, N, m0 + wm, n0 + wn, lane);
}

// ---- direct-to-LDS kernel (bf16 operands, K a multiple of the stage) ------
// The operand tiles go from global memory straight into LDS (one
// global_load_lds_dwordx4 per 1 KB block of tile rows: lane l writes bytes
// 16 l .. 16 l + 15 of the block and fetches the chunk the swizzle puts there),
// through a ring of NS stages: NS - 1 stages are in flight while one is read.
// A stage is complete once this wave's own loads of it have retired
// (s_waitcnt vmcnt) and every wave has passed the barrier that follows.
// 16 bytes per lane from global memory into LDS: lane l's bytes land at
// dst + 16 l (dst is the same for the whole wave)
__device__ __forceinline__ void lds_dma16(const void *src, void *dst)
{
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}


// A workgroup is 2 x NWN waves, each owning WM x 64 of C: 2 WM rows by 64 NWN
// columns.  A ring stage holds BK (32 or 64) columns of K: tile rows of RB =
// 2 BK bytes, 1 KB blocks of 1024 / RB rows; with BK = 64 a row is a whole
// 128-byte cache line.  Chunk kc of row r sits at position kc ^ swz(r mod 16):
// swz4 for 4 chunks a row, swz8(r) = (r ^ (r >> 3)) mod 8 for 8, which keeps
// the fragment reads free of bank conflicts for 8 or 16 lanes a cycle alike.
__device__ __forceinline__ int swz8(int r)
{
    return (r ^ (r >> 3)) & 7;
}

// One ring step: start the copy of a later stage into `fill` (null when there
// is none) and multiply the fragments of stage `cur`.  The two buffers reach
// this function as distinct restrict pointers, so the compiler knows that its
// LDS reads do not touch what the copy writes and adds no wait on the copy
// before them; the kernel itself waits for a stage's copy (vmcnt) and for
// every wave (barrier) before it is read.  The fragment reads are ordinary
// loads, which the compiler interleaves with the MFMAs.
template <int FI, int PA, int RB, int BK, int TILE_A, int LA, int LB>
__device__ __forceinline__ void gemm_ring_step(unsigned char *__restrict__ fill,
                                               const unsigned char *__restrict__ cur,
                                               const bf16_t *const (&pa)[PA][LA],
                                               const bf16_t *const (&pb)[LB], int k0, int wave,
                                               const int (&a_rel)[BK / 32],
                                               const int (&b_rel)[BK / 32], floatx4 (&acc)[FI][4])
{
    if (fill) {
#pragma unroll
        for (int p = 0; p < PA; ++p)
#pragma unroll
            for (int l = 0; l < LA; ++l)
                lds_dma16(pa[p][l] + k0, fill + p * TILE_A + (wave * LA + l) * 1024);
#pragma unroll
        for (int l = 0; l < LB; ++l)
            lds_dma16(pb[l] + k0, fill + PA * TILE_A + (wave * LB + l) * 1024);
    }
#pragma unroll
    for (int h = 0; h < BK / 32; ++h) {
        uint4 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const uint4 *>(cur + b_rel[h] + j * 16 * RB);
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            uint4 a[PA];
#pragma unroll
            for (int p = 0; p < PA; ++p)
                a[p] = *reinterpret_cast<const uint4 *>(cur + a_rel[h] + p * TILE_A + i * 16 * RB);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < PA; ++p)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a[p]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j],
                        0, 0, 0);
        }
    }
}

template <int MODE, int WM, int NWN, int NS, int BK>
__global__ __launch_bounds__(2 * NWN * kWave) void gemm_lds_kernel(const bf16_t *__restrict__ A,
                                                                  const bf16_t *__restrict__ A2,
                                                                  const bf16_t *__restrict__ B,
                                                                  float *__restrict__ Cm, int M,
                                                                  int N, int K, int64_t lda,
                                                                  int64_t ldb, int k_slice, int gx,
                                                                  int gy)
{
    constexpr int PA = GTile<MODE>::parts;
    constexpr int WAVES = 2 * NWN;
    constexpr int BM = 2 * WM, BN = 64 * NWN, FI = WM / 16;
    constexpr int RB = 2 * BK;                                  // bytes per tile row
    constexpr int CPR = RB / 16;                                // 16-byte chunks per row
    constexpr int RPB = 1024 / RB;                              // rows per 1 KB block
    constexpr int TILE_A = BM * RB, TILE_B = BN * RB;
    constexpr int STAGE = PA * TILE_A + TILE_B;
    constexpr int LA = BM / RPB / WAVES, LB = BN / RPB / WAVES; // blocks per wave
    static_assert(LA * RPB * WAVES == BM && LB * RPB * WAVES == BN, "whole blocks per wave");
    constexpr int LPS = PA * LA + LB;                           // loads per wave per stage
    static_assert(NS >= 2 && NS <= 4 && (NS - 2) * LPS < 64, "ring depth");
    static_assert(BK == 32 || BK == 64, "stage width");
    __shared__ __align__(1024) unsigned char lds[NS * STAGE];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    int tx, ty, tz;
    gemm_tile(gx, gy, tx, ty, tz);
    const int m0 = ty * BM, n0 = tx * BN;
    const int wm = (wave & 1) * WM, wn = (wave >> 1) * 64;
    const int r16 = lane & 15, kg = lane >> 4;
    auto swz = [](int r) { return CPR == 4 ? swz4(r & 15) : swz8(r & 15); };

    // this lane's source rows (clamped into the matrix: rows past M or N are
    // computed from repeated data and never stored) and the chunk the swizzle
    // puts at its position (lane l writes row l / CPR, position l % CPR of
    // its block)
    const int lrow = lane / CPR, lpos = lane % CPR;
    const bf16_t *pa[PA][LA];
    const bf16_t *pb[LB];
#pragma unroll
    for (int l = 0; l < LA; ++l) {
        const int row = (wave * LA + l) * RPB + lrow;
        const int gr = m0 + row < M ? m0 + row : M - 1;
        const int kc = lpos ^ swz(row);
        pa[0][l] = A + (int64_t)gr * lda + 8 * kc;
        if constexpr (PA == 2)
            pa[1][l] = A2 + (int64_t)gr * lda + 8 * kc;
    }
#pragma unroll
    for (int l = 0; l < LB; ++l) {
        const int row = (wave * LB + l) * RPB + lrow;
        const int gr = n0 + row < N ? n0 + row : N - 1;
        pb[l] = B + (int64_t)gr * ldb + 8 * (lpos ^ swz(row));
    }
    const int kb = tz * k_slice;
    const int ke = kb + k_slice < K ? kb + k_slice : K;
    Cm += (int64_t)tz * M * N;
    const int nk = (ke - kb) / BK;

    auto issue = [&](int c) {
        unsigned char *st = lds + (c % NS) * STAGE;
        const int k0 = kb + c * BK;
#pragma unroll
        for (int p = 0; p < PA; ++p)
#pragma unroll
            for (int l = 0; l < LA; ++l)
                lds_dma16(pa[p][l] + k0, st + p * TILE_A + (wave * LA + l) * 1024);
#pragma unroll
        for (int l = 0; l < LB; ++l)
            lds_dma16(pb[l] + k0, st + PA * TILE_A + (wave * LB + l) * 1024);
    };

    floatx4 acc[FI][4];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // byte offsets of this lane's fragments in a stage, per 32-wide K half
    // (the swizzle of rows wm + 16 i + r16 does not depend on i)
    int a_rel[BK / 32], b_rel[BK / 32];
#pragma unroll
    for (int h = 0; h < BK / 32; ++h) {
        const int sw = ((kg + 4 * h) ^ swz(r16)) * 16;
        a_rel[h] = (wm + r16) * RB + sw;
        b_rel[h] = PA * TILE_A + (wn + r16) * RB + sw;
    }

#pragma unroll
    for (int c = 0; c < NS - 1; ++c)
        if (c < nk)
            issue(c);
    for (int c = 0; c < nk; ++c) {
        // stage c is this wave's oldest outstanding one: wait until at most
        // the loads of the stages issued after it are in flight
        const int after = nk - 1 - c < NS - 2 ? nk - 1 - c : NS - 2;
        if (after >= 2)
            wait_vmcnt<2 * LPS>();
        else if (after == 1)
            wait_vmcnt<LPS>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");      // no LDS access moves above the barrier
        // every wave is done with stage c - 1: its buffer takes stage c + NS - 1
        const int nxt = c + NS - 1;
        gemm_ring_step<FI, PA, RB, BK, TILE_A, LA, LB>(
            nxt < nk ? lds + (nxt % NS) * STAGE : nullptr, lds + (c % NS) * STAGE, pa, pb,
            kb + nxt * BK, wave, a_rel, b_rel, acc);
    }
    gemm_store<FI>(acc, Cm, M, N, m0 + wm, n0 + wn, lane);
}

// C = A B^T with both operands K-contiguous.  With splits > 1 the K range is
// cut into `splits` slices whose partial products go to `parts`
// ([splits][M][N]) and are then summed into C.
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

template <int MODE>
static int gemm_rows_per_tile()
{
    return 2 * GTile<MODE>::WM;
}

// tile shape (2 WM x 64 NWN) and ring depth of the direct-to-LDS kernel per mode
template <int MODE> struct GLds;
template <> struct GLds<kBf16> { static constexpr int WM = 128, NWN = 4, NS = 2, BK = 64; };
template <> struct GLds<kBf16SplitA> { static constexpr int WM = 64, NWN = 4, NS = 2, BK = 64; };

static bool aligned16(const void *p)
{
    return ((uintptr_t)p & 15) == 0;
}

template <typename TA, typename TB, int MODE>
static hipError_t gemm(const TA *A, const TA *A2, const TB *B, float *Cm, int M, int N, int K,
                       int64_t lda, int64_t ldb, hipStream_t stream, int splits = 1,
                       float *parts = nullptr)
{
    bool direct = false;
    int gran = kGBK;                    // K slices are whole stages
    if constexpr (MODE != kF32) {
        direct = K % GLds<MODE>::BK == 0 && lda % 8 == 0 && ldb % 8 == 0 && aligned16(A) &&
                 aligned16(B) && (A2 == nullptr || aligned16(A2));
        if (direct)
            gran = GLds<MODE>::BK;
    }
    int k_slice = K;
    if (splits > 1) {
        k_slice = (K + splits - 1) / splits;
        k_slice = (k_slice + gran - 1) / gran * gran;
        splits = (K + k_slice - 1) / k_slice;
    }
    float *out = splits > 1 ? parts : Cm;
    if constexpr (MODE != kF32) {
        if (direct) {
            typedef GLds<MODE> G;
            const int BM = 2 * G::WM, BN = 64 * G::NWN;
            const int gx = (N + BN - 1) / BN, gy = (M + BM - 1) / BM;
            hipLaunchKernelGGL((gemm_lds_kernel<MODE, G::WM, G::NWN, G::NS, G::BK>),
                               dim3((unsigned)((int64_t)gx * gy * splits)), dim3(2 * G::NWN * kWave),
                               0, stream, A, A2, B, out, M, N, K, lda, ldb, k_slice, gx, gy);
        }
    }
    if (!direct) {
        const int BM = gemm_rows_per_tile<MODE>();
        const int gx = (N + kGBN - 1) / kGBN, gy = (M + BM - 1) / BM;
        hipLaunchKernelGGL((gemm_kernel<TA, TB, MODE>), dim3((unsigned)((int64_t)gx * gy * splits)),
                           dim3(kGThreads), 0, stream, A, A2, B, out, M, N, K, lda, ldb, k_slice, gx,
                           gy);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || splits <= 1)
        return err;
    const int64_t count = (int64_t)M * N;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256),
                       0, stream, parts, splits, count, Cm);
    return hipGetLastError();
}

// out[c][r] = in[r][c] for an R x C matrix of 4-byte elements, through
// 64 x 64 LDS tiles (both sides coalesced); out rows have pitch ldo >= R and
// their tail r in [R, ldo) is written with zeros.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E *__restrict__ in, E *__restrict__ out,
                                                        int64_t R, int64_t C, int64_t ldo)
{
    __shared__ E tile[64][65];
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    for (int64_t r0 = (int64_t)blockIdx.y * 64; r0 < ldo; r0 += (int64_t)gridDim.y * 64) {
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
        __syncthreads();
    }
}

// K of the GEMM that runs over the tokens (dW = dz^T x): the token count
// rounded up to 64, a whole number of 64-wide K steps of 16-byte aligned
// pieces (8 bf16 or 4 float32 elements), plus 64 more when that is a multiple
// of 512 (rows a power-of-two number of kilobytes apart put the rows one load
// touches into the same memory channels); the padding holds zeros.
static int64_t token_pitch(int64_t T)
{
    const int64_t p = (T + 63) & ~(int64_t)63;
    return p % 512 == 0 ? p + 64 : p;
}

// 16-bit elements: 64 x 64 tiles moved in 16-byte pieces on both sides.  The
// tile sits in LDS with a row pitch of 65 elements, so that the 8 rows 8
// apart that one read instruction touches (per column) fall in distinct banks.
constexpr int kTrPitch = 65;

// out[(c0 + c) ldo + r0 + r] = t[r][c] for the 64 x 64 tile t, 8 consecutive
// r per lane (one 16-byte store; ldo and r0 are multiples of 8): columns past
// C and rows past ldo are skipped.
__device__ __forceinline__ void tile16_store_t(const uint16_t (*t)[kTrPitch], uint16_t *__restrict__ out,
                                               int64_t r0, int64_t c0, int64_t C, int64_t ldo, int tid)
{
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int c = pass * 32 + tid / 8, rs = (tid % 8) * 8;
        if (c0 + c >= C || r0 + rs >= ldo)
            continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)t[rs + 2 * e][c] | ((uint32_t)t[rs + 2 * e + 1][c] << 16);
        *reinterpret_cast<uint4 *>(out + (c0 + c) * ldo + r0 + rs) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// out[c][r] = in[r][c] for an R x C matrix of 16-bit elements (C a multiple
// of 8), out pitch ldo >= R (a multiple of 8), the tail r in [R, ldo) zeros
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t *__restrict__ in,
                                                          uint16_t *__restrict__ out, int64_t R,
                                                          int64_t C, int64_t ldo)
{
    __shared__ uint16_t tile[64][kTrPitch];
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int tid = threadIdx.x;
    for (int64_t r0 = (int64_t)blockIdx.y * 64; r0 < ldo; r0 += (int64_t)gridDim.y * 64) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int r = pass * 32 + tid / 8, cs = (tid % 8) * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r0 + r < R && c0 + cs < C)
                v = *reinterpret_cast<const uint4 *>(in + (r0 + r) * C + c0 + cs);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tile[r][cs + 2 * e] = (uint16_t)w[e];
                tile[r][cs + 2 * e + 1] = (uint16_t)(w[e] >> 16);
            }
        }
        __syncthreads();
        tile16_store_t(tile, out, r0, c0, C, ldo, tid);
        __syncthreads();
    }
}

// transposes and the fused batch-norm step walk 64-row tiles from blockIdx.y
// by gridDim.y, which stays within the launch limit of the y dimension
static unsigned row_tiles_grid(int64_t rows)
{
    const int64_t t = (rows + 63) / 64;
    return (unsigned)(t < 65535 ? t : 65535);
}

template <typename E>
static hipError_t transpose(const E *in, E *out, int64_t R, int64_t C, hipStream_t stream,
                            int64_t ldo = -1)
{
    if (ldo < 0)
        ldo = R;
    const dim3 grid((unsigned)((C + 63) / 64), row_tiles_grid(ldo));
    if constexpr (sizeof(E) == 2)
        hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, stream,
                           reinterpret_cast<const uint16_t *>(in), reinterpret_cast<uint16_t *>(out), R,
                           C, ldo);
    else
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

// The same step for bf16 storage, fused with the transposes the dW product
// needs: over a 64 x 64 tile of (token, feature), dz is split into two bf16
// planes, hi = bf16(dz) and lo = bf16(dz - hi) (the operand form of the bf16
// products that follow), written row-major ([T][D], for dx) and transposed
// ([D][Tp], for dW; tokens past T are zeros).  D is a multiple of 8.
__global__ __launch_bounds__(256) void bn_bwd_apply_split_kernel(
    const float *__restrict__ z, const float *__restrict__ dq, int64_t T, int D,
    const float *__restrict__ mean, const float *__restrict__ rstd, const float *__restrict__ gamma,
    const float *__restrict__ coef, uint16_t *__restrict__ dz_hi, uint16_t *__restrict__ dz_lo,
    uint16_t *__restrict__ dzt_hi, uint16_t *__restrict__ dzt_lo, int64_t Tp)
{
    __shared__ uint16_t th[64][kTrPitch], tl[64][kTrPitch];
    const int c0 = blockIdx.x * 64, tid = threadIdx.x;
    const int cl = 4 * (tid % 16), c = c0 + cl;           // this thread's 4 features
    const bool cok = c < D;
    float mu[4], rs[4], gr[4], k0[4], k1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mu[e] = cok ? mean[c + e] : 0.f;
        rs[e] = cok ? rstd[c + e] : 0.f;
        gr[e] = (gamma && cok ? gamma[c + e] : 1.f) * rs[e];
        k0[e] = cok ? coef[2 * (c + e)] : 0.f;
        k1[e] = cok ? coef[2 * (c + e) + 1] : 0.f;
    }
    for (int64_t r0 = (int64_t)blockIdx.y * 64; r0 < Tp; r0 += (int64_t)gridDim.y * 64) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = tid / 16 + 16 * j;
            const int64_t t = r0 + r;
            uint32_t h[4] = {0u, 0u, 0u, 0u}, l[4] = {0u, 0u, 0u, 0u};
            if (t < T && cok) {
                const float4 zv = *reinterpret_cast<const float4 *>(z + t * D + c);
                const float4 gv = *reinterpret_cast<const float4 *>(dq + t * D + c);
                const float zz[4] = {zv.x, zv.y, zv.z, zv.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float zh = (zz[e] - mu[e]) * rs[e];
                    const float o = gr[e] * (gg[e] - k0[e] - zh * k1[e]);
                    h[e] = f32_to_bf16_bits(o);
                    l[e] = f32_to_bf16_bits(o - bf16_to_f32(h[e]));
                }
                *reinterpret_cast<uint2 *>(dz_hi + t * D + c) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                *reinterpret_cast<uint2 *>(dz_lo + t * D + c) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                th[r][cl + e] = (uint16_t)h[e];
                tl[r][cl + e] = (uint16_t)l[e];
            }
        }
        __syncthreads();
        tile16_store_t(th, dzt_hi, r0, c0, D, Tp, tid);
        tile16_store_t(tl, dzt_lo, r0, c0, D, Tp, tid);
        __syncthreads();
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
    S.dw_splits = dw_splits(T, d_model, D, elt);
    S.total = backward ? a256(S.off_dwp + (size_t)S.dw_splits * D * d_model * 4) : S.off_coef;
    return S;
}

// dW = dz^T x has only (D / BM) (d_model / BN) output tiles and a long K (the
// tokens): cut K so that about kDwWorkgroups workgroups run.  (bf16 tiles are
// those of the direct-to-LDS kernel; when a product falls back to the
// register-staged one, the split count is only less well matched.)
constexpr int kDwWorkgroups = 1024;
int dw_splits(int64_t T, int d_model, int D, int elt)
{
    const int bm = elt == 2 ? 2 * GLds<kBf16SplitA>::WM : gemm_rows_per_tile<kF32>();
    const int bn = elt == 2 ? 64 * GLds<kBf16SplitA>::NWN : kGBN;
    const int64_t tiles = (int64_t)((D + bm - 1) / bm) * ((d_model + bn - 1) / bn);
    int64_t s = (kDwWorkgroups + tiles - 1) / tiles;
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
    hipError_t err = gemm<DT, DT, MODE>(x, nullptr, W, z, (int)T, D, d_model, d_model, d_model,
                                        stream);
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
    constexpr bool SPLIT = sizeof(DT) == 2;
    uint16_t *dzh = reinterpret_cast<uint16_t *>(dz), *dzl = dzh + T * D;
    uint16_t *dzth = reinterpret_cast<uint16_t *>(dzt), *dztl = dzth + Tp * D;
    if constexpr (SPLIT)
        hipLaunchKernelGGL(bn_bwd_apply_split_kernel,
                           dim3((unsigned)((D + 63) / 64), row_tiles_grid(Tp)), dim3(256), 0,
                           stream, z, dq, T, D, mean, rstd, gamma, coef, dzh, dzl, dzth, dztl, Tp);
    else
        hipLaunchKernelGGL(bn_bwd_apply_kernel, bn_rows_grid(T, D), dim3(256), 0, stream, z, dq, T,
                           D, mean, rstd, gamma, coef, dz);
    hipError_t err = hipGetLastError();
    // every GEMM operand K-contiguous: W^T [d_model][D], x^T [d_model][Tp], dz^T [D][Tp]
    if (err == hipSuccess)
        err = transpose<E>(reinterpret_cast<const E *>(W), reinterpret_cast<E *>(Wt), D, d_model, stream);
    if (err == hipSuccess)
        err = transpose<E>(reinterpret_cast<const E *>(x), reinterpret_cast<E *>(xt), T, d_model, stream,
                           Tp);
    if constexpr (SPLIT) {
        if (err != hipSuccess)
            return err;
        const bf16_t *h = reinterpret_cast<const bf16_t *>(dzh), *l = reinterpret_cast<const bf16_t *>(dzl);
        const bf16_t *th = reinterpret_cast<const bf16_t *>(dzth), *tl = reinterpret_cast<const bf16_t *>(dztl);
        // dx [T][d_model] = dz [T][D] . (W^T)^T
        err = gemm<bf16_t, bf16_t, kBf16SplitA>(h, l, reinterpret_cast<const bf16_t *>(Wt), dx, (int)T,
                                                d_model, D, D, D, stream);
        if (err != hipSuccess)
            return err;
        // dW [D][d_model] = dz^T [D][Tp] . (x^T)^T, K = Tp (zero-padded tokens)
        // cut into slices
        return gemm<bf16_t, bf16_t, kBf16SplitA>(th, tl, reinterpret_cast<const bf16_t *>(xt), dW, D,
                                                 d_model, (int)Tp, Tp, Tp, stream, S.dw_splits, dwp);
    } else {
        if (err == hipSuccess)
            err = transpose<float>(dz, dzt, T, D, stream, Tp);
        if (err != hipSuccess)
            return err;
        const float *wt = reinterpret_cast<const float *>(Wt), *xtf = reinterpret_cast<const float *>(xt);
        err = gemm<float, float, kF32>(dz, nullptr, wt, dx, (int)T, d_model, D, D, D, stream);
        if (err != hipSuccess)
            return err;
        return gemm<float, float, kF32>(dzt, nullptr, xtf, dW, D, d_model, (int)Tp, Tp, Tp, stream,
                                        S.dw_splits, dwp);
    }
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

// pkm_device.hpp -- device-side building blocks shared by the PKM kernels:
// storage-type conversions, order-preserving selection keys, and wave64
// primitives (reductions, scans, bitonic sorts across the 64 lanes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// bfloat16 storage is carried as raw 16-bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Unpack 16 bytes of storage into float32 lanes.
__device__ __forceinline__ void unpack16(const uint4 v, float (&out)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4 v, float (&out)[4])
{
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
}

// Elements of a storage type per 16-byte chunk.
template <typename DT> struct Elt;
template <> struct Elt<float> { static constexpr int per16 = 4; };
template <> struct Elt<bf16_t> { static constexpr int per16 = 8; };

// ---------------------------------------------------------------------------
// Selection keys.  A 64-bit key orders (score descending, index ascending) as
// plain unsigned integer descending: high word = order-preserving image of the
// float score (-0 folded onto +0), low word = bitwise NOT of the index.  Every
// key of a finite score is > 0, so 0 pads a sort and sinks to the end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_f32(float s)
{
    // s + 0 turns -0 into +0 (round to nearest) and leaves every other value
    // as it is; then flip the sign bit of a positive pattern and every bit of
    // a negative one -- integer ops only, no compare-and-select
    const uint32_t u = __float_as_uint(s + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t index)
{
    return ((uint64_t)ord_f32(s) << 32) | (uint64_t)(~index);
}
__device__ __forceinline__ float key_score(uint64_t key) { return unord_f32((uint32_t)(key >> 32)); }
__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// Keys that sort as float64 values.  For an index below 2^IB (IB <= 20) the
// key 2^52 + ord * 2^IB + (2^IB - 1 - index) has bit 52 set and nothing above
// it, so its bit pattern is a positive normal float64 (biased exponent 1),
// and float64 order, integer order and (score descending, index ascending)
// all agree.  A sort then exchanges two keys with one v_max_f64 and one
// v_min_f64 instead of a 64-bit compare and four selects.  0 (+0.0) is below
// every key and pads a sort.
template <int IB>
__device__ __forceinline__ uint64_t dkey(uint32_t ord, uint32_t index)
{
    static_assert(IB >= 1 && IB <= 20, "the key must stay below 2^53");
    return (1ull << 52) | ((uint64_t)ord << IB) | (uint64_t)((1u << IB) - 1u - index);
}
template <int IB>
__device__ __forceinline__ uint32_t dkey_ord(uint64_t key) { return (uint32_t)(key >> IB); }
template <int IB>
__device__ __forceinline__ uint32_t dkey_index(uint64_t key)
{
    return (1u << IB) - 1u - ((uint32_t)key & ((1u << IB) - 1u));
}
// max / min of two such keys.  Written as instructions so that the compiler
// adds no canonicalisation of the operands (they are bit patterns of normal
// numbers, never NaN, so the IEEE max / min is the plain order).
__device__ __forceinline__ uint64_t dkey_max(uint64_t a, uint64_t b)
{
    uint64_t r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ uint64_t dkey_min(uint64_t a, uint64_t b)
{
    uint64_t r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// ---------------------------------------------------------------------------
// wave64 primitives
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Workgroups are dealt to the 8 XCDs (each with its own L2) in turn.  The id
// below renumbers a 1-D grid so that each XCD gets one contiguous range of
// ids, walked in order: work items next to each other in id run on the same
// XCD at about the same time and share its L2.  A bijection for any grid, so
// correctness does not depend on how workgroups are actually dealt.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous_id()
{
    const int total = (int)gridDim.x;
    const int g = (int)blockIdx.x;
    const int q = total / kXcds, r = total % kXcds;
    const int xcd = g % kXcds, pos = g / kXcds;
    return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    const uint32_t lo = __shfl_xor((int)(uint32_t)v, mask);
    const uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), mask);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src)
{
    const uint32_t lo = __shfl((int)(uint32_t)v, src);
    const uint32_t hi = __shfl((int)(uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m);
    return v;
}

// Sums of U values over the 64 lanes at once (U a power of two <= 64).  On
// return v[0] of lane l holds the total of value (l / (64 / U)).  Each halving
// step exchanges half of the remaining values, so U sums cost about
// U + log2(64 / U) cross-lane moves instead of 6 U.
template <int U>
__device__ __forceinline__ void wave_multi_sum(float (&v)[U])
{
    const int lane = lane_id();
    int width = U;
#pragma unroll
    for (int stride = 32; stride >= 1; stride >>= 1) {
        if (width > 1) {
            // lanes with the stride bit set keep the upper half of the values
            // bit masks instead of a select between two array elements, which
            // the compiler may turn into a private-memory indexed load
            const uint32_t up = (lane & stride) != 0 ? 0xffffffffu : 0u;
            const int h = width / 2;
#pragma unroll
            for (int j = 0; j < U / 2; ++j) {
                if (j < h) {
                    const uint32_t a = __float_as_uint(v[j]), b = __float_as_uint(v[j + h]);
                    const float send = __uint_as_float((a & up) | (b & ~up));
                    const float keep = __uint_as_float((b & up) | (a & ~up));
                    v[j] = keep + __shfl_xor(send, stride);
                }
            }
            width = h;
        } else {
            v[0] += __shfl_xor(v[0], stride);
        }
    }
}

// Buffer descriptor over `bytes` bytes at p: loads that reach past the end
// return zeros, so loads can be issued unconditionally (a fixed count of
// memory operations per loop trip keeps the compiler's waits partial).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 l (dst is the same for the whole wave); a lane reaching past the
// buffer's end reads zeros.  The copy counts on the vector memory counter.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void *dst, int voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16,
                                             voffset, 0, 0, 0);
}

// s_waitcnt on the vector memory counter alone (vmcnt bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Exclusive prefix sum over the 64 lanes; *total receives the wave total.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total)
{
    const int lane = lane_id();
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d);
        if (lane >= d)
            inc += o;
    }
    *total = __shfl(inc, kWave - 1);
    return inc - v;
}

// The lanes of this wave whose `key` equals this lane's (keys < 2^bits; lanes
// with valid == false match nothing and get 0): one ballot per key bit.
// `bits` must be the same in every lane.
__device__ __forceinline__ uint64_t wave_match(uint32_t key, bool valid, int bits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
        const bool on = (key >> b) & 1u;
        const uint64_t set = __ballot(on);
        m &= on ? set : ~set;
    }
    return valid ? m : 0ull;
}

// Lanes below this one: bit l set for every lane l < lane_id().
__device__ __forceinline__ uint64_t lanes_below() { return (1ull << lane_id()) - 1ull; }

// Make this wave's LDS stores visible to its own later LDS loads.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort, descending, of 64 floats (one per lane).  Lane i ends with
// the i-th largest.
__device__ __forceinline__ float wave_sort64_desc(float v)
{
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const float o = __shfl_xor(v, stride);
            const bool desc = (lane & size) == 0 || size == kWave;
            const bool lower = (lane & stride) == 0;
            v = (lower == desc) ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return v;
}

// Bitonic sort, descending, of R*64 keys held R per lane; element i = r*64 + lane.
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&v)[R])
{
    const int lane = lane_id();
    constexpr int P = R * kWave;
#pragma unroll
    for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= kWave) {
                const int rs = stride / kWave;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & rs) == 0) {
                        const bool desc = ((r * kWave) & size) == 0;
                        const uint64_t a = v[r], b = v[r | rs];
                        const bool swap = desc ? (a < b) : (a > b);
                        v[r] = swap ? b : a;
                        v[r | rs] = swap ? a : b;
                    }
                }
            } else {
                const bool lower = (lane & stride) == 0;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint64_t o = shfl_xor_u64(v[r], stride);
                    const bool desc = ((r * kWave + lane) & size) == 0;
                    const bool keep_max = (lower == desc);
                    v[r] = keep_max ? (v[r] > o ? v[r] : o) : (v[r] < o ? v[r] : o);
                }
            }
        }
    }
}

// Bitonic sort, descending, inside each group of 4 lanes {l, l^16, l^32, l^48}
// (the lanes that share l % 16), of the 4R values the group holds: element
// e = (lane / 16) * R + r lives in register r of lane group lane / 16.
__device__ __forceinline__ float g4_shfl(float v, int m) { return __shfl_xor(v, m); }
__device__ __forceinline__ uint32_t g4_shfl(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m); }
__device__ __forceinline__ uint64_t g4_shfl(uint64_t v, int m) { return shfl_xor_u64(v, m); }
__device__ __forceinline__ float g4_bcast(float v, int src) { return __shfl(v, src); }
__device__ __forceinline__ uint32_t g4_bcast(uint32_t v, int src) { return (uint32_t)__shfl((int)v, src); }

// Sum over the 4 lanes that share lane % 16.
__device__ __forceinline__ int group4_sum(int v)
{
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float vmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float vmin(float a, float b) { return fminf(a, b); }
__device__ __forceinline__ uint32_t vmax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t vmin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// The k-th largest (1 <= k <= 64) of the 64 values a 4-lane group holds (16
// a lane, element e = 16 (lane / 16) + r), returned in all 4 lanes; v is
// left permuted.  A bitonic network whose every merge of size `size` starts
// by exchanging element e with its mirror e ^ (size - 1): every exchange then
// keeps the larger value at the lower position, so in-lane exchanges are one
// max and one min with no compare.  For k = 32 the last merge stops after its
// mirror exchange: positions 0..31 then hold the 32 largest values, and the
// 32nd is their least.
template <typename T>
__device__ __forceinline__ T group4_kth(T (&v)[16], int k)
{
    const int g = lane_id() >> 4;
    auto inlane = [&](int r, int r2) {
        const T a = v[r], b = v[r2];
        v[r] = vmax(a, b);
        v[r2] = vmin(a, b);
    };
    // the stride exchanges 8 .. 1 of 16-runs inside the lane
    auto runs16 = [&](int from) {
#pragma unroll
        for (int stride = 8; stride > 0; stride >>= 1)
            if (stride <= from)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((r & stride) == 0)
                        inlane(r, r | stride);
    };
    // with lane group g ^ (lanes / 16): the mirror register 15 - r or the
    // same register; the lower lane group keeps the larger value
    auto cross = [&](int lanes, bool mirror, bool lower) {
        T o[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[r] = g4_shfl(v[mirror ? 15 - r : r], lanes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const T hi = vmax(v[r], o[r]), lo = vmin(v[r], o[r]);
            v[r] = lower ? hi : lo;
        }
    };
#pragma unroll
    for (int size = 2; size <= 16; size <<= 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r & (size >> 1)) == 0)
                inlane(r, r ^ (size - 1));
        runs16(size >> 2);
    }
    cross(16, true, (g & 1) == 0);      // size 32: e ^ 31 = lane group g ^ 1, register 15 - r
    runs16(8);
    cross(48, true, g < 2);             // size 64: e ^ 63 = lane group g ^ 3, register 15 - r
    T x;
    if (k == 32) {
        x = v[0];
#pragma unroll
        for (int r = 1; r < 16; ++r)
            x = vmin(x, v[r]);
        x = vmin(x, g4_shfl(x, 16));
        // lane groups 0 and 1 hold the 32 largest: every lane reads group 0's
        return g4_bcast(x, lane_id() & 15);
    }
    cross(16, false, (g & 1) == 0);     // stride 16
    runs16(8);
    x = v[0];
#pragma unroll
    for (int r = 1; r < 16; ++r)
        if (r == ((k - 1) & 15))
            x = v[r];
    return g4_bcast(x, (lane_id() & 15) + 16 * ((k - 1) >> 4));
}

// Descending sort of the 64 keys (dkey format, or 0) a 4-lane group holds,
// 16 a lane (element e = 16 (lane / 16) + r in register r).  The network is
// group4_kth's: every merge of size s starts by exchanging element e with its
// mirror e ^ (s - 1), so every exchange keeps the larger key at the lower
// position -- in-lane exchanges are one max and one min, with no compare and
// no direction.
__device__ __forceinline__ void group4_sort_desc_dkey(uint64_t (&v)[16])
{
    const int g = lane_id() >> 4;
    auto inlane = [&](int r, int r2) {
        const uint64_t a = v[r], b = v[r2];
        v[r] = dkey_max(a, b);
        v[r2] = dkey_min(a, b);
    };
    auto runs16 = [&](int from) {
#pragma unroll
        for (int stride = 8; stride > 0; stride >>= 1)
            if (stride <= from)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if ((r & stride) == 0)
                        inlane(r, r | stride);
    };
    // with lane group g ^ (lanes / 16), register 15 - r (mirror) or r; the
    // lower lane group keeps the larger key
    auto cross = [&](int lanes, bool mirror, bool lower) {
        uint64_t o[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[r] = shfl_xor_u64(v[mirror ? 15 - r : r], lanes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            v[r] = lower ? dkey_max(v[r], o[r]) : dkey_min(v[r], o[r]);
    };
#pragma unroll
    for (int size = 2; size <= 16; size <<= 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r & (size >> 1)) == 0)
                inlane(r, r ^ (size - 1));
        runs16(size >> 2);
    }
    cross(16, true, (g & 1) == 0);      // size 32: e ^ 31 = lane group g ^ 1, register 15 - r
    runs16(8);
    cross(48, true, g < 2);             // size 64: e ^ 63 = lane group g ^ 3, register 15 - r
    cross(16, false, (g & 1) == 0);     // stride 16
    runs16(8);
}

template <int R, typename T>
__device__ __forceinline__ void group4_sort_desc(T (&v)[R])
{
    const int g = lane_id() >> 4;
    constexpr int P = 4 * R;
    // Every compare-exchange is one compare, at most one lane-mask XOR (a
    // scalar op) and plain selects: the direction of a stage, where it depends
    // on the lane group, is a lane mask computed once per stage.
#pragma unroll
    for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= R) {
                // partner in lane group g ^ (stride / R); the lane keeps the
                // larger value iff (lower half) == (descending block)
                const int lm = 16 * (stride / R);
                const bool keep_min = (((g * R) & stride) == 0) != (((g * R) & size) == 0);
                // all R exchanges are issued before the first is used, so their
                // LDS round trips overlap
                T o[R];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    o[r] = g4_shfl(v[r], lm);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const bool take = (v[r] < o[r]) != keep_min;   // o is the one to keep
                    v[r] = take ? o[r] : v[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & stride) == 0) {
                        // ascending block: swap when a >= b (equal keys are identical)
                        const bool asc = ((g * R + r) & size) != 0;
                        const T a = v[r], b = v[r | stride];
                        const bool swap = (a < b) != asc;
                        v[r] = swap ? b : a;
                        v[r | stride] = swap ? a : b;
                    }
                }
            }
        }
    }
}

}  // namespace pkm

// dd_device.hpp - wave64 / workgroup building blocks shared by the gfx950
// kernels of libdmadesc (scans, reductions, key grouping, owner search).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dd {

constexpr int kWave = 64;

__device__ __forceinline__ int lane() { return (int)__lane_id(); }
__device__ __forceinline__ int wave() { return (int)(threadIdx.x / kWave); }

// Page rounding of one request range (NCCL course page, "IB Backend MR
// Cache": floor of the start to the page, cover of the end): the absolute
// start a = va_base + o widened to [lo, hi) of whole pages (in_page = page
// size - 1). Returns false, with lo = hi = 0, for an empty range or one
// whose start, end or rounded end wraps 2^64.
__device__ __forceinline__ bool page_round(uint64_t va_base, uint64_t o, uint64_t l,
                                           uint64_t in_page, uint64_t &lo, uint64_t &hi)
{
    const uint64_t a = va_base + o;
    const uint64_t last = a + l - 1;
    const bool bad = (l == 0) | (a < va_base) | (l > ~a) | ((last | in_page) == ~0ull);
    lo = bad ? 0 : (a & ~in_page);             // page floor of the start
    hi = bad ? 0 : (last | in_page) + 1;       // page cover of the end
    return !bad;
}

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v)
{
    const int ln = lane();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        T u = __shfl_up(v, (unsigned)d, kWave);
        if (ln >= d) v += u;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Exclusive prefix sum across a workgroup of kThreads threads. `scratch`
// holds kThreads/64 elements of LDS. Returns this thread's exclusive prefix
// and writes the workgroup total to *total (same value in every thread).
// Contains two barriers; every thread of the workgroup must call it.
template <int kThreads, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T *scratch, T *total)
{
    constexpr int kWaves = kThreads / kWave;
    T inc = wave_incl_scan(v);
    const int w = wave();
    if (lane() == kWave - 1) scratch[w] = inc;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        T s = scratch[k];
        before += (k < w) ? s : T(0);
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Largest r in [0, kN) with pre[r] <= key, for a non-decreasing pre[0..kN]
// whose first element is <= key. kN is a power of two.
template <int kN, typename T>
__device__ __forceinline__ int owner_of(const T *pre, T key)
{
    int r = 0;
#pragma unroll
    for (int step = kN / 2; step > 0; step >>= 1)
        r = (pre[r + step] <= key) ? r + step : r;
    return r;
}

// Lanes of this wave (among `active`) whose `key` equals this lane's key,
// from one ballot per key bit: a lane matches when it agrees on every bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key, bool on, int nbits, uint64_t active)
{
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t vote = __ballot(on && bit);
        m &= bit ? vote : ~vote;
    }
    return m;
}

}  // namespace dd

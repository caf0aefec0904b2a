// mr_lookup.hip - page-rounded containment lookup of request ranges in a
// sorted table of registered memory regions, for gfx950.
//
// Method ("NCCL 专家课程 26：GPUDirect RDMA、DMA-BUF、MR 与注册缓存",
// "IB Backend MR Cache" and "Communicator User Registration Cache"): widen the
// range to whole pages, then a region that fully contains the widened range
// is a hit (exact when both bounds coincide); partial overlap is a miss.
//
// Layout: one lane per request over structure-of-arrays columns, so each
// column load/store of a wave is one contiguous 64-element run. Every block
// first stages a splitter array -- every S-th region start, S a power of two
// chosen so at most kMaxSplitters fit in LDS -- then each lane does a
// branch-free binary search over the splitters in LDS followed by one over
// the <= S starts of the selected run in global memory (L2-resident: the
// whole table is at most a few MiB). Blocks loop over the batch so the
// splitter staging is paid once per block, not per 256 requests.
#include "dd_device.hpp"
#include "dd_internal.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMaxSplitters = 8192;   // 64 KiB of LDS

// Index of the last element <= key in a[0..cnt), given a[0] <= key; the trip
// count depends only on cnt, so lanes with equal cnt never diverge.
template <typename Ptr>
__device__ __forceinline__ uint64_t last_le(Ptr a, uint64_t cnt, uint64_t key)
{
    uint64_t idx = 0;
    while (cnt > 1) {
        const uint64_t half = cnt >> 1;
        idx = (a[idx + half] <= key) ? idx + half : idx;
        cnt -= half;
    }
    return idx;
}

__global__ __launch_bounds__(kThreads) void k_mr_lookup(
    const uint64_t *__restrict__ rs, const uint64_t *__restrict__ re,
    const uint32_t *__restrict__ rk, uint32_t nregions,
    uint32_t split_shift, uint32_t nsplit, uint32_t page_shift,
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len,
    uint64_t n, uint64_t va_base,
    int32_t *__restrict__ handle, uint32_t *__restrict__ lkey,
    uint8_t *__restrict__ kind, uint64_t *__restrict__ rbase,
    uint64_t *__restrict__ rend)
{
    extern __shared__ uint64_t spl[];
    for (uint32_t k = threadIdx.x; k < nsplit; k += kThreads)
        spl[k] = rs[(uint64_t)k << split_shift];
    __syncthreads();

    const uint64_t in_page = (1ull << page_shift) - 1;
    const uint64_t run = 1ull << split_shift;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const uint64_t o = off[i], l = len[i];
        const uint64_t a = va_base + o;
        int32_t h = -1;
        uint32_t key = 0;
        uint8_t kd = 0;        // MISS
        uint64_t lo = 0, hi = 0;

        // Invalid: empty, start wraps, end wraps, or rounded end wraps.
        bool bad = (l == 0) | (a < va_base) | (l > ~a);
        const uint64_t last = a + l - 1;
        bad |= ((last | in_page) == ~0ull);
        if (bad) {
            kd = 3;            // INVALID
        } else {
            lo = a & ~in_page;             // page floor of the start
            hi = (last | in_page) + 1;     // page cover of the end
            if (nsplit > 0 && spl[0] <= lo) {
                const uint64_t c = last_le(spl, nsplit, lo);      // splitter run
                const uint64_t b0 = c << split_shift;
                const uint64_t left = (uint64_t)nregions - b0;
                const uint64_t cnt = left < run ? left : run;
                const uint64_t r = b0 + last_le(rs + b0, cnt, lo); // last start <= lo
                const uint64_t e = re[r];
                if (hi <= e) {
                    h = (int32_t)r;
                    key = rk[r];
                    kd = (lo == rs[r] && hi == e) ? 1 : 2;   // EXACT : CONTAINED
                }
            }
        }
        handle[i] = h;
        lkey[i] = key;
        kind[i] = kd;
        rbase[i] = lo;
        rend[i] = hi;
    }
}

}  // namespace

hipError_t launch_mr_lookup(const LookupArgs &a, hipStream_t s)
{
    uint32_t shift = 0;
    while (((uint64_t)a.nregions + (1ull << shift) - 1) >> shift > kMaxSplitters) ++shift;
    const uint32_t nsplit = (uint32_t)(((uint64_t)a.nregions + (1ull << shift) - 1) >> shift);
    uint64_t blocks = (a.n + kThreads - 1) / kThreads;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_mr_lookup, dim3((unsigned)blocks), dim3(kThreads),
                       (size_t)nsplit * sizeof(uint64_t), s,
                       a.reg_start, a.reg_end, a.reg_lkey, a.nregions, shift, nsplit,
                       a.page_shift, a.off, a.len, a.n, a.va_base,
                       a.handle, a.lkey, a.kind, a.rbase, a.rend);
    return hipGetLastError();
}

}  // namespace dd

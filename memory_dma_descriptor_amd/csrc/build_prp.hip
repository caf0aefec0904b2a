// build_prp.hip - 64 KiB GPU-page physical-address table -> 4 KiB NVMe
// PRP1/PRP2 and chained PRP lists, for gfx950.
//
// Method (xNVMe "uPCIe CUDA", introduction and "Limitations"): GPU memory is
// described by one physical address per 64 KiB GPU page, and PRP entries are
// formed at 4 KiB granularity from the sub-page offsets inside each 64 KiB
// entry; a list page holds 512 entries. Chaining follows the NVMe PRP rule:
// the last entry of every non-final list page points to the next list page,
// so a non-final page carries 511 data entries and the final one up to 512.
//
// Three kernels, stream-ordered, no atomics:
//   k_prp_count  one lane per request: validity and list pages L; per-block sum
//   k_prp_scan   one workgroup: exclusive scan of the block sums -> first list
//                page of every block, and the batch total
//   k_prp_emit   per block of 256 requests: PRP1/PRP2/status, then the list
//                entries, load-balanced over entries (not requests): the
//                block's data entries form one index space that all 256 lanes
//                walk in steps of 256, each lane finding its request by a
//                binary search over the per-request entry offsets in LDS. The
//                table entries the block needs are staged in LDS once per
//                window of kWin GPU pages (each request's pages form one
//                contiguous run of the table), so every entry reads LDS, not
//                global memory.
#include "dd_device.hpp"
#include "dd_internal.h"

namespace dd {
namespace {

constexpr int kTile = 256;        // requests per block (= threads)
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 16;
constexpr int kWin = 2048;        // GPU pages staged per window (16 KiB LDS)

enum : uint8_t { kOk = 0, kEinval = 1, kErange = 2, kEnospc = 3 };

// Status and 4 KiB page count of one request.
__device__ __forceinline__ uint8_t decode(uint64_t o, uint64_t l, uint64_t heap,
                                          uint64_t &pages)
{
    pages = 0;
    if (l == 0 || (o & 3u) || l > ~o) return kEinval;
    if (o + l > heap) return kErange;
    pages = ((o & 4095u) + l + 4095u) >> 12;
    return kOk;
}

// List pages of a request with `pages` 4 KiB pages: entries m = pages - 1,
// pages L = ceil((m - 1) / 511) when pages >= 3.
__device__ __forceinline__ uint64_t list_pages(uint64_t pages)
{
    return pages >= 3 ? (pages - 2 + 510) / 511 : 0;
}

__global__ __launch_bounds__(kTile) void k_prp_count(
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len, uint64_t n,
    uint64_t heap, uint64_t *__restrict__ partial)
{
    __shared__ uint64_t wsum[kTile / kWave];
    const uint64_t i = (uint64_t)blockIdx.x * kTile + threadIdx.x;
    uint64_t lp = 0;
    if (i < n) {
        uint64_t pages;
        if (decode(off[i], len[i], heap, pages) == kOk) lp = list_pages(pages);
    }
    lp = wave_sum(lp);
    if (lane() == 0) wsum[wave()] = lp;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t s = 0;
        for (int k = 0; k < kTile / kWave; ++k) s += wsum[k];
        partial[blockIdx.x] = s;
    }
}

// Single workgroup: in-place exclusive scan of partial[0..nb), total -> *total.
__global__ __launch_bounds__(kScanThreads) void k_prp_scan(
    uint64_t *__restrict__ partial, uint64_t nb, uint64_t *__restrict__ total)
{
    __shared__ uint64_t scratch[kScanThreads / kWave];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nb; base += (uint64_t)kScanThreads * kScanItems) {
        const uint64_t b0 = base + (uint64_t)threadIdx.x * kScanItems;
        uint64_t v[kScanItems];
        uint64_t s = 0;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            v[k] = (b0 + k < nb) ? partial[b0 + k] : 0;
            s += v[k];
        }
        uint64_t chunk;
        uint64_t run = carry + block_excl_scan<kScanThreads>(s, scratch, &chunk);
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            if (b0 + k < nb) partial[b0 + k] = run;
            run += v[k];
        }
        carry += chunk;
    }
    if (threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(kTile) void k_prp_emit(
    const uint64_t *__restrict__ lut, uint64_t heap,
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len, uint64_t n,
    uint64_t bus, uint64_t *__restrict__ pool, uint64_t pool_pages,
    uint64_t *__restrict__ prp1, uint64_t *__restrict__ prp2,
    uint8_t *__restrict__ status, const uint64_t *__restrict__ block_slot)
{
    __shared__ uint64_t s_moff[kTile + 1];   // exclusive prefix of data entries
    __shared__ uint64_t s_foff[kTile + 1];   // exclusive prefix of staged GPU pages
    __shared__ uint64_t s_pb[kTile];         // heap offset of the request's 4 KiB page 0
    __shared__ uint64_t s_slot[kTile];       // first list page
    __shared__ uint64_t s_lp[kTile];         // list pages
    __shared__ uint64_t s_lut[kWin];
    __shared__ uint64_t s_red[kTile / kWave];
    __shared__ uint64_t s_bound[2];

    const int t = threadIdx.x;
    const uint64_t i = (uint64_t)blockIdx.x * kTile + t;

    uint64_t o = 0, l = 0, pages = 0;
    uint8_t st = kEinval;
    if (i < n) {
        o = off[i];
        l = len[i];
        st = decode(o, l, heap, pages);
    }
    const uint64_t lp = (st == kOk) ? list_pages(pages) : 0;
    uint64_t lp_tot;
    const uint64_t slot = block_slot[blockIdx.x] + block_excl_scan<kTile>(lp, s_red, &lp_tot);
    if (lp != 0 && slot + lp > pool_pages) st = kEnospc;     // refused; still took its slots
    const bool lists = (st == kOk) && lp != 0;

    const uint64_t pb = o & ~4095ull;
    const uint64_t fa = (pb + 4096) >> 16;                    // GPU page of 4 KiB page 1
    const uint64_t m = lists ? pages - 1 : 0;
    const uint64_t fr = lists ? ((o + l - 1) >> 16) - fa + 1 : 0;
    uint64_t m_tot, f_tot;
    const uint64_t moff = block_excl_scan<kTile>(m, s_red, &m_tot);
    const uint64_t foff = block_excl_scan<kTile>(fr, s_red, &f_tot);
    s_moff[t] = moff;
    s_foff[t] = foff;
    if (t == 0) {
        s_moff[kTile] = m_tot;
        s_foff[kTile] = f_tot;
    }
    s_pb[t] = pb;
    s_slot[t] = slot;
    s_lp[t] = lp;

    if (i < n) {
        uint64_t p1 = 0, p2 = 0;
        if (st == kOk) {
            p1 = lut[o >> 16] + (o & 0xFFFFu);
            if (pages == 2) {
                const uint64_t x = pb + 4096;
                p2 = lut[x >> 16] + (x & 0xFFFFu);
            } else if (pages >= 3) {
                p2 = bus + slot * 4096;
            }
        }
        prp1[i] = p1;
        prp2[i] = p2;
        status[i] = st;
    }
    __syncthreads();
    if (m_tot == 0) return;                                    // uniform

    for (uint64_t w0 = 0; w0 < f_tot; w0 += kWin) {
        const uint64_t wn = (f_tot - w0 < (uint64_t)kWin) ? f_tot - w0 : (uint64_t)kWin;
        // Stage the table entries of GPU-page positions [w0, w0 + wn).
        for (uint64_t j = t; j < wn; j += kTile) {
            const uint64_t g = w0 + j;
            const int r = owner_of<kTile>(s_foff, g);
            s_lut[j] = lut[((s_pb[r] + 4096) >> 16) + (g - s_foff[r])];
        }
        // Entry range whose GPU pages fall in this window: first entry at or
        // after GPU-page position w0 and w0 + kWin.
        if (t < 2) {
            const uint64_t g = w0 + (t ? (uint64_t)kWin : 0);
            uint64_t e = m_tot;
            if (g < f_tot) {
                const int r = owner_of<kTile>(s_foff, g);
                const uint64_t frame = ((s_pb[r] + 4096) >> 16) + (g - s_foff[r]);
                const uint64_t start = frame << 16;
                const uint64_t j = (start <= s_pb[r] + 4096) ? 0 : (start - s_pb[r]) / 4096 - 1;
                e = s_moff[r] + j;
            }
            s_bound[t] = e;
        }
        __syncthreads();
        const uint64_t e_hi = s_bound[1];
        for (uint64_t e = s_bound[0] + t; e < e_hi; e += kTile) {
            const int r = owner_of<kTile>(s_moff, e);
            const uint64_t j = e - s_moff[r];                   // data entry j = page j+1
            const uint64_t pb_r = s_pb[r];
            const uint64_t x = pb_r + 4096 * (j + 1);
            const uint64_t g = s_foff[r] + (x >> 16) - ((pb_r + 4096) >> 16);
            const uint64_t v = s_lut[g - w0] + (x & 0xFFFFu);
            const uint64_t lp_r = s_lp[r];
            uint64_t tp = j / 511;
            if (tp > lp_r - 1) tp = lp_r - 1;
            const uint64_t pos = j - 511 * tp;
            const uint64_t sl = s_slot[r] + tp;
            pool[sl * 512 + pos] = v;
            if (pos == 510 && tp + 1 < lp_r) pool[sl * 512 + 511] = bus + (sl + 1) * 4096;
        }
        __syncthreads();
    }
}

}  // namespace

size_t ws_build_prp(uint64_t n)
{
    const uint64_t nb = (n + kTile - 1) / kTile;
    return align256(nb * sizeof(uint64_t));
}

hipError_t launch_build_prp(const PrpArgs &a, hipStream_t s)
{
    const uint64_t heap = a.lut_entries << 16;
    const uint64_t nb = (a.n + kTile - 1) / kTile;
    uint64_t *partial = static_cast<uint64_t *>(a.ws);
    if (nb > 0) {
        hipLaunchKernelGGL(k_prp_count, dim3((unsigned)nb), dim3(kTile), 0, s,
                           a.off, a.len, a.n, heap, partial);
    }
    hipLaunchKernelGGL(k_prp_scan, dim3(1), dim3(kScanThreads), 0, s, partial, nb,
                       a.total_pages);
    if (nb > 0) {
        hipLaunchKernelGGL(k_prp_emit, dim3((unsigned)nb), dim3(kTile), 0, s,
                           a.lut, heap, a.off, a.len, a.n, a.list_bus_base, a.pool,
                           a.pool_pages, a.prp1, a.prp2, a.status, partial);
    }
    return hipGetLastError();
}

}  // namespace dd

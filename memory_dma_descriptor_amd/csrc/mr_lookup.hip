// mr_lookup.hip - page-rounded containment lookup of request ranges in a
// sorted table of registered memory regions, for gfx950.
//
// Method ("NCCL 专家课程 26：GPUDirect RDMA、DMA-BUF、MR 与注册缓存",
// "IB Backend MR Cache" and "Communicator User Registration Cache"): widen the
// range to whole pages, then a region that fully contains the widened range
// is a hit (exact when both bounds coincide); partial overlap is a miss.
//
// Layout: structure-of-arrays columns; every column load and store of a wave
// covers one contiguous run. Two kernels:
//
//  * k_lookup_lds, for tables of up to 4,096 regions (20 bytes per region;
//    MI355X has 160 KiB of LDS per CU): one 1,024-thread block per CU copies
//    the whole table into LDS once, builds a bucket index over the region
//    starts, and then answers requests in a grid-stride loop. A query reads
//    two index entries and searches only its bucket's run of regions (one or
//    two on evenly spread tables) instead of the whole table: a wave's random
//    LDS reads then collide in far fewer banks. All table reads are LDS
//    reads, so no random global gathers reach the texture address unit.
//  * k_lookup_big, for larger tables: every block stages every 8th region
//    start in LDS (at most kMaxSplitters splitters = 64 KiB, with a bucket
//    index over them); a lane finds its splitter in LDS, then reads the 8
//    starts of that run in one 64-byte read (the table is L2-resident).
//    With a workspace, k_rec_build first writes one 64-byte record per run
//    of 4 regions (the other three starts as page deltas from the first, the
//    four ends and the four keys), LDS holds every 4th start, and a request
//    is answered from its run's record in one round of four independent
//    16-byte loads. The time of this kernel goes to dependent rounds of
//    gathers (each waits behind the column stream's HBM misses in the vector
//    memory pipeline), not to the number of loads in a round.
//
// The searches are branch-free: the trip count depends only on the length
// searched, so lanes of a wave never diverge in them.
#include "dd_device.hpp"
#include "dd_internal.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr int kThreadsLds = 1024;            // one block per CU: 16 waves
constexpr uint32_t kBuckets = 4096;          // bucket index over the region starts (LDS kernel)
constexpr int kPerLane = 4;                  // requests per lane per trip (LDS kernel)
static_assert(kPerLane % 2 == 0, "lanes take requests in pairs");

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kMaxSplitters = 8192;   // 64 KiB of LDS
constexpr uint32_t kMaxRecSplitters = 16384;   // 128 KiB of LDS (record path)
constexpr uint32_t kRecRun = 4;              // regions per 64-byte record
constexpr uint32_t kRecBytes = 64;
constexpr uint32_t kLdsRegions = 4096;       // largest table k_lookup_lds holds

// Index of the last element <= key in a[0..cnt), given a[0] <= key.
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

__device__ __forceinline__ void put(uint64_t i, int32_t h, uint32_t key, uint8_t kd,
                                    uint64_t lo, uint64_t hi, int32_t *__restrict__ handle,
                                    uint32_t *__restrict__ lkey, uint8_t *__restrict__ kind,
                                    uint64_t *__restrict__ rbase, uint64_t *__restrict__ rend)
{
    handle[i] = h;
    lkey[i] = key;
    kind[i] = kd;
    rbase[i] = lo;
    rend[i] = hi;
}

__global__ __launch_bounds__(kThreadsLds) void k_lookup_lds(
    const uint64_t *__restrict__ rs, const uint64_t *__restrict__ re,
    const uint32_t *__restrict__ rk, uint32_t nregions, uint32_t page_shift,
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len,
    uint64_t n, uint64_t va_base,
    int32_t *__restrict__ handle, uint32_t *__restrict__ lkey,
    uint8_t *__restrict__ kind, uint64_t *__restrict__ rbase,
    uint64_t *__restrict__ rend, bool aligned)
{
    extern __shared__ uint64_t lds[];
    uint64_t *s_start = lds;
    uint64_t *s_end = lds + nregions;
    uint32_t *s_key = reinterpret_cast<uint32_t *>(lds + 2 * (uint64_t)nregions);
    uint16_t *s_idx = reinterpret_cast<uint16_t *>(s_key + nregions + (nregions & 1));
    for (uint32_t k = threadIdx.x; k < nregions; k += kThreadsLds) {
        s_start[k] = rs[k];
        s_end[k] = re[k];
        s_key[k] = rk[k];
    }
    __syncthreads();
    // Bucket index: the starts' span [base, last start] cut into kBuckets
    // buckets of 2^bs bytes; s_idx[b] = first region whose start is at or
    // past bucket b. The last region starting at or before x then lies in
    // [s_idx[b] - 1, s_idx[b + 1]) for x's bucket b: a query reads two index
    // entries and searches that short run (usually one or two regions)
    // instead of the whole table, so far fewer of a wave's random LDS reads
    // collide in the same banks.
    const uint64_t base = nregions ? s_start[0] : 0;
    uint32_t bs = 0;
    if (nregions) {
        const uint64_t span = s_start[nregions - 1] - base;
        while ((span >> bs) >= kBuckets) ++bs;
        for (uint32_t b = threadIdx.x; b <= kBuckets; b += kThreadsLds) {
            // Start of bucket b, saturating at 2^64 - 1 (then no region is past it).
            const bool over = bs && ((uint64_t)b >> (64 - bs)) != 0;
            const uint64_t width = over ? ~0ull : (uint64_t)b << bs;
            const uint64_t x = width > ~base ? ~0ull : base + width;
            uint32_t lo = 0, cnt = nregions;                  // first start >= x
            while (cnt > 0) {
                const uint32_t half = cnt >> 1;
                if (s_start[lo + half] < x) {
                    lo += half + 1;
                    cnt -= half + 1;
                } else {
                    cnt = half;
                }
            }
            s_idx[b] = (uint16_t)lo;
        }
    }
    __syncthreads();

    // A wave takes 256 consecutive requests per trip; request k of a lane is
    // wb + (k >> 1) * 128 + 2 * lane + (k & 1), so each of the wave's column
    // loads and stores covers one contiguous run (1 KiB for the 8-byte
    // columns, 16 bytes per lane) and every 64-byte segment is written whole
    // by one instruction: a mapping whose store instruction fills only part
    // of each segment (4 consecutive requests per lane: half of every
    // 32 bytes of rbase) costs about 10 % more, 8 consecutive requests per
    // lane 3x. All loads are issued before any search.
    const uint64_t in_page = (1ull << page_shift) - 1;
    const uint64_t span = (uint64_t)kThreadsLds * kPerLane;
    const int ln = (int)(threadIdx.x & 63), wv = (int)(threadIdx.x >> 6);
    for (uint64_t c = (uint64_t)blockIdx.x * span; c < n; c += (uint64_t)gridDim.x * span) {
        const uint64_t wb = c + (uint64_t)wv * (64 * kPerLane);     // the wave's requests
        if (wb >= n) break;
        const bool whole = aligned && wb + 64 * kPerLane <= n;      // uniform per wave
        uint64_t o[kPerLane], l[kPerLane];
        if (whole) {
            // Columns are streamed (non-temporal): nothing reads them again.
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const u64x2 oa = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(off + wb + p * 128 + 2 * ln));
                o[2 * p] = oa.x; o[2 * p + 1] = oa.y;
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const u64x2 la = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(len + wb + p * 128 + 2 * ln));
                l[2 * p] = la.x; l[2 * p + 1] = la.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const uint64_t i = wb + (k >> 1) * 128 + 2 * ln + (k & 1);
                o[k] = i < n ? off[i] : 0;
                l[k] = i < n ? len[i] : 0;
            }
        }
        int32_t h[kPerLane];
        uint32_t key[kPerLane];
        uint8_t kd[kPerLane];
        uint64_t lo[kPerLane], hi[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const bool ok = page_round(va_base, o[k], l[k], in_page, lo[k], hi[k]);
            h[k] = -1;
            key[k] = 0;
            kd[k] = ok ? 0 : 3;                  // MISS : INVALID
            if (ok && nregions > 0 && base <= lo[k]) {
                uint64_t b = (lo[k] - base) >> bs;
                b = b < kBuckets ? b : kBuckets - 1;
                const uint32_t i0 = s_idx[b], i1 = s_idx[b + 1];
                const uint32_t first = i0 ? i0 - 1 : 0;
                const uint32_t r = first + (uint32_t)last_le(s_start + first, i1 - first, lo[k]);
                const uint64_t e = s_end[r];
                if (hi[k] <= e) {
                    h[k] = (int32_t)r;
                    key[k] = s_key[r];
                    kd[k] = (lo[k] == s_start[r] && hi[k] == e) ? 1 : 2;   // EXACT : CONTAINED
                }
            }
        }
        if (whole) {
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store(u64x2{lo[2 * p], lo[2 * p + 1]}, reinterpret_cast<u64x2 *>(rbase + i));
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store(u64x2{hi[2 * p], hi[2 * p + 1]}, reinterpret_cast<u64x2 *>(rend + i));
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store(
                    (uint64_t)(uint32_t)h[2 * p] | ((uint64_t)(uint32_t)h[2 * p + 1] << 32),
                    reinterpret_cast<uint64_t *>(handle + i));
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store((uint64_t)key[2 * p] | ((uint64_t)key[2 * p + 1] << 32),
                                            reinterpret_cast<uint64_t *>(lkey + i));
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store((uint16_t)(kd[2 * p] | (kd[2 * p + 1] << 8)),
                                            reinterpret_cast<uint16_t *>(kind + i));
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const uint64_t i = wb + (k >> 1) * 128 + 2 * ln + (k & 1);
                if (i < n) put(i, h[k], key[k], kd[k], lo[k], hi[k], handle, lkey, kind, rbase, rend);
            }
        }
    }
}

// Larger tables (k_lookup_big): the region starts do not fit LDS, so LDS
// holds every 8th start ("splitters", up to kMaxSplitters = 64 KiB) and a
// bucket index over them; a request finds its splitter c in LDS, then reads
// the 8 starts of run c as one 64-byte read (four 16-byte loads), counts
// those at or below its rounded base, and reads the end and key of that
// region. Three dependent global rounds per request (columns, run, region),
// four requests per lane in flight, columns read and written as in
// k_lookup_lds. Tables with more than 8 * kMaxSplitters regions put every
// 2^s-th start in LDS and narrow the run by a global binary search first.
constexpr uint32_t kRun = 8;                 // starts read per request in one go

__device__ __forceinline__ uint32_t count_le(const uint64_t (&t)[kRun], uint64_t key)
{
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < (int)kRun; ++j) c += t[j] <= key ? 1u : 0u;
    return c;
}

// Record copy of the table for k_lookup_big<true>. With P = 2^page_shift
// and B = ceil(start[4j] / P), record j (64 bytes) describes regions
// 4j .. 4j + 3:
//   u32 d[1..3]  ceil(start[4j + i] / P) - B: for a page-aligned rounded base
//                lo, start <= lo exactly when its d <= lo / P - B.
//                0xFFFFFFFF past the table (never at or below a base).
//   u32 flags    bit i: start[4j + i] is a multiple of P (with d equal to
//                lo / P - B this makes start == lo: an EXACT bound); bit 4
//                ("wide"): some delta does not fit 32 bits, and the lookup
//                reads that run's starts from the table instead.
//   u64 end[0..3], then u32 key[0..3] (0 past the table).
// One thread per record.
constexpr uint32_t kWide = 16u;

__global__ __launch_bounds__(kThreads) void k_rec_build(
    const uint64_t *__restrict__ rs, const uint64_t *__restrict__ re,
    const uint32_t *__restrict__ rk, uint32_t nregions, uint32_t page_shift,
    uint32_t *__restrict__ rec)
{
    const uint64_t nrec = ((uint64_t)nregions + kRecRun - 1) / kRecRun;
    const uint64_t in_page = (1ull << page_shift) - 1;
    for (uint64_t j = (uint64_t)blockIdx.x * kThreads + threadIdx.x; j < nrec;
         j += (uint64_t)gridDim.x * kThreads) {
        const uint64_t r0 = j * kRecRun;
        uint64_t e[kRecRun];
        uint32_t k[kRecRun], d[kRecRun], flags = 0;
        const uint64_t s0 = rs[r0];
        const uint64_t base = (s0 >> page_shift) + ((s0 & in_page) != 0);
#pragma unroll
        for (uint32_t i = 0; i < kRecRun; ++i) {
            const bool in = r0 + i < nregions;
            const uint64_t st = in ? rs[r0 + i] : 0;
            e[i] = in ? re[r0 + i] : 0;
            k[i] = in ? rk[r0 + i] : 0;
            const uint64_t up = (st >> page_shift) + ((st & in_page) != 0);
            const uint64_t delta = up - base;      // wraps on an unsorted table: then "wide"
            d[i] = !in ? 0xFFFFFFFFu : delta >= 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)delta;
            if (in && delta >= 0xFFFFFFFFull) flags |= kWide;
            if (in && (st & in_page) == 0) flags |= 1u << i;
        }
        u32x4 *q = reinterpret_cast<u32x4 *>(rec + j * (kRecBytes / 4));
        q[0] = u32x4{d[1], d[2], d[3], flags};
        reinterpret_cast<u64x2 *>(q)[1] = u64x2{e[0], e[1]};
        reinterpret_cast<u64x2 *>(q)[2] = u64x2{e[2], e[3]};
        q[3] = u32x4{k[0], k[1], k[2], k[3]};
    }
}

template <bool kRec>
__global__ __launch_bounds__(kThreadsLds) void k_lookup_big(
    const uint64_t *__restrict__ rs, const uint64_t *__restrict__ re,
    const uint32_t *__restrict__ rk, uint32_t nregions, uint32_t split_shift,
    uint32_t nsplit, uint32_t page_shift,
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len,
    uint64_t n, uint64_t va_base,
    int32_t *__restrict__ handle, uint32_t *__restrict__ lkey,
    uint8_t *__restrict__ kind, uint64_t *__restrict__ rbase,
    uint64_t *__restrict__ rend, bool aligned, const uint32_t *__restrict__ rec)
{
    constexpr uint32_t kNarrow = kRec ? kRecRun : kRun;   // run length after narrowing
    extern __shared__ uint64_t lds[];
    uint64_t *spl = lds;                                          // nsplit starts
    uint16_t *s_idx = reinterpret_cast<uint16_t *>(lds + nsplit); // kBuckets + 1
    for (uint32_t k = threadIdx.x; k < nsplit; k += kThreadsLds)
        spl[k] = rs[(uint64_t)k << split_shift];
    __syncthreads();
    // Bucket index over the splitters, as k_lookup_lds builds over starts:
    // s_idx[b] = first splitter at or past bucket b of the splitters' span.
    const uint64_t base = spl[0];
    uint32_t bs = 0;
    {
        const uint64_t span = spl[nsplit - 1] - base;
        while ((span >> bs) >= kBuckets) ++bs;
        for (uint32_t b = threadIdx.x; b <= kBuckets; b += kThreadsLds) {
            const bool over = bs && ((uint64_t)b >> (64 - bs)) != 0;
            const uint64_t width = over ? ~0ull : (uint64_t)b << bs;
            const uint64_t x = width > ~base ? ~0ull : base + width;
            uint32_t lo = 0, cnt = nsplit;
            while (cnt > 0) {
                const uint32_t half = cnt >> 1;
                if (spl[lo + half] < x) {
                    lo += half + 1;
                    cnt -= half + 1;
                } else {
                    cnt = half;
                }
            }
            s_idx[b] = (uint16_t)lo;
        }
    }
    __syncthreads();

    const uint64_t in_page = (1ull << page_shift) - 1;
    const uint64_t span = (uint64_t)kThreadsLds * kPerLane;
    const uint64_t runlen = 1ull << split_shift;                  // starts per splitter
    const int ln = (int)(threadIdx.x & 63), wv = (int)(threadIdx.x >> 6);
    for (uint64_t c0 = (uint64_t)blockIdx.x * span; c0 < n; c0 += (uint64_t)gridDim.x * span) {
        const uint64_t wb = c0 + (uint64_t)wv * (64 * kPerLane);
        if (wb >= n) break;
        const bool whole = aligned && wb + 64 * kPerLane <= n;   // uniform per wave
        uint64_t o[kPerLane], l[kPerLane];
        if (whole) {
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const u64x2 oa = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(off + wb + p * 128 + 2 * ln));
                o[2 * p] = oa.x; o[2 * p + 1] = oa.y;
            }
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const u64x2 la = __builtin_nontemporal_load(reinterpret_cast<const u64x2 *>(len + wb + p * 128 + 2 * ln));
                l[2 * p] = la.x; l[2 * p + 1] = la.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const uint64_t i = wb + (k >> 1) * 128 + 2 * ln + (k & 1);
                o[k] = i < n ? off[i] : 0;
                l[k] = i < n ? len[i] : 0;
            }
        }
        uint64_t lo[kPerLane], hi[kPerLane], at[kPerLane], sat[kPerLane];
        bool valid[kPerLane], cand[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            valid[k] = page_round(va_base, o[k], l[k], in_page, lo[k], hi[k]);
            cand[k] = valid[k] && lo[k] >= base;
            // Splitter c: the last splitter at or before lo (LDS).
            uint32_t c = 0;
            if (cand[k]) {
                uint64_t b = (lo[k] - base) >> bs;
                b = b < kBuckets ? b : kBuckets - 1;
                const uint32_t i0 = s_idx[b], i1 = s_idx[b + 1];
                const uint32_t first = i0 ? i0 - 1 : 0;
                c = first + (uint32_t)last_le(spl + first, i1 - first, lo[k]);
            }
            at[k] = (uint64_t)c << split_shift;
            sat[k] = spl[c];                      // start of region at[k]
            // Runs of more than kNarrow starts: narrow to kNarrow by a search
            // over every kNarrow-th start of the run in global memory.
            uint64_t cnt = (uint64_t)nregions - at[k];
            cnt = cnt < runlen ? cnt : runlen;
            if (cand[k] && runlen > kNarrow) {
                uint64_t step_at = 0, m = (cnt + kNarrow - 1) / kNarrow;
                while (m > 1) {
                    const uint64_t half = m >> 1;
                    const uint64_t v = rs[at[k] + (step_at + half) * kNarrow];
                    if (v <= lo[k]) {
                        step_at += half;
                        sat[k] = v;
                    }
                    m -= half;
                }
                at[k] += step_at * kNarrow;
            }
        }
        int32_t h[kPerLane];
        uint32_t key[kPerLane];
        uint8_t kd[kPerLane];
        if constexpr (kRec) {
            // One round: the run's whole record (a non-candidate reads record
            // 0, so the loads stay unconditional).
            u32x4 hd[kPerLane], kk[kPerLane];
            u64x2 ea[kPerLane], eb[kPerLane];
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const u32x4 *q = reinterpret_cast<const u32x4 *>(
                    rec + (cand[k] ? at[k] / kRecRun : 0) * (kRecBytes / 4));
                hd[k] = q[0];
                ea[k] = reinterpret_cast<const u64x2 *>(q)[1];
                eb[k] = reinterpret_cast<const u64x2 *>(q)[2];
                kk[k] = q[3];
            }
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const uint64_t base_pg = (sat[k] >> page_shift) + ((sat[k] & in_page) != 0);
                const uint64_t qd = (lo[k] >> page_shift) - base_pg;     // >= 0: sat <= lo
                const uint32_t q32 = qd < 0xFFFFFFFEull ? (uint32_t)qd : 0xFFFFFFFEu;
                uint32_t c = (hd[k].x <= q32 ? 1u : 0u) + (hd[k].y <= q32 ? 1u : 0u) +
                             (hd[k].z <= q32 ? 1u : 0u);
                const uint32_t dc = c == 0 ? 0u : c == 1 ? hd[k].x : c == 2 ? hd[k].y : hd[k].z;
                bool exact_lo = ((hd[k].w >> c) & 1u) && (uint64_t)dc == qd;
                if (cand[k] && (hd[k].w & kWide)) {
                    // Deltas beyond 32 bits: count the run's starts exactly.
                    uint64_t sc = sat[k];
                    c = 0;
#pragma unroll
                    for (uint32_t i = 1; i < kRecRun; ++i) {
                        const bool in = at[k] + i < nregions;
                        const uint64_t v = in ? rs[at[k] + i] : ~0ull;
                        if (in && v <= lo[k]) {
                            c = i;
                            sc = v;
                        }
                    }
                    exact_lo = lo[k] == sc;
                }
                const uint64_t e = c == 0 ? ea[k].x : c == 1 ? ea[k].y : c == 2 ? eb[k].x : eb[k].y;
                const uint32_t kv = c == 0 ? kk[k].x : c == 1 ? kk[k].y : c == 2 ? kk[k].z : kk[k].w;
                const bool hit = cand[k] && hi[k] <= e;
                h[k] = hit ? (int32_t)(at[k] + c) : -1;
                key[k] = hit ? kv : 0;
                kd[k] = !valid[k] ? 3 : !hit ? 0 : (exact_lo && hi[k] == e) ? 1 : 2;
            }
        } else {
            // The kRun starts from `at` (past the table: never at or below lo).
            uint32_t r[kPerLane];
            uint64_t s0[kPerLane];
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                uint64_t t[kRun];
                if (cand[k] && at[k] + kRun <= nregions && aligned) {
                    const u64x2 *q = reinterpret_cast<const u64x2 *>(rs + at[k]);
#pragma unroll
                    for (int j = 0; j < (int)kRun / 2; ++j) {
                        const u64x2 v = q[j];
                        t[2 * j] = v.x;
                        t[2 * j + 1] = v.y;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < (int)kRun; ++j)
                        t[j] = cand[k] && at[k] + j < nregions ? rs[at[k] + j] : ~0ull;
                }
                const uint32_t c = cand[k] ? count_le(t, lo[k]) : 1u;   // >= 1: t[0] <= lo
                r[k] = (uint32_t)at[k] + c - 1;
                uint64_t sel = t[0];
#pragma unroll
                for (int j = 1; j < (int)kRun; ++j) sel = (uint32_t)j == c - 1 ? t[j] : sel;
                s0[k] = sel;
            }
            uint64_t e0[kPerLane];
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                e0[k] = cand[k] ? re[r[k]] : 0;
                key[k] = cand[k] ? rk[r[k]] : 0;
            }
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const bool hit = cand[k] && hi[k] <= e0[k];
                h[k] = hit ? (int32_t)r[k] : -1;
                key[k] = hit ? key[k] : 0;
                kd[k] = !valid[k] ? 3 : !hit ? 0 : (lo[k] == s0[k] && hi[k] == e0[k]) ? 1 : 2;
            }
        }
        if (whole) {
#pragma unroll
            for (int p = 0; p < kPerLane / 2; ++p) {
                const uint64_t i = wb + p * 128 + 2 * ln;
                __builtin_nontemporal_store(u64x2{lo[2 * p], lo[2 * p + 1]}, reinterpret_cast<u64x2 *>(rbase + i));
                __builtin_nontemporal_store(u64x2{hi[2 * p], hi[2 * p + 1]}, reinterpret_cast<u64x2 *>(rend + i));
                __builtin_nontemporal_store(
                    (uint64_t)(uint32_t)h[2 * p] | ((uint64_t)(uint32_t)h[2 * p + 1] << 32),
                    reinterpret_cast<uint64_t *>(handle + i));
                __builtin_nontemporal_store((uint64_t)key[2 * p] | ((uint64_t)key[2 * p + 1] << 32),
                                            reinterpret_cast<uint64_t *>(lkey + i));
                __builtin_nontemporal_store((uint16_t)(kd[2 * p] | (kd[2 * p + 1] << 8)),
                                            reinterpret_cast<uint16_t *>(kind + i));
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const uint64_t i = wb + (k >> 1) * 128 + 2 * ln + (k & 1);
                if (i < n) put(i, h[k], key[k], kd[k], lo[k], hi[k], handle, lkey, kind, rbase, rend);
            }
        }
    }
}

// Region r breaks the table rules when it is empty, a bound is not a page
// multiple, or it overlaps region r + 1 (or starts before it ends). The
// smallest such r lands in *first_bad (a minimum is order-independent).
__global__ __launch_bounds__(kThreads) void k_table_check(
    const uint64_t *__restrict__ rs, const uint64_t *__restrict__ re, uint32_t nregions,
    uint64_t in_page, unsigned long long *__restrict__ first_bad)
{
    for (uint64_t r = (uint64_t)blockIdx.x * kThreads + threadIdx.x; r < nregions;
         r += (uint64_t)gridDim.x * kThreads) {
        const uint64_t s0 = rs[r], e0 = re[r];
        bool bad = s0 >= e0 || ((s0 | e0) & in_page) != 0;
        if (r + 1 < nregions) bad = bad || e0 > rs[r + 1];
        if (bad) atomicMin(first_bad, (unsigned long long)r);
    }
}

__global__ void k_set_u64(unsigned long long *p, unsigned long long v) { *p = v; }

}  // namespace

hipError_t launch_table_check(const uint64_t *rs, const uint64_t *re, uint32_t nregions,
                              uint32_t page_shift, uint64_t *scratch, uint64_t *host_result,
                              hipStream_t s)
{
    auto *fb = reinterpret_cast<unsigned long long *>(scratch);
    hipLaunchKernelGGL(k_set_u64, dim3(1), dim3(1), 0, s, fb, ~0ull);
    if (nregions > 0) {
        uint64_t blocks = ((uint64_t)nregions + kThreads - 1) / kThreads;
        if (blocks > 1024) blocks = 1024;
        hipLaunchKernelGGL(k_table_check, dim3((unsigned)blocks), dim3(kThreads), 0, s, rs, re,
                           nregions, (1ull << page_shift) - 1, fb);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(host_result, scratch, sizeof(uint64_t),
                                            hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

hipError_t launch_mr_lookup(const LookupArgs &a, hipStream_t s)
{
    int dev = 0, cus = 0, lds_max = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&lds_max, hipDeviceAttributeSharedMemPerBlockOptin, dev);
    if (e != hipSuccess) return e;

    const size_t table_bytes = (size_t)a.nregions * 20 + (a.nregions & 1) * 4 +
                               (size_t)(kBuckets + 1) * sizeof(uint16_t);
    if (a.nregions <= kLdsRegions && table_bytes <= (size_t)lds_max) {
        // One 1,024-thread block per CU holds the table and its bucket index;
        // each answers a grid-stride share.
        const size_t bytes = table_bytes;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_lookup_lds),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        uint64_t blocks = (a.n + (uint64_t)kThreadsLds * kPerLane - 1) / ((uint64_t)kThreadsLds * kPerLane);
        const uint64_t cap = (uint64_t)cus;
        if (blocks > cap) blocks = cap;
        // Columns that allow the vector accesses (16 bytes for off, len,
        // rbase and rend, 8 for handle and lkey, 2 for kind) take the vector
        // path; any other alignment is served element by element.
        auto al = [](const void *p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) == 0; };
        const bool aligned = al(a.off, 15) && al(a.len, 15) && al(a.handle, 15) &&
                             al(a.lkey, 7) && al(a.kind, 1) && al(a.rbase, 15) && al(a.rend, 15);
        hipLaunchKernelGGL(k_lookup_lds, dim3((unsigned)blocks), dim3(kThreadsLds), bytes, s,
                           a.reg_start, a.reg_end, a.reg_lkey, a.nregions, a.page_shift,
                           a.off, a.len, a.n, a.va_base, a.handle, a.lkey, a.kind, a.rbase,
                           a.rend, aligned);
        return hipGetLastError();
    }
    auto al = [](const void *p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) == 0; };
    const bool cols_aligned = al(a.off, 15) && al(a.len, 15) && al(a.handle, 15) &&
                              al(a.lkey, 7) && al(a.kind, 1) && al(a.rbase, 15) && al(a.rend, 15);
    uint64_t blocks = (a.n + (uint64_t)kThreadsLds * kPerLane - 1) / ((uint64_t)kThreadsLds * kPerLane);
    if (blocks > (uint64_t)cus) blocks = (uint64_t)cus;
    // Record path: every 2^shift-th start in LDS (at least every 4th).
    uint32_t rshift = 2;
    while (((uint64_t)a.nregions + (1ull << rshift) - 1) >> rshift > kMaxRecSplitters) ++rshift;
    const uint32_t rsplit = (uint32_t)(((uint64_t)a.nregions + (1ull << rshift) - 1) >> rshift);
    const size_t rbytes = (size_t)rsplit * sizeof(uint64_t) + (size_t)(kBuckets + 1) * sizeof(uint16_t);
    if (a.rec && rbytes <= (size_t)lds_max) {
        const uint32_t shift = rshift, nsplit = rsplit;
        const size_t bytes = rbytes;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_lookup_big<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        const uint64_t nrec = ((uint64_t)a.nregions + kRecRun - 1) / kRecRun;
        uint64_t rb = (nrec + kThreads - 1) / kThreads;
        if (rb > 1024) rb = 1024;
        auto *rec = reinterpret_cast<uint32_t *>(a.rec);
        hipLaunchKernelGGL(k_rec_build, dim3((unsigned)rb), dim3(kThreads), 0, s,
                           a.reg_start, a.reg_end, a.reg_lkey, a.nregions, a.page_shift, rec);
        hipLaunchKernelGGL(k_lookup_big<true>, dim3((unsigned)blocks), dim3(kThreadsLds), bytes, s,
                           a.reg_start, a.reg_end, a.reg_lkey, a.nregions, shift, nsplit,
                           a.page_shift, a.off, a.len, a.n, a.va_base,
                           a.handle, a.lkey, a.kind, a.rbase, a.rend, cols_aligned,
                           (const uint32_t *)rec);
        return hipGetLastError();
    }
    // Every 2^shift-th start in LDS (at least every kRun-th).
    uint32_t shift = 3;
    while (((uint64_t)a.nregions + (1ull << shift) - 1) >> shift > kMaxSplitters) ++shift;
    const uint32_t nsplit = (uint32_t)(((uint64_t)a.nregions + (1ull << shift) - 1) >> shift);
    const size_t bytes = (size_t)nsplit * sizeof(uint64_t) + (size_t)(kBuckets + 1) * sizeof(uint16_t);
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_lookup_big<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    const bool aligned = cols_aligned && al(a.reg_start, 15);
    hipLaunchKernelGGL(k_lookup_big<false>, dim3((unsigned)blocks), dim3(kThreadsLds), bytes, s,
                       a.reg_start, a.reg_end, a.reg_lkey, a.nregions, shift, nsplit,
                       a.page_shift, a.off, a.len, a.n, a.va_base,
                       a.handle, a.lkey, a.kind, a.rbase, a.rend, aligned,
                       (const uint32_t *)nullptr);
    return hipGetLastError();
}

size_t ws_mr_lookup(uint32_t nregions)
{
    return nregions > kLdsRegions ? ((size_t)nregions + kRecRun - 1) / kRecRun * kRecBytes : 0;
}

}  // namespace dd

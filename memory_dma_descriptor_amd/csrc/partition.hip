// partition.hip - stable split of request indices by destination queue, for
// gfx950.
//
// Method: every queue's requests are placed contiguously in increasing
// request index. The grouping of a wave's lanes by key follows the idea of the
// MORI thread-scope put kernel ("mori通信库分析(一)——对称内存RDMA数据发送过程"),
// which ballots the lanes that share a destination and lets one of them act
// for the group, and of its warp-level WQE reservation, where one lane
// reserves for the whole group and the others take consecutive slots by
// their rank. Here each lane learns the lanes sharing its queue id from one
// ballot per key bit (a lane matches when it agrees on every bit), its rank is
// the popcount of that group below it, and the lowest lane of the group bumps
// a wave-private running counter by the group size; scans over (bucket,
// block) and over the waves of a block turn counts into positions. No atomic
// decides a position, so the output is deterministic.
//
// A block owns kTile consecutive requests; wave w of it owns the kWaveItems
// consecutive requests [w * kWaveItems, (w + 1) * kWaveItems) of the tile,
// read as kItems rounds of 64 consecutive requests, so equal ids meet in
// (wave, round, lane) order -- request order.
//
// Kernels: k_split_hist (per-block bucket counts, bucket-major),
// k_split_colscan (one block per bucket: exclusive scan over blocks), then a
// scatter: ranks, a block-local stable sort in LDS, and perm written as
// contiguous runs, one per bucket, so stores coalesce. Two scatters compute
// the same ranks: k_split_scatter_cnt, for up to kCntQueues queues, counts
// each thread's consecutive requests into a (bucket, thread) matrix of LDS
// counters and scans it (a few VALU per request); k_split_scatter, for any
// count, ranks with the per-bit ballots above (one per key bit per request).
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Requests per thread: 32 (8,192 per block) with the counter ranking, whose
// registers allow it and whose per-bucket runs of perm get twice as long
// (fewer partly written 64-byte segments); 16 with the ballot ranking,
// which at 32 would need 225 VGPRs. The histogram uses the scatter's tile.
constexpr int kItemsCnt = 32;
constexpr int kItemsBallot = 16;
constexpr int kMaxBuckets = DMADESC_MAX_QUEUES + 1;
constexpr int kBucketSlots = 2 * kThreads;      // >= kMaxBuckets, two per thread

__device__ __forceinline__ int key_bits(uint32_t nq)
{
    return 32 - __clz(nq);                       // bits of the largest bucket id
}

// Buckets of a thread's kItems requests base + 64 k. In a tile that lies
// wholly inside the batch (every tile but the last) the loads carry no
// condition, so all of them are in flight at once; a guarded load would wait
// for each before issuing the next.
template <int kItems>
__device__ __forceinline__ void load_buckets(const uint32_t *__restrict__ qid, uint64_t base,
                                             uint64_t n, uint32_t nq, bool full,
                                             uint32_t (&b)[kItems])
{
    if (full) {
#pragma unroll
        for (int k = 0; k < kItems; ++k) b[k] = qid[base + (uint64_t)k * kWave];
#pragma unroll
        for (int k = 0; k < kItems; ++k) b[k] = b[k] < nq ? b[k] : nq;
    } else {
        // Clamped, not guarded (requests past the batch take bucket 0; their
        // callers skip them).
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint64_t i = base + (uint64_t)k * kWave;
            const uint32_t v = qid[i < n ? i : n - 1];
            b[k] = i < n ? (v < nq ? v : nq) : 0u;
        }
    }
}

// Copies of the block histogram: lane l adds into copy l % kCopies, so the
// lanes of a wave that share a popular queue spread over kCopies addresses
// instead of serializing on one (the copies lie in different LDS banks).
constexpr int kCopies = 8;

template <int kItems>
__global__ __launch_bounds__(kThreads) void k_split_hist(
    const uint32_t *__restrict__ qid, uint64_t n, uint32_t nq, uint64_t nb,
    uint32_t *__restrict__ counts)
{
    constexpr int kWaveItems = kWave * kItems;          // requests per wave
    constexpr int kTile = kThreads * kItems;            // requests per block
    __shared__ uint32_t h[kCopies][kMaxBuckets];
    const uint32_t nbk = nq + 1;
    for (uint32_t b = threadIdx.x; b < kCopies * kMaxBuckets; b += kThreads) (&h[0][0])[b] = 0;
    __syncthreads();
    // Counts only (no ranks), so LDS atomics suffice here.
    const uint64_t base = (uint64_t)blockIdx.x * kTile + (uint64_t)wave() * kWaveItems + lane();
    uint32_t *hc = h[lane() % kCopies];
    uint32_t b[kItems];
    load_buckets(qid, base, n, nq, (uint64_t)(blockIdx.x + 1) * kTile <= n, b);
#pragma unroll
    for (int k = 0; k < kItems; ++k)
        if (base + (uint64_t)k * kWave < n) atomicAdd(&hc[b[k]], 1u);
    __syncthreads();
    // Bucket-major: bucket k's counts over all blocks are contiguous.
    for (uint32_t k = threadIdx.x; k < nbk; k += kThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < kCopies; ++j) c += h[j][k];
        counts[(uint64_t)k * nb + blockIdx.x] = c;
    }
}

// One block per bucket: in-place exclusive scan of that bucket's per-block
// counts (one contiguous row of the bucket-major matrix) and the bucket
// total. Thread t takes a contiguous segment of the row; all its loads are
// issued before the first is used.
__global__ __launch_bounds__(kThreads) void k_split_colscan(
    uint32_t *__restrict__ counts, uint64_t nb, uint32_t nbk, uint64_t *__restrict__ total)
{
    __shared__ uint64_t scratch[kWaves];
    uint32_t *row = counts + (uint64_t)blockIdx.x * nb;
    const uint64_t seg = (nb + kThreads - 1) / kThreads;
    const uint64_t b0 = (uint64_t)threadIdx.x * seg;
    const uint64_t b1 = (b0 + seg < nb) ? b0 + seg : nb;
    uint64_t s = 0;
    for (uint64_t k = b0; k < b1; ++k) s += row[k];
    uint64_t tot;
    uint64_t run = block_excl_scan<kThreads>(s, scratch, &tot);
    for (uint64_t k = b0; k < b1; ++k) {
        const uint32_t c = row[k];
        row[k] = (uint32_t)run;
        run += c;
    }
    if (threadIdx.x == 0) total[blockIdx.x] = tot;
}

template <int kItems>
__global__ __launch_bounds__(kThreads) void k_split_scatter(
    const uint32_t *__restrict__ qid, uint64_t n, uint32_t nq,
    const uint32_t *__restrict__ offs, const uint64_t *__restrict__ total,
    uint32_t *__restrict__ perm, uint64_t *__restrict__ qoff,
    uint64_t *__restrict__ n_invalid)
{
    constexpr int kWaveItems = kWave * kItems;          // requests per wave
    constexpr int kTile = kThreads * kItems;            // requests per block
    __shared__ uint64_t s_scr[kWaves];
    __shared__ uint32_t s_wcnt[kWaves][kMaxBuckets];   // running, then prefix, per wave
    __shared__ uint32_t s_lstart[kBucketSlots];        // bucket start in the block's sorted tile
    __shared__ uint64_t s_gpos[kBucketSlots];          // bucket start in perm for this block
    __shared__ uint32_t s_sorted[kTile];               // request indices, block-local stable order
    __shared__ uint16_t s_sbkt[kTile];                 // their buckets

    const uint32_t nbk = nq + 1;
    const int t = threadIdx.x, w = wave(), ln = lane();
    for (uint32_t b = ln; b < nbk; b += kWave) s_wcnt[w][b] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Wave-private stable ranks: round k of wave w covers 64 consecutive requests.
    const int nbits = key_bits(nq);
    const uint64_t tile = (uint64_t)blockIdx.x * kTile;
    const uint64_t base = tile + (uint64_t)w * kWaveItems + ln;
    const uint64_t below = __lanemask_lt();
    uint32_t b[kItems], rank[kItems];
    load_buckets(qid, base, n, nq, (uint64_t)(blockIdx.x + 1) * kTile <= n, b);
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const bool on = base + (uint64_t)k * kWave < n;
        const uint64_t m = match_key(b[k], on, nbits, __ballot(on));
        const uint32_t before = s_wcnt[w][b[k]];
        rank[k] = before + (uint32_t)__popcll(m & below);
        __builtin_amdgcn_wave_barrier();
        if (on && (m & below) == 0) s_wcnt[w][b[k]] = before + (uint32_t)__popcll(m);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();

    // Per bucket: waves' prefix inside the block, the block's total, and the
    // bucket's start in perm (all buckets' totals scanned across the block).
    uint64_t pair_tot[2] = {0, 0}, pair_off[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t bk = 2 * t + h;
        if (bk < nbk) {
            uint32_t run = 0;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const uint32_t c = s_wcnt[ww][bk];
                s_wcnt[ww][bk] = run;
                run += c;
            }
            pair_tot[h] = run;                           // this block's count in bucket bk
            pair_off[h] = total[bk];                     // whole batch's count in bucket bk
        }
    }
    uint64_t ltot, gtot;
    const uint64_t lex = block_excl_scan<kThreads>(pair_tot[0] + pair_tot[1], s_scr, &ltot);
    const uint64_t gex = block_excl_scan<kThreads>(pair_off[0] + pair_off[1], s_scr, &gtot);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t bk = 2 * t + h;
        if (bk < nbk) {
            const uint64_t gbase = gex + (h ? pair_off[0] : 0);
            s_lstart[bk] = (uint32_t)(lex + (h ? pair_tot[0] : 0));
            s_gpos[bk] = gbase + offs[(uint64_t)bk * gridDim.x + blockIdx.x];
            if (blockIdx.x == 0) qoff[bk] = gbase;
        }
    }
    if (blockIdx.x == 0 && t == 0) {
        qoff[nbk] = n;
        *n_invalid = total[nq];
    }
    __syncthreads();

    // Block-local stable order in LDS, then perm written run by run.
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kWave;
        if (i < n) {
            const uint32_t sidx = s_lstart[b[k]] + s_wcnt[w][b[k]] + rank[k];
            s_sorted[sidx] = (uint32_t)i;
            s_sbkt[sidx] = (uint16_t)b[k];
        }
    }
    __syncthreads();
    const uint64_t cnt = n - tile < (uint64_t)kTile ? n - tile : (uint64_t)kTile;
    for (uint32_t j = t; j < cnt; j += kThreads) {
        const uint32_t bk = s_sbkt[j];
        perm[s_gpos[bk] + (j - s_lstart[bk])] = s_sorted[j];
    }
}

// Counter ranking. Thread t of a block owns the kItems consecutive requests
// of chunk c(t) of the tile and counts them, in request order, into its own
// column of a (bucket, chunk) matrix of 16-bit LDS counters: the count it
// reads is the request's rank among the chunk's requests of its bucket. One
// exclusive scan of the matrix in bucket-major order then gives (bucket b,
// chunk c) the number of the tile's requests that sort before chunk c's
// requests of bucket b -- those of lower buckets, and those of bucket b in
// earlier chunks -- so scan value + rank is a request's place in the block's
// stable order. Buckets are padded to a multiple of 8 (a thread scans whole
// 16-byte rows) with at least one spare bucket, which takes the requests past
// the end of the batch in the last tile.
constexpr int kCntBuckets = 72;                 // padded bucket limit of the counter path
constexpr uint32_t kCntQueues = kCntBuckets - 2;   // nq + 1 buckets + a spare fit
static_assert(kCntBuckets % 8 == 0, "scan rows are 8 counters");
static_assert(kThreads * kItemsCnt * 4 <= kCntBuckets * kThreads * 2,
              "sorted tile fits over the counters");

// Lanes l and l + 32 of a wave own adjacent chunks, so the 32 lanes an LDS
// cycle serves touch 32 different dwords of a 16-bit counter row.
__device__ __forceinline__ uint32_t chunk_of(int t)
{
    const int l = t & (kWave - 1), w = t / kWave;
    return (uint32_t)(w * kWave + 2 * (l & 31) + (l >> 5));
}

// kSingle: the whole batch is this one tile (the histogram and column scan
// are then not launched): the bucket totals and their starts in perm are the
// tile's own, from its counter scan.
template <int kItems, bool kSingle>
__global__ __launch_bounds__(kThreads) void k_split_scatter_cnt(
    const uint32_t *__restrict__ qid, uint64_t n, uint32_t nq, bool vec,
    const uint32_t *__restrict__ offs, const uint64_t *__restrict__ total,
    uint32_t *__restrict__ perm, uint64_t *__restrict__ qoff,
    uint64_t *__restrict__ n_invalid)
{
    constexpr int kTile = kThreads * kItems;            // requests per block
    __shared__ uint32_t s_scr32[kWaves];
    __shared__ uint64_t s_scr64[kWaves];
    // Counters, then their bucket-major exclusive scan; at the end the sorted
    // tile (16-bit request index inside the tile, then 8-bit bucket) over it.
    __shared__ __align__(16) uint16_t s_cnt[kCntBuckets * kThreads];
    __shared__ uint32_t s_lstart[kCntBuckets];         // bucket start in the sorted tile
    __shared__ uint64_t s_gpos[kCntBuckets];           // bucket start in perm for this block

    const uint32_t nbk = nq + 1;
    const uint32_t nbp = (nbk + 8) & ~7u;              // padded, >= nbk + 1
    const uint32_t rows = nbp / 8;                     // 16-byte scan rows per thread
    const int t = threadIdx.x;
    const uint32_t c = chunk_of(t);
    const uint64_t tile = (uint64_t)blockIdx.x * kTile;
    const uint64_t base = tile + (uint64_t)c * kItems;
    uint4 *s4 = reinterpret_cast<uint4 *>(s_cnt);
    for (uint32_t k = t; k < rows * kThreads; k += kThreads) s4[k] = make_uint4(0, 0, 0, 0);

    // Buckets of the chunk's requests; past the batch: the spare bucket.
    uint32_t b[kItems];
    if (vec && tile + kTile <= n) {
#pragma unroll
        for (int q = 0; q < kItems / 4; ++q) {
            const uint4 x = *reinterpret_cast<const uint4 *>(qid + base + 4 * q);
            b[4 * q] = x.x;
            b[4 * q + 1] = x.y;
            b[4 * q + 2] = x.z;
            b[4 * q + 3] = x.w;
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) b[k] = b[k] < nq ? b[k] : nq;
    } else if (vec && base + kItems <= n) {
        // A chunk wholly inside the batch (in the last, partial tile).
#pragma unroll
        for (int q = 0; q < kItems / 4; ++q) {
            const uint4 x = *reinterpret_cast<const uint4 *>(qid + base + 4 * q);
            b[4 * q] = x.x;
            b[4 * q + 1] = x.y;
            b[4 * q + 2] = x.z;
            b[4 * q + 3] = x.w;
        }
#pragma unroll
        for (int k = 0; k < kItems; ++k) b[k] = b[k] < nq ? b[k] : nq;
    } else {
        // Clamped, not guarded, so that all of the chunk's loads are in
        // flight at once (a one-tile batch: 10.3 -> 8.0 us for 4,096 requests).
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint64_t i = base + k;
            const uint32_t v = qid[i < n ? i : n - 1];
            b[k] = i < n ? (v < nq ? v : nq) : nbp - 1;
        }
    }
    __syncthreads();

    // Ranks inside the chunk: each request bumps its own counter with an LDS
    // atomic add that returns the old value. The counters of chunks 2m and
    // 2m + 1 share a dword, so the add goes to this chunk's half; a chunk
    // counts at most kItems per bucket, so no carry reaches the other half.
    // A wave's LDS operations complete in order, so the ranks follow request
    // order, and the adds need not wait for each other (a load and a store
    // per request made a dependent round trip each).
    uint16_t *col = s_cnt + c;
    uint32_t *col32 = reinterpret_cast<uint32_t *>(s_cnt) + (c >> 1);
    const uint32_t half = (c & 1u) * 16u;
    uint32_t rank[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k)
        rank[k] = (atomicAdd(col32 + b[k] * (kThreads / 2), 1u << half) >> half) & 0xFFFFu;
    __syncthreads();

    // Exclusive scan of the matrix, bucket-major: thread t scans counters
    // [t * nbp, (t + 1) * nbp) of the flattened matrix. A chunk's count in a
    // bucket is <= kItems, so the 16-bit halves of a dword sum without carry.
    uint32_t sum = 0;
    for (uint32_t q = 0; q < rows; ++q) {
        const uint4 x = s4[t * rows + q];
        const uint32_t s2 = x.x + x.y + x.z + x.w;
        sum += (s2 & 0xFFFFu) + (s2 >> 16);
    }
    uint32_t tile_tot;
    uint32_t run = block_excl_scan<kThreads>(sum, s_scr32, &tile_tot);
    for (uint32_t q = 0; q < rows; ++q) {
        uint4 x = s4[t * rows + q];
        uint32_t *xw = &x.x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = xw[j] & 0xFFFFu, hi = xw[j] >> 16;
            xw[j] = run | ((run + lo) << 16);
            run += lo + hi;
        }
        s4[t * rows + q] = x;
    }
    __syncthreads();

    // Bucket starts: in the sorted tile (scan value of chunk 0), and in perm
    // (all buckets' batch totals scanned, plus the blocks before this one).
    if constexpr (kSingle) {
        // One tile: a bucket starts in perm where it starts in the tile; the
        // spare bucket (past the batch) starts at n.
        if ((uint32_t)t < nbk) {
            const uint32_t st = s_cnt[t * kThreads];
            s_lstart[t] = st;
            s_gpos[t] = st;
            qoff[t] = st;
        }
        if (t == 0) {
            qoff[nbk] = n;
            *n_invalid = n - (uint64_t)s_cnt[nq * kThreads];
        }
    } else {
        const uint64_t gv = (uint32_t)t < nbk ? total[t] : 0;
        uint64_t gtot;
        const uint64_t gex = block_excl_scan<kThreads>(gv, s_scr64, &gtot);
        if ((uint32_t)t < nbk) {
            s_lstart[t] = s_cnt[t * kThreads];
            s_gpos[t] = gex + offs[(uint64_t)t * gridDim.x + blockIdx.x];
            if (blockIdx.x == 0) qoff[t] = gex;
        }
        if (blockIdx.x == 0 && t == 0) {
            qoff[nbk] = n;
            *n_invalid = total[nq];
        }
    }
    uint32_t sidx[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) sidx[k] = col[b[k] * kThreads] + rank[k];
    __syncthreads();
    // Where the tile's place j of bucket bk goes in perm: s_gpos[bk] - s_lstart[bk] + j.
    if ((uint32_t)t < nbk) s_gpos[t] -= s_lstart[t];

    // The sorted tile: one dword per place, (bucket << 16) | request index in
    // the tile. Requests past the batch (spare bucket, sorted last) land past
    // its count, where nothing reads them, so no request needs a guard.
    uint32_t *s_sorted = reinterpret_cast<uint32_t *>(s_cnt);
#pragma unroll
    for (int k = 0; k < kItems; ++k) s_sorted[sidx[k]] = (b[k] << 16) | (c * kItems + k);
    __syncthreads();
    const uint64_t cnt = n - tile < (uint64_t)kTile ? n - tile : (uint64_t)kTile;
    if (cnt == (uint64_t)kTile) {
        // Eight places per lane at a time: their LDS reads are in flight
        // together instead of one dependent pair per place.
        constexpr int kU = 8;
#pragma unroll 1
        for (int m0 = 0; m0 < kItems; m0 += kU) {
            uint32_t e[kU];
            uint64_t d[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) e[u] = s_sorted[t + (m0 + u) * kThreads];
#pragma unroll
            for (int u = 0; u < kU; ++u) d[u] = s_gpos[e[u] >> 16];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                perm[d[u] + (uint32_t)(t + (m0 + u) * kThreads)] = (uint32_t)(tile + (e[u] & 0xFFFFu));
        }
    } else {
        for (uint32_t j = t; j < cnt; j += kThreads) {
            const uint32_t e = s_sorted[j];
            perm[s_gpos[e >> 16] + j] = (uint32_t)(tile + (e & 0xFFFFu));
        }
    }
}

__global__ void k_split_empty(uint32_t nq, uint64_t *__restrict__ qoff, uint64_t *__restrict__ n_invalid)
{
    for (uint32_t b = threadIdx.x; b < nq + 2; b += blockDim.x) qoff[b] = 0;
    if (threadIdx.x == 0) *n_invalid = 0;
}

// Requests per block of the split for nq queues (the ranking it uses).
uint64_t split_tile(uint32_t nq)
{
    return (uint64_t)kThreads * (nq <= kCntQueues ? kItemsCnt : kItemsBallot);
}
static_assert(kThreads * kItemsCnt == 1 << 13 && kThreads * kItemsBallot == 1 << 12,
              "split_tile_shift matches split_tile");

}  // namespace

size_t ws_partition(uint64_t n, uint32_t nq)
{
    const uint64_t tile = split_tile(nq);
    const uint64_t nb = (n + tile - 1) / tile;
    return align256((uint64_t)(nq + 1) * nb * sizeof(uint32_t)) +
           align256((uint64_t)(nq + 1) * sizeof(uint64_t));
}

bool split_single(uint64_t n, uint32_t nq)
{
    return n > 0 && n <= split_tile(nq) && nq <= kCntQueues;
}

uint32_t split_tile_shift(uint32_t nq)
{
    return nq <= kCntQueues ? 13 : 12;
}

hipError_t launch_partition(const SplitArgs &a, hipStream_t s)
{
    if (a.n == 0) {
        hipLaunchKernelGGL(k_split_empty, dim3(1), dim3(kThreads), 0, s, a.nqueues, a.qoff,
                           a.n_invalid);
        return hipGetLastError();
    }
    const uint64_t tile = split_tile(a.nqueues);
    const uint64_t nb = (a.n + tile - 1) / tile;
    uint32_t *counts = static_cast<uint32_t *>(a.ws);
    if (split_single(a.n, a.nqueues)) {
        // One tile: the scatter alone (no histogram, no column scan).
        const bool vec = (reinterpret_cast<uintptr_t>(a.qid) & 15u) == 0;
        hipLaunchKernelGGL((k_split_scatter_cnt<kItemsCnt, true>), dim3(1), dim3(kThreads), 0, s,
                           a.qid, a.n, a.nqueues, vec, counts, nullptr, a.perm, a.qoff,
                           a.n_invalid);
        return hipGetLastError();
    }
    if (a.nqueues <= kCntQueues)
        hipLaunchKernelGGL(k_split_hist<kItemsCnt>, dim3((unsigned)nb), dim3(kThreads), 0, s,
                           a.qid, a.n, a.nqueues, nb, counts);
    else
        hipLaunchKernelGGL(k_split_hist<kItemsBallot>, dim3((unsigned)nb), dim3(kThreads), 0, s,
                           a.qid, a.n, a.nqueues, nb, counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_partition_counted(a, s);
}

hipError_t launch_partition_counted(const SplitArgs &a, hipStream_t s)
{
    const uint64_t tile = split_tile(a.nqueues);
    const uint64_t nb = (a.n + tile - 1) / tile;
    const uint32_t nbk = a.nqueues + 1;
    const bool cnt_path = a.nqueues <= kCntQueues;
    uint32_t *counts = static_cast<uint32_t *>(a.ws);
    uint64_t *total = reinterpret_cast<uint64_t *>(
        static_cast<char *>(a.ws) + align256((uint64_t)nbk * nb * sizeof(uint32_t)));
    hipLaunchKernelGGL(k_split_colscan, dim3(nbk), dim3(kThreads), 0, s,
                       counts, nb, nbk, total);
    if (cnt_path) {
        const bool vec = (reinterpret_cast<uintptr_t>(a.qid) & 15u) == 0;
        hipLaunchKernelGGL((k_split_scatter_cnt<kItemsCnt, false>), dim3((unsigned)nb), dim3(kThreads), 0, s,
                           a.qid, a.n, a.nqueues, vec, counts, total, a.perm, a.qoff,
                           a.n_invalid);
    } else {
        hipLaunchKernelGGL(k_split_scatter<kItemsBallot>, dim3((unsigned)nb), dim3(kThreads), 0, s,
                           a.qid, a.n, a.nqueues, counts, total, a.perm, a.qoff, a.n_invalid);
    }
    return hipGetLastError();
}

}  // namespace dd

// registry.hip - the registration cache on the device: batches of register
// and deregister calls applied to a refcounted record table, for gfx950.
//
// Method (NCCL GDR/MR course page, "Communicator User Registration Cache" and
// "IB Backend MR Cache"): a registration widens its range to whole pages; a
// record that fully contains the widened range gains a reference and its
// handle is returned, otherwise a new record is inserted in start order; a
// deregistration drops a reference and frees the record at zero, and a handle
// no record holds is an error. The record table grows 0 -> 32 -> 64 -> ...
//
// A batch means what its calls made one after another mean. In parallel:
//  * A range that some record of the table before the batch contains hits
//    the first such record in start order: with PM[p] the running maximum of
//    the records' ends in start order, that record is the first p with
//    PM[p] >= end, provided its start is <= the range's start.
//  * A miss is inserted exactly when no earlier miss of the batch contains
//    it (an earlier miss either was inserted or was itself contained by an
//    inserted record, which then contains this one too; an earlier hit's range
//    lies inside an old record, so it never contains a miss). Every other
//    range goes to the record that comes first in start order among the old
//    record it hit (if any) and the earlier inserts that contain it: the
//    insert with the smallest (start, batch index) wins over the old record
//    only when its start is strictly smaller, since an insert goes after the
//    records with the same start. These relations are found through a
//    bucketed index of the batch's ranges (a containing range that is no
//    longer than a bucket lies in one of two buckets), and by comparing
//    every pair in LDS tiles only for the ranges that are longer than a
//    bucket or overflow theirs (a batch is at most DMADESC_REG_MAX_BATCH
//    calls).
//  * New records get handles next_id + their rank among the batch's inserts,
//    take storage slots after the live records (storage is in handle order,
//    so a handle is found by binary search), and are merged into the
//    start-ordered index behind existing records with the same start.
//  * A deregistration of a record with r references is stale when r earlier
//    calls of the batch already named it; live records are compacted stably.
// A register batch that would leave more records than the capacity applies
// nothing and reports the capacity the growth rule reaches.
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPer = 4;                              // records per thread in scans
constexpr uint32_t kChunk = kThreads * kPer;         // records per scan block
constexpr int kTopThreads = 1024;
constexpr uint32_t kMaxChunks = DMADESC_REG_MAX_CAPACITY / kChunk;   // 16384
constexpr uint32_t kItemChunks = DMADESC_REG_MAX_BATCH / kChunk;      // 64
static_assert(kItemChunks <= kThreads, "item chunk totals scan in one block");
static_assert(kMaxChunks % kTopThreads == 0, "chunk totals scan in one block");

enum : uint8_t { kInvalid = DMADESC_REG_INVALID, kHit = DMADESC_REG_HIT, kNew = DMADESC_REG_NEW,
                 kHitNew = DMADESC_REG_HIT_NEW, kNospace = DMADESC_REG_NOSPACE };
enum : uint8_t { kMiss = 5 };                        // internal class before inserts are known

// Pair kernels: items per block (one per lane of a wave), and entries of a
// tile read from LDS before they are compared.
constexpr uint32_t kPairItems = kWave;
constexpr uint32_t kPairStep = 8;
static_assert(kWave % (4 * kPairStep) == 0, "a wave's quarter is whole steps");

// A rounded range in LDS; kNoRange contains nothing and sorts after every
// valid start (a valid range has base < 2^64 - 1 and top > 0).
struct alignas(16) Range {
    uint64_t base, top;
};
constexpr Range kNoRange{~0ull, 0};

// Range index of the batch's misses, and one of its inserts: buckets of
// width W = 2^shift over [lo, hi], the smallest and largest start among the
// misses (inserts are misses, so the same buckets serve both), each bucket
// holding up to kSlots ranges inline. A range longer than W, or one that
// finds its bucket full, is flagged long instead. A range of length at most
// W that contains [b, t) starts in [b + 1 - W, b], so a query reads at most
// two buckets, plus the long ranges, which the pair kernels walk in rank
// order through LDS tiles as they walked every earlier range before,
// skipping the 256-rank tiles that hold none.
constexpr uint32_t kSlots = 8;
constexpr uint32_t kMinBuckets = 64, kMaxBuckets = 16384;
static_assert((kMaxBuckets & (kMaxBuckets - 1)) == 0, "bucket counts are powers of two");

struct RIdx {
    uint32_t *cnt;          // ranges filed to each bucket (past kSlots: flagged long)
    Range *rec;             // [bucket * kSlots + s]: a range of the bucket
    uint32_t *key;          // [bucket * kSlots + s]: its rank (miss rank or insert rank)
    uint8_t *lflag;         // by rank: 1 if the range is long (not in a bucket)
    uint32_t *tlong;        // long ranges per 256-rank tile
    uint32_t *pre;          // inserts only: in-table ranges of the earlier buckets
};
constexpr uint32_t kRankTiles = DMADESC_REG_MAX_BATCH / 256;

// Workspace pieces (pointers into the caller's workspace).
struct RegWs {
    // per batch item
    uint64_t *base, *top;
    uint8_t *cls;           // kInvalid / kHit / kMiss, then kNew / kHitNew
    uint32_t *hit;          // storage slot of the hit record (kHit)
    uint64_t *hstart;       // start of the hit record (kHit)
    uint32_t *rank;         // rank among inserts (kNew)
    uint32_t *brank;        // rank of an insert in (start, batch index) order
    uint32_t *owner;        // rank of the containing insert (kHitNew)
    uint32_t *newrefs;      // references of each insert, by rank
    uint64_t *newbase;      // start of each insert, by brank
    uint64_t *ibase, *itop; // rounded range of each insert, by rank
    uint64_t *mbase, *mtop; // rounded range of each miss, by miss rank
    uint32_t *mrank;        // misses before each item
    // range indexes (misses, inserts); rinfo = {lo, hi}; rcnt = long ranges
    // of each index
    RIdx xm, xi;
    uint64_t *rinfo;
    uint64_t *bmin, *bmax;  // per classification block: smallest / largest miss start
    uint32_t *rcnt;
    uint32_t nbk;           // buckets per index (a power of two)
    // per record (capacity)
    uint64_t *sstart;       // starts in start order
    uint64_t *pm;           // running maximum of ends in start order
    uint32_t *merged;       // next start-ordered index / kept flags
    uint32_t *newslot;      // storage slot after compaction
    uint64_t *tmp64a, *tmp64b, *tmp64c;
    uint32_t *tmp32;
    // per scan chunk
    uint64_t *chunk;        // chunk totals, then exclusive prefixes
    uint64_t *ichunk;       // the same for batch items (ranking misses, inserts)
    // scalars: [0] inserts, [1] fits, [2] live count after deregistration
    uint64_t *scal;
};

struct RegState {
    uint64_t *start, *end, *id;
    uint32_t *refs, *by_start;
    uint64_t *state;        // [0] live records, [1] next handle
    uint64_t capacity;
};

// ---------------------------------------------------------------- scans ---

template <bool kMax>
__device__ __forceinline__ uint64_t combine(uint64_t a, uint64_t b)
{
    return kMax ? (a > b ? a : b) : a + b;
}

template <bool kMax, int kT>
__device__ __forceinline__ uint64_t block_excl(uint64_t v, uint64_t *scr, uint64_t *total)
{
    constexpr int kW = kT / kWave;
    uint64_t inc = v;
    const int ln = lane();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t u = __shfl_up(inc, (unsigned)d, kWave);
        if (ln >= d) inc = combine<kMax>(inc, u);
    }
    const int w = wave();
    if (ln == kWave - 1) scr[w] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kW; ++k) {
        const uint64_t s = scr[k];
        if (k < w) before = combine<kMax>(before, s);
        all = combine<kMax>(all, s);
    }
    __syncthreads();
    *total = all;
    // exclusive: the wave-exclusive value combined with the earlier waves'
    const uint64_t wex = __shfl_up(inc, 1u, kWave);
    return combine<kMax>(before, ln ? wex : 0ull);
}

// Values of the records in start order, for the running maximum of ends.
struct EndsInOrder {
    const uint64_t *end;
    const uint32_t *by_start;
    __device__ uint64_t operator()(uint64_t p) const { return end[by_start[p]]; }
};
// Kept flags (refs > 0) of storage slots, for the compaction.
struct KeptSlots {
    const uint32_t *refs;
    __device__ uint64_t operator()(uint64_t p) const { return refs[p] != 0; }
};
// Kept flags of the start-ordered index.
struct KeptInOrder {
    const uint32_t *refs;
    const uint32_t *by_start;
    __device__ uint64_t operator()(uint64_t p) const { return refs[by_start[p]] != 0; }
};

// Pass 1: per-chunk totals of f(p) for p < count.
template <bool kMax, class F>
__global__ __launch_bounds__(kThreads) void k_scan_chunks(F f, const uint64_t *state,
                                                          uint64_t *chunk)
{
    __shared__ uint64_t scr[kWaves];
    const uint64_t count = state[0];
    const uint64_t p0 = (uint64_t)blockIdx.x * kChunk;
    if (p0 >= count) return;                         // uniform over the block
    uint64_t v = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint64_t p = p0 + (uint64_t)threadIdx.x * kPer + k;
        if (p < count) v = combine<kMax>(v, f(p));
    }
    uint64_t tot;
    block_excl<kMax, kThreads>(v, scr, &tot);
    if (threadIdx.x == 0) chunk[blockIdx.x] = tot;
}

// Pass 2: one block turns the chunk totals into exclusive prefixes; the grand
// total goes to *total.
template <bool kMax>
__global__ __launch_bounds__(kTopThreads) void k_scan_top(const uint64_t *state, uint64_t *chunk,
                                                          uint64_t *total)
{
    __shared__ uint64_t scr[kTopThreads / kWave];
    const uint64_t count = state[0];
    const uint32_t nch = (uint32_t)((count + kChunk - 1) / kChunk);
    constexpr uint32_t kEach = kMaxChunks / kTopThreads;
    uint64_t v[kEach], s = 0;
#pragma unroll
    for (uint32_t k = 0; k < kEach; ++k) {
        const uint32_t c = threadIdx.x * kEach + k;
        v[k] = c < nch ? chunk[c] : 0;
        s = combine<kMax>(s, v[k]);
    }
    uint64_t tot;
    uint64_t run = block_excl<kMax, kTopThreads>(s, scr, &tot);
#pragma unroll
    for (uint32_t k = 0; k < kEach; ++k) {
        const uint32_t c = threadIdx.x * kEach + k;
        if (c < nch) chunk[c] = run;
        run = combine<kMax>(run, v[k]);
    }
    if (threadIdx.x == 0 && total) *total = count ? tot : 0;
}

// Pass 3: out[p] = prefix of f over records before p (exclusive) or up to p
// (inclusive).
template <bool kMax, bool kIncl, class F>
__global__ __launch_bounds__(kThreads) void k_scan_apply(F f, const uint64_t *state,
                                                         const uint64_t *chunk, uint64_t *out)
{
    __shared__ uint64_t scr[kWaves];
    const uint64_t count = state[0];
    const uint64_t p0 = (uint64_t)blockIdx.x * kChunk;
    if (p0 >= count) return;
    uint64_t v[kPer], s = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint64_t p = p0 + (uint64_t)threadIdx.x * kPer + k;
        v[k] = p < count ? f(p) : 0;
        s = combine<kMax>(s, v[k]);
    }
    uint64_t tot;
    uint64_t run = combine<kMax>(chunk[blockIdx.x], block_excl<kMax, kThreads>(s, scr, &tot));
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint64_t p = p0 + (uint64_t)threadIdx.x * kPer + k;
        const uint64_t nxt = combine<kMax>(run, v[k]);
        if (p < count) out[p] = kIncl ? nxt : run;
        run = nxt;
    }
}

template <bool kMax, bool kIncl, class F>
void scan_records(F f, const uint64_t *state, uint64_t capacity, uint64_t *chunk, uint64_t *out,
                  uint64_t *total, hipStream_t s)
{
    const unsigned nb = (unsigned)((capacity + kChunk - 1) / kChunk);
    if (nb == 0) return;
    hipLaunchKernelGGL((k_scan_chunks<kMax, F>), dim3(nb), dim3(kThreads), 0, s, f, state, chunk);
    hipLaunchKernelGGL((k_scan_top<kMax>), dim3(1), dim3(kTopThreads), 0, s, state, chunk, total);
    hipLaunchKernelGGL((k_scan_apply<kMax, kIncl, F>), dim3(nb), dim3(kThreads), 0, s, f, state,
                       chunk, out);
}

// ---------------------------------------------------------- range index ---

// The smallest shift s with (hi - lo) >> s < nbk (nbk a power of two).
__device__ __forceinline__ uint32_t idx_shift(uint64_t lo, uint64_t hi, uint32_t nbk)
{
    const uint64_t span = hi > lo ? hi - lo : 0;
    const uint32_t bl = span ? 64u - (uint32_t)__clzll((long long)span) : 0u;
    const uint32_t lb = 31u - (uint32_t)__clz((int)nbk);
    return bl > lb ? bl - lb : 0u;
}

// Files range [b, t) (b in [lo, hi]) of rank r into index X, or flags it
// long; returns whether it is long. The caller counts long ranges per
// 256-rank tile and in all with a few atomics per wave (an atomic per long
// range on one shared word would serialize).
__device__ __forceinline__ bool idx_put(const RIdx &X, uint64_t lo, uint32_t shift, uint64_t b,
                                        uint64_t t, uint32_t r)
{
    if (t - b <= (1ull << shift)) {
        const uint32_t c = (uint32_t)((b - lo) >> shift);
        const uint32_t s = atomicAdd(&X.cnt[c], 1u);
        if (s < kSlots) {
            X.rec[(uint64_t)c * kSlots + s] = Range{b, t};
            X.key[(uint64_t)c * kSlots + s] = r;
            X.lflag[r] = 0;
            return false;
        }
    }
    X.lflag[r] = 1;
    return true;
}

// Buckets [c0, c1] (of either index: both share lo, hi and shift) that can
// hold a range of length <= 2^shift containing a range starting at b;
// c0 > c1 when there are none.
__device__ __forceinline__ void idx_window(uint64_t lo, uint64_t hi, uint32_t shift, uint64_t b,
                                          uint32_t &c0, uint32_t &c1)
{
    const uint64_t wd = 1ull << shift;
    uint64_t xlo = b + 1 >= wd ? b + 1 - wd : 0;       // b is a page start: b + 1 does not wrap
    if (xlo < lo) xlo = lo;
    const uint64_t xhi = b < hi ? b : hi;
    if (xlo > xhi) {
        c0 = 1;
        c1 = 0;
        return;
    }
    c0 = (uint32_t)((xlo - lo) >> shift);
    c1 = (uint32_t)((xhi - lo) >> shift);
}

// Clears both indexes' bucket counts, long-tile counts and long counts.
__global__ __launch_bounds__(kThreads) void k_ridx_clear(RegWs w)
{
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g < w.nbk) {
        w.xm.cnt[g] = 0;
        w.xi.cnt[g] = 0;
    }
    if (g < kRankTiles) {
        w.xm.tlong[g] = 0;
        w.xi.tlong[g] = 0;
    }
    if (g == 0) {
        w.rcnt[0] = 0;
        w.rcnt[1] = 0;
    }
}

// One block: pre[c] = in-table inserts of buckets before c. Thread t takes
// buckets [16t, 16t + 16) (nbk is a multiple of 64, so a thread's buckets
// are all inside or all past the index) as four 16-byte loads issued
// together.
__global__ __launch_bounds__(kTopThreads) void k_ridx_scan(RegWs w)
{
    __shared__ uint64_t scr[kTopThreads / kWave];
    constexpr uint32_t kEach = kMaxBuckets / kTopThreads;
    static_assert(kEach == 16 && kMinBuckets % kEach == 0, "whole 16-byte rows per thread");
    const uint32_t c0 = threadIdx.x * kEach;
    const bool mine = c0 < w.nbk;
    uint32_t v[kEach], sum = 0;
    if (mine) {
        uint4 x[kEach / 4];
#pragma unroll
        for (uint32_t q = 0; q < kEach / 4; ++q) x[q] = reinterpret_cast<const uint4 *>(w.xi.cnt + c0)[q];
#pragma unroll
        for (uint32_t q = 0; q < kEach / 4; ++q) {
            v[4 * q] = x[q].x;
            v[4 * q + 1] = x[q].y;
            v[4 * q + 2] = x[q].z;
            v[4 * q + 3] = x[q].w;
        }
    } else {
#pragma unroll
        for (uint32_t k = 0; k < kEach; ++k) v[k] = 0;
    }
#pragma unroll
    for (uint32_t k = 0; k < kEach; ++k) {
        v[k] = v[k] < kSlots ? v[k] : kSlots;
        sum += v[k];
    }
    uint64_t tot;
    uint32_t run = (uint32_t)block_excl<false, kTopThreads>(sum, scr, &tot);
    if (mine) {
        uint4 y[kEach / 4];
#pragma unroll
        for (uint32_t q = 0; q < kEach / 4; ++q) {
            y[q].x = run; run += v[4 * q];
            y[q].y = run; run += v[4 * q + 1];
            y[q].z = run; run += v[4 * q + 2];
            y[q].w = run; run += v[4 * q + 3];
        }
#pragma unroll
        for (uint32_t q = 0; q < kEach / 4; ++q) reinterpret_cast<uint4 *>(w.xi.pre + c0)[q] = y[q];
    }
}

// ------------------------------------------------------------- register ---

__global__ __launch_bounds__(kThreads) void k_reg_starts(RegState g, RegWs w)
{
    const uint64_t count = g.state[0];
    for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < count;
         p += (uint64_t)gridDim.x * kThreads)
        w.sstart[p] = g.start[g.by_start[p]];
}

// Rounding and the lookup in the table as it was before the batch; each
// block also stores the smallest and largest start among its misses, which
// the misses' ranking kernel reduces to the range indexes' bounds.
__global__ __launch_bounds__(kThreads) void k_reg_classify(RegState g, RegWs w, uint32_t shift,
                                                           const uint64_t *addr, const uint64_t *size,
                                                           uint32_t n)
{
    __shared__ uint64_t s_lo[kWaves], s_hi[kWaves];
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    uint64_t mlo = ~0ull, mhi = 0;
    if (i < n) {
        const uint64_t count = g.state[0];
        const uint64_t a = addr[i], l = size[i];
        const uint64_t page = 1ull << shift;
        uint8_t c = kMiss;
        uint64_t base = 0, top = 0;
        if (l == 0 || l > ~a) {
            c = kInvalid;
        } else {
            base = a & ~(page - 1);
            const uint64_t last = a + l - 1;              // no wrap: l <= ~a
            const uint64_t lastp = last & ~(page - 1);
            if (lastp > ~0ull - page) c = kInvalid;       // the rounded end would wrap
            else top = lastp + page;
        }
        uint32_t hit = 0;
        uint64_t hstart = 0;
        if (c == kMiss && count) {
            // First p with pm[p] >= top (pm is non-decreasing).
            uint64_t lo = 0, hi = count;
            while (lo < hi) {
                const uint64_t mid = (lo + hi) >> 1;
                if (w.pm[mid] >= top) hi = mid;
                else lo = mid + 1;
            }
            if (lo < count && w.sstart[lo] <= base) {
                c = kHit;
                hit = g.by_start[lo];
                hstart = w.sstart[lo];
            }
        }
        w.hstart[i] = hstart;
        w.base[i] = base;
        w.top[i] = top;
        w.cls[i] = c;
        w.hit[i] = hit;
        if (c == kMiss) {
            mlo = base;
            mhi = base;
        }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
        const uint64_t a = __shfl_xor(mlo, d, kWave), b = __shfl_xor(mhi, d, kWave);
        mlo = a < mlo ? a : mlo;
        mhi = b > mhi ? b : mhi;
    }
    if (lane() == 0) {
        s_lo[wave()] = mlo;
        s_hi[wave()] = mhi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 1; k < kWaves; ++k) {
            mlo = s_lo[k] < mlo ? s_lo[k] : mlo;
            mhi = s_hi[k] > mhi ? s_hi[k] : mhi;
        }
        w.bmin[blockIdx.x] = mlo;                        // ~0 and 0 for a block without misses
        w.bmax[blockIdx.x] = mhi;
    }
}

// Ranking batch items of one class (misses, then inserts) in batch order: a
// device-wide exclusive scan over chunks of kChunk items in three kernels
// (count per chunk, scan of the chunk counts in one block, ranks and
// scatter), so that no wave walks a long chunk round by round. Thread t of a
// block takes the 4 consecutive items p0 + 4t .. p0 + 4t + 3.
template <uint8_t kCls>
__device__ __forceinline__ void item_flags(const RegWs &w, uint32_t n, uint32_t p, uint32_t (&f)[kPer])
{
    if (p + kPer <= n) {
        const uint32_t c4 = *reinterpret_cast<const uint32_t *>(w.cls + p);
#pragma unroll
        for (int k = 0; k < kPer; ++k) f[k] = ((c4 >> (8 * k)) & 0xFFu) == kCls;
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) f[k] = p + k < n && w.cls[p + k] == kCls;
    }
}

template <uint8_t kCls>
__global__ __launch_bounds__(kThreads) void k_rank_chunks(RegWs w, uint32_t n)
{
    __shared__ uint64_t scr[kWaves];
    const uint32_t p = blockIdx.x * kChunk + threadIdx.x * kPer;
    uint32_t f[kPer];
    item_flags<kCls>(w, n, p, f);
    uint64_t tot;
    block_excl<false, kThreads>((uint64_t)(f[0] + f[1] + f[2] + f[3]), scr, &tot);
    if (threadIdx.x == 0) w.ichunk[blockIdx.x] = tot;
}

// One block: the chunk counts become exclusive prefixes. For the misses it
// also reduces the classification blocks' start bounds to the range
// indexes' [lo, hi] (lo > hi when there is no miss); for the inserts
// (kCount) it records their number, whether the table has room, and the
// capacity the growth rule reaches (reported either way).
template <bool kCount>
__global__ __launch_bounds__(kThreads) void k_rank_top(RegState g, RegWs w, uint32_t n,
                                                       uint64_t *needed)
{
    __shared__ uint64_t scr[kWaves];
    const uint32_t nch = (n + kChunk - 1) / kChunk;
    const uint64_t v = threadIdx.x < nch ? w.ichunk[threadIdx.x] : 0;
    uint64_t tot;
    const uint64_t ex = block_excl<false, kThreads>(v, scr, &tot);
    if (threadIdx.x < nch) w.ichunk[threadIdx.x] = ex;
    if (!kCount) {
        const uint32_t ncb = (n + kThreads - 1) / kThreads;        // classification blocks
        const uint64_t nlo = threadIdx.x < ncb ? ~w.bmin[threadIdx.x] : 0;   // min as ~max(~x)
        const uint64_t mhi = threadIdx.x < ncb ? w.bmax[threadIdx.x] : 0;
        uint64_t a, b;
        block_excl<true, kThreads>(nlo, scr, &a);
        block_excl<true, kThreads>(mhi, scr, &b);
        if (threadIdx.x == 0) {
            w.rinfo[0] = ~a;
            w.rinfo[1] = b;
        }
    }
    if (kCount && threadIdx.x == 0) {
        const uint64_t after = g.state[0] + tot;
        uint64_t need = g.capacity;
        while (need < after) need = need == 0 ? 32 : 2 * need;
        *needed = need;
        w.scal[0] = tot;
        w.scal[1] = after <= g.capacity;
    }
}

// Ranks and scatter. Misses: mrank[i] = misses before item i, and each
// miss's range goes to its rank and into the misses' index. Inserts:
// rank[i] = inserts before item i, newrefs[i] = 1 (by rank; ranks < n), and
// each insert's range goes to its rank and into the inserts' index.
template <uint8_t kCls>
__global__ __launch_bounds__(kThreads) void k_rank_apply(RegWs w, uint32_t n)
{
    __shared__ uint64_t scr[kWaves];
    const uint32_t p = blockIdx.x * kChunk + threadIdx.x * kPer;
    uint32_t f[kPer];
    item_flags<kCls>(w, n, p, f);
    // The ranges of all four items, read at once (clamped, not guarded).
    uint64_t b[kPer], t[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t i = p + k < n ? p + k : 0u;
        b[k] = w.base[i];
        t[k] = w.top[i];
    }
    uint64_t tot;
    uint32_t run = (uint32_t)(w.ichunk[blockIdx.x] +
                              block_excl<false, kThreads>((uint64_t)(f[0] + f[1] + f[2] + f[3]),
                                                          scr, &tot));
    uint32_t *rk_out = kCls == kMiss ? w.mrank : w.rank;
    uint64_t *ob = kCls == kMiss ? w.mbase : w.ibase;
    uint64_t *ot = kCls == kMiss ? w.mtop : w.itop;
    const RIdx &X = kCls == kMiss ? w.xm : w.xi;
    uint32_t *nlong = w.rcnt + (kCls == kMiss ? 0 : 1);
    const uint64_t lo = w.rinfo[0];
    const uint32_t sh = idx_shift(lo, w.rinfo[1], w.nbk);
    // The wave's ranks are at most 256 consecutive ones from lane 0's first:
    // they fall in 256-rank tile bt or bt + 1.
    const uint32_t bt = __shfl(run, 0, kWave) / 256;
    uint32_t l0 = 0, l1 = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t i = p + k;
        if (i < n) {
            rk_out[i] = run;
            if (kCls == kNew) w.newrefs[i] = 1;
            if (f[k]) {
                ob[run] = b[k];
                ot[run] = t[k];
                if (idx_put(X, lo, sh, b[k], t[k], run)) {
                    if (run / 256 == bt) ++l0;
                    else ++l1;
                }
            }
        }
        run += f[k];
    }
    const uint32_t w0 = wave_sum(l0), w1 = wave_sum(l1);
    if (lane() == 0) {
        if (w0 + w1) atomicAdd(nlong, w0 + w1);
        if (w0) atomicAdd(&X.tlong[bt], w0);
        if (w1) atomicAdd(&X.tlong[bt + 1], w1);
    }
}

// Reads the in-table ranges of bucket c of index X (all kSlots slots at
// once; those past the bucket's count are not used) and calls f(range, rank)
// for each one the bucket holds.
template <class F>
__device__ __forceinline__ void idx_bucket(const RIdx &X, uint32_t c, F f)
{
    const uint32_t m = X.cnt[c] < kSlots ? X.cnt[c] : kSlots;
    Range r[kSlots];
    uint32_t q[kSlots];
#pragma unroll
    for (uint32_t s = 0; s < kSlots; ++s) {
        r[s] = X.rec[(uint64_t)c * kSlots + s];
        q[s] = X.key[(uint64_t)c * kSlots + s];
    }
#pragma unroll
    for (uint32_t s = 0; s < kSlots; ++s)
        if (s < m) f(r[s], q[s]);
}

// Range of rank r for a tile of the long walk: the range itself if it is
// flagged long, else one that contains nothing (its bucket already answered
// for it). r is clamped, not guarded, so the three loads go out together.
__device__ __forceinline__ Range long_range(const RIdx &X, const uint64_t *rb, const uint64_t *rt,
                                            uint32_t r, uint32_t jend)
{
    const uint32_t q = r < jend ? r : jend - 1;
    const uint8_t f = X.lflag[q];
    const Range x{rb[q], rt[q]};
    return r < jend && f ? x : kNoRange;
}
static_assert(kRankTiles == kThreads, "one long-tile count per thread");

// The 256-rank tiles that hold a long range, listed in rank order so that the
// walks visit only those: thread t tests tile t; part 1 counts each wave's
// tiles (a ballot), part 2 (after a barrier) writes the list and returns its
// length.
struct TileList {
    uint32_t list[kRankTiles];
    uint32_t wcnt[kWaves];
};
__device__ __forceinline__ uint64_t tiles_part1(TileList &L, const uint32_t *tlong)
{
    const uint64_t bal = __ballot(tlong[threadIdx.x] != 0);
    if (lane() == 0) L.wcnt[wave()] = (uint32_t)__popcll(bal);
    return bal;
}
// Listed tiles that start before rank jend (the list is in rank order).
__device__ __forceinline__ uint32_t tiles_before(const TileList &L, uint32_t ntl, uint32_t jend)
{
    uint32_t lo = 0, hi = ntl;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (L.list[mid] * kThreads < jend) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ uint32_t tiles_part2(TileList &L, uint64_t bal)
{
    uint32_t off = 0, all = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        off += v < wave() ? L.wcnt[v] : 0u;
        all += L.wcnt[v];
    }
    const uint64_t below = lane() ? (~0ull >> (64 - lane())) : 0ull;
    if ((bal >> lane()) & 1ull) L.list[off + (uint32_t)__popcll(bal & below)] = threadIdx.x;
    return all;
}

// inserted(i) = miss and no earlier miss contains it. A containing earlier
// miss is either in the buckets of the misses' index that can hold it,
// which wave 0 reads for the block's kPairItems items, or long; the long
// ones are walked in rank order through LDS 256 ranks at a time (tiles
// without one are skipped), each wave comparing the items still open with
// its own quarter of the tile, up to the largest miss rank among them.
// s_done[l] turns 1 once item l is decided.
__global__ __launch_bounds__(kThreads) void k_reg_inserted(RegWs w, uint32_t n)
{
    __shared__ Range s_r[kThreads];
    __shared__ uint32_t s_done[kPairItems];
    __shared__ TileList s_tl;
    __shared__ uint32_t s_jend;
    const uint32_t ln = threadIdx.x % kWave, k0 = threadIdx.x / kWave * kWave;
    const uint32_t i = blockIdx.x * kPairItems + ln;
    const bool me = i < n && w.cls[i] == kMiss;
    const uint64_t b = me ? w.base[i] : 0, t = me ? w.top[i] : 0;
    const uint32_t mi = me ? w.mrank[i] : 0;             // misses before item i
    const bool walk = w.rcnt[0] != 0;                    // any long miss (uniform)
    if (!walk && k0 != 0) return;                        // the buckets alone decide
    if (threadIdx.x == 0) s_jend = 0;
    const uint64_t bal = walk ? tiles_part1(s_tl, w.xm.tlong) : 0;
    if (k0 == 0) {
        bool in = false;
        if (me) {
            const uint64_t lo = w.rinfo[0], hi = w.rinfo[1];
            const uint32_t sh = idx_shift(lo, hi, w.nbk);
            uint32_t c0, c1;
            idx_window(lo, hi, sh, b, c0, c1);
            for (uint32_t c = c0; c <= c1; ++c)
                idx_bucket(w.xm, c, [&](const Range &r, uint32_t q) {
                    in |= q < mi && r.base <= b && t <= r.top;
                });
        }
        if (!walk) {
            if (me && !in) w.cls[i] = kNew;
            return;
        }
        s_done[ln] = !me || in;
    }
    __syncthreads();
    const uint32_t ntl = tiles_part2(s_tl, bal);
    if (k0 == 0 && s_done[ln] == 0) atomicMax(&s_jend, mi);
    __syncthreads();
    const uint32_t jend = s_jend;                        // ranks the open items need
    const uint32_t nt = tiles_before(s_tl, ntl, jend);   // tiles to walk
    Range nx = nt ? long_range(w.xm, w.mbase, w.mtop, s_tl.list[0] * kThreads + threadIdx.x, jend)
                  : kNoRange;
    for (uint32_t u = 0; u < nt; ++u) {
        const uint32_t j0 = s_tl.list[u] * kThreads;     // a tile holding a long miss
        const bool open = s_done[ln] == 0;
        if (__syncthreads_or(open) == 0) break;          // every item here is decided
        s_r[threadIdx.x] = nx;
        if (u + 1 < nt)                                  // the next tile, loaded while this one is used
            nx = long_range(w.xm, w.mbase, w.mtop, s_tl.list[u + 1] * kThreads + threadIdx.x, jend);
        __syncthreads();
        if (open) {
            const uint32_t lim = mi > j0 ? (mi - j0 < kThreads ? mi - j0 : kThreads) : 0;   // rank < mi
            const uint32_t ke = lim < k0 + kWave ? lim : k0 + kWave;
            bool in = false;
            uint32_t k = k0;
            for (; k + kPairStep <= ke && !in; k += kPairStep) {   // reads in flight together
                Range r[kPairStep];
#pragma unroll
                for (uint32_t u = 0; u < kPairStep; ++u) r[u] = s_r[k + u];
#pragma unroll
                for (uint32_t u = 0; u < kPairStep; ++u) in |= r[u].base <= b && t <= r[u].top;
            }
            for (; k < ke && !in; ++k) in = s_r[k].base <= b && t <= s_r[k].top;
            if (in) s_done[ln] = 1;
        }
        __syncthreads();
    }
    if (k0 == 0 && me && s_done[ln] == 0) w.cls[i] = kNew;
}

// For every range that is not inserted, the earlier insert with the smallest
// (start, rank) that contains it decides between that insert and the old
// record it hit; and the (start, rank) rank of each insert. Both questions
// are about inserts only: wave 0 reads the buckets of the inserts' index
// that can hold a containing insert (or, for an insert, its own bucket, the
// earlier buckets being counted by the index's prefix), and the long
// inserts are walked in rank order through LDS 256 ranks at a time (tiles
// without one are skipped), each wave on a quarter of every tile, partial
// answers merged at the end: item i meets the rank[i] inserts before it, an
// insert meets all of them. (start, rank) orders inserts as (start, batch
// index) does.
__global__ __launch_bounds__(kThreads) void k_reg_owner(RegWs w, uint32_t n)
{
    __shared__ Range s_r[kThreads];
    __shared__ uint64_t s_bb[kThreads];
    __shared__ uint32_t s_bj[kThreads];
    __shared__ TileList s_tl;
    __shared__ uint32_t s_jend;
    const uint32_t ln = threadIdx.x % kWave, k0 = threadIdx.x / kWave * kWave;
    const uint32_t i = blockIdx.x * kPairItems + ln;
    const uint8_t c = i < n ? w.cls[i] : kInvalid;
    const bool look = c == kMiss || c == kHit;           // looks for a containing insert
    const bool ins = c == kNew;                          // ranks itself among inserts
    const uint64_t b = look || ins ? w.base[i] : 0;
    const uint64_t t = look || ins ? w.top[i] : 0;
    const uint32_t ri = look || ins ? w.rank[i] : 0;     // inserts before item i
    uint32_t best = UINT32_MAX, brank = 0;
    uint64_t bbase = 0;
    // Takes insert q (range r) if it contains item i and comes first so far.
    auto consider = [&](const Range &r, uint32_t q) {
        if (q < ri && r.base <= b && t <= r.top &&
            (best == UINT32_MAX || r.base < bbase || (r.base == bbase && q < best))) {
            best = q;
            bbase = r.base;
        }
    };
    // Whether insert q (range r) comes before this insert in (start, rank)
    // order; a range that contains nothing never does.
    auto before = [&](const Range &r, uint32_t q) -> uint32_t {
        return r.base < b || (r.base == b && q < ri);
    };
    const bool walk = w.rcnt[1] != 0;                    // any long insert (uniform)
    if (!walk && k0 != 0) return;                        // wave 0's buckets alone decide
    if (threadIdx.x == 0) s_jend = 0;
    const uint64_t bal = walk ? tiles_part1(s_tl, w.xi.tlong) : 0;
    if (k0 == 0 && (look || ins)) {
        const uint64_t lo = w.rinfo[0], hi = w.rinfo[1];
        const uint32_t sh = idx_shift(lo, hi, w.nbk);
        if (look) {
            uint32_t c0, c1;
            idx_window(lo, hi, sh, b, c0, c1);
            for (uint32_t cb = c0; cb <= c1; ++cb) idx_bucket(w.xi, cb, consider);
        } else {
            const uint32_t cb = (uint32_t)((b - lo) >> sh);   // an insert's start is in [lo, hi]
            brank = w.xi.pre[cb];
            idx_bucket(w.xi, cb, [&](const Range &r, uint32_t q) { brank += before(r, q); });
        }
    }
    bool walked = false;                                 // uniform over the block
    if (walk) {                                          // the long inserts, in rank order
        __syncthreads();
        const uint32_t ntl = tiles_part2(s_tl, bal);
        // Inserts the block needs: all of them if it holds one, else those
        // before its last looking item.
        if (k0 == 0 && (look || ins)) atomicMax(&s_jend, ins ? (uint32_t)w.scal[0] : ri);
        __syncthreads();
        const uint32_t jend = s_jend;
        const uint32_t nt = tiles_before(s_tl, ntl, jend);   // tiles to walk
        Range nx = nt ? long_range(w.xi, w.ibase, w.itop, s_tl.list[0] * kThreads + threadIdx.x, jend)
                      : kNoRange;
        for (uint32_t u = 0; u < nt; ++u) {
            const uint32_t j0 = s_tl.list[u] * kThreads;     // a tile holding a long insert
            walked = true;
            s_r[threadIdx.x] = nx;
            if (u + 1 < nt)                              // the next tile, loaded while this one is used
                nx = long_range(w.xi, w.ibase, w.itop, s_tl.list[u + 1] * kThreads + threadIdx.x, jend);
            __syncthreads();
            const uint32_t lim = jend - j0 < kThreads ? jend - j0 : kThreads;
            if (look) {
                const uint32_t jl = ri > j0 ? (ri - j0 < lim ? ri - j0 : lim) : 0;   // rank < ri
                const uint32_t ke = jl < k0 + kWave ? jl : k0 + kWave;
                uint32_t k = k0;
                for (; k + kPairStep <= ke; k += kPairStep) {
                    Range r[kPairStep];
    #pragma unroll
                    for (uint32_t u = 0; u < kPairStep; ++u) r[u] = s_r[k + u];
    #pragma unroll
                    for (uint32_t u = 0; u < kPairStep; ++u) consider(r[u], j0 + k + u);
                }
                for (; k < ke; ++k) consider(s_r[k], j0 + k);
            } else if (ins) {
                const uint32_t ke = lim < k0 + kWave ? lim : k0 + kWave;
                uint32_t k = k0;
                for (; k + kPairStep <= ke; k += kPairStep) {
                    uint64_t rb[kPairStep];
    #pragma unroll
                    for (uint32_t u = 0; u < kPairStep; ++u) rb[u] = s_r[k + u].base;
    #pragma unroll
                    for (uint32_t u = 0; u < kPairStep; ++u) brank += before(Range{rb[u], 0}, j0 + k + u);
                }
                for (; k < ke; ++k) brank += before(s_r[k], j0 + k);
            }
            __syncthreads();
        }
        if (walked) {
            s_bb[threadIdx.x] = bbase;
            s_bj[threadIdx.x] = look ? best : brank;
            __syncthreads();
        }
    }
    if (k0 != 0 || !(look || ins)) return;
    if (walked) {
        for (uint32_t v = kWave; v < kThreads; v += kWave) {
            const uint32_t oj = s_bj[v + ln];
            const uint64_t ob = s_bb[v + ln];
            if (ins) {
                brank += oj;
            } else if (oj != UINT32_MAX &&
                       (best == UINT32_MAX || ob < bbase || (ob == bbase && oj < best))) {
                best = oj;
                bbase = ob;
            }
        }
    }
    if (c == kMiss || (c == kHit && best != UINT32_MAX && bbase < w.hstart[i])) {
        w.owner[i] = best;                               // a miss always finds one
        w.cls[i] = kHitNew;
    } else if (ins) {
        w.brank[i] = brank;
    }
}

// Atomic update (add, subtract or minimum) of word base[idx] by v for every
// lane with `on`, made once per wave, with the wave's total (or minimum), when
// all such lanes of the wave name the same word: a record that every call
// of a batch names would otherwise take one atomic per call, all on one
// word, one after another. Every lane of the wave must call it.
enum class Upd { kAdd, kSub, kMin };
template <Upd kOp>
__device__ __forceinline__ void wave_update(uint32_t *base, uint32_t idx, bool on, uint32_t v)
{
    const uint64_t act = __ballot(on);
    if (act == 0) return;
    const int first = __ffsll((unsigned long long)act) - 1;
    const uint32_t i0 = __shfl(idx, first, kWave);
    if (__ballot(on && idx != i0) == 0) {
        uint32_t x = on ? v : (kOp == Upd::kMin ? UINT32_MAX : 0u);
#pragma unroll
        for (int d = kWave / 2; d > 0; d >>= 1) {
            const uint32_t y = __shfl_xor(x, d, kWave);
            x = kOp == Upd::kMin ? (y < x ? y : x) : x + y;
        }
        if (lane() == first) {
            if (kOp == Upd::kAdd) atomicAdd(base + i0, x);
            else if (kOp == Upd::kSub) atomicSub(base + i0, x);
            else atomicMin(base + i0, x);
        }
    } else if (on) {
        if (kOp == Upd::kAdd) atomicAdd(base + idx, v);
        else if (kOp == Upd::kSub) atomicSub(base + idx, v);
        else atomicMin(base + idx, v);
    }
}

// Handles, kinds and reference counts (or NOSPACE for every item).
__global__ __launch_bounds__(kThreads) void k_reg_apply(RegState g, RegWs w, uint32_t n,
                                                        uint64_t *handle, uint8_t *kind)
{
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    const bool valid = i < n;
    const uint8_t c = valid ? w.cls[i] : kInvalid;
    if (!w.scal[1]) {                                    // uniform: the batch did not fit
        if (valid) {
            handle[i] = 0;
            kind[i] = kNospace;
        }
        return;
    }
    const uint64_t next = g.state[1];
    uint64_t h = 0;
    const uint32_t hs = c == kHit ? w.hit[i] : 0u;       // storage slot of the hit record
    const uint32_t o = c == kHitNew ? w.owner[i] : 0u;   // rank of the containing insert (< n)
    if (c == kHit) {
        h = g.id[hs];
    } else if (c == kNew) {
        h = next + w.rank[i];
        w.newbase[w.brank[i]] = w.base[i];
    } else if (c == kHitNew) {
        h = next + o;
    }
    wave_update<Upd::kAdd>(g.refs, hs, c == kHit, 1u);
    wave_update<Upd::kAdd>(w.newrefs, o, c == kHitNew && o < n, 1u);
    if (valid) {
        handle[i] = h;
        kind[i] = c;
    }
}

// New records in storage after the live ones, and the merged start order.
__global__ __launch_bounds__(kThreads) void k_reg_insert(RegState g, RegWs w, uint32_t n)
{
    if (!w.scal[1]) return;
    const uint64_t count = g.state[0], T = w.scal[0], next = g.state[1];
    const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    // Existing records: shift by the inserts that start strictly before.
    for (uint64_t p = tid; p < count; p += stride) {
        const uint64_t st = w.sstart[p];
        uint64_t lo = 0, hi = T;                         // inserts with start < st
        while (lo < hi) {
            const uint64_t mid = (lo + hi) >> 1;
            if (w.newbase[mid] < st) lo = mid + 1;
            else hi = mid;
        }
        w.merged[p + lo] = g.by_start[p];
    }
    // Inserts: after the existing records that start at or before them.
    for (uint64_t i = tid; i < n; i += stride) {
        if (w.cls[i] != kNew) continue;
        const uint64_t b = w.base[i];
        uint64_t lo = 0, hi = count;                     // existing with start <= b
        while (lo < hi) {
            const uint64_t mid = (lo + hi) >> 1;
            if (w.sstart[mid] <= b) lo = mid + 1;
            else hi = mid;
        }
        const uint64_t slot = count + w.rank[i];
        w.merged[w.brank[i] + lo] = (uint32_t)slot;
        g.start[slot] = b;
        g.end[slot] = w.top[i];
        g.id[slot] = next + w.rank[i];
        g.refs[slot] = w.newrefs[w.rank[i]];
    }
}

__global__ __launch_bounds__(kThreads) void k_reg_commit(RegState g, RegWs w)
{
    if (!w.scal[1]) return;
    const uint64_t count = g.state[0] + w.scal[0];
    for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < count;
         p += (uint64_t)gridDim.x * kThreads)
        g.by_start[p] = w.merged[p];
}

__global__ void k_reg_state(RegState g, RegWs w)
{
    if (threadIdx.x == 0 && w.scal[1]) {
        g.state[0] += w.scal[0];
        g.state[1] += w.scal[0];
    }
}

// ----------------------------------------------------------- deregister ---

__global__ __launch_bounds__(kThreads) void k_dereg_find(RegState g, RegWs w, const uint64_t *h,
                                                         uint32_t n)
{
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const uint64_t count = g.state[0], key = h[i];
    uint64_t lo = 0, hi = count;                         // storage is in handle order
    while (lo < hi) {
        const uint64_t mid = (lo + hi) >> 1;
        if (g.id[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    const bool found = lo < count && g.id[lo] == key;
    w.hit[i] = found ? (uint32_t)lo : UINT32_MAX;
    if (found) w.tmp32[lo] = UINT32_MAX;                 // its first call, set next
}

// The first call of the batch on each named record (tmp32 by storage slot).
__global__ __launch_bounds__(kThreads) void k_dereg_first(RegWs w, uint32_t n)
{
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t me = i < n ? w.hit[i] : UINT32_MAX;
    wave_update<Upd::kMin>(w.tmp32, me, me != UINT32_MAX, i);
}

// Calls before i naming the same record decide whether call i succeeds. No
// call before the record's first call of the batch names it, so the first
// call has none before it, and a later call on a record of one reference
// has at least one: neither counts. The others count the calls in [first,
// i): blocks of kPairItems calls, each wave over its quarter of every tile,
// adding its count to s_before; a call that has seen as many earlier calls
// as its record has references is stale whatever follows, so it stops there.
__global__ __launch_bounds__(kThreads) void k_dereg_status(RegState g, RegWs w, uint32_t n,
                                                           uint8_t *status)
{
    __shared__ __align__(16) uint32_t s_slot[kThreads];
    __shared__ uint32_t s_before[kPairItems];
    __shared__ uint32_t s_from;
    const uint32_t ln = threadIdx.x % kWave, k0 = threadIdx.x / kWave * kWave;
    const uint32_t i = blockIdx.x * kPairItems + ln;
    const uint32_t me = i < n ? w.hit[i] : UINT32_MAX;
    const uint32_t r = me != UINT32_MAX ? g.refs[me] : 0u;
    const uint32_t first = me != UINT32_MAX ? w.tmp32[me] : i;
    const bool counts = me != UINT32_MAX && first < i && r > 1;
    if (threadIdx.x == 0) s_from = UINT32_MAX;
    if (k0 == 0) s_before[ln] = first < i ? (r > 1 ? 0u : 1u) : 0u;
    __syncthreads();
    if (k0 == 0 && counts) atomicMin(&s_from, first);
    __syncthreads();
    const uint32_t jend = blockIdx.x * kPairItems + kPairItems;
    const uint32_t jfrom = s_from == UINT32_MAX ? jend : s_from / kThreads * kThreads;
    uint32_t hj = jfrom + threadIdx.x < n ? w.hit[jfrom + threadIdx.x] : UINT32_MAX;   // one tile ahead
    for (uint32_t j0 = jfrom; j0 < jend; j0 += kThreads) {
        const bool open = counts && s_before[ln] < r;
        if (__syncthreads_or(open) == 0) break;          // every call here is decided
        s_slot[threadIdx.x] = hj;
        const uint32_t jn = j0 + kThreads + threadIdx.x;
        hj = j0 + kThreads < jend && jn < n ? w.hit[jn] : UINT32_MAX;
        __syncthreads();
        if (open) {
            const uint32_t lim = i > j0 ? (i - j0 < kThreads ? i - j0 : kThreads) : 0;
            const uint32_t ke = lim < k0 + kWave ? lim : k0 + kWave;
            uint32_t c = 0, k = k0;
            for (; k + 4 * kPairStep <= ke; k += 4 * kPairStep) {   // 16-byte reads in flight together
                uint4 v[kPairStep];
#pragma unroll
                for (uint32_t u = 0; u < kPairStep; ++u)
                    v[u] = *reinterpret_cast<const uint4 *>(&s_slot[k + 4 * u]);
#pragma unroll
                for (uint32_t u = 0; u < kPairStep; ++u)
                    c += (v[u].x == me) + (v[u].y == me) + (v[u].z == me) + (v[u].w == me);
            }
            for (; k < ke; ++k) c += s_slot[k] == me;
            if (c) atomicAdd(&s_before[ln], c);
        }
        __syncthreads();
    }
    if (k0 != 0 || i >= n) return;
    const uint32_t before = s_before[ln];                 // exact unless already >= r
    uint8_t st = DMADESC_DEREG_STALE;
    if (me != UINT32_MAX) {
        if (before + 1 < r) st = DMADESC_DEREG_OK;
        else if (before + 1 == r) st = DMADESC_DEREG_REMOVED;
    }
    status[i] = st;
    w.cls[i] = st;
}

__global__ __launch_bounds__(kThreads) void k_dereg_drop(RegState g, RegWs w, uint32_t n)
{
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    const bool on = i < n && w.cls[i] != DMADESC_DEREG_STALE;
    wave_update<Upd::kSub>(g.refs, on ? w.hit[i] : 0u, on, 1u);
}

// Stable compaction: kept storage slots move to their exclusive prefix, and
// the start-ordered index keeps its kept entries, renamed to the new slots.
__global__ __launch_bounds__(kThreads) void k_dereg_gather(RegState g, RegWs w)
{
    const uint64_t count = g.state[0];
    for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < count;
         p += (uint64_t)gridDim.x * kThreads) {
        w.tmp64a[p] = g.start[p];
        w.tmp64b[p] = g.end[p];
        w.tmp64c[p] = g.id[p];
        w.tmp32[p] = g.refs[p];
        w.merged[p] = g.by_start[p];
    }
}

__global__ __launch_bounds__(kThreads) void k_dereg_scatter(RegState g, RegWs w,
                                                            const uint64_t *slot_pre,
                                                            const uint64_t *order_pre)
{
    const uint64_t count = g.state[0];
    for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < count;
         p += (uint64_t)gridDim.x * kThreads) {
        if (w.tmp32[p] != 0) {
            const uint64_t q = slot_pre[p];
            g.start[q] = w.tmp64a[p];
            g.end[q] = w.tmp64b[p];
            g.id[q] = w.tmp64c[p];
            g.refs[q] = w.tmp32[p];
        }
        const uint32_t s = w.merged[p];
        if (w.tmp32[s] != 0) g.by_start[order_pre[p]] = (uint32_t)slot_pre[s];
    }
}

__global__ void k_dereg_state(RegState g, RegWs w)
{
    if (threadIdx.x == 0) g.state[0] = w.scal[2];
}

// ------------------------------------------------------------ workspace ---

struct Carver {
    // Walks the layout by offset, so the same walk both sizes the workspace
    // (base == nullptr) and hands out its pieces.
    char *base;
    size_t off;
    template <typename T>
    T *take(uint64_t count)
    {
        T *r = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += align256(count * sizeof(T));
        return r;
    }
};

// Buckets of the range indexes for a batch of n: a power of two near n / 4.
uint32_t reg_buckets(uint64_t n)
{
    uint32_t b = kMinBuckets;
    while (b < n / 4 && b < kMaxBuckets) b <<= 1;
    return b;
}

// Lays the workspace out for a batch of n items and a table of cap records;
// *bytes receives the end of the walk, which is what the workspace must hold.
RegWs carve(void *ws, uint64_t n, uint64_t cap, size_t *bytes = nullptr)
{
    Carver c{static_cast<char *>(ws), 0};
    RegWs w;
    w.base = c.take<uint64_t>(n);
    w.top = c.take<uint64_t>(n);
    w.cls = c.take<uint8_t>(n);
    w.hit = c.take<uint32_t>(n);
    w.hstart = c.take<uint64_t>(n);
    w.rank = c.take<uint32_t>(n);
    w.brank = c.take<uint32_t>(n);
    w.owner = c.take<uint32_t>(n);
    w.newrefs = c.take<uint32_t>(n);
    w.newbase = c.take<uint64_t>(n);
    w.ibase = c.take<uint64_t>(n);
    w.itop = c.take<uint64_t>(n);
    w.mbase = c.take<uint64_t>(n);
    w.mtop = c.take<uint64_t>(n);
    w.mrank = c.take<uint32_t>(n);
    w.nbk = reg_buckets(n);
    for (RIdx *x : {&w.xm, &w.xi}) {
        x->cnt = c.take<uint32_t>(w.nbk);
        x->rec = c.take<Range>((uint64_t)w.nbk * kSlots);
        x->key = c.take<uint32_t>((uint64_t)w.nbk * kSlots);
        x->lflag = c.take<uint8_t>(n);
        x->tlong = c.take<uint32_t>(kRankTiles);
    }
    w.xm.pre = nullptr;
    w.xi.pre = c.take<uint32_t>(w.nbk);
    w.rinfo = c.take<uint64_t>(2);
    w.bmin = c.take<uint64_t>(kRankTiles);
    w.bmax = c.take<uint64_t>(kRankTiles);
    w.rcnt = c.take<uint32_t>(2);
    w.sstart = c.take<uint64_t>(cap);
    w.pm = c.take<uint64_t>(cap);
    w.merged = c.take<uint32_t>(cap + n);
    w.newslot = c.take<uint32_t>(cap);
    w.tmp64a = c.take<uint64_t>(cap);
    w.tmp64b = c.take<uint64_t>(cap);
    w.tmp64c = c.take<uint64_t>(cap);
    w.tmp32 = c.take<uint32_t>(cap);
    w.chunk = c.take<uint64_t>(kMaxChunks);
    w.ichunk = c.take<uint64_t>(kItemChunks);
    w.scal = c.take<uint64_t>(4);
    if (bytes) *bytes = c.off;
    return w;
}

size_t carve_bytes(uint64_t n, uint64_t cap)
{
    size_t bytes = 0;
    carve(nullptr, n, cap, &bytes);
    return bytes;
}

}  // namespace

size_t ws_registry(uint64_t n, uint64_t capacity)
{
    return carve_bytes(n < 1 ? 1 : n, capacity < 1 ? 1 : capacity);
}

hipError_t launch_reg_register(const RegArgs &a, hipStream_t s)
{
    const uint64_t cap = a.capacity;
    RegState g{a.start, a.end, a.id, a.refs, a.by_start, a.state, cap};
    RegWs w = carve(a.ws, a.n < 1 ? 1 : a.n, cap < 1 ? 1 : cap);
    const uint32_t n = (uint32_t)a.n;
    const unsigned nb = (n + kThreads - 1) / kThreads;
    const unsigned pb = (n + kPairItems - 1) / kPairItems;
    const unsigned cb = (n + kChunk - 1) / kChunk;       // item chunks of the rankings
    const unsigned rb = (unsigned)((cap + kThreads - 1) / kThreads < 4096 ? (cap + kThreads - 1) / kThreads : 4096);
    if (rb) {
        hipLaunchKernelGGL(k_reg_starts, dim3(rb), dim3(kThreads), 0, s, g, w);
        scan_records<true, true>(EndsInOrder{a.end, a.by_start}, a.state, cap, w.chunk, w.pm,
                                 nullptr, s);
    }
    if (nb) {
        const uint32_t cl = w.nbk > kRankTiles ? w.nbk : kRankTiles;
        hipLaunchKernelGGL(k_ridx_clear, dim3((cl + kThreads - 1) / kThreads), dim3(kThreads), 0,
                           s, w);
        hipLaunchKernelGGL(k_reg_classify, dim3(nb), dim3(kThreads), 0, s, g, w, a.page_shift,
                           a.addr, a.size, n);
        hipLaunchKernelGGL(k_rank_chunks<kMiss>, dim3(cb), dim3(kThreads), 0, s, w, n);
        hipLaunchKernelGGL(k_rank_top<false>, dim3(1), dim3(kThreads), 0, s, g, w, n, a.needed);
        hipLaunchKernelGGL(k_rank_apply<kMiss>, dim3(cb), dim3(kThreads), 0, s, w, n);
        hipLaunchKernelGGL(k_reg_inserted, dim3(pb), dim3(kThreads), 0, s, w, n);
        hipLaunchKernelGGL(k_rank_chunks<kNew>, dim3(cb), dim3(kThreads), 0, s, w, n);
    }
    hipLaunchKernelGGL(k_rank_top<true>, dim3(1), dim3(kThreads), 0, s, g, w, n, a.needed);
    if (nb) hipLaunchKernelGGL(k_rank_apply<kNew>, dim3(cb), dim3(kThreads), 0, s, w, n);
    if (nb) {
        hipLaunchKernelGGL(k_ridx_scan, dim3(1), dim3(kTopThreads), 0, s, w);
        hipLaunchKernelGGL(k_reg_owner, dim3(pb), dim3(kThreads), 0, s, w, n);
        hipLaunchKernelGGL(k_reg_apply, dim3(nb), dim3(kThreads), 0, s, g, w, n, a.handle,
                           a.kind);
        const unsigned ib = (unsigned)((cap + n + kThreads - 1) / kThreads < 4096
                                           ? (cap + n + kThreads - 1) / kThreads : 4096);
        hipLaunchKernelGGL(k_reg_insert, dim3(ib), dim3(kThreads), 0, s, g, w, n);
        hipLaunchKernelGGL(k_reg_commit, dim3(ib), dim3(kThreads), 0, s, g, w);
        hipLaunchKernelGGL(k_reg_state, dim3(1), dim3(64), 0, s, g, w);
    }
    return hipGetLastError();
}

hipError_t launch_reg_deregister(const RegArgs &a, hipStream_t s)
{
    const uint64_t cap = a.capacity;
    RegState g{a.start, a.end, a.id, a.refs, a.by_start, a.state, cap};
    RegWs w = carve(a.ws, a.n < 1 ? 1 : a.n, cap < 1 ? 1 : cap);
    const uint32_t n = (uint32_t)a.n;
    const unsigned nb = (n + kThreads - 1) / kThreads;
    const unsigned pb = (n + kPairItems - 1) / kPairItems;
    if (nb == 0 || cap == 0) {
        if (nb) {                                        // nothing is live: all stale
            hipLaunchKernelGGL(k_dereg_find, dim3(nb), dim3(kThreads), 0, s, g, w, a.handle_in, n);
            hipLaunchKernelGGL(k_dereg_status, dim3(pb), dim3(kThreads), 0, s, g, w, n, a.status);
        }
        return hipGetLastError();
    }
    const unsigned rb = (unsigned)((cap + kThreads - 1) / kThreads < 4096 ? (cap + kThreads - 1) / kThreads : 4096);
    hipLaunchKernelGGL(k_dereg_find, dim3(nb), dim3(kThreads), 0, s, g, w, a.handle_in, n);
    hipLaunchKernelGGL(k_dereg_first, dim3(nb), dim3(kThreads), 0, s, w, n);
    hipLaunchKernelGGL(k_dereg_status, dim3(pb), dim3(kThreads), 0, s, g, w, n, a.status);
    hipLaunchKernelGGL(k_dereg_drop, dim3(nb), dim3(kThreads), 0, s, g, w, n);
    // Prefixes of kept slots (storage) and kept entries (start order).
    scan_records<false, false>(KeptSlots{a.refs}, a.state, cap, w.chunk, w.pm, &w.scal[2], s);
    scan_records<false, false>(KeptInOrder{a.refs, a.by_start}, a.state, cap, w.chunk, w.sstart,
                               nullptr, s);
    hipLaunchKernelGGL(k_dereg_gather, dim3(rb), dim3(kThreads), 0, s, g, w);
    hipLaunchKernelGGL(k_dereg_scatter, dim3(rb), dim3(kThreads), 0, s, g, w, w.pm, w.sstart);
    hipLaunchKernelGGL(k_dereg_state, dim3(1), dim3(64), 0, s, g, w);
    return hipGetLastError();
}

}  // namespace dd

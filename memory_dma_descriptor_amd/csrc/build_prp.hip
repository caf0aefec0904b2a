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
// One pass, one kernel (after a small workspace-clearing kernel):
//
//  * Request phase, T threads per block and one or four requests per thread
//    (prp_shape below: 256-1,024 requests per block by batch size), item k
//    of thread t being request block_base + T k + t (so every column load
//    is contiguous per wave):
//    validity, 4 KiB page count, list pages L. List pages are handed out in
//    request order by a device-wide exclusive scan done in the same pass
//    with decoupled look-back: each block publishes its aggregate, then
//    reads its predecessors' published values until it meets an inclusive
//    prefix. Block order comes from an atomic ticket, so a block only ever
//    waits on blocks that are already running; waits are bounded.
//  * Because a request's list pages are consecutive slots, its written
//    entries (data entries plus chain pointers) are ONE contiguous run of
//    E = m + L - 1 words starting at word 512 * slot of the pool: word q of
//    the run is the chain pointer when q % 512 == 511 on a non-final page,
//    else data entry j = q - q / 512. No division is needed anywhere.
//  * List phase, per wave and per item round: the wave's 64 consecutive
//    requests of that round are emitted in pairs of consecutive words
//    (16 bytes), load-balanced over pairs, not requests: lane k of each step
//    takes pair c + k, finds its request by a 6-step search over the wave's
//    pair offsets in LDS, and writes it with one non-temporal 16-byte store,
//    so that each store instruction fills whole 64-byte segments (a lane
//    writing 32 bytes as two stores would fill half of every 32 bytes per
//    instruction). Two consecutive 4 KiB pages lie in at most two 64 KiB GPU
//    pages, so each pair reads at most two table entries, staged in LDS.
//    Rounds with a list of 2^24 words or more take a 64-bit path in groups
//    of 4 words.
//
// Packed layout (the same kernel, kPacked = true): lists lie back to back in
// data slots, 511 to a page (words 0..510); a request's list starts where the
// previous one ended, and PRP2 may carry that qword offset, as NVMe allows for
// the list pointer in a command. The scan hands out data slots (entries)
// instead of pages, and a wave writes the words of its 64 consecutive
// requests as one range [word(S), word(E)) of the pool: aligned 4-word groups,
// each word's owner found by a search over the requests' first slots. Word
// 511 of a page is written by the owner of the page's last slot: a chain
// pointer when two or more of its entries remain, its final entry when one
// remains (the next page's word 0 is then 0), else 0. The list writes become
// one dense stream instead of one short run per 4 KiB list page.
#include <type_traits>

#include "dd_device.hpp"
#include "dd_internal.h"
#include "dd_lookback.hpp"

namespace dd {
namespace {

// Requests per thread: 4 for large batches; 1 for batches of at most
// kSmallBatch requests, whose blocks would otherwise be too few to fill the
// chip (a 262,144-request batch of long lists makes 256 blocks of 1,024:
// one block, four waves, per CU).
constexpr int kItemsLarge = 4;
constexpr int kItemsSmall = 1;
constexpr uint64_t kSmallBatch = 1ull << 19;
// A request's list run is written in whole units of kPadWords words (a
// multiple of 4 dividing 512, so padding never leaves the request's final
// list page): whole 64-byte segments. Words past the last entry are
// written as 0.
constexpr uint64_t kPadWords = 8;
// GPU pages of the table staged in LDS per wave and round (4 KiB).
constexpr int kTileFrames = 512;
enum : uint8_t { kOk = 0, kEinval = 1, kErange = 2, kEnospc = 3, kEbusy = 4 };

// ---- the fused batch (dmadesc_build_batch) --------------------------------
// The region lookup and the queue histogram of the split ride along the PRP
// build's request phase, so off, len and qid are read once. The region table
// stays in global memory: a bucket index over the region starts (built by
// k_batch_prep) holds, per bucket, the first two regions that can contain an
// address of the bucket, so on evenly spread tables one 48-byte record read
// answers a lookup; longer runs are searched in the table.
struct IndexHdr {
    uint64_t base;                // start of region 0: bucket 0 begins here
    uint32_t bs;                  // log2 of the bucket width in bytes
    uint32_t pad;
};
// Bucket b of the index: the regions that can hold the last start at or
// before an address in the bucket are [at, at + cnt) (at = the last region
// starting before the bucket, or 0); the first two of them are copied in, so
// a lookup whose run has one or two candidates reads one record.
struct alignas(16) BucketRec {
    uint64_t s0, e0;              // region at: start, end
    uint64_t s1, e1;              // region at + 1 (cnt >= 2)
    uint32_t k0, k1;              // their keys
    uint32_t at, cnt;
};
static_assert(sizeof(BucketRec) == 48, "three 16-byte loads");
struct Fuse {
    const uint64_t *rs, *re;      // region table (nregions entries)
    const uint32_t *rk;
    uint32_t nregions, nbuckets;
    const IndexHdr *ihdr;
    const BucketRec *idx;
    uint64_t in_page, va_base;
    int32_t *handle;              // lookup columns; handle == nullptr: no lookup
    uint32_t *lkey;
    uint8_t *kind;
    uint64_t *rbase, *rend;
    const uint32_t *qid;          // queue id of each request
    uint32_t nq;                  // queues; bucket nq takes ids >= nq
    uint32_t tile_shift;          // log2 of the split's requests per tile
    uint64_t ntiles;              // split tiles: the row length of counts
    uint32_t *counts;             // bucket-major per-tile counts, zeroed; nullptr: the
                                  // split counts its single tile itself
};
constexpr int kHistCopies = 4;                    // lane l counts into copy l % 4
constexpr int kHistStride = DMADESC_MAX_QUEUES + 1;

// Looks up kN requests of this thread (items k0 .. k0 + kN - 1, item k being
// request base + k * (threads per block) + t) and writes the five lookup columns. Every
// load of one stage is issued for all kN items before any is used.
// Looks one request up (item k of this thread: request i) and writes the
// five lookup columns. Only a range at or past the first region's start can
// have a containing region, and only such a range reads the index, whose
// records exist only when the table has regions.
__device__ __forceinline__ void fused_lookup(const Fuse &F, const IndexHdr &H, uint64_t o,
                                             uint64_t l, uint64_t i, uint64_t n)
{
    typedef uint64_t u64x2v __attribute__((ext_vector_type(2)));
    uint64_t lo, hi;
    const bool valid = page_round(F.va_base, o, l, F.in_page, lo, hi);
    const bool cand = valid && F.nregions > 0 && lo >= H.base;
    u64x2v a = u64x2v{0, 0}, c = u64x2v{0, 0};
    uint4 m = make_uint4(0, 0, 0, 0);
    if (cand) {
        uint64_t bkt = (lo - H.base) >> H.bs;
        bkt = bkt < F.nbuckets ? bkt : F.nbuckets - 1;
        const u64x2v *rec = reinterpret_cast<const u64x2v *>(F.idx + bkt);
        a = rec[0];
        c = rec[1];
        m = reinterpret_cast<const uint4 *>(rec)[2];
    }
    // One or two candidates: the record decides. More: search the table's
    // starts over [at, at + cnt), then read the region (rare on spread
    // tables; at + cnt <= nregions).
    uint32_t r = 0, key = 0;
    uint64_t s0 = 0, e0 = 0;
    if (cand && m.w <= 2) {
        const bool second = m.w == 2 && c.x <= lo;
        r = m.z + (second ? 1u : 0u);
        s0 = second ? c.x : a.x;
        e0 = second ? c.y : a.y;
        key = second ? m.y : m.x;
    } else if (cand) {
        uint32_t at = m.z, cnt = m.w;
        while (cnt > 1) {
            const uint32_t half = cnt >> 1;
            at = (F.rs[at + half] <= lo) ? at + half : at;
            cnt -= half;
        }
        r = at;
        s0 = F.rs[r];
        e0 = F.re[r];
        key = F.rk[r];
    }
    const bool hit = cand && hi <= e0;
    const uint8_t kd = !valid ? 3 : !hit ? 0 : (lo == s0 && hi == e0) ? 1 : 2;
    if (i < n) {
        // Streamed: nothing reads the lookup columns again here.
        __builtin_nontemporal_store(hit ? (int32_t)r : -1, F.handle + i);
        __builtin_nontemporal_store(hit ? key : 0u, F.lkey + i);
        __builtin_nontemporal_store(kd, F.kind + i);
        __builtin_nontemporal_store(lo, F.rbase + i);
        __builtin_nontemporal_store(hi, F.rend + i);
    }
}

// The lookups of this thread's kItems requests, one after another (one
// record and its answer live at a time).
template <int kItems, int kT>
__device__ __forceinline__ void fused_lookups(const Fuse &F, const uint64_t (&o)[kItems],
                                              const uint64_t (&l)[kItems], uint64_t base, int t,
                                              uint64_t n)
{
    const IndexHdr H = *F.ihdr;
#pragma unroll
    for (int k = 0; k < kItems; ++k)
        fused_lookup(F, H, o[k], l[k], base + (uint64_t)k * kT + t, n);
}

// First region whose start is at or past bucket b (b may be nbuckets).
__device__ __forceinline__ uint32_t first_at_or_past(const uint64_t *__restrict__ rs,
                                                     uint32_t nregions, uint64_t base,
                                                     uint32_t bs, uint64_t b)
{
    const bool over = bs && (b >> (64 - bs)) != 0;
    const uint64_t width = over ? ~0ull : b << bs;
    const uint64_t x = width > ~base ? ~0ull : base + width;   // saturating
    uint32_t lo = 0, cnt = nregions;
    while (cnt > 0) {
        const uint32_t half = cnt >> 1;
        if (rs[lo + half] < x) {
            lo += half + 1;
            cnt -= half + 1;
        } else {
            cnt = half;
        }
    }
    return lo;
}

// Before the fused kernel: clears the slot scan's header and status words
// and the split's per-tile counts, and builds the bucket index over the
// region starts (span from region 0's start to the last start, nbuckets
// buckets of 2^bs bytes; the last bucket also takes everything past it).
__global__ __launch_bounds__(256) void k_batch_prep(
    uint64_t *__restrict__ scan_words, uint64_t nscan, uint32_t *__restrict__ counts,
    uint64_t ncounts, const uint64_t *__restrict__ rs, uint32_t nregions, uint32_t nbuckets,
    const uint64_t *__restrict__ re, const uint32_t *__restrict__ rk,
    IndexHdr *__restrict__ ihdr, BucketRec *__restrict__ idx)
{
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t k = g; k < nscan; k += stride) scan_words[k] = 0;
    for (uint64_t k = g; k < ncounts; k += stride) counts[k] = 0;
    if (nregions == 0) return;
    const uint64_t base = rs[0], span = rs[nregions - 1] - base;
    uint32_t bs = 0;
    while (bs < 63 && (span >> bs) >= nbuckets) ++bs;
    if (g == 0) *ihdr = IndexHdr{base, bs, 0};
    for (uint64_t b = g; b < nbuckets; b += stride) {
        const uint32_t x = first_at_or_past(rs, nregions, base, bs, b);
        const uint32_t y = b + 1 == nbuckets ? nregions
                                             : first_at_or_past(rs, nregions, base, bs, b + 1);
        // The last region starting at or before an address of this bucket
        // lies in [x - 1, y) (region x - 1 starts before the bucket).
        const uint32_t at = x ? x - 1 : 0;
        const uint32_t nx = at + 1 < nregions ? at + 1 : at;
        BucketRec R;
        R.s0 = rs[at];
        R.e0 = re[at];
        R.k0 = rk[at];
        R.s1 = rs[nx];
        R.e1 = re[nx];
        R.k1 = rk[nx];
        R.at = at;
        R.cnt = y - at;
        idx[b] = R;
    }
}

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

// Per-wave table of one round of 64 requests, in LDS.
struct RoundTable {
    uint64_t goff[kWave + 1];   // exclusive prefix of 4-word groups
    uint64_t foff[kWave + 1];   // exclusive prefix of staged GPU pages
    uint64_t xb[kWave];         // heap offset of data entry 0 (4 KiB page 1)
    uint64_t word[kWave];       // first pool word (512 * slot)
    uint64_t ent[kWave];        // words holding entries or pointers (m + L - 1)
    uint64_t plim[kWave];       // 512 * (L - 1): chain pointers lie below this
    uint64_t lut[kTileFrames];  // staged table entries of the round's requests
};

// Compact round table for rounds whose lists are all shorter than 2^24
// words: every offset inside a list then fits 32-bit arithmetic.
constexpr uint64_t kFastWords = 1ull << 24;
struct ReqRec {                 // 32 bytes, read with two 16-byte LDS loads
    uint64_t word;              // first pool word (512 * slot)
    uint64_t f0;                // GPU page holding data entry 0
    uint32_t ent;               // words holding entries or pointers
    uint32_t plim;              // 512 * (L - 1): chain pointers lie below this
    uint32_t fbase;             // staged-tile index of GPU page f0
    uint32_t ph;                // 4 KiB page of data entry 0 within GPU page f0
};
struct FastTable {
    uint32_t goff[kWave + 1];   // exclusive prefix of 2-word pairs
    uint32_t foff[kWave + 1];   // exclusive prefix of staged GPU pages
    ReqRec rec[kWave];
    uint64_t lut[kTileFrames];
};
union RoundLds {
    RoundTable wide;
    FastTable fast;
};

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reads through explicitly typed pointers. Where a branch chooses between a
// staged (LDS) copy of the table and the table itself, plain reads let the
// compiler merge both into one generic-pointer (flat) load, which also counts
// against the LDS counter; loads of different address spaces cannot merge.
__device__ __forceinline__ uint64_t lds_read(const uint64_t *p)
{
    return *(const __attribute__((address_space(3))) uint64_t *)p;
}
__device__ __forceinline__ uint64_t global_read(const uint64_t *p)
{
    return *(const __attribute__((address_space(1))) uint64_t *)p;
}

// Writes the list runs of the wave's 64 requests of one round. Lane k's
// request is described by (xb, word, ent, lp); ent == 0 for no list.
__device__ __forceinline__ void emit_round_wide(RoundTable &T, uint64_t xb, uint64_t word, uint64_t ent,
                                           uint64_t lp, uint64_t last_frame, uint64_t o,
                                           uint64_t &p1, const uint64_t *__restrict__ lut,
                                           uint64_t *__restrict__ pool, uint64_t bus)
{
    const int ln = lane();
    if (ent) p1 = global_read(&lut[o >> 16]) + (o & 0xFFFFu);
    const uint64_t groups = ((ent + kPadWords - 1) / kPadWords) * (kPadWords / 4);
    const uint64_t ginc = wave_incl_scan(groups);
    const uint64_t gtot = __shfl(ginc, kWave - 1, kWave);
    if (gtot == 0) {                                         // uniform per wave
        return;
    }
    const uint64_t frames = ent ? last_frame - (xb >> 16) + 1 : 0;
    const uint64_t finc = wave_incl_scan(frames);
    const uint64_t ftot = __shfl(finc, kWave - 1, kWave);
    const bool staged = ftot <= (uint64_t)kTileFrames;      // uniform per wave
    T.goff[ln] = ginc - groups;
    T.foff[ln] = finc - frames;
    if (ln == kWave - 1) {
        T.goff[kWave] = ginc;
        T.foff[kWave] = finc;
    }
    T.xb[ln] = xb;
    T.word[ln] = word;
    T.ent[ln] = ent;
    T.plim[ln] = lp ? (lp - 1) << 9 : 0;
    wave_sync_lds();
    if (staged) {
        // Each request's data entries read one contiguous run of the table.
        for (uint64_t j = ln; j < ftot; j += kWave) {
            const int r = owner_of<kWave>(T.foff, j);
            T.lut[j] = lut[(T.xb[r] >> 16) + (j - T.foff[r])];
        }
        wave_sync_lds();
    }
    for (uint64_t g = ln; g < gtot; g += kWave) {
        const int r = owner_of<kWave>(T.goff, g);
        const uint64_t q = (g - T.goff[r]) << 2;             // first word of the group
        const uint64_t e = T.ent[r];
        const uint64_t page = q >> 9;
        const uint64_t w0 = T.word[r];
        const uint64_t xr = T.xb[r];
        const uint64_t x0 = xr + ((q - page) << 12);         // data entry q - page
        const bool has_ptr = ((q & 511u) == 508u) && (q < T.plim[r]);
        const uint64_t left = e > q ? e - q : 0;             // 0 for a padding-only group
        const uint32_t nd = has_ptr ? 3u : (uint32_t)(left < 4 ? left : 4);
        const uint64_t f = x0 >> 16;
        const bool two = nd && (((x0 + ((uint64_t)(nd - 1) << 12)) >> 16) != f);
        uint64_t l0 = 0, l1 = 0;
        if (nd) {
            if (staged) {
                const uint64_t fs = T.foff[r] + f - (xr >> 16);
                l0 = lds_read(&T.lut[fs]);
                l1 = two ? lds_read(&T.lut[fs + 1]) : l0;
            } else {
                l0 = global_read(&lut[f]);
                l1 = two ? global_read(&lut[f + 1]) : l0;
            }
        }
        uint64_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t x = x0 + ((uint64_t)k << 12);
            const uint64_t d = (((x >> 16) != f) ? l1 : l0) + (x & 0xFFFFu);
            v[k] = (uint32_t)k < nd ? d : 0;                 // padding words are 0
        }
        if (has_ptr) v[3] = bus + (((w0 >> 9) + page + 1) << 12);
        uint64_t *dst = pool + w0 + q;
        *reinterpret_cast<u64x2 *>(dst) = u64x2{v[0], v[1]};
        *reinterpret_cast<u64x2 *>(dst + 2) = u64x2{v[2], v[3]};
    }
    wave_sync_lds();                                         // the next round rewrites T
}

// Writes one 2-word pair of a fast round (one 16-byte store: the lanes of a
// wave write consecutive pairs, so each store instruction fills whole lines).
// Data entry j of a request lies in GPU page f0 + ((ph + j) >> 4) at in-page
// offset ((ph + j) & 15) * 4 KiB.
template <bool kStaged>
__device__ __forceinline__ void fast_group(const FastTable &T, uint32_t g, int r,
                                           const uint64_t *__restrict__ lut,
                                           uint64_t *__restrict__ pool, uint64_t bus)
{
    const ReqRec R = T.rec[r];
    const uint32_t q = (g - T.goff[r]) << 1;                 // first word of the pair
    const uint32_t page = q >> 9;
    const uint32_t j0 = q - page;                            // its data entry
    const bool has_ptr = ((q & 511u) == 510u) && (q < R.plim);
    const uint32_t left = R.ent > q ? R.ent - q : 0;         // 0 for a padding-only pair
    const uint32_t nd = has_ptr ? 1u : (left < 2u ? left : 2u);
    const uint32_t t0 = R.ph + j0;
    const uint32_t fi = t0 >> 4, u = t0 & 15u;
    uint64_t l0 = 0, l1 = 0;
    if (nd) {
        const bool two = (u + nd - 1u) >= 16u;
        if (kStaged) {
            l0 = lds_read(&T.lut[R.fbase + fi]);
            l1 = two ? lds_read(&T.lut[R.fbase + fi + 1]) : l0;
        } else {
            l0 = global_read(&lut[R.f0 + fi]);
            l1 = two ? global_read(&lut[R.f0 + fi + 1]) : l0;
        }
    }
    uint64_t v[2];
#pragma unroll
    for (uint32_t k = 0; k < 2; ++k) {
        const uint32_t wk = u + k;
        const uint64_t d = (wk >= 16u ? l1 : l0) + (uint64_t)((wk & 15u) << 12);
        v[k] = k < nd ? d : 0;                               // padding words are 0
    }
    if (has_ptr) v[1] = bus + (((R.word >> 9) + page + 1) << 12);
    // Non-temporal: the list words are not read again by this kernel.
    __builtin_nontemporal_store(u64x2{v[0], v[1]},
                                reinterpret_cast<u64x2 *>(pool + R.word + q));
}

// Writes the pairs of a fast round, two per lane per step: pairs g and
// g + 64 are searched in lockstep so that their LDS reads overlap.
template <bool kStaged>
__device__ __forceinline__ void fast_groups(const FastTable &T, uint32_t gtot,
                                            const uint64_t *__restrict__ lut,
                                            uint64_t *__restrict__ pool, uint64_t bus)
{
    const uint32_t ln = lane();
    for (uint32_t c = 0; c < gtot; c += 2 * kWave) {
        const uint32_t ga = c + ln, gb = c + kWave + ln;
        const uint32_t ka = ga < gtot ? ga : gtot - 1;       // clamped search keys
        const uint32_t kb = gb < gtot ? gb : gtot - 1;
        int ra = 0, rb = 0;
#pragma unroll
        for (int step = kWave / 2; step > 0; step >>= 1) {
            const uint32_t pa = T.goff[ra + step], pbv = T.goff[rb + step];
            ra = (pa <= ka) ? ra + step : ra;
            rb = (pbv <= kb) ? rb + step : rb;
        }
        if (ga < gtot) fast_group<kStaged>(T, ga, ra, lut, pool, bus);
        if (gb < gtot) fast_group<kStaged>(T, gb, rb, lut, pool, bus);
    }
}

__device__ __forceinline__ void emit_round_fast(FastTable &T, uint64_t xb, uint64_t word,
                                                uint32_t ent, uint64_t lp, uint64_t last_frame,
                                                uint64_t o, uint64_t &p1,
                                                const uint64_t *__restrict__ lut,
                                                uint64_t *__restrict__ pool, uint64_t bus)
{
    const int ln = lane();
    const uint32_t groups = ((ent + (uint32_t)kPadWords - 1) / (uint32_t)kPadWords) *
                            (uint32_t)(kPadWords / 2);
    const uint32_t ginc = wave_incl_scan(groups);
    const uint32_t gtot = __shfl(ginc, kWave - 1, kWave);
    if (gtot == 0) {                                         // uniform per wave
        return;
    }
    // Staged from PRP1's GPU page, so that PRP1 comes from the tile too; data
    // entry 0 then lies in 4 KiB page ph (< 32) counted from that GPU page.
    const uint64_t f0 = o >> 16;
    const uint32_t frames = ent ? (uint32_t)(last_frame - f0 + 1) : 0;
    const uint32_t finc = wave_incl_scan(frames);
    const uint32_t ftot = __shfl(finc, kWave - 1, kWave);
    T.goff[ln] = ginc - groups;
    T.foff[ln] = finc - frames;
    if (ln == kWave - 1) {
        T.goff[kWave] = ginc;
        T.foff[kWave] = finc;
    }
    T.rec[ln] = ReqRec{word, f0, ent, lp ? (uint32_t)((lp - 1) << 9) : 0u, finc - frames,
                       (uint32_t)((xb >> 12) & 15u) + (uint32_t)(((xb >> 16) - f0) << 4)};
    wave_sync_lds();
    if (ftot <= (uint32_t)kTileFrames) {
        // Four reads in flight per lane before any lands in LDS.
        for (uint32_t j0 = 0; j0 < ftot; j0 += 4 * kWave) {
            uint64_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t j = j0 + u * kWave + ln;
                const uint32_t jj = j < ftot ? j : 0;
                const int r = owner_of<kWave>(T.foff, jj);
                v[u] = lut[T.rec[r].f0 + (jj - T.foff[r])];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t j = j0 + u * kWave + ln;
                if (j < ftot) T.lut[j] = v[u];
            }
        }
        wave_sync_lds();
        if (ent) p1 = lds_read(&T.lut[finc - frames]) + (o & 0xFFFFu);
        fast_groups<true>(T, gtot, lut, pool, bus);
    } else {
        if (ent) p1 = global_read(&lut[f0]) + (o & 0xFFFFu);
        fast_groups<false>(T, gtot, lut, pool, bus);
    }
    wave_sync_lds();                                         // the next round rewrites T
}

// Writes the list runs of the wave's 64 requests of one round (lane k: one
// request; ent == 0 for no list).
// Sets p1 to PRP1 of each request with a list.
__device__ __forceinline__ void emit_round(RoundLds &T, uint64_t xb, uint64_t word, uint64_t ent,
                                           uint64_t lp, uint64_t last_frame, uint64_t o,
                                           uint64_t &p1, const uint64_t *__restrict__ lut,
                                           uint64_t *__restrict__ pool, uint64_t bus)
{
    if (__ballot(ent >= kFastWords) == 0)
        emit_round_fast(T.fast, xb, word, (uint32_t)ent, lp, last_frame, o, p1, lut, pool, bus);
    else
        emit_round_wide(T.wide, xb, word, ent, lp, last_frame, o, p1, lut, pool, bus);
}

// Per-wave table of one round of 64 requests for the packed layout. T holds
// slot offsets relative to the round's first slot S: 32-bit when the round
// spans fewer than 2^31 slots, else 64-bit.
template <typename T>
struct PackTab {
    T start[kWave + 1];         // first data slot of each request, - S (clamped to E - S)
    T foff[kWave + 1];          // exclusive prefix of staged GPU pages
    T m[kWave];                 // list entries (0: none)
    uint64_t f0[kWave];         // GPU page of PRP1, the first staged page
    uint32_t ph[kWave];         // 4 KiB page of data entry 0 counted from f0 (< 32)
    uint4 rec[kWave];           // 32-bit rounds: {start, m, foff, ph} of each request
    uint2 rec2[kWave];          // 32-bit rounds: {ph - start, foff} of each request
    // 32-bit rounds: 1 + request whose list starts at a word of a 256-word
    // window (the 64-bit rounds do not use it; their table is the larger).
    uint8_t mark[sizeof(T) == 4 ? 4 * kWave : 2 * kWave];
    uint64_t lut[kTileFrames];
};
union PackLds {
    PackTab<uint32_t> fast;
    PackTab<uint64_t> wide;
};

// Value of pool word w of a packed round whose owner is request r (record
// st, mm, f0, ph, fb; rel = the slot the word stands for, relative to S).
template <typename T, bool kStaged>
__device__ __forceinline__ uint64_t pack_word(const PackTab<T> &P, uint64_t w, T rel, T st,
                                              T mm, uint64_t f0, uint32_t ph, T fb,
                                              const uint64_t *__restrict__ lut, uint64_t bus)
{
    const uint32_t o = (uint32_t)(w & 511u);
    const T j = rel - st;                                    // entry at this slot
    T e = j;                                                 // entry to write, if any
    if (o == 511u) {
        const T rem = mm - j - 1;                            // entries after the slot
        if (rem >= 2) return bus + (((w >> 9) + 1) << 12);   // chain pointer
        if (rem == 0) return 0;                              // list ended in word 510
        e = mm - 1;                                          // the final entry moves up
    } else if (o == 0u && j > 0 && j == mm - 1) {
        return 0;                                            // vacated by the final entry
    }
    const T t0 = (T)ph + e;
    const T fi = t0 >> 4;
    const uint64_t l = kStaged ? P.lut[fb + fi] : lut[f0 + fi];
    return l + ((uint64_t)(t0 & 15u) << 12);
}

// Writes the aligned 2-word pairs covering pool words [wlo, whi) of one
// packed round; words outside the range belong to other rounds. Each lane
// takes kPairs pairs per step, pair c + 64 k + lane, so each of the wave's
// 16-byte stores covers 1 KiB of the pool contiguously, and the pairs' owner
// searches run in lockstep, so their LDS latencies overlap.
template <typename T, bool kStaged>
__device__ __forceinline__ void pack_groups(const PackTab<T> &P, uint64_t S, uint64_t wlo,
                                            uint64_t whi, const uint64_t *__restrict__ lut,
                                            uint64_t *__restrict__ pool, uint64_t bus)
{
    constexpr int kPairs = 4;
    const uint64_t c0 = wlo >> 1, chi = (whi + 1) >> 1;
    const T last = (T)(P.start[kWave] - 1);                  // last slot of the round
    for (uint64_t c = c0; c < chi; c += kPairs * kWave) {
        T key[kPairs];
        int r[kPairs];
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            // The slot of the pair's first word inside the range (clamped).
            uint64_t w = (c + (uint64_t)k * kWave + lane()) << 1;
            w = w < wlo ? wlo : w;
            const uint32_t o = (uint32_t)(w & 511u);
            const uint64_t d = (w >> 9) * 511 + (o == 511u ? 510u : o) - S;
            key[k] = d < (uint64_t)last ? (T)d : last;
            r[k] = 0;
        }
#pragma unroll
        for (int step = kWave / 2; step > 0; step >>= 1) {
#pragma unroll
            for (int k = 0; k < kPairs; ++k)
                r[k] = (P.start[r[k] + step] <= key[k]) ? r[k] + step : r[k];
        }
#pragma unroll
        for (int k = 0; k < kPairs; ++k) {
            const uint64_t C = c + (uint64_t)k * kWave + lane();
            if (C >= chi) continue;
            const uint64_t w0 = C << 1;
            int rr = r[k];
            T st = P.start[rr], nx = P.start[rr + 1], mm = P.m[rr], fb = P.foff[rr];
            uint64_t f0 = P.f0[rr];
            uint32_t ph = P.ph[rr];
            uint64_t v[2];
            bool all = true;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint64_t w = w0 + q;
                v[q] = 0;
                if (w < wlo || w >= whi) {
                    all = false;
                    continue;
                }
                const uint32_t o = (uint32_t)(w & 511u);
                const T rel = (T)((w >> 9) * 511 + (o == 511u ? 510u : o) - S);
                if (nx <= rel) {                             // the pair's second word
                    do {                                     // begins a later list
                        ++rr;                                // (requests with no list
                        st = nx;                             // own no slot: skip them)
                        nx = P.start[rr + 1];
                    } while (nx <= rel);
                    mm = P.m[rr];
                    fb = P.foff[rr];
                    f0 = P.f0[rr];
                    ph = P.ph[rr];
                }
                v[q] = pack_word<T, kStaged>(P, w, rel, st, mm, f0, ph, fb, lut, bus);
            }
            // Non-temporal: the list words are not read again by this kernel,
            // and streaming them frees L2 for the table and the columns.
            uint64_t *dst = pool + w0;
            if (all) {
                __builtin_nontemporal_store(u64x2{v[0], v[1]}, reinterpret_cast<u64x2 *>(dst));
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    if (w0 + q >= wlo && w0 + q < whi) __builtin_nontemporal_store(v[q], dst + q);
            }
        }
    }
}

// Inclusive maximum over lanes 0..l of the wave (row shifts within rows of 16
// lanes, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
    return x;
}

// The value of lane l - 1 (0 in lane 0).
__device__ __forceinline__ uint32_t wave_shr1(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x138, 0xF, 0xF, false);
}

// Writes pool words [wlo, whi) of a packed round whose slots, relative to S,
// fit 32 bits, in windows of 256 words, each two halves of 128: lane l writes
// words 2l, 2l + 1 of each half, so each 16-byte store of the wave covers
// 1 KiB contiguously, and the window's fixed work (the owner map below) is
// shared by four words per lane. A word's owner is the last list that starts
// at or before it: every list marks its first word in an LDS map of the
// window, and a prefix maximum across the wave (plus the owner carried from
// before) hands each word its owner, with no search. Every word of a window
// lies in one pool page, so a non-511 word W holds slot W - W / 512, and its
// entry is (slot - S) + (ph - start) of its owner's staged GPU pages. Word 511
// (lane 63) and word 0 (lane 0) of a page get their special values in a
// branch taken only in the windows that hold them. `wst` is the first word of
// this lane's list (a value no window reaches when it has none); `first` is
// the first list lane.
template <bool kStaged>
__device__ __forceinline__ void pack_marks(PackTab<uint32_t> &P, uint64_t S, uint64_t wlo,
                                           uint64_t whi, uint64_t wst, int first,
                                           uint64_t lut_entries,
                                           const uint64_t *__restrict__ lut,
                                           uint64_t *__restrict__ pool, uint64_t bus)
{
    constexpr uint64_t kWin = 4 * kWave;
    const uint32_t ln = (uint32_t)lane();
    uint32_t carry = (uint32_t)first + 1;                    // owner mark before the window
    uint32_t *mark32 = reinterpret_cast<uint32_t *>(P.mark);
    const uint16_t *mark16 = reinterpret_cast<const uint16_t *>(P.mark);
    for (uint64_t Wb = wlo & ~(kWin - 1); Wb < whi; Wb += kWin) {
        mark32[ln] = 0;
        if (wst - Wb < kWin) P.mark[wst - Wb] = (uint8_t)(ln + 1);
        wave_sync_lds();
        const uint32_t ma = mark16[ln], mb = mark16[kWave + ln];
        const uint32_t a0 = ma & 0xFFu, a1 = ma >> 8, b0 = mb & 0xFFu, b1 = mb >> 8;
        // Prefix maxima of both halves side by side; the second half carries
        // the first half's last owner.
        const uint32_t pa = max(wave_incl_max(max(a0, a1)), carry);
        const uint32_t pb0 = wave_incl_max(max(b0, b1));
        const uint32_t ca = (uint32_t)__builtin_amdgcn_readlane((int)pa, kWave - 1);
        const uint32_t pb = max(pb0, ca);
        int r[4];
        r[0] = (int)max(max(wave_shr1(pa), carry), a0) - 1;
        r[1] = max(r[0], (int)a1 - 1);
        r[2] = (int)max(max(wave_shr1(pb), ca), b0) - 1;
        r[3] = max(r[2], (int)b1 - 1);
        carry = (uint32_t)__builtin_amdgcn_readlane((int)pb, kWave - 1);
        // Slot of this lane's first word, relative to S (mod 2^32; words
        // outside the range compute anything and are not stored).
        const uint32_t sb = (uint32_t)(Wb - (Wb >> 9) - S) + 2 * ln;
        uint64_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint2 a = P.rec2[r[k]];
            const uint32_t t = sb + (uint32_t)((k >> 1) * 128 + (k & 1)) + a.x;
            uint64_t l;
            if (kStaged) {
                l = P.lut[(a.y + (t >> 4)) & (kTileFrames - 1)];
            } else {
                const uint64_t i = P.f0[r[k]] + (t >> 4);
                l = lut[i < lut_entries ? i : 0];
            }
            v[k] = l + ((uint64_t)(t & 15u) << 12);
        }
        if ((Wb & 511u) == 256u && ln == kWave - 1) {
            // Word 511 (second half, second word of lane 63): the owner of
            // slot 510 writes a chain pointer if two or more of its entries
            // remain, its final entry if exactly one does (v[3] is then that
            // entry), else 0.
            const uint4 R = P.rec[r[3]];
            const uint32_t rem = R.y - ((sb + 128u) - R.x) - 1u;
            if (rem >= 2) v[3] = bus + ((((Wb + 255) >> 9) + 1) << 12);
            else if (rem == 0) v[3] = 0;
        }
        if ((Wb & 511u) == 0u && ln == 0) {
            // Word 0: 0 when its slot's entry is its owner's final one, which
            // then sits in word 511 of the page before.
            const uint4 R = P.rec[r[0]];
            const uint32_t j = sb - R.x;
            if (j > 0 && j == R.y - 1) v[0] = 0;
        }
        // Non-temporal: the list words are not read again by this kernel.
        if (Wb >= wlo && Wb + kWin <= whi) {
            __builtin_nontemporal_store(u64x2{v[0], v[1]},
                                        reinterpret_cast<u64x2 *>(pool + Wb + 2 * ln));
            __builtin_nontemporal_store(u64x2{v[2], v[3]},
                                        reinterpret_cast<u64x2 *>(pool + Wb + 128 + 2 * ln));
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint64_t W0 = Wb + 2 * ln + 128 * h, W1 = W0 + 1;
                const bool in0 = W0 >= wlo && W0 < whi, in1 = W1 >= wlo && W1 < whi;
                if (in0 && in1) {
                    __builtin_nontemporal_store(u64x2{v[2 * h], v[2 * h + 1]},
                                                reinterpret_cast<u64x2 *>(pool + W0));
                } else {
                    if (in0) __builtin_nontemporal_store(v[2 * h], pool + W0);
                    if (in1) __builtin_nontemporal_store(v[2 * h + 1], pool + W1);
                }
            }
        }
        wave_sync_lds();                                     // the map is rewritten next
    }
}

template <typename T>
__device__ __forceinline__ void emit_packed_t(PackTab<T> &P, uint64_t d, uint64_t m,
                                              uint64_t S, uint64_t E, int first, uint64_t o,
                                              uint64_t xb, uint64_t last_frame, uint64_t &p1,
                                              uint64_t lut_entries,
                                              const uint64_t *__restrict__ lut,
                                              uint64_t *__restrict__ pool, uint64_t bus)
{
    // A request's staged GPU pages run from PRP1's (o >> 16) to its last one;
    // data entry e then lies in staged page (ph + e) >> 4, with ph < 32 the
    // 4 KiB page of entry 0 counted from the start of PRP1's GPU page.
    const int ln = lane();
    const uint64_t f0 = o >> 16;
    const uint64_t frames = m ? last_frame - f0 + 1 : 0;
    const uint64_t finc = wave_incl_scan(frames);
    const uint64_t ftot = __shfl(finc, kWave - 1, kWave);
    const uint64_t rs = d - S < E - S ? d - S : E - S;       // d >= S for every lane
    P.start[ln] = (T)rs;
    P.foff[ln] = (T)(finc - frames);
    P.m[ln] = (T)m;
    P.f0[ln] = f0;
    P.ph[ln] = (uint32_t)((xb >> 12) & 15u) + (uint32_t)(((xb >> 16) - f0) << 4);
    if constexpr (std::is_same<T, uint32_t>::value) {
        const uint32_t ph = (uint32_t)((xb >> 12) & 15u) + (uint32_t)(((xb >> 16) - f0) << 4);
        P.rec[ln] = make_uint4((uint32_t)rs, (uint32_t)m, (uint32_t)(finc - frames), ph);
        P.rec2[ln] = make_uint2(ph - (uint32_t)rs, (uint32_t)(finc - frames));
    }
    if (ln == kWave - 1) {
        P.start[kWave] = (T)(E - S);
        P.foff[kWave] = (T)finc;
    }
    wave_sync_lds();
    const uint64_t wlo = S + S / 511, whi = E + E / 511;
    const uint64_t wst = m ? d + d / 511 : ~0ull;            // first word of this lane's list
    if (ftot <= (uint64_t)kTileFrames) {
        for (uint32_t j0 = 0; j0 < (uint32_t)ftot; j0 += 4 * kWave) {
            uint64_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t j = j0 + u * kWave + ln;
                const T jj = j < ftot ? (T)j : (T)0;
                const int r = owner_of<kWave>(P.foff, jj);
                v[u] = lut[P.f0[r] + (jj - P.foff[r])];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t j = j0 + u * kWave + ln;
                if (j < ftot) P.lut[j] = v[u];
            }
        }
        wave_sync_lds();
        if (m) p1 = P.lut[P.foff[ln]] + (o & 0xFFFFu);
        if constexpr (std::is_same<T, uint32_t>::value)
            pack_marks<true>(P, S, wlo, whi, wst, first, lut_entries, lut, pool, bus);
        else
            pack_groups<T, true>(P, S, wlo, whi, lut, pool, bus);
    } else {
        if (m) p1 = lut[f0] + (o & 0xFFFFu);
        if constexpr (std::is_same<T, uint32_t>::value)
            pack_marks<false>(P, S, wlo, whi, wst, first, lut_entries, lut, pool, bus);
        else
            pack_groups<T, false>(P, S, wlo, whi, lut, pool, bus);
    }
    wave_sync_lds();                                         // the next round rewrites P
}

// Writes the packed words of the wave's 64 requests of one round (lane k: one
// request at heap offset o with list entries m from data slot d; m == 0 for
// no list); sets p1 to PRP1 of each request with a list.
__device__ __forceinline__ void emit_round_packed(PackLds &L, uint64_t d, uint64_t m,
                                                  uint64_t o, uint64_t xb, uint64_t last_frame,
                                                  uint64_t &p1, uint64_t lut_entries,
                                                  const uint64_t *__restrict__ lut,
                                                  uint64_t *__restrict__ pool, uint64_t bus)
{
    const uint64_t has = __ballot(m != 0);
    if (has == 0) {                                          // uniform per wave
        return;
    }
    const int first = __ffsll((unsigned long long)has) - 1;
    const int last = 63 - __clzll((unsigned long long)has);
    const uint64_t S = __shfl(d, first, kWave);
    const uint64_t E = __shfl(d + m, last, kWave);
    if (E - S < (1ull << 31))
        emit_packed_t<uint32_t>(L.fast, d, m, S, E, first, o, xb, last_frame, p1, lut_entries,
                                lut, pool, bus);
    else
        emit_packed_t<uint64_t>(L.wide, d, m, S, E, first, o, xb, last_frame, p1, lut_entries,
                                lut, pool, bus);
}

template <bool kPacked, bool kFused, int kItems, int kT>
__global__ __launch_bounds__(kT, 4) void k_prp_build(
    const uint64_t *__restrict__ lut, uint64_t heap,
    const uint64_t *__restrict__ off, const uint64_t *__restrict__ len, uint64_t n,
    uint64_t nblocks, uint64_t bus, uint64_t *__restrict__ pool, uint64_t pool_pages,
    uint64_t *__restrict__ prp1, uint64_t *__restrict__ prp2,
    uint8_t *__restrict__ status, uint64_t *__restrict__ total,
    Header *__restrict__ hdr, uint64_t *__restrict__ bstat, uint32_t max_polls, Fuse F)
{
    constexpr int kWv = kT / kWave;                  // waves per block
    using RoundT = typename std::conditional<kPacked, PackLds, RoundLds>::type;
    __shared__ uint64_t s_red[kItems * kWv];
    __shared__ uint64_t s_bid, s_excl;
    __shared__ uint32_t s_dead;
    __shared__ uint64_t s_v2[kItems * kT];   // table entry of PRP2's page (two pages)
    __shared__ RoundT s_round[kWv];
    // The fused split's block histogram lives in the round tables' memory,
    // which the list rounds only use after the request phase.
    static_assert(sizeof(RoundT) * kWv >= kHistCopies * kHistStride * sizeof(uint32_t),
                  "the histogram fits in the round tables");
    uint32_t *hist = reinterpret_cast<uint32_t *>(&s_round[0]);

    const int t = threadIdx.x, w = wave(), ln = lane();
    const bool split_hist = kFused && F.counts != nullptr;
    if (split_hist) {
        for (int k = t; k < kHistCopies * kHistStride; k += kT) hist[k] = 0;
    }
    if (t == 0) s_bid = atomicAdd(&hdr->ticket, 1u);
    __syncthreads();
    const uint64_t b = s_bid;
    constexpr int kTile = kT * kItems;       // requests per block
    const uint64_t base = b * kTile;

    // ---- request phase: item k of thread t is request base + k*256 + t ----
    // The request phase (column loads, scan, look-back, table gathers) runs
    // at a raised wave priority, so that a SIMD issues a block's loads ahead
    // of the list stores of the blocks beside it in their list rounds: the
    // look-back chain and the next list rounds wait less (Mixed build 1.096
    // -> 1.085 ms; priority 2 the same, raising it for the rounds' table
    // staging too was slower).
    __builtin_amdgcn_s_setprio(3);
    uint64_t o[kItems], l[kItems], pre[kItems];
    uint32_t q[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kT + t;
        o[k] = i < n ? __builtin_nontemporal_load(off + i) : 0;
        l[k] = i < n ? __builtin_nontemporal_load(len + i) : 0;   // len 0 decodes as invalid
        // Clamped, not guarded, and loaded even when the split counts its
        // one tile itself: a load behind a condition is a branch whose result
        // the compiler waits for before the next item's loads are issued.
        if constexpr (kFused) q[k] = __builtin_nontemporal_load(F.qid + (i < n ? i : n - 1));
    }
    if (split_hist) {
        // Queue histogram of the block (LDS atomics; counts only, so their
        // order does not matter).
        uint32_t *hc = hist + (ln % kHistCopies) * kHistStride;
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint64_t i = base + (uint64_t)k * kT + t;
            if (i < n) atomicAdd(&hc[q[k] < F.nq ? q[k] : F.nq], 1u);
        }
    }
    // Scanned per request: list pages (page layout) or list entries (packed).
    // Request order is (item, wave, lane): wave scans per item, then one
    // barrier to combine the waves' totals. The scan needs only the request
    // columns, so it comes first and the block's aggregate is published
    // before any table read: blocks looking back at this one wait less.
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        uint64_t pages;
        const uint8_t st = decode(o[k], l[k], heap, pages);
        const uint64_t cnt = (st == kOk && pages >= 3)
                                 ? (kPacked ? pages - 1 : (pages - 2 + 510) / 511) : 0;
        const uint64_t inc = wave_incl_scan(cnt);
        pre[k] = inc - cnt;
        if (ln == kWave - 1) s_red[k * kWv + w] = inc;
    }
    __syncthreads();
    uint64_t agg = 0;
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        uint64_t before = 0, all = 0;
#pragma unroll
        for (int v = 0; v < kWv; ++v) {
            const uint64_t x = s_red[k * kWv + v];
            before += v < w ? x : 0ull;
            all += x;
        }
        pre[k] += agg + before;
        agg += all;
    }
    if (w == 0 && ln == 0) store_status(bstat + b, (b == 0 ? kFlagInc : kFlagAgg) | agg);

    // PRP1, PRP2 and the status of a request are written once, in the list
    // round of its item: every 64-request segment of the three columns goes
    // out whole, in one pass, instead of in two passes with holes (a column
    // written in parts costs whole-segment writes twice). The table reads for
    // PRP1 and a two-page PRP2 are issued here, branch-free (index 0 stands
    // in for a request that needs none) so that all of them are in flight
    // together; waves 1..3 issue theirs before wave 0 looks back, wave 0
    // after (its look-back polls would otherwise wait for its table reads).
    // A list (either layout) takes PRP1 from the table entries its round
    // stages, so its table read is not repeated here. The second page's table entry of
    // a two-page request waits in LDS (8 bytes per request), which keeps the
    // packed build within 128 VGPRs, four waves per SIMD.
    uint64_t v1[kItems];
    auto gather = [&]() {
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            uint64_t pages;
            const uint8_t st = decode(o[k], l[k], heap, pages);
            const uint64_t x = (o[k] & ~4095ull) + 4096;
            const bool staged_prp1 = pages >= 3;
            const uint64_t i1 = (st == kOk && !staged_prp1) ? o[k] >> 16 : 0;
            const uint64_t i2 = (st == kOk && pages == 2) ? x >> 16 : 0;
            v1[k] = heap ? lut[i1] : 0;
            s_v2[k * kT + t] = heap ? lut[i2] : 0;
        }
    };
    if (w != 0) {
        gather();
        if constexpr (kFused) {
            // Waves 1..3 add the block histogram to its split tile's counts
            // while wave 0 looks back, then look their requests up.
            const uint64_t tile = base >> F.tile_shift;
            for (uint32_t bk = t - kWave; split_hist && bk <= F.nq; bk += kT - kWave) {
                uint32_t c = 0;
#pragma unroll
                for (int j = 0; j < kHistCopies; ++j) c += hist[j * kHistStride + bk];
                if (c) atomicAdd(F.counts + (uint64_t)bk * F.ntiles + tile, c);
            }
            if (F.handle) fused_lookups<kItems, kT>(F, o, l, base, t, n);
        }
    }
    if (w == 0) {
        uint64_t excl = 0;
        bool dead = false;
        if (b != 0) {
            excl = look_back(bstat, (int64_t)b, &hdr->timeouts, max_polls, dead);
            // An expired wait leaves the aggregate published, so later blocks
            // still find their prefixes; this block's list requests are refused.
            if (ln == 0 && !dead) store_status(bstat + b, kFlagInc | (excl + agg));
        }
        if (ln == 0) {
            s_excl = excl;
            s_dead = dead;
            if (b == nblocks - 1)
                *total = dead ? ~0ull : (kPacked ? (excl + agg + 510) / 511 : excl + agg);
        }
        gather();
        if constexpr (kFused) {
            if (F.handle) fused_lookups<kItems, kT>(F, o, l, base, t, n);
        }
    }
    __syncthreads();
    const uint64_t excl = s_excl;
    const bool dead = s_dead != 0;

    __builtin_amdgcn_s_setprio(0);
    const uint64_t cap = kPacked ? pool_pages * 511 : pool_pages;   // slots of the pool
#pragma unroll 1
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kT + t;
        uint64_t pages;
        uint8_t st = decode(o[k], l[k], heap, pages);
        const uint64_t cnt = (st == kOk && pages >= 3)
                                 ? (kPacked ? pages - 1 : (pages - 2 + 510) / 511) : 0;
        const uint64_t slot = excl + pre[k];
        if (cnt != 0 && dead) st = kEbusy;                   // its slots are unknown
        else if (cnt != 0 && slot + cnt > cap) st = kEnospc; // refused; its slots stay taken
        const bool lists = (st == kOk) && cnt != 0;
        const uint64_t xb = (o[k] & ~4095ull) + 4096;
        const uint64_t last_frame = (o[k] + l[k] - 1) >> 16;
        uint64_t p1 = v1[k] + (o[k] & 0xFFFFu);
        if constexpr (kPacked)
            emit_round_packed(s_round[w], slot, lists ? cnt : 0, o[k], xb, last_frame, p1,
                              heap >> 16, lut, pool, bus);
        else
            emit_round(s_round[w], xb, slot << 9, lists ? (pages - 1) + (cnt - 1) : 0,
                       lists ? cnt : 0, last_frame, o[k], p1, lut, pool, bus);
        if (i < n) {
            const uint64_t list = kPacked ? bus + 8 * (slot + slot / 511) : bus + (slot << 12);
            const uint64_t p2 = lists ? list : (pages == 2 ? s_v2[k * kT + t] + (xb & 0xFFFFu) : 0);
            // Output columns and input columns are streamed (non-temporal):
            // neither is read again by this kernel.
            __builtin_nontemporal_store(st == kOk ? p1 : 0, prp1 + i);
            __builtin_nontemporal_store(st == kOk ? p2 : 0, prp2 + i);
            __builtin_nontemporal_store(st, status + i);
        }
    }
}

}  // namespace

// Buckets of the fused lookup's index: two per region (rounded up to a
// power of two), at least 4,096 and at most 2^21 (96 MiB of records).
// Requests per block of the PRP build for a batch of n (the launch and the
// workspace size agree on it).
// Block shape of the build for a batch of n (threads per block, requests per
// thread): one request per thread up to 2^19 requests, four above; 512-thread
// blocks from 2^16 to 2^22 requests (half as many blocks take tickets from
// the one ticket word than with 256 threads, which the launch's first round
// of blocks otherwise takes one after another: 1,048,576 requests 36 -> 30
// us, 262,144 large ones 0.487 -> 0.482 ms), 256-thread blocks outside that
// (a 512-thread block's scan spills a few registers, which large batches pay
// in every block; tiny ones want more blocks).
constexpr uint64_t kMidBatch = 1ull << 22;
void prp_shape(uint64_t n, int &threads, int &items)
{
    threads = n > (1ull << 16) && n <= kMidBatch ? 512 : 256;
    items = n <= kSmallBatch ? kItemsSmall : kItemsLarge;
}

uint64_t prp_tile(uint64_t n)
{
    int threads = 0, items = 0;
    prp_shape(n, threads, items);
    return (uint64_t)threads * (uint64_t)items;
}

// Launches the k_prp_build instantiation for the layout and the batch size.
template <bool kFused>
void launch_prp_kernel(const PrpArgs &a, uint64_t nb, Header *hdr, uint64_t *bstat,
                       const Fuse &F, hipStream_t s)
{
    const uint64_t heap = a.lut_entries << 16;
    int threads = 0, items = 0;
    prp_shape(a.n, threads, items);
#define DD_PRP_LAUNCH(P, I, T)                                                                \
    hipLaunchKernelGGL((k_prp_build<P, kFused, I, T>), dim3((unsigned)nb), dim3(T), 0, s,      \
                       a.lut, heap, a.off, a.len, a.n, nb, a.list_bus_base, a.pool,            \
                       a.pool_pages, a.prp1, a.prp2, a.status, a.total_pages, hdr, bstat,     \
                       wait_limit(), F)
    if (a.packed) {
        if (items == kItemsSmall && threads == 512) DD_PRP_LAUNCH(true, kItemsSmall, 512);
        else if (items == kItemsSmall) DD_PRP_LAUNCH(true, kItemsSmall, 256);
        else if (threads == 512) DD_PRP_LAUNCH(true, kItemsLarge, 512);
        else DD_PRP_LAUNCH(true, kItemsLarge, 256);
    } else {
        if (items == kItemsSmall && threads == 512) DD_PRP_LAUNCH(false, kItemsSmall, 512);
        else if (items == kItemsSmall) DD_PRP_LAUNCH(false, kItemsSmall, 256);
        else if (threads == 512) DD_PRP_LAUNCH(false, kItemsLarge, 512);
        else DD_PRP_LAUNCH(false, kItemsLarge, 256);
    }
#undef DD_PRP_LAUNCH
}

uint32_t index_buckets(uint32_t nregions)
{
    uint64_t b = 4096;
    while (b < 2ull * nregions && b < (1ull << 21)) b <<= 1;
    return (uint32_t)b;
}

size_t ws_batch_index(uint32_t nregions)
{
    return align256(sizeof(IndexHdr)) +
           align256((uint64_t)index_buckets(nregions) * sizeof(BucketRec));
}

hipError_t launch_build_batch(const LookupArgs &lk, const PrpArgs &a, const SplitArgs &sp,
                              void *index_ws, hipStream_t s)
{
    const uint64_t nb = (a.n + prp_tile(a.n) - 1) / prp_tile(a.n);
    if (nb == 0) {
        hipLaunchKernelGGL(k_ws_clear, dim3(1), dim3(64), 0, s, a.total_pages, (uint64_t)1);
        return launch_partition(sp, s);                   // an empty split
    }
    Header *hdr = static_cast<Header *>(a.ws);
    uint64_t *bstat = reinterpret_cast<uint64_t *>(static_cast<char *>(a.ws) + kHeaderBytes);
    const uint64_t words = kHeaderBytes / sizeof(uint64_t) + nb;
    const uint32_t shift = split_tile_shift(sp.nqueues);
    const uint64_t ntiles = (a.n + (1ull << shift) - 1) >> shift;
    uint32_t *counts = static_cast<uint32_t *>(sp.ws);
    const uint64_t ncounts = (uint64_t)(sp.nqueues + 1) * ntiles;
    const uint32_t nbuckets = index_buckets(lk.nregions);
    IndexHdr *ihdr = static_cast<IndexHdr *>(index_ws);
    BucketRec *idx = reinterpret_cast<BucketRec *>(static_cast<char *>(index_ws) +
                                                   align256(sizeof(IndexHdr)));
    const bool lookup = lk.handle != nullptr;
    uint64_t pb = (words > ncounts ? words : ncounts);
    if (lookup && nbuckets > pb) pb = nbuckets;
    pb = (pb + 255) / 256;
    if (pb > 1024) pb = 1024;
    hipLaunchKernelGGL(k_batch_prep, dim3((unsigned)pb), dim3(256), 0, s,
                       static_cast<uint64_t *>(a.ws), words, counts, ncounts, lk.reg_start,
                       lookup ? lk.nregions : 0u, nbuckets, lk.reg_end, lk.reg_lkey, ihdr, idx);
    Fuse F{};
    F.rs = lk.reg_start;
    F.re = lk.reg_end;
    F.rk = lk.reg_lkey;
    F.nregions = lk.nregions;
    F.nbuckets = nbuckets;
    F.ihdr = ihdr;
    F.idx = idx;
    F.in_page = (1ull << lk.page_shift) - 1;
    F.va_base = lk.va_base;
    F.handle = lk.handle;
    F.lkey = lk.lkey;
    F.kind = lk.kind;
    F.rbase = lk.rbase;
    F.rend = lk.rend;
    F.qid = sp.qid;
    F.nq = sp.nqueues;
    F.tile_shift = shift;
    F.ntiles = ntiles;
    // A batch of one split tile is ranked by the split's own one-tile kernel
    // (it counts its tile itself): the build then adds no histogram.
    const bool single = split_single(sp.n, sp.nqueues);
    F.counts = single ? nullptr : counts;
    launch_prp_kernel<true>(a, nb, hdr, bstat, F, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return single ? launch_partition(sp, s) : launch_partition_counted(sp, s);
}

size_t ws_build_prp(uint64_t n)
{
    if (n == 0) return 0;
    const uint64_t nb = (n + prp_tile(n) - 1) / prp_tile(n);
    return align256(kHeaderBytes + nb * sizeof(uint64_t));
}

hipError_t launch_build_prp(const PrpArgs &a, hipStream_t s)
{
    const uint64_t nb = (a.n + prp_tile(a.n) - 1) / prp_tile(a.n);
    if (nb == 0) {
        // Nothing to build; the batch needs no list pages.
        hipLaunchKernelGGL(k_ws_clear, dim3(1), dim3(64), 0, s, a.total_pages, (uint64_t)1);
        return hipGetLastError();
    }
    Header *hdr = static_cast<Header *>(a.ws);
    uint64_t *bstat = reinterpret_cast<uint64_t *>(static_cast<char *>(a.ws) + kHeaderBytes);
    const uint64_t words = kHeaderBytes / sizeof(uint64_t) + nb;
    uint64_t cblocks = (words + 255) / 256;
    if (cblocks > 1024) cblocks = 1024;
    hipLaunchKernelGGL(k_ws_clear, dim3((unsigned)cblocks), dim3(256), 0, s,
                       static_cast<uint64_t *>(a.ws), words);
    launch_prp_kernel<false>(a, nb, hdr, bstat, Fuse{}, s);
    return hipGetLastError();
}

}  // namespace dd

// emit_sqe.hip - NVMe submission entries per queue, one window of the split
// per call, for gfx950.
//
// Method: the xNVMe "uPCIe CUDA" page ("GPU-Resident Queue API") has a kernel
// fill the submission queue itself, one 64-byte entry per command, written as
// four 16-byte stores that the L2 merges into whole sectors. The MORI page
// ("mori通信库分析(一)——对称内存RDMA数据发送过程", warp-level WQE reservation)
// reserves a run of consecutive slots from a queue's tail for the lanes bound
// to it and then moves the tail on by their number. Here the run of slots a
// queue takes in one call is its window of the split (at most its free slots),
// and each placeable request's slot is the tail plus the number of placeable
// requests before it in the window: a count per tile, a sum over the tiles
// before, and ballots inside the tile. No atomic decides a slot, so the rings
// are deterministic.
//
// Layout: tile g = 64 q + t owns positions [t * kTile, (t + 1) * kTile) of
// queue q's window. A window is shorter than the deepest ring (65536 entries),
// so kTilesPerQueue tiles cover any window. Round k of a tile covers kThreads
// consecutive positions, wave w the 64 positions [k * kThreads + 64 w, ...),
// so lanes meet positions in (round, wave, lane) order -- the window's order.
//
// Schedule: a queue's window is a sparse, increasing run of request indices,
// so the gathers of one tile touch many cache lines that tiles of other
// queues touch as well. Launched queue by queue, the resident tiles would
// span the whole batch and re-read each line from HBM once per queue; instead
// the non-empty tiles are ordered by their first request index, and block b of
// the two passes takes the b-th tile of that order, so the resident tiles
// sweep the batch together and share its lines in the caches. The order only
// affects speed: a slot depends on the per-tile counts, never on which block
// ran first.
//
// Kernels: k_sqe_order (tile order, one record per tile and per queue),
// k_sqe_count (placeable requests per tile; it gathers status and length and
// keeps, for the next pass, each round's placeable lanes and each position's
// block-count field), k_sqe_emit (slots, entries, request map; it gathers
// only PRP1, PRP2 and the starting block, since every gathered column costs
// a cache line per entry of a sparse queue), k_sqe_finish (placed counts,
// tails and cursors). The records spare the two passes the chain of
// dependent reads (tile, queue state, bucket bounds, cursor, free slots) that
// finding a tile's window takes: a block reads its record and starts its
// gathers.
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRounds = 4;
constexpr uint32_t kTile = kThreads * kRounds;                  // window positions per block
constexpr uint32_t kTilesPerQueue = DMADESC_SQ_MAX_DEPTH / kTile;
static_assert(kTilesPerQueue == 64, "tile ids are 64 q + t");
constexpr int kOrderThreads = 1024;
constexpr uint32_t kBins = 4096;                 // tile-order buckets over the batch
constexpr int kBinsPerThread = kBins / kOrderThreads;
constexpr int kMaxTiles = DMADESC_MAX_QUEUES * kTilesPerQueue;

// A non-empty tile in schedule order: where its entries start in perm, how
// many there are, and its id g = 64 q + t.
struct TileRec {
    uint64_t pos;
    uint32_t cnt, g;
};
static_assert(sizeof(TileRec) == 16, "one 16-byte load");

// A queue's ring as this call sees it.
struct QueueRec {
    uint64_t ring;
    uint32_t tail, depth;
};
static_assert(sizeof(QueueRec) == 16, "one 16-byte load");

// Workspace: per-tile counts and placeable masks, the block-count fields,
// the tile records in schedule order, the queue records, and the number of
// non-empty tiles.
struct SqeWs {
    uint32_t *counts;     // [nq * 64], by tile id
    uint64_t *mask;       // [nq * 64 * kRounds * kWaves]: placeable lanes of each
                          // (tile, round, wave), by tile id
    uint16_t *nlb;        // [schedule index * kTile + position]: blocks - 1 of each
                          // placeable position of a tile
    TileRec *tiles;       // [nq * 64], the first *ntiles in schedule order
    QueueRec *queues;     // [nq]
    uint32_t *ntiles;     // scalar
};

struct Window {
    uint64_t start;     // position in perm of the window's first entry
    uint64_t ring;      // device address of the queue's ring
    uint32_t w;         // window length; 0 for a refused queue
    uint32_t tail, depth;
};

// The window of queue q for this call (identical in every kernel: all of them
// read tail/cursor before k_sqe_finish, the last, writes them).
__device__ __forceinline__ Window window_of(const SqeArgs &a, uint32_t q)
{
    Window v{0, a.ring[q], 0, a.tail[q], a.depth[q]};
    if (v.ring == 0 || (v.ring & 63u) || v.depth < 2 || v.depth > DMADESC_SQ_MAX_DEPTH ||
        v.tail >= v.depth)
        return v;
    // Bucket bounds, clamped to the batch so that a damaged qoff stays in bounds.
    const uint64_t b1 = a.qoff[q + 1] < a.n ? a.qoff[q + 1] : a.n;
    const uint64_t b0 = a.qoff[q] < b1 ? a.qoff[q] : b1;
    const uint64_t c = a.cursor[q];
    const uint64_t left = c < b1 - b0 ? b1 - b0 - c : 0;
    const uint32_t room = a.free_slots[q] < v.depth - 1 ? a.free_slots[q] : v.depth - 1;
    v.w = left < room ? (uint32_t)left : room;
    v.start = b0 + c;
    return v;
}

// A command can carry the request: PRPs built, and a whole number of logical
// blocks, from 1 to 65536.
__device__ __forceinline__ bool placeable(uint8_t st, uint64_t len, uint32_t shift)
{
    return st == DMADESC_PRP_OK && len != 0 && (len & ((1ull << shift) - 1)) == 0 &&
           (len >> shift) <= 65536u;
}

// One block: counting sort of the non-empty tiles by the bucket of their first
// request index (bucket = index * kBins / n). Ties in a bucket take the order
// of the LDS atomics; only the schedule depends on it.
__global__ __launch_bounds__(kOrderThreads) void k_sqe_order(SqeArgs a, SqeWs ws)
{
    __shared__ uint64_t s_start[DMADESC_MAX_QUEUES];
    __shared__ uint32_t s_w[DMADESC_MAX_QUEUES];
    __shared__ uint32_t s_bin[kBins];
    __shared__ uint32_t s_scr[kOrderThreads / kWave];
    const uint32_t nq = a.nqueues, ntile = nq * kTilesPerQueue;
    for (uint32_t q = threadIdx.x; q < nq; q += kOrderThreads) {
        const Window win = window_of(a, q);
        s_start[q] = win.start;
        s_w[q] = win.w;
        ws.queues[q] = QueueRec{win.ring, win.tail, win.depth};
    }
    for (uint32_t b = threadIdx.x; b < kBins; b += kOrderThreads) s_bin[b] = 0;
    __syncthreads();
    // Each thread owns tiles threadIdx.x + k * kOrderThreads. The first
    // entries of all of them are read at once, from a clamped position (a
    // read behind a condition would wait for the one before it); with an
    // empty batch no tile is non-empty and nothing is read.
    constexpr int kPer = kMaxTiles / kOrderThreads;
    uint32_t bin[kPer];
    bool live[kPer];
    uint64_t first[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const uint32_t g = threadIdx.x + k * kOrderThreads;
        const uint32_t q = g < ntile ? g / kTilesPerQueue : 0u;
        const uint32_t lo = (g % kTilesPerQueue) * kTile;
        live[k] = g < ntile && lo < s_w[q];
        first[k] = live[k] ? s_start[q] + lo : 0;
    }
    if (a.n != 0) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) first[k] = a.perm[first[k]];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        bin[k] = UINT32_MAX;
        if (live[k]) {
            bin[k] = (uint32_t)(first[k] * kBins / a.n);     // first < n, so bin < kBins
            atomicAdd(&s_bin[bin[k]], 1u);
        }
    }
    __syncthreads();
    uint32_t v[kBinsPerThread], sum = 0;
#pragma unroll
    for (int k = 0; k < kBinsPerThread; ++k) {
        v[k] = s_bin[threadIdx.x * kBinsPerThread + k];
        sum += v[k];
    }
    uint32_t total;
    uint32_t run = block_excl_scan<kOrderThreads>(sum, s_scr, &total);
#pragma unroll
    for (int k = 0; k < kBinsPerThread; ++k) {
        s_bin[threadIdx.x * kBinsPerThread + k] = run;
        run += v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (bin[k] != UINT32_MAX) {
            const uint32_t g = threadIdx.x + k * kOrderThreads;
            const uint32_t q = g / kTilesPerQueue, lo = (g % kTilesPerQueue) * kTile;
            const uint32_t cnt = s_w[q] - lo < kTile ? s_w[q] - lo : kTile;
            ws.tiles[atomicAdd(&s_bin[bin[k]], 1u)] = TileRec{s_start[q] + lo, cnt, g};
        }
    if (threadIdx.x == 0) *ws.ntiles = total;
}

// The tile block b works on, or false when b has none. Blocks are dealt to
// the 8 XCDs in turn; XCD x takes the x-th eighth of the tile order, so the
// tiles that share an XCD's L2 cover neighbouring request ranges.
__device__ __forceinline__ bool tile_of(const SqeWs &ws, TileRec &r, uint32_t &idx)
{
    const uint32_t nt = *ws.ntiles, per = (nt + 7) / 8;
    const uint32_t x = blockIdx.x & 7, k = blockIdx.x >> 3;
    idx = x * per + k;
    if (k >= per || idx >= nt) return false;
    r = ws.tiles[idx];
    return true;
}

__global__ __launch_bounds__(kThreads) void k_sqe_count(SqeArgs a, SqeWs ws)
{
    __shared__ uint32_t s_sum[kWaves];
    TileRec r;
    uint32_t ti;
    if (!tile_of(ws, r, ti)) return;                   // uniform over the block
    const uint32_t cnt = r.cnt;
    const uint32_t *__restrict__ pos = a.perm + r.pos;

    uint32_t idx[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t j = k * kThreads + threadIdx.x;
        idx[k] = j < cnt ? pos[j] : UINT32_MAX;
    }
    // Gathers from a clamped index, all issued before any is used (a load
    // behind an i < n branch would wait for the one before it).
    uint8_t st[kRounds];
    uint64_t len[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t i = idx[k] < a.n ? idx[k] : 0u;
        st[k] = a.status[i];
        len[k] = a.len[i];
    }
    // The placeable lanes of each round, kept for the emit pass (which then
    // gathers no status) and counted.
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint64_t mk = __ballot(idx[k] < a.n && placeable(st[k], len[k], a.lba_shift));
        if (lane() == 0) ws.mask[((uint64_t)r.g * kRounds + k) * kWaves + wave()] = mk;
        c += (uint32_t)__popcll(mk);
        // The block count field of each position, stored contiguously for
        // the emit pass (which then gathers no length either).
        const uint32_t j = k * kThreads + threadIdx.x;
        if (j < cnt)
            ws.nlb[(uint64_t)ti * kTile + j] =
                (mk >> lane()) & 1u ? (uint16_t)((len[k] >> a.lba_shift) - 1u) : (uint16_t)0;
    }
    if (lane() == 0) s_sum[wave()] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += s_sum[w];
        ws.counts[r.g] = s;
    }
}

__global__ __launch_bounds__(kThreads) void k_sqe_emit(SqeArgs a, SqeWs ws)
{
    __shared__ uint32_t s_cnt[kRounds][kWaves];
    // A wave's entries of one round, by rank: 64 x 64 bytes per wave.
    __shared__ uint4 s_ent[kWaves][kWave * 4];
    TileRec r;
    uint32_t ti;
    if (!tile_of(ws, r, ti)) return;                   // uniform over the block
    const uint32_t q = r.g / kTilesPerQueue, t = r.g % kTilesPerQueue;
    const QueueRec win = ws.queues[q];
    const uint32_t cnt = r.cnt;
    const uint32_t *__restrict__ pos = a.perm + r.pos;
    const int w = wave(), ln = lane();

    // Placeable requests of the window before this tile (t < 64 tiles).
    uint32_t before = (uint32_t)ln < t ? ws.counts[(uint64_t)q * kTilesPerQueue + ln] : 0u;
    before = wave_sum(before);

    // Every gather of the tile is issued before the first ring store: the
    // compiler cannot prove that a ring aliases no input column, so a load
    // placed after a store would wait for it.
    uint32_t idx[kRounds];
    uint64_t p1[kRounds], p2[kRounds], lba[kRounds];
    uint32_t nlb[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t j = k * kThreads + threadIdx.x;
        idx[k] = j < cnt ? pos[j] : UINT32_MAX;
    }
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t i = idx[k] < a.n ? idx[k] : 0u;
        const bool in = idx[k] < a.n;
        const uint32_t j = k * kThreads + threadIdx.x;
        nlb[k] = ws.nlb[(uint64_t)ti * kTile + (j < cnt ? j : 0u)];
        p1[k] = in ? a.prp1[i] : 0;
        p2[k] = in ? a.prp2[i] : 0;
        lba[k] = in ? a.slba[i] : 0;
    }
    uint64_t m[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        m[k] = ws.mask[((uint64_t)r.g * kRounds + k) * kWaves + w];   // the count pass's
        if (ln == 0) s_cnt[k][w] = (uint32_t)__popcll(m[k]);
    }
    __syncthreads();

    // Each round: the wave's placeable requests take consecutive slots (from
    // s0, wrapping at the ring's end) in lane order. A lane builds its entry
    // in the wave's LDS area at its rank; then lane l copies 16-byte quarter
    // l % 4 of entries l / 4, l / 4 + 16, ... to the ring, so each store
    // instruction writes 16 whole entries (1 KiB) back to back instead of
    // one quarter of 64 entries 64 bytes apart.
    const uint64_t below = __lanemask_lt();
    uint32_t run = before;                             // placeable before round k
    // The ring address comes from memory, so the compiler cannot infer its
    // address space; as a generic pointer its stores would be flat stores,
    // which also count against the LDS counter and so make every staging
    // read wait for them. Rings are device (global) memory.
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) u32x4 global_u32x4;
    global_u32x4 *ring = (global_u32x4 *)(uintptr_t)win.ring;
    uint4 *ent = s_ent[w];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        uint32_t wpre = 0, rtot = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const uint32_t c = s_cnt[k][v];
            wpre += v < w ? c : 0u;
            rtot += c;
        }
        uint32_t s0 = win.tail + run + wpre;           // slot of the wave's rank 0
        if (s0 >= win.depth) s0 -= win.depth;          // tail < depth, rank < depth - 1
        if ((m[k] >> ln) & 1u) {
            const uint32_t r = (uint32_t)__popcll(m[k] & below);
            uint32_t s = s0 + r;
            if (s >= win.depth) s -= win.depth;
            const uint32_t nlb0 = nlb[k];
            uint4 *e = ent + r * 4;
            e[0] = make_uint4(a.opcode | (s << 16), a.nsid, 0u, 0u);
            e[1] = make_uint4(0u, 0u, (uint32_t)p1[k], (uint32_t)(p1[k] >> 32));
            e[2] = make_uint4((uint32_t)p2[k], (uint32_t)(p2[k] >> 32), (uint32_t)lba[k],
                              (uint32_t)(lba[k] >> 32));
            e[3] = make_uint4(nlb0, 0u, 0u, 0u);
            if (a.req_of_slot) a.req_of_slot[(uint64_t)q * DMADESC_SQ_MAX_DEPTH + s] = idx[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t cw = (uint32_t)__popcll(m[k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t r = (uint32_t)(ln >> 2) + 16u * j;
            if (r < cw) {
                uint32_t s = s0 + r;
                if (s >= win.depth) s -= win.depth;
                const uint4 x = ent[r * 4 + (ln & 3)];
                ring[(uint64_t)s * 4 + (ln & 3)] = u32x4{x.x, x.y, x.z, x.w};
            }
        }
        // The next round reuses the area: its writes wait for these reads.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        run += rtot;
    }
}

// One wave per queue: lane t adds tile t's count (64 tiles cover a window).
__global__ __launch_bounds__(kThreads) void k_sqe_finish(SqeArgs a, SqeWs ws)
{
    const uint32_t q = blockIdx.x * kWaves + wave();
    if (q >= a.nqueues) return;                         // uniform per wave
    const Window win = window_of(a, q);
    const uint32_t tiles = (win.w + kTile - 1) / kTile;
    const uint32_t ln = lane();
    uint32_t placed = ln < tiles ? ws.counts[(uint64_t)q * kTilesPerQueue + ln] : 0u;
    placed = wave_sum(placed);
    if (ln == 0) {
        a.placed[q] = placed;
        if (win.w > 0) {
            uint32_t nt = win.tail + placed;
            if (nt >= win.depth) nt -= win.depth;
            a.tail[q] = nt;
            a.cursor[q] += win.w;
        }
    }
}

}  // namespace

// Per (queue, tile): a count, the masks and a record, and the block counts
// of its positions (2 bytes per ring slot a call can fill, 64 tiles per
// queue whatever qoff holds, so every schedule index stays in bounds); per
// queue a record. Under 1/16 of the rings the call can fill.
size_t ws_emit_sqe(uint32_t nq)
{
    const uint64_t tiles = (uint64_t)nq * kTilesPerQueue;
    return align256(tiles * sizeof(uint32_t)) + align256(tiles * kRounds * kWaves * 8) +
           align256(tiles * kTile * sizeof(uint16_t)) + align256(tiles * sizeof(TileRec)) +
           align256((uint64_t)nq * sizeof(QueueRec)) + 256;
}

hipError_t launch_emit_sqe(const SqeArgs &a, hipStream_t s)
{
    char *base = static_cast<char *>(a.ws);
    const uint64_t tiles = (uint64_t)a.nqueues * kTilesPerQueue;
    const uint64_t at_mask = align256(tiles * sizeof(uint32_t));
    const uint64_t at_nlb = at_mask + align256(tiles * kRounds * kWaves * 8);
    const uint64_t at_tiles = at_nlb + align256(tiles * kTile * sizeof(uint16_t));
    const uint64_t at_queues = at_tiles + align256(tiles * sizeof(TileRec));
    const uint64_t at_count = at_queues + align256((uint64_t)a.nqueues * sizeof(QueueRec));
    SqeWs ws{reinterpret_cast<uint32_t *>(base), reinterpret_cast<uint64_t *>(base + at_mask),
             reinterpret_cast<uint16_t *>(base + at_nlb), reinterpret_cast<TileRec *>(base + at_tiles),
             reinterpret_cast<QueueRec *>(base + at_queues),
             reinterpret_cast<uint32_t *>(base + at_count)};
    hipLaunchKernelGGL(k_sqe_order, dim3(1), dim3(kOrderThreads), 0, s, a, ws);
    hipLaunchKernelGGL(k_sqe_count, dim3((unsigned)tiles), dim3(kThreads), 0, s, a, ws);
    hipLaunchKernelGGL(k_sqe_emit, dim3((unsigned)tiles), dim3(kThreads), 0, s, a, ws);
    hipLaunchKernelGGL(k_sqe_finish, dim3((a.nqueues + kWaves - 1) / kWaves), dim3(kThreads), 0,
                       s, a, ws);
    return hipGetLastError();
}

}  // namespace dd

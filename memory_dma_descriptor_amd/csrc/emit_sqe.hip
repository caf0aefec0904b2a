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
// Layout: block (t, q) owns positions [t * kTile, (t + 1) * kTile) of queue
// q's window. A window is shorter than the deepest ring (65536 entries), so
// kTilesPerQueue blocks cover any window; blocks past the window's end return
// at once. Round k of a block covers kThreads consecutive positions, wave w
// the 64 positions [k * kThreads + 64 w, ...), so lanes meet positions in
// (round, wave, lane) order -- the window's order.
//
// Kernels: k_sqe_count (placeable requests per tile), k_sqe_emit (slots,
// entries, request map), k_sqe_finish (placed counts, tails and cursors).
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
static_assert(kTilesPerQueue <= kWave, "a wave sums the tile counts of one queue");

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

__global__ __launch_bounds__(kThreads) void k_sqe_count(SqeArgs a, uint32_t *__restrict__ counts)
{
    __shared__ uint32_t s_sum[kWaves];
    const uint32_t t = blockIdx.x, q = blockIdx.y;
    const Window win = window_of(a, q);
    const uint32_t lo = t * kTile;
    if (lo >= win.w) return;                           // uniform over the block
    const uint32_t cnt = win.w - lo < kTile ? win.w - lo : kTile;
    const uint32_t *__restrict__ pos = a.perm + win.start + lo;

    uint32_t idx[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t j = k * kThreads + threadIdx.x;
        idx[k] = j < cnt ? pos[j] : UINT32_MAX;
    }
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t i = idx[k];
        if (i < a.n && placeable(a.status[i], a.len[i], a.lba_shift)) ++c;
    }
    c = wave_sum(c);
    if (lane() == 0) s_sum[wave()] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += s_sum[w];
        counts[(uint64_t)q * kTilesPerQueue + t] = s;
    }
}

__global__ __launch_bounds__(kThreads) void k_sqe_emit(SqeArgs a, const uint32_t *__restrict__ counts)
{
    __shared__ uint32_t s_cnt[kRounds][kWaves];
    const uint32_t t = blockIdx.x, q = blockIdx.y;
    const Window win = window_of(a, q);
    const uint32_t lo = t * kTile;
    if (lo >= win.w) return;                           // uniform over the block
    const uint32_t cnt = win.w - lo < kTile ? win.w - lo : kTile;
    const uint32_t *__restrict__ pos = a.perm + win.start + lo;
    const int w = wave(), ln = lane();

    // Placeable requests of the window before this tile (t < 64 tiles).
    uint32_t before = (uint32_t)ln < t ? counts[(uint64_t)q * kTilesPerQueue + ln] : 0u;
    before = wave_sum(before);

    uint32_t idx[kRounds];
    uint64_t len[kRounds];
    bool ok[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t j = k * kThreads + threadIdx.x;
        idx[k] = j < cnt ? pos[j] : UINT32_MAX;
    }
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        const uint32_t i = idx[k];
        const bool in = i < a.n;
        len[k] = in ? a.len[i] : 0;
        ok[k] = in && placeable(a.status[i], len[k], a.lba_shift);
    }
    uint64_t m[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        m[k] = __ballot(ok[k]);
        if (ln == 0) s_cnt[k][w] = (uint32_t)__popcll(m[k]);
    }
    __syncthreads();

    const uint64_t below = __lanemask_lt();
    uint32_t run = before;                             // placeable before round k
    uint4 *ring = reinterpret_cast<uint4 *>(win.ring);
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
        uint32_t wpre = 0, rtot = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const uint32_t c = s_cnt[k][v];
            wpre += v < w ? c : 0u;
            rtot += c;
        }
        if (ok[k]) {
            const uint32_t i = idx[k];
            uint32_t s = win.tail + run + wpre + (uint32_t)__popcll(m[k] & below);
            if (s >= win.depth) s -= win.depth;        // tail < depth, rank < depth - 1
            const uint64_t p1 = a.prp1[i], p2 = a.prp2[i], lba = a.slba[i];
            const uint32_t nlb0 = (uint32_t)(len[k] >> a.lba_shift) - 1u;
            uint4 *e = ring + (uint64_t)s * 4;
            e[0] = make_uint4(a.opcode | (s << 16), a.nsid, 0u, 0u);
            e[1] = make_uint4(0u, 0u, (uint32_t)p1, (uint32_t)(p1 >> 32));
            e[2] = make_uint4((uint32_t)p2, (uint32_t)(p2 >> 32), (uint32_t)lba,
                              (uint32_t)(lba >> 32));
            e[3] = make_uint4(nlb0, 0u, 0u, 0u);
            if (a.req_of_slot) a.req_of_slot[(uint64_t)q * DMADESC_SQ_MAX_DEPTH + s] = i;
        }
        run += rtot;
    }
}

__global__ __launch_bounds__(kThreads) void k_sqe_finish(SqeArgs a, const uint32_t *__restrict__ counts)
{
    for (uint32_t q = threadIdx.x; q < a.nqueues; q += kThreads) {
        const Window win = window_of(a, q);
        const uint32_t tiles = (win.w + kTile - 1) / kTile;
        uint32_t placed = 0;
        for (uint32_t t = 0; t < tiles; ++t) placed += counts[(uint64_t)q * kTilesPerQueue + t];
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

size_t ws_emit_sqe(uint32_t nq)
{
    return align256((uint64_t)nq * kTilesPerQueue * sizeof(uint32_t));
}

hipError_t launch_emit_sqe(const SqeArgs &a, hipStream_t s)
{
    uint32_t *counts = static_cast<uint32_t *>(a.ws);
    const dim3 grid(kTilesPerQueue, a.nqueues);
    hipLaunchKernelGGL(k_sqe_count, grid, dim3(kThreads), 0, s, a, counts);
    hipLaunchKernelGGL(k_sqe_emit, grid, dim3(kThreads), 0, s, a, counts);
    hipLaunchKernelGGL(k_sqe_finish, dim3(1), dim3(kThreads), 0, s, a, counts);
    return hipGetLastError();
}

}  // namespace dd

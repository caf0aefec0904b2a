// partition.hip - stable split of request indices by destination queue, for
// gfx950.
//
// Method: every queue's requests are placed contiguously in increasing
// request index. The grouping of a wave's lanes by key follows the idea of the
// MORI thread-scope put kernel ("mori通信库分析(一)——对称内存RDMA数据发送过程"),
// which ballots the lanes that share a destination and lets one of them act
// for the group, and of its warp-level WQE reservation, where one lane
// reserves for the whole group and the others take consecutive slots by
// their rank. Here the group of each lane comes from one ballot per key bit
// (a lane matches when it agrees on every bit), its rank is the popcount of
// the group below it, and the lowest lane of each group publishes the count;
// a scan over (queue, block, item-round, wave) in that order turns counts
// into positions, which keeps equal keys in index order. No atomic decides a
// position, so the output is deterministic.
//
// Kernels: k_split_hist (per-block bucket counts, bucket-major),
// k_split_rowscan (one block per bucket: exclusive scan over blocks),
// k_split_scatter (bucket bases, intra-block ranks, perm writes).
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;                       // requests per thread
constexpr int kTile = kThreads * kItems;        // requests per block
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxBuckets = DMADESC_MAX_QUEUES + 1;

__device__ __forceinline__ int key_bits(uint32_t nq)
{
    return 32 - __clz(nq);                       // bits of the largest bucket id
}

__global__ __launch_bounds__(kThreads) void k_split_hist(
    const uint32_t *__restrict__ qid, uint64_t n, uint32_t nq, uint64_t nb,
    uint32_t *__restrict__ counts)
{
    __shared__ uint32_t h[kMaxBuckets];
    const uint32_t nbk = nq + 1;
    for (uint32_t b = threadIdx.x; b < nbk; b += kThreads) h[b] = 0;
    __syncthreads();
    const int nbits = key_bits(nq);
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
    const uint64_t below = __lanemask_lt();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kThreads + threadIdx.x;
        const bool on = i < n;
        uint32_t b = 0;
        if (on) {
            const uint32_t q = qid[i];
            b = q < nq ? q : nq;
        }
        const uint64_t m = match_key(b, on, nbits, __ballot(on));
        if (on && (m & below) == 0) atomicAdd(&h[b], (uint32_t)__popcll(m));
    }
    __syncthreads();
    for (uint32_t b = threadIdx.x; b < nbk; b += kThreads) counts[(uint64_t)b * nb + blockIdx.x] = h[b];
}

// One block per bucket: exclusive scan of that bucket's per-block counts.
__global__ __launch_bounds__(kThreads) void k_split_rowscan(
    uint32_t *__restrict__ counts, uint64_t nb, uint64_t *__restrict__ rowtotal)
{
    __shared__ uint64_t scratch[kWaves];
    uint32_t *row = counts + (uint64_t)blockIdx.x * nb;
    const uint64_t seg = (nb + kThreads - 1) / kThreads;
    const uint64_t b0 = (uint64_t)threadIdx.x * seg;
    const uint64_t b1 = (b0 + seg < nb) ? b0 + seg : nb;
    uint64_t s = 0;
    for (uint64_t b = b0; b < b1; ++b) s += row[b];
    uint64_t tot;
    uint64_t run = block_excl_scan<kThreads>(s, scratch, &tot);
    for (uint64_t b = b0; b < b1; ++b) {
        const uint32_t c = row[b];
        row[b] = (uint32_t)run;
        run += c;
    }
    if (threadIdx.x == 0) rowtotal[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kThreads) void k_split_scatter(
    const uint32_t *__restrict__ qid, uint64_t n, uint32_t nq, uint64_t nb,
    const uint32_t *__restrict__ counts, const uint64_t *__restrict__ rowtotal,
    uint32_t *__restrict__ perm, uint64_t *__restrict__ qoff,
    uint64_t *__restrict__ n_invalid)
{
    __shared__ uint64_t s_base[kMaxBuckets];
    __shared__ uint32_t s_cnt[kItems * kWaves][kMaxBuckets];
    const uint32_t nbk = nq + 1;
    const int t = threadIdx.x, w = wave();

    for (uint32_t b = t; b < nbk; b += kThreads) s_base[b] = rowtotal[b];
    for (int kw = 0; kw < kItems * kWaves; ++kw)
        for (uint32_t b = t; b < nbk; b += kThreads) s_cnt[kw][b] = 0;
    __syncthreads();
    if (t == 0) {                                  // bucket starts over the whole batch
        uint64_t run = 0;
        for (uint32_t b = 0; b < nbk; ++b) {
            const uint64_t c = s_base[b];
            s_base[b] = run;
            run += c;
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (uint32_t b = t; b < nbk; b += kThreads) qoff[b] = s_base[b];
        if (t == 0) {
            qoff[nbk] = n;
            *n_invalid = rowtotal[nq];
        }
    }

    const int nbits = key_bits(nq);
    const uint64_t base = (uint64_t)blockIdx.x * kTile;
    const uint64_t below = __lanemask_lt();
    uint32_t bkt[kItems], rank[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kThreads + t;
        const bool on = i < n;
        uint32_t b = 0;
        if (on) {
            const uint32_t q = qid[i];
            b = q < nq ? q : nq;
        }
        const uint64_t m = match_key(b, on, nbits, __ballot(on));
        const uint32_t r = (uint32_t)__popcll(m & below);
        if (on && r == 0) s_cnt[k * kWaves + w][b] = (uint32_t)__popcll(m);
        bkt[k] = b;
        rank[k] = r;
    }
    __syncthreads();
    // Positions: bucket start + this block's offset in the bucket + earlier
    // (item-round, wave) groups of this block.
    for (uint32_t b = t; b < nbk; b += kThreads) {
        uint64_t run = s_base[b] + counts[(uint64_t)b * nb + blockIdx.x];
        for (int kw = 0; kw < kItems * kWaves; ++kw) {
            const uint32_t c = s_cnt[kw][b];
            s_cnt[kw][b] = (uint32_t)run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = base + (uint64_t)k * kThreads + t;
        if (i < n) perm[s_cnt[k * kWaves + w][bkt[k]] + rank[k]] = (uint32_t)i;
    }
}

__global__ void k_split_empty(uint32_t nq, uint64_t *__restrict__ qoff, uint64_t *__restrict__ n_invalid)
{
    for (uint32_t b = threadIdx.x; b < nq + 2; b += blockDim.x) qoff[b] = 0;
    if (threadIdx.x == 0) *n_invalid = 0;
}

}  // namespace

size_t ws_partition(uint64_t n, uint32_t nq)
{
    const uint64_t nb = (n + kTile - 1) / kTile;
    return align256((uint64_t)(nq + 1) * nb * sizeof(uint32_t)) +
           align256((uint64_t)(nq + 1) * sizeof(uint64_t));
}

hipError_t launch_partition(const SplitArgs &a, hipStream_t s)
{
    if (a.n == 0) {
        hipLaunchKernelGGL(k_split_empty, dim3(1), dim3(kThreads), 0, s, a.nqueues, a.qoff,
                           a.n_invalid);
        return hipGetLastError();
    }
    const uint64_t nb = (a.n + kTile - 1) / kTile;
    uint32_t *counts = static_cast<uint32_t *>(a.ws);
    uint64_t *rowtotal = reinterpret_cast<uint64_t *>(
        static_cast<char *>(a.ws) + align256((uint64_t)(a.nqueues + 1) * nb * sizeof(uint32_t)));
    hipLaunchKernelGGL(k_split_hist, dim3((unsigned)nb), dim3(kThreads), 0, s,
                       a.qid, a.n, a.nqueues, nb, counts);
    hipLaunchKernelGGL(k_split_rowscan, dim3(a.nqueues + 1), dim3(kThreads), 0, s,
                       counts, nb, rowtotal);
    hipLaunchKernelGGL(k_split_scatter, dim3((unsigned)nb), dim3(kThreads), 0, s,
                       a.qid, a.n, a.nqueues, nb, counts, rowtotal, a.perm, a.qoff,
                       a.n_invalid);
    return hipGetLastError();
}

}  // namespace dd

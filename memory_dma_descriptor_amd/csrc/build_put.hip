// build_put.hip - RDMA put descriptors for a symmetric heap, static or VMM,
// for gfx950.
//
// Method (MORI page, "mori通信库分析(一)", thread-scope put and QueryRemoteAddr):
// the remote address of a heap offset is the peer's heap base plus the same
// offset. In a static heap one local key and one remote key per peer cover the
// heap and the whole remainder goes in one transfer. In a VMM heap every chunk
// has its own keys, and each round of the put loop sends min(bytes left in the
// source chunk, bytes left in the destination chunk, remaining), so that a key
// always covers what it is used for. No transfer exceeds 2^31 bytes (the RDMA
// message limit), which only binds for a static heap.
//
// The rounds have a closed form. With chunk size C, the source boundaries
// after the start lie at a, a + C, ... (a = C - src % C) and the destination
// ones at b, b + C, ...; both progressions have period C, so when a != b they
// alternate: min(a, b), max(a, b), min(a, b) + C, ... Piece j ends at the j-th
// boundary (or at the end of the request); the piece count is 1 + source
// boundaries crossed + destination boundaries crossed - the shared ones (all
// of them when a == b). Every descriptor is therefore computed on its own.
//
// One pass: 4,096 requests per block (16 waves, one block per CU), 256
// consecutive ones per wave; the
// descriptor slots of a request are a device-wide exclusive scan of the piece
// counts in request order (decoupled look-back, dd_lookback.hpp); then each
// wave writes the descriptors of its requests in two halves of 128, each one
// contiguous range, load-balanced over descriptors: lane j of a step takes
// descriptor S + 64 j + lane and finds its request by a 7-step search over
// the requests' first slots in LDS. The key reads of up to kSub steps are
// issued before any of them is used, so a half waits about one gather round
// trip, not one per step; a step's 64 descriptors go out through LDS as two
// 1 KiB store instructions.
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dd_lookback.hpp"
#include "dmadesc.h"

namespace dd {
namespace {

// Blocks of 1,024 threads: a block's look-back waits for its youngest
// predecessors' aggregates (their column loads) while its waves idle, so
// fewer, larger blocks pay that wait less often (256-thread blocks: 0.515 ms
// on 16.8 M puts, 512: 0.480, 1,024: 0.422).
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kItems = 4;
constexpr int kTile = kThreads * kItems;
constexpr uint32_t kMsgShift = 31;                   // largest transfer: 2^31 bytes

enum : uint8_t { kOk = 0, kEinval = 1, kErange = 2, kEnospc = 3, kEbusy = 4 };

// Pieces of one put (shift 0: static heap).
__device__ __forceinline__ uint64_t put_pieces(uint64_t s, uint64_t d, uint64_t b, uint32_t shift)
{
    if (shift == 0) return (b + (1ull << kMsgShift) - 1) >> kMsgShift;
    const uint64_t cs = ((s + b - 1) >> shift) - (s >> shift);
    const uint64_t cd = ((d + b - 1) >> shift) - (d >> shift);
    const uint64_t common = ((s - d) & ((1ull << shift) - 1)) == 0 ? cs : 0;
    return 1 + cs + cd - common;
}

// Offset (from the put's start) at which piece j ends, before clipping to the
// put's length.
__device__ __forceinline__ uint64_t put_boundary(uint64_t s, uint64_t d, uint32_t shift, uint64_t j)
{
    if (shift == 0) return (j + 1) << kMsgShift;
    const uint64_t c = 1ull << shift, mask = c - 1;
    const uint64_t a = c - (s & mask), bb = c - (d & mask);
    if (a == bb) return a + (j << shift);
    const uint64_t lo = a < bb ? a : bb, hi = a < bb ? bb : a;
    return ((j & 1) ? hi : lo) + ((j >> 1) << shift);
}

constexpr int kHalf = 2 * kWave;          // requests per emission table
constexpr int kSub = 4;                   // descriptor steps whose key reads fly together

struct PutTab {
    uint64_t start[kHalf + 1];   // first descriptor slot of each request ([kHalf]: end)
    uint64_t s[kHalf], d[kHalf], b[kHalf];
    uint32_t pe[kHalf];
    u64x2 out[2 * kWave];        // one step's 64 descriptors, in order, for the stores
};

struct PutKeys {
    const uint32_t *lkeys;
    const uint64_t *peer_base;
    const uint32_t *rkeys;
    uint64_t local_base, nchunks;
    uint32_t shift;
};

__device__ __forceinline__ void wave_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes the descriptors of 128 consecutive requests, request r = 64 h + lane
// for h = 0, 1 (first[h], m[h] descriptors from slot first[h]; m == 0 for
// none); req0 is the index of request 0.
__device__ __forceinline__ void emit_put_half(PutTab &T, const uint64_t (&first)[2],
                                              const uint64_t (&m)[2], const uint64_t (&s)[2],
                                              const uint64_t (&d)[2], const uint64_t (&b)[2],
                                              const uint32_t (&pe)[2], uint64_t req0,
                                              const PutKeys &K, uint64_t *__restrict__ desc)
{
    const int ln = lane();
    const uint64_t has0 = __ballot(m[0] != 0), has1 = __ballot(m[1] != 0);
    if ((has0 | has1) == 0) return;                      // uniform per wave
    const uint64_t S = has0 ? __shfl(first[0], __ffsll((unsigned long long)has0) - 1, kWave)
                            : __shfl(first[1], __ffsll((unsigned long long)has1) - 1, kWave);
    const uint64_t E = has1 ? __shfl(first[1] + m[1], 63 - __clzll((unsigned long long)has1), kWave)
                            : __shfl(first[0] + m[0], 63 - __clzll((unsigned long long)has0), kWave);
    // Requests before the first one with descriptors start at S; those after
    // the last one (none, or refused) at E: the search never picks them.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = h * kWave + ln;
        T.start[r] = first[h] < S ? S : (first[h] > E ? E : first[h]);
        T.s[r] = s[h];
        T.d[r] = d[h];
        T.b[r] = b[h];
        T.pe[r] = pe[h];
    }
    if (ln == kWave - 1) T.start[kHalf] = E;
    wave_fence();
    for (uint64_t c = S; c < E; c += (uint64_t)kSub * kWave) {   // uniform per wave
        // Every step's descriptor and key reads first (lanes past the end
        // compute the last descriptor again; not stored).
        int r[kSub];
        uint64_t x0[kSub], x1[kSub], pb[kSub];
        uint32_t lkey[kSub], rkey[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            const uint64_t pu = c + (uint64_t)u * kWave + ln;
            const uint64_t p = pu < E ? pu : E - 1;
            r[u] = owner_of<kHalf>(T.start, p);
            const uint64_t j = p - T.start[r[u]];
            const uint64_t rs = T.s[r[u]], rd = T.d[r[u]], rb = T.b[r[u]];
            const uint32_t rpe = T.pe[r[u]];
            x0[u] = j ? put_boundary(rs, rd, K.shift, j - 1) : 0;
            const uint64_t e = put_boundary(rs, rd, K.shift, j);
            x1[u] = e < rb ? e : rb;
            // Key indices without a branch (a static heap has one local key
            // and one remote key per PE: nchunks is 1 and the chunk is 0),
            // so all of the steps' reads are in flight together; behind a
            // branch each join waited for every read issued before it.
            const uint64_t lc = K.shift ? (rs + x0[u]) >> K.shift : 0;
            const uint64_t rc = K.shift ? (rd + x0[u]) >> K.shift : 0;
            lkey[u] = K.lkeys[lc];
            rkey[u] = K.rkeys[(uint64_t)rpe * K.nchunks + rc];
            pb[u] = K.peer_base[rpe];
        }
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            const uint64_t cu = c + (uint64_t)u * kWave;
            if (cu >= E) break;                              // uniform per wave
            const uint64_t rs = T.s[r[u]], rd = T.d[r[u]];
            const uint64_t w2 = (x1[u] - x0[u]) | ((uint64_t)lkey[u] << 32);
            const uint64_t w3 = rkey[u] | ((req0 + (uint64_t)r[u]) << 32);
            // Through LDS, so that each of the wave's two 16-byte store
            // instructions covers 1 KiB contiguously (a lane storing its own
            // 32-byte descriptor would fill half of every 32 bytes per
            // instruction, which non-temporal stores pay for twice).
            T.out[2 * ln] = u64x2{K.local_base + rs + x0[u], pb[u] + rd + x0[u]};
            T.out[2 * ln + 1] = u64x2{w2, w3};
            wave_fence();
            const u64x2 h0 = T.out[ln], h1 = T.out[kWave + ln];
            u64x2 *dst = reinterpret_cast<u64x2 *>(desc + 4 * cu);
            if (cu + (ln >> 1) < E) __builtin_nontemporal_store(h0, dst + ln);
            if (cu + kWave / 2 + (ln >> 1) < E) __builtin_nontemporal_store(h1, dst + kWave + ln);
            wave_fence();                                    // out is rewritten next
        }
    }
    wave_fence();                                            // the next half rewrites T
}

__global__ __launch_bounds__(kThreads) void k_put_build(
    const uint64_t *__restrict__ src, const uint64_t *__restrict__ dst,
    const uint64_t *__restrict__ bytes, const uint32_t *__restrict__ pe, uint64_t n,
    uint64_t heap, uint32_t npes, PutKeys K, uint64_t *__restrict__ desc, uint64_t cap,
    uint64_t *__restrict__ first_out, uint32_t *__restrict__ count_out,
    uint8_t *__restrict__ status, uint64_t *__restrict__ total, uint64_t nblocks,
    Header *__restrict__ hdr, uint64_t *__restrict__ bstat, uint32_t max_polls)
{
    __shared__ uint64_t s_red[kWaves];
    __shared__ uint64_t s_bid, s_excl;
    __shared__ uint32_t s_dead;
    __shared__ PutTab s_tab[kWaves];
    const int t = threadIdx.x, w = wave(), ln = lane();
    if (t == 0) s_bid = atomicAdd(&hdr->ticket, 1u);
    __syncthreads();
    const uint64_t blk = s_bid;
    const uint64_t base = blk * kTile;
    // Wave w owns requests wbase .. wbase + 255; item k of a lane is request
    // wbase + 64 k + lane (request order is (wave, item, lane) order).
    const uint64_t wbase = base + (uint64_t)w * (kWave * kItems);
    const bool full = base + kTile <= n;                 // uniform per block

    uint64_t s[kItems], d[kItems], b[kItems], cnt[kItems], pre[kItems];
    uint32_t q[kItems];
    uint8_t st[kItems];
    if (full) {
        // Every load in flight at once (a guarded load would wait for the
        // one before it).
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint64_t i = wbase + (uint64_t)k * kWave + ln;
            s[k] = __builtin_nontemporal_load(src + i);
            d[k] = __builtin_nontemporal_load(dst + i);
            b[k] = __builtin_nontemporal_load(bytes + i);
            q[k] = __builtin_nontemporal_load(pe + i);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kItems; ++k) {
            const uint64_t i = wbase + (uint64_t)k * kWave + ln;
            const bool in = i < n;
            s[k] = in ? src[i] : 0;
            d[k] = in ? dst[i] : 0;
            b[k] = in ? bytes[i] : 0;
            q[k] = in ? pe[i] : 0;
        }
    }
    uint64_t carry = 0;                                  // the wave's pieces before item k
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        st[k] = kOk;
        if (b[k] == 0 || q[k] >= npes) st[k] = kEinval;
        else if (b[k] > heap || s[k] > heap - b[k] || d[k] > heap - b[k]) st[k] = kErange;
        cnt[k] = st[k] == kOk ? put_pieces(s[k], d[k], b[k], K.shift) : 0;
        const uint64_t inc = wave_incl_scan(cnt[k]);
        pre[k] = carry + inc - cnt[k];
        carry += __shfl(inc, kWave - 1, kWave);
    }
    if (ln == 0) s_red[w] = carry;
    __syncthreads();
    uint64_t agg = 0, wpre = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const uint64_t x = s_red[v];
        wpre += v < w ? x : 0ull;
        agg += x;
    }
    if (w == 0) {
        uint64_t excl = 0;
        bool dead = false;
        if (blk == 0) {
            if (ln == 0) store_status(bstat, kFlagInc | agg);
        } else {
            if (ln == 0) store_status(bstat + blk, kFlagAgg | agg);
            excl = look_back(bstat, (int64_t)blk, &hdr->timeouts, max_polls, dead);
            // An expired wait leaves the aggregate published (later blocks
            // still find their prefixes); this block's puts are refused.
            if (ln == 0 && !dead) store_status(bstat + blk, kFlagInc | (excl + agg));
        }
        if (ln == 0) {
            s_excl = excl;
            s_dead = dead;
            if (blk == nblocks - 1) *total = dead ? ~0ull : excl + agg;
        }
    }
    __syncthreads();
    const uint64_t excl = s_excl + wpre;
    const bool dead = s_dead != 0;

    uint64_t f[kItems], m[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        const uint64_t i = wbase + (uint64_t)k * kWave + ln;
        f[k] = excl + pre[k];
        uint8_t sk = st[k];
        if (cnt[k] != 0 && dead) {
            sk = kEbusy;                                      // its slots are unknown
            f[k] = ~0ull;
        } else if (cnt[k] != 0 && f[k] + cnt[k] > cap) {
            sk = kEnospc;                                     // refused; its slots stay taken
        }
        m[k] = sk == kOk ? cnt[k] : 0;
        if (i < n) {
            __builtin_nontemporal_store(f[k], first_out + i);
            __builtin_nontemporal_store((uint32_t)cnt[k], count_out + i);
            __builtin_nontemporal_store(sk, status + i);
        }
    }
#pragma unroll 1
    for (int h = 0; h < kItems / 2; ++h) {
        const uint64_t fh[2] = {f[2 * h], f[2 * h + 1]}, mh[2] = {m[2 * h], m[2 * h + 1]};
        const uint64_t sh[2] = {s[2 * h], s[2 * h + 1]}, dh[2] = {d[2 * h], d[2 * h + 1]};
        const uint64_t bh[2] = {b[2 * h], b[2 * h + 1]};
        const uint32_t qh[2] = {q[2 * h], q[2 * h + 1]};
        emit_put_half(s_tab[w], fh, mh, sh, dh, bh, qh, wbase + (uint64_t)h * kHalf, K, desc);
    }
}

}  // namespace

size_t ws_build_put(uint64_t n)
{
    if (n == 0) return 0;
    const uint64_t nb = (n + kTile - 1) / kTile;
    return align256(kHeaderBytes + nb * sizeof(uint64_t));
}

hipError_t launch_build_put(const PutArgs &a, hipStream_t s)
{
    const uint64_t nb = (a.n + kTile - 1) / kTile;
    if (nb == 0) {
        hipLaunchKernelGGL(k_ws_clear, dim3(1), dim3(64), 0, s, a.total, (uint64_t)1);
        return hipGetLastError();
    }
    Header *hdr = static_cast<Header *>(a.ws);
    uint64_t *bstat = reinterpret_cast<uint64_t *>(static_cast<char *>(a.ws) + kHeaderBytes);
    const uint64_t words = kHeaderBytes / sizeof(uint64_t) + nb;
    uint64_t cblocks = (words + 255) / 256;
    if (cblocks > 1024) cblocks = 1024;
    hipLaunchKernelGGL(k_ws_clear, dim3((unsigned)cblocks), dim3(256), 0, s,
                       static_cast<uint64_t *>(a.ws), words);
    const PutKeys K{a.lkeys, a.peer_base, a.rkeys, a.local_base,
                    a.chunk_shift ? a.heap_bytes >> a.chunk_shift : 1, a.chunk_shift};
    hipLaunchKernelGGL(k_put_build, dim3((unsigned)nb), dim3(kThreads), 0, s, a.src, a.dst,
                       a.bytes, a.pe, a.n, a.heap_bytes, a.npes, K, a.desc, a.desc_cap,
                       a.first, a.count, a.status, a.total, nb, hdr, bstat, wait_limit());
    return hipGetLastError();
}

}  // namespace dd

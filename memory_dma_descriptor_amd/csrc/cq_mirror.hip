// cq_mirror.hip - completion-queue mirror: a resident kernel copies NVMe
// completions from device-memory completion queues into mirror queues as their
// phase bit turns, for gfx950.
//
// Method (xNVMe "uPCIe CUDA" page, "Completions in device memory"): one
// kernel serves every mirrored queue (up to 64), one warp -- here one wave --
// per queue; it copies completions into the host queue as their phase bit
// turns. Host and kernel share a slot per queue holding the two queue
// addresses, the depth, a generation and an acknowledgement: the host raises
// the generation to an odd value to attach a queue, the wave copies until the
// generation changes and then acknowledges the value it worked under, and a
// wave finding an even generation acknowledges the odd value before it. The
// completion entry is NVMe's: 16 bytes, phase tag in bit 16 of dword 3, written
// as 1 on the controller's first pass through the queue and inverted on every
// later pass.
//
// A wave polls the next min(256, depth) entries at once: lane l reads dword 3
// of entries head + l, head + 64 + l, ... and compares each phase with the one
// expected there (it flips past the wrap); the leading run of matches is copied:
// each entry whole but with the old phase bit, then -- after a release fence --
// dword 3 with the new one, so a consumer polling the mirror's phase bits never
// sees a partial entry, whatever the width at which the writes land. Loads of the
// device queue are system-scope atomics after a system-scope acquire, so a
// writer on another agent (the controller, the host, another stream) is seen.
//
// The kernel is resident only for one call: every wave leaves when the stop
// flag is set (after a last drain), after `idle_polls` polls in a row that
// copied nothing, or after kMaxPolls polls in all, so the grid always drains.
// The slot keeps the next position, the expected phase and the count copied,
// so successive calls continue where the last one stopped.
#include "dd_device.hpp"
#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr uint32_t kMaxPolls = 1u << 22;

__device__ __forceinline__ uint32_t load_sys(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void store_sys(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Entries a lane watches per poll: a wave looks at up to 256 at once, so a
// burst of completions costs one poll round trip per 256 rather than per 64.
constexpr uint32_t kPerLane = 4;

// One poll of one queue: copies the leading run of entries whose phase is the
// expected one; returns how many (wave-uniform).
__device__ __forceinline__ uint32_t drain_once(const uint32_t *src, uint32_t *dst, uint32_t depth,
                                               uint32_t &head, uint32_t &phase)
{
    const uint32_t ln = (uint32_t)lane();
    const uint32_t span = (uint32_t)kWave * kPerLane;
    const uint32_t width = depth < span ? depth : span;
    uint32_t pos[kPerLane], dw3[kPerLane];
    uint64_t m[kPerLane];
#pragma unroll
    for (uint32_t j = 0; j < kPerLane; ++j) {
        const uint32_t i = j * (uint32_t)kWave + ln;      // window index, < width if on
        const bool on = i < width;
        uint32_t p = head + i;
        const bool wrapped = p >= depth;
        if (wrapped) p -= depth;                           // i < depth: at most one wrap
        pos[j] = p;
        const uint32_t want = phase ^ (wrapped ? 1u : 0u);
        dw3[j] = on ? load_sys(src + 4 * (uint64_t)p + 3) : 0u;
        m[j] = __ballot(on && ((dw3[j] >> 16) & 1u) == want);
    }
    // Leading matches over the window, <= width (lanes past it never match).
    uint32_t k = 0;
#pragma unroll
    for (uint32_t j = 0; j < kPerLane; ++j) {
        if (m[j] != ~0ull) {
            k += (uint32_t)__builtin_ctzll(~m[j]);
            break;
        }
        k += (uint32_t)kWave;
    }
    if (k == 0) return 0;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");          // entry data after its phase
    uint32_t d[kPerLane][3];
#pragma unroll
    for (uint32_t j = 0; j < kPerLane; ++j) {
        if (j * (uint32_t)kWave + ln < k) {
            const uint32_t *e = src + 4 * (uint64_t)pos[j];
            d[j][0] = load_sys(e);
            d[j][1] = load_sys(e + 1);
            d[j][2] = load_sys(e + 2);
        }
    }
    // Each entry is written whole with its phase bit still the old one, then
    // -- after a release -- its dword 3 with the new phase, then released
    // again so the poll's completions are visible at once. Plain stores and
    // fences: system-scope stores to host memory each wait for the write to
    // land (about a microsecond apiece), fences wait once per poll.
#pragma unroll
    for (uint32_t j = 0; j < kPerLane; ++j) {
        if (j * (uint32_t)kWave + ln < k) {
            uint4 *o = reinterpret_cast<uint4 *>(dst + 4 * (uint64_t)pos[j]);
            *o = make_uint4(d[j][0], d[j][1], d[j][2], dw3[j] ^ (1u << 16));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");          // data before the phase words
#pragma unroll
    for (uint32_t j = 0; j < kPerLane; ++j)
        if (j * (uint32_t)kWave + ln < k) dst[4 * (uint64_t)pos[j] + 3] = dw3[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");          // publish now, not at the next poll
    uint32_t nh = head + k;
    if (nh >= depth) {
        nh -= depth;
        phase ^= 1u;
    }
    head = nh;
    return k;
}

// The queue a slot describes, as the host last filled it.
struct Queue {
    const uint32_t *src;
    uint32_t *dst;
    uint32_t depth, head, phase;
    uint64_t copied;
    bool usable;
};

__device__ __forceinline__ Queue read_slot(const dmadesc_cq_slot *sl)
{
    Queue v;
    v.depth = sl->depth;
    const uint64_t srca = sl->src, dsta = sl->dst;
    v.usable = v.depth >= 2 && v.depth <= DMADESC_CQ_MAX_DEPTH && srca && dsta &&
               !(srca & 15u) && !(dsta & 15u);
    v.src = reinterpret_cast<const uint32_t *>(srca);
    v.dst = reinterpret_cast<uint32_t *>(dsta);
    v.head = sl->head;
    v.phase = sl->phase & 1u;
    if (v.head >= v.depth) v.usable = false;
    v.copied = sl->copied;
    return v;
}

__global__ __launch_bounds__(kWave) void k_cq_mirror(dmadesc_cq_slot *slots, uint32_t nslots,
                                                     const uint32_t *stop, uint32_t idle_polls)
{
    const uint32_t q = blockIdx.x;
    if (q >= nslots) return;
    dmadesc_cq_slot *sl = slots + q;
    uint32_t work_gen = 0;                               // odd generation being served
    Queue v{};
    uint32_t idle = 0, acked_gen = 0;
    bool acked = false;
    for (uint32_t poll = 0; poll < kMaxPolls; ++poll) {
        // Each poll starts with a system-scope acquire: the loads after it see
        // what other agents wrote even where this GPU's caches hold an older
        // copy (a controller writing the queue over PCIe bypasses them), and
        // a wave that sees the stop flag also sees every generation and entry
        // written before it.
        const bool stopping = load_sys(stop) != 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
        const uint32_t gen = load_sys(&sl->generation);
        uint32_t got = 0;
        if (gen & 1u) {
            if (gen != work_gen) {
                if (work_gen != 0) {                     // re-attached: finish the old queue
                    if (lane() == 0) {
                        sl->head = v.head;
                        sl->phase = v.phase;
                        sl->copied = v.copied;
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
                        store_sys(&sl->ack, work_gen);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // slot fields after gen
                v = read_slot(sl);                       // the host filled it before gen
                work_gen = gen;
            }
            if (v.usable) got = drain_once(v.src, v.dst, v.depth, v.head, v.phase);
            v.copied += got;
        } else {
            if (work_gen != 0 && lane() == 0) {          // detached while served
                sl->head = v.head;
                sl->phase = v.phase;
                sl->copied = v.copied;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
            }
            if (!acked || gen != acked_gen) {            // once per detached generation
                if (lane() == 0) store_sys(&sl->ack, gen - 1);
                acked = true;
                acked_gen = gen;
            }
            work_gen = 0;
        }
        if (got) {
            idle = 0;
            continue;                                    // more may be waiting
        }
        if (stopping || ++idle >= idle_polls) break;
        __builtin_amdgcn_s_sleep(8);
    }
    if (work_gen != 0 && lane() == 0) {                  // keep the position for the next call
        sl->head = v.head;
        sl->phase = v.phase;
        sl->copied = v.copied;
    }
}

}  // namespace

hipError_t launch_cq_mirror(dmadesc_cq_slot *slots, uint32_t nslots, const uint32_t *stop,
                            uint32_t idle_polls, hipStream_t s)
{
    hipLaunchKernelGGL(k_cq_mirror, dim3(nslots), dim3(kWave), 0, s, slots, nslots, stop,
                       idle_polls);
    return hipGetLastError();
}

}  // namespace dd

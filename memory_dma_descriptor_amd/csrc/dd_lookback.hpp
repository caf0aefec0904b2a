// dd_lookback.hpp - a device-wide exclusive scan in one pass (decoupled
// look-back) shared by the kernels that hand out output slots in request
// order: each block publishes its aggregate, then reads its predecessors'
// published values until it meets an inclusive prefix. Block order comes from
// an atomic ticket in the workspace header, so a block only ever waits on
// blocks that are already running. Waits are bounded: a block whose wait
// runs out does not know its prefix, counts itself in the header and
// reports it to its caller, which then refuses the outputs that need the
// prefix (a distinct status), so an expired wait is never silent. Blocks
// after it still find their own prefixes, since its aggregate is published.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dd_device.hpp"

namespace dd {
namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;     // status word: aggregate published
constexpr uint64_t kFlagInc = 2ull << 62;     // status word: inclusive prefix published
constexpr uint64_t kValue = (1ull << 62) - 1;

// Workspace layout: a 256-byte header, then one status word per block.
struct Header {
    uint32_t ticket;     // next block order
    uint32_t timeouts;   // blocks whose look-back wait hit the bound (never
                         // expected at the default bound)
};
constexpr size_t kHeaderBytes = 256;

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t load_status(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_status(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of the values of all blocks before `b` (called by one
// whole wave; lane k inspects block b-1-k of the current window). When a
// wait takes more than max_polls polls, `expired` is set (in every lane) and
// the value returned is meaningless.
__device__ uint64_t look_back(uint64_t *status, int64_t b, uint32_t *timeouts,
                              uint32_t max_polls, bool &expired)
{
    const int ln = lane();
    uint64_t excl = 0;
    int64_t top = b - 1;
    uint32_t polls = 0;
    expired = false;
    for (;;) {
        const int64_t idx = top - ln;
        uint64_t s = idx >= 0 ? load_status(status + idx) : kFlagInc;   // before block 0: 0
        while (__ballot((s >> 62) == 0) != 0) {
            if (++polls > max_polls) {
                if (ln == 0) atomicAdd(timeouts, 1u);
                expired = true;
                return 0;
            }
            __builtin_amdgcn_s_sleep(2);
            if ((s >> 62) == 0) s = load_status(status + idx);
        }
        const uint64_t inc = __ballot((s >> 62) == 2);
        if (inc != 0) {
            const int first = __ffsll((unsigned long long)inc) - 1;   // nearest inclusive
            excl += wave_sum(ln <= first ? (s & kValue) : 0ull);
            return excl;
        }
        excl += wave_sum(s & kValue);
        top -= kWave;
    }
}

__global__ void k_ws_clear(uint64_t *ws_words, uint64_t words)
{
    for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < words;
         k += (uint64_t)gridDim.x * blockDim.x)
        ws_words[k] = 0;
}

}  // namespace
}  // namespace dd

// dd_internal.h - launchers behind the C ABI (host side). The public entry
// points in api.hip validate arguments and then call these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dmadesc.h"

namespace dd {

struct LookupArgs {
    const uint64_t *reg_start, *reg_end;
    const uint32_t *reg_lkey;
    uint32_t nregions, page_shift;
    const uint64_t *off, *len;
    uint64_t n, va_base;
    int32_t *handle;
    uint32_t *lkey;
    uint8_t *kind;
    uint64_t *rbase, *rend;
    uint64_t *rec = nullptr;   // record copy of a large table (workspace), or none
};

struct PrpArgs {
    const uint64_t *lut;
    uint64_t lut_entries;
    const uint64_t *off, *len;
    uint64_t n, list_bus_base;
    uint64_t *pool;
    uint64_t pool_pages;
    uint64_t *prp1, *prp2;
    uint8_t *status;
    uint64_t *total_pages;
    void *ws;
    bool packed;          // lists back to back (dmadesc_build_prp_packed)
};

struct SplitArgs {
    const uint32_t *qid;
    uint64_t n;
    uint32_t nqueues;
    uint32_t *perm;
    uint64_t *qoff, *n_invalid;
    void *ws;
};

struct SqeArgs {
    const uint32_t *perm;
    const uint64_t *qoff;
    uint32_t nqueues;
    const uint8_t *status;
    const uint64_t *len, *slba, *prp1, *prp2;
    uint64_t n;
    uint32_t opcode, nsid, lba_shift;
    const uint64_t *ring;
    const uint32_t *depth, *free_slots;
    uint32_t *tail;
    uint64_t *cursor;
    uint32_t *placed, *req_of_slot;
    void *ws;
};

struct RegArgs {
    uint64_t *start, *end, *id;
    uint32_t *refs, *by_start;
    uint64_t *state;
    uint64_t capacity;
    uint32_t page_shift;
    const uint64_t *addr, *size;      // register
    const uint64_t *handle_in;        // deregister
    uint64_t n;
    uint64_t *handle;                 // register outputs
    uint8_t *kind;
    uint64_t *needed;
    uint8_t *status;                  // deregister output
    void *ws;
};

struct PutArgs {
    const uint64_t *src, *dst, *bytes;
    const uint32_t *pe;
    uint64_t n, local_base, heap_bytes;
    uint32_t chunk_shift, npes;
    const uint32_t *lkeys;
    const uint64_t *peer_base;
    const uint32_t *rkeys;
    uint64_t *desc;             // 4 words per descriptor
    uint64_t desc_cap;
    uint64_t *first;
    uint32_t *count;
    uint8_t *status;
    uint64_t *total;
    void *ws;
};

hipError_t launch_mr_lookup(const LookupArgs &a, hipStream_t s);
hipError_t launch_table_check(const uint64_t *rs, const uint64_t *re, uint32_t nregions,
                              uint32_t page_shift, uint64_t *scratch, uint64_t *host_result,
                              hipStream_t s);
hipError_t launch_build_prp(const PrpArgs &a, hipStream_t s);
hipError_t launch_partition(const SplitArgs &a, hipStream_t s);
// The split's column scan and scatter, with the per-tile counts (bucket
// major, a row of ceil(n / 2^split_tile_shift) tiles per bucket) already in
// the first part of a.ws.
hipError_t launch_partition_counted(const SplitArgs &a, hipStream_t s);
uint32_t split_tile_shift(uint32_t nq);
// The batch is one split tile ranked by the counter path: the split runs its
// one-tile kernel alone (no histogram, no column scan).
bool split_single(uint64_t n, uint32_t nq);
// The fused batch: lookup (lk.handle == nullptr: none), PRP build (a.packed
// selects the layout) and split; a.ws, sp.ws and index_ws are the three
// parts of the call's workspace.
hipError_t launch_build_batch(const LookupArgs &lk, const PrpArgs &a, const SplitArgs &sp,
                              void *index_ws, hipStream_t s);
size_t ws_batch_index(uint32_t nregions);
hipError_t launch_emit_sqe(const SqeArgs &a, hipStream_t s);
hipError_t launch_cq_mirror(dmadesc_cq_slot *slots, uint32_t nslots, const uint32_t *stop,
                            uint32_t idle_polls, hipStream_t s);
hipError_t launch_build_put(const PutArgs &a, hipStream_t s);
hipError_t launch_reg_register(const RegArgs &a, hipStream_t s);
hipError_t launch_reg_deregister(const RegArgs &a, hipStream_t s);

size_t ws_mr_lookup(uint32_t nregions);
size_t ws_build_prp(uint64_t n);
size_t ws_partition(uint64_t n, uint32_t nqueues);
size_t ws_emit_sqe(uint32_t nqueues);
size_t ws_build_put(uint64_t n);
size_t ws_registry(uint64_t n, uint64_t capacity);

// Device address and size of the allocation-free entry point's scratch on
// the current device (looked up on the first call on each device).
hipError_t noalloc_scratch(void **ptr, size_t *bytes);

// Polls a look-back wait may take before it gives up (process-wide; set by
// dmadesc_debug_wait_limit, default 2^22).
uint32_t wait_limit();

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace dd

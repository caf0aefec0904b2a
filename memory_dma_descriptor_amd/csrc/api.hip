// api.hip - the C ABI of libdmadesc: argument validation, workspace sizing
// and kernel launches. Every check here runs on the host before anything is
// launched, so a rejected call touches no memory and needs no GPU.
#include <errno.h>

#include <atomic>

#include "dd_internal.h"
#include "dmadesc.h"

namespace {

// Bound on the polls of one look-back wait (about seconds at the default).
std::atomic<uint32_t> g_wait_polls{DMADESC_DEFAULT_WAIT_POLLS};

constexpr uint64_t kMaxN = 1ull << 32;           // indices are u32
constexpr uint64_t kMaxLutEntries = 1ull << 48;  // heap < 2^64 bytes

int launched(hipError_t e) { return e == hipSuccess ? 0 : -EIO; }

// A workspace is present, at least `need` bytes and 256-byte aligned (the
// kernels keep 64-bit atomics and 16-byte columns in it).
bool ws_ok(const void *ws, size_t ws_bytes, size_t need)
{
    return ws && ws_bytes >= need && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0;
}

// Arguments of a PRP build (both layouts), checked on the host.
bool prp_args_ok(const uint64_t *lut, uint64_t lut_entries, const uint64_t *off,
                 const uint64_t *len, uint64_t n, uint64_t list_bus_base, uint64_t *list_pool,
                 uint64_t pool_pages, uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                 uint64_t *total_pages, bool packed)
{
    if (n >= kMaxN || lut_entries >= kMaxLutEntries) return false;
    if (list_bus_base & 4095u) return false;
    if (!total_pages) return false;
    if (lut_entries > 0 && !lut) return false;
    if (pool_pages > 0 && !list_pool) return false;
    if (reinterpret_cast<uintptr_t>(list_pool) & 15u) return false;   // 16-byte stores
    if (pool_pages > (~0ull >> 12)) return false;        // pool byte size fits 64 bits
    // The scan carries 62-bit counts: every request has at most 16 lut_entries
    // + 1 list entries, so n of them must stay below 2^62.
    if (packed && (unsigned __int128)(lut_entries * 16 + 2) * n >= ((unsigned __int128)1 << 62))
        return false;
    if (n > 0 && (!off || !len || !prp1 || !prp2 || !status)) return false;
    return true;
}

// The fused batch's workspace: the PRP slot scan, the split's counts and
// totals, and the lookup's bucket index, each 256-byte aligned.
size_t batch_ws(uint64_t n, uint32_t nqueues, uint32_t nregions, size_t *split_at,
                size_t *index_at)
{
    const size_t a = dd::align256(dd::ws_build_prp(n));
    const size_t b = dd::align256(dd::ws_partition(n, nqueues));
    if (split_at) *split_at = a;
    if (index_at) *index_at = a + b;
    return a + b + dd::ws_batch_index(nregions);
}

int build_prp_common(const uint64_t *lut, uint64_t lut_entries, const uint64_t *off,
                     const uint64_t *len, uint64_t n, uint64_t list_bus_base,
                     uint64_t *list_pool, uint64_t pool_pages, uint64_t *prp1, uint64_t *prp2,
                     uint8_t *status, uint64_t *total_pages, void *ws, size_t ws_bytes,
                     void *stream, bool packed)
{
    if (!prp_args_ok(lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages, prp1,
                     prp2, status, total_pages, packed))
        return -EINVAL;
    const size_t need = dd::ws_build_prp(n);
    if (need > 0 && !ws_ok(ws, ws_bytes, need)) return -EINVAL;
    dd::PrpArgs a{lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages,
                  prp1, prp2, status, total_pages, ws, packed};
    return launched(dd::launch_build_prp(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

namespace dd {
uint32_t wait_limit() { return g_wait_polls.load(std::memory_order_relaxed); }
}  // namespace dd

extern "C" {

int dmadesc_version(void) { return 1; }

uint32_t dmadesc_debug_wait_limit(uint32_t polls)
{
    return g_wait_polls.exchange(polls);
}

const char *dmadesc_strerror(int err)
{
    switch (err) {
    case 0: return "success";
    case -EINVAL: return "invalid argument (null pointer, size or parameter out of range, or workspace too small)";
    case -EIO: return "the HIP runtime refused a kernel launch";
    case -E2BIG: return "batch larger than the allocation-free entry point's scratch allows";
    default: return "unknown error";
    }
}

size_t dmadesc_workspace_bytes(int op, uint64_t n, uint32_t param)
{
    switch (op) {
    case DMADESC_OP_MR_LOOKUP: return dd::ws_mr_lookup(param);
    case DMADESC_OP_BUILD_PRP: return dd::ws_build_prp(n);
    case DMADESC_OP_PARTITION:
        if (param == 0 || param > DMADESC_MAX_QUEUES) return 0;
        return dd::ws_partition(n, param);
    case DMADESC_OP_EMIT_SQE:
        if (param == 0 || param > DMADESC_MAX_QUEUES) return 0;
        return dd::ws_emit_sqe(param);
    case DMADESC_OP_BUILD_PUT: return dd::ws_build_put(n);
    case DMADESC_OP_REGISTRY:
        if (n > DMADESC_REG_MAX_BATCH || param > DMADESC_REG_MAX_CAPACITY) return 0;
        return dd::ws_registry(n, param);
    default: return 0;
    }
}

int dmadesc_mr_lookup(const uint64_t *reg_start, const uint64_t *reg_end,
                      const uint32_t *reg_lkey, uint32_t nregions, uint32_t page_shift,
                      const uint64_t *off, const uint64_t *len, uint64_t n, uint64_t va_base,
                      int32_t *handle, uint32_t *lkey, uint8_t *kind,
                      uint64_t *rbase, uint64_t *rend,
                      void *ws, size_t ws_bytes, void *stream)
{
    if (page_shift < 12 || page_shift > 30) return -EINVAL;
    if (n >= kMaxN || nregions >= (1u << 31)) return -EINVAL;
    if (nregions > 0 && (!reg_start || !reg_end || !reg_lkey)) return -EINVAL;
    const size_t need = dd::ws_mr_lookup(nregions);
    if (ws && need > 0 && !ws_ok(ws, ws_bytes, need)) return -EINVAL;
    if (n == 0) return 0;
    if (!off || !len || !handle || !lkey || !kind || !rbase || !rend) return -EINVAL;
    dd::LookupArgs a{reg_start, reg_end, reg_lkey, nregions, page_shift, off, len, n, va_base,
                     handle, lkey, kind, rbase, rend};
    if (ws && need > 0) a.rec = static_cast<uint64_t *>(ws);
    return launched(dd::launch_mr_lookup(a, static_cast<hipStream_t>(stream)));
}

int dmadesc_mr_table_check(const uint64_t *reg_start, const uint64_t *reg_end,
                           uint32_t nregions, uint32_t page_shift, uint64_t *scratch,
                           uint64_t *first_bad, void *stream)
{
    if (first_bad) *first_bad = ~0ull;
    if (page_shift < 12 || page_shift > 30 || nregions >= (1u << 31) || !scratch) return -EINVAL;
    if (reinterpret_cast<uintptr_t>(scratch) & 7u) return -EINVAL;
    if (nregions > 0 && (!reg_start || !reg_end)) return -EINVAL;
    uint64_t bad = ~0ull;
    if (dd::launch_table_check(reg_start, reg_end, nregions, page_shift, scratch, &bad,
                               static_cast<hipStream_t>(stream)) != hipSuccess)
        return -EIO;
    if (first_bad) *first_bad = bad;
    return bad == ~0ull ? 0 : -EINVAL;
}

int dmadesc_build_prp(const uint64_t *lut, uint64_t lut_entries,
                      const uint64_t *off, const uint64_t *len, uint64_t n,
                      uint64_t list_bus_base, uint64_t *list_pool, uint64_t pool_pages,
                      uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                      uint64_t *total_pages,
                      void *ws, size_t ws_bytes, void *stream)
{
    return build_prp_common(lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages,
                            prp1, prp2, status, total_pages, ws, ws_bytes, stream, false);
}

int dmadesc_build_prp_packed(const uint64_t *lut, uint64_t lut_entries,
                             const uint64_t *off, const uint64_t *len, uint64_t n,
                             uint64_t list_bus_base, uint64_t *list_pool, uint64_t pool_pages,
                             uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                             uint64_t *total_pages,
                             void *ws, size_t ws_bytes, void *stream)
{
    return build_prp_common(lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages,
                            prp1, prp2, status, total_pages, ws, ws_bytes, stream, true);
}

size_t dmadesc_batch_workspace_bytes(uint64_t n, uint32_t nqueues, uint32_t nregions)
{
    if (nqueues == 0 || nqueues > DMADESC_MAX_QUEUES || n >= kMaxN || nregions >= (1u << 31))
        return 0;
    return batch_ws(n, nqueues, nregions, nullptr, nullptr);
}

int dmadesc_build_batch(const uint64_t *reg_start, const uint64_t *reg_end,
                        const uint32_t *reg_lkey, uint32_t nregions, uint32_t page_shift,
                        uint64_t va_base, const uint64_t *lut, uint64_t lut_entries,
                        const uint64_t *off, const uint64_t *len, const uint32_t *qid,
                        uint64_t n, uint32_t nqueues, uint64_t list_bus_base,
                        uint64_t *list_pool, uint64_t pool_pages, uint32_t flags,
                        int32_t *handle, uint32_t *lkey, uint8_t *kind, uint64_t *rbase,
                        uint64_t *rend, uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                        uint64_t *total_pages, uint32_t *perm, uint64_t *qoff,
                        uint64_t *n_invalid, void *ws, size_t ws_bytes, void *stream)
{
    if (flags & ~(uint32_t)DMADESC_BATCH_PACKED) return -EINVAL;
    const bool packed = (flags & DMADESC_BATCH_PACKED) != 0;
    if (!prp_args_ok(lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages, prp1,
                     prp2, status, total_pages, packed))
        return -EINVAL;
    if (nqueues == 0 || nqueues > DMADESC_MAX_QUEUES || !qoff || !n_invalid) return -EINVAL;
    if (n > 0 && (!qid || !perm)) return -EINVAL;
    // The lookup columns come all or none (none: the batch has no region table).
    const int given = !!handle + !!lkey + !!kind + !!rbase + !!rend;
    if (given != 0 && given != 5) return -EINVAL;
    const bool lookup = given == 5;
    if (lookup) {
        if (page_shift < 12 || page_shift > 30 || nregions >= (1u << 31)) return -EINVAL;
        if (nregions > 0 && (!reg_start || !reg_end || !reg_lkey)) return -EINVAL;
    }
    const uint32_t nreg = lookup ? nregions : 0;
    size_t split_at = 0, index_at = 0;
    const size_t need = batch_ws(n, nqueues, nreg, &split_at, &index_at);
    if (!ws_ok(ws, ws_bytes, need)) return -EINVAL;
    char *w = static_cast<char *>(ws);
    dd::LookupArgs lk{reg_start, reg_end, reg_lkey, nreg, page_shift, off, len, n, va_base,
                      lookup ? handle : nullptr, lkey, kind, rbase, rend};
    dd::PrpArgs a{lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages,
                  prp1, prp2, status, total_pages, ws, packed};
    dd::SplitArgs sp{qid, n, nqueues, perm, qoff, n_invalid, w + split_at};
    return launched(dd::launch_build_batch(lk, a, sp, w + index_at,
                                           static_cast<hipStream_t>(stream)));
}

int dmadesc_build_prp_packed_noalloc(const uint64_t *lut, uint64_t lut_entries,
                                     const uint64_t *off, const uint64_t *len, uint64_t n,
                                     uint64_t list_bus_base, uint64_t *list_pool,
                                     uint64_t pool_pages, uint64_t *prp1, uint64_t *prp2,
                                     uint8_t *status, uint64_t *total_pages, void *stream)
{
    if (n > DMADESC_NOALLOC_MAX_N) return -E2BIG;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (dd::noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return -EIO;
    return build_prp_common(lut, lut_entries, off, len, n, list_bus_base, list_pool, pool_pages,
                            prp1, prp2, status, total_pages, ws, ws_bytes, stream, true);
}

int dmadesc_partition_by_queue(const uint32_t *qid, uint64_t n, uint32_t nqueues,
                               uint32_t *perm, uint64_t *qoff, uint64_t *n_invalid,
                               void *ws, size_t ws_bytes, void *stream)
{
    if (nqueues == 0 || nqueues > DMADESC_MAX_QUEUES) return -EINVAL;
    if (n >= kMaxN) return -EINVAL;
    if (!qoff || !n_invalid) return -EINVAL;
    if (n > 0 && (!qid || !perm)) return -EINVAL;
    const size_t need = dd::ws_partition(n, nqueues);
    if (n > 0 && !ws_ok(ws, ws_bytes, need)) return -EINVAL;
    dd::SplitArgs a{qid, n, nqueues, perm, qoff, n_invalid, ws};
    return launched(dd::launch_partition(a, static_cast<hipStream_t>(stream)));
}

int dmadesc_emit_sqe(const uint32_t *perm, const uint64_t *qoff, uint32_t nqueues,
                     const uint8_t *status, const uint64_t *len, const uint64_t *slba,
                     const uint64_t *prp1, const uint64_t *prp2, uint64_t n,
                     uint32_t opcode, uint32_t nsid, uint32_t lba_shift,
                     const uint64_t *ring, const uint32_t *depth, const uint32_t *free_slots,
                     uint32_t *tail, uint64_t *cursor, uint32_t *placed,
                     uint32_t *req_of_slot, void *ws, size_t ws_bytes, void *stream)
{
    if (nqueues == 0 || nqueues > DMADESC_MAX_QUEUES) return -EINVAL;
    if (n >= kMaxN || opcode > 0xFFu || lba_shift < 9 || lba_shift > 16) return -EINVAL;
    if (!qoff || !ring || !depth || !free_slots || !tail || !cursor || !placed) return -EINVAL;
    if (n > 0 && (!perm || !status || !len || !slba || !prp1 || !prp2)) return -EINVAL;
    const size_t need = dd::ws_emit_sqe(nqueues);
    if (!ws_ok(ws, ws_bytes, need)) return -EINVAL;
    dd::SqeArgs a{perm, qoff, nqueues, status, len, slba, prp1, prp2, n, opcode, nsid, lba_shift,
                  ring, depth, free_slots, tail, cursor, placed, req_of_slot, ws};
    return launched(dd::launch_emit_sqe(a, static_cast<hipStream_t>(stream)));
}

int dmadesc_build_put(const uint64_t *src, const uint64_t *dst, const uint64_t *bytes,
                      const uint32_t *pe, uint64_t n, uint64_t local_base, uint64_t heap_bytes,
                      uint32_t chunk_shift, const uint32_t *lkeys, const uint64_t *peer_base,
                      const uint32_t *rkeys, uint32_t npes, dmadesc_put_desc *desc,
                      uint64_t desc_cap, uint64_t *first, uint32_t *count, uint8_t *status,
                      uint64_t *total, void *ws, size_t ws_bytes, void *stream)
{
    if (n >= kMaxN || npes == 0 || npes > 65536) return -EINVAL;
    if (chunk_shift != 0 && (chunk_shift < 12 || chunk_shift > 31)) return -EINVAL;
    if (chunk_shift != 0 &&
        ((heap_bytes & ((1ull << chunk_shift) - 1)) || (heap_bytes >> chunk_shift) >= (1ull << 30)))
        return -EINVAL;
    if (!lkeys || !peer_base || !rkeys || !total) return -EINVAL;
    if (desc_cap > 0 && !desc) return -EINVAL;
    if (reinterpret_cast<uintptr_t>(desc) & 15u) return -EINVAL;
    if (desc_cap > (~0ull >> 5)) return -EINVAL;                 // byte size fits 64 bits
    const unsigned __int128 most = chunk_shift ? 2 * (heap_bytes >> chunk_shift) + 1
                                               : (heap_bytes >> 31) + 1;
    if (most * n >= ((unsigned __int128)1 << 62)) return -EINVAL;
    if (n > 0 && (!src || !dst || !bytes || !pe || !first || !count || !status)) return -EINVAL;
    const size_t need = dd::ws_build_put(n);
    if (need > 0 && !ws_ok(ws, ws_bytes, need)) return -EINVAL;
    dd::PutArgs a{src, dst, bytes, pe, n, local_base, heap_bytes, chunk_shift, npes, lkeys,
                  peer_base, rkeys, reinterpret_cast<uint64_t *>(desc), desc_cap, first, count,
                  status, total, ws};
    return launched(dd::launch_build_put(a, static_cast<hipStream_t>(stream)));
}

int dmadesc_cq_mirror(dmadesc_cq_slot *slots, uint32_t nslots, const uint32_t *stop,
                      uint32_t idle_polls, void *stream)
{
    if (!slots || !stop || nslots == 0 || nslots > DMADESC_CQ_MAX_SLOTS) return -EINVAL;
    if (idle_polls == 0 || idle_polls > (1u << 24)) return -EINVAL;
    if (reinterpret_cast<uintptr_t>(slots) & 7u) return -EINVAL;
    return launched(dd::launch_cq_mirror(slots, nslots, stop, idle_polls,
                                         static_cast<hipStream_t>(stream)));
}

int dmadesc_reg_register(uint64_t *start, uint64_t *end, uint64_t *id, uint32_t *refs,
                         uint32_t *by_start, uint64_t *state, uint64_t capacity,
                         uint32_t page_shift, const uint64_t *addr, const uint64_t *size,
                         uint64_t n, uint64_t *handle, uint8_t *kind, uint64_t *needed,
                         void *ws, size_t ws_bytes, void *stream)
{
    if (page_shift < 12 || page_shift > 30) return -EINVAL;
    if (n > DMADESC_REG_MAX_BATCH || capacity > DMADESC_REG_MAX_CAPACITY) return -EINVAL;
    if (!state || !needed) return -EINVAL;
    if (capacity > 0 && (!start || !end || !id || !refs || !by_start)) return -EINVAL;
    if (n > 0 && (!addr || !size || !handle || !kind)) return -EINVAL;
    if (!ws_ok(ws, ws_bytes, dd::ws_registry(n, capacity))) return -EINVAL;
    dd::RegArgs a{start, end, id, refs, by_start, state, capacity, page_shift, addr, size,
                  nullptr, n, handle, kind, needed, nullptr, ws};
    return launched(dd::launch_reg_register(a, static_cast<hipStream_t>(stream)));
}

int dmadesc_reg_deregister(uint64_t *start, uint64_t *end, uint64_t *id, uint32_t *refs,
                           uint32_t *by_start, uint64_t *state, uint64_t capacity,
                           const uint64_t *handle, uint64_t n, uint8_t *status,
                           void *ws, size_t ws_bytes, void *stream)
{
    if (n > DMADESC_REG_MAX_BATCH || capacity > DMADESC_REG_MAX_CAPACITY) return -EINVAL;
    if (!state) return -EINVAL;
    if (capacity > 0 && (!start || !end || !id || !refs || !by_start)) return -EINVAL;
    if (n > 0 && (!handle || !status)) return -EINVAL;
    if (!ws_ok(ws, ws_bytes, dd::ws_registry(n, capacity))) return -EINVAL;
    dd::RegArgs a{start, end, id, refs, by_start, state, capacity, 12, nullptr, nullptr,
                  handle, n, nullptr, nullptr, nullptr, status, ws};
    return launched(dd::launch_reg_deregister(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

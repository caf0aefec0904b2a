/*
 * oracle.h - plain, single-threaded CPU reference for batched DMA-descriptor
 * building.
 *
 * TEST INFRASTRUCTURE ONLY. This is the checker the GPU library is compared
 * against; it is not part of the product. Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it. It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [NCCL-26]  "NCCL 专家课程 26：GPUDirect RDMA、DMA-BUF、MR 与注册缓存"
 *              (blog.cptz.space), sections "IB Backend MR Cache",
 *              "Communicator User Registration Cache" and
 *              "真实 ncclCommRegister 语义实验".
 *   [UPCIE]    xNVMe "uPCIe CUDA" backend (xnvme.io), introduction,
 *              "Memory Architecture", "Completions in device memory" and
 *              "Limitations".
 *   [MORI]     "mori通信库分析(一)——对称内存RDMA数据发送过程", the
 *              thread-scope put kernel and the warp-level WQE reservation.
 *   [NVMe]     NVM Express Base Specification, PRP entry / PRP list rules
 *              (not on the pages; used where they stop).
 *
 * Every function computes one fully determined result; see oracle.c for the
 * step-by-step definitions and the readings taken where the pages are silent.
 */
#ifndef DMADESC_ORACLE_H
#define DMADESC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Lookup outcome per request. */
enum { ORC_MISS = 0, ORC_EXACT = 1, ORC_CONTAINED = 2, ORC_INVALID = 3 };

/* PRP build status per request. */
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ERANGE = 2, ORC_ENOSPC = 3 };

/*
 * O1: page-rounded containment lookup of each request range in a sorted,
 * non-overlapping region table [start[r], end[r]).
 * Outputs per request: handle (region index, -1 on miss/invalid), lkey
 * (0 on miss/invalid), kind, rounded base and rounded end (0/0 on invalid).
 */
void orc_mr_lookup(const uint64_t *start, const uint64_t *end, const uint32_t *lkey,
                   uint64_t nregions, unsigned page_shift,
                   const uint64_t *off, const uint64_t *len, uint64_t n, uint64_t va_base,
                   int32_t *handle, uint32_t *lkey_out, uint8_t *kind,
                   uint64_t *rbase, uint64_t *rend);

/*
 * O2: 64 KiB GPU-page table -> 4 KiB NVMe PRP1/PRP2 and chained PRP lists.
 * pool (may be NULL: lists are then not written) is u64[pool_pages][512];
 * list page s has bus address list_bus_base + 4096*s. *total receives the
 * number of list pages the batch needs (including those refused with ENOSPC).
 */
void orc_build_prp(const uint64_t *lut, uint64_t lut_entries,
                   const uint64_t *off, const uint64_t *len, uint64_t n,
                   uint64_t list_bus_base, uint64_t *pool, uint64_t pool_pages,
                   uint64_t *prp1, uint64_t *prp2, uint8_t *status, uint64_t *total);

/*
 * O2p: the same PRP entries with the lists packed back to back. List entries
 * are numbered by data slots: request i with m = pages - 1 >= 2 entries takes
 * slots [D, D + m), D = running count of earlier requests' entries (refused
 * ones included). A pool page holds data slots 511 p .. 511 p + 510 in words
 * 0..510; slot d lies in word d + floor(d / 511). PRP2 = list_bus_base +
 * 8 * word(D). Word 511 of a page is set by the request owning the page's
 * last data slot: a pointer to the next page if two or more of its entries
 * remain, its final entry if exactly one remains (the next page's word 0 is
 * then 0), and 0 if its list ended in word 510. ENOSPC when D + m >
 * 511 * pool_pages. *total = ceil(all entries / 511) pages.
 */
void orc_build_prp_packed(const uint64_t *lut, uint64_t lut_entries,
                          const uint64_t *off, const uint64_t *len, uint64_t n,
                          uint64_t list_bus_base, uint64_t *pool, uint64_t pool_pages,
                          uint64_t *prp1, uint64_t *prp2, uint8_t *status, uint64_t *total);

/*
 * O3: stable split of request indices by queue id. Queue ids >= nqueues go to
 * an overflow bucket nqueues. qoff has nqueues+2 entries: bucket b occupies
 * perm[qoff[b] .. qoff[b+1]). *n_invalid = size of the overflow bucket.
 */
void orc_partition(const uint32_t *qid, uint64_t n, uint32_t nqueues,
                   uint32_t *perm, uint64_t *qoff, uint64_t *n_invalid);

/*
 * O5: NVMe submission entries per queue, one window of the split per call.
 * Inputs are the split of O3 (perm, qoff with nqueues+2 entries) and, per
 * request, the PRP status, length, starting LBA and PRP1/PRP2 of O2.
 * Queue q is refused (nothing consumed or placed) when ring[q] is NULL,
 * depth[q] is outside [2, 65536] or tail[q] >= depth[q]. Otherwise the call
 * consumes the next W = min(free_slots[q], depth[q] - 1, left) entries of
 * bucket q, starting after the cursor[q] entries consumed by earlier calls
 * (left = bucket size - cursor[q], or 0). In bucket order, each consumed
 * request that is placeable (status OK; length a positive multiple of
 * 2^lba_shift of at most 65536 blocks) takes ring slot (tail[q] + k) % depth[q]
 * for k = 0, 1, ... and gets a 64-byte entry there, and
 * req_of_slot[q * 65536 + slot] (if req_of_slot is not NULL) receives its
 * request index. Afterwards placed[q] = k, tail[q] = (tail[q] + k) % depth[q]
 * and cursor[q] += W. ring[q] is u8[depth[q]][64].
 */
void orc_emit_sqe(const uint32_t *perm, const uint64_t *qoff, uint32_t nqueues,
                  const uint8_t *status, const uint64_t *len, const uint64_t *slba,
                  const uint64_t *prp1, const uint64_t *prp2, uint64_t n,
                  uint8_t opcode, uint32_t nsid, unsigned lba_shift,
                  uint8_t *const *ring, const uint32_t *depth, const uint32_t *free_slots,
                  uint32_t *tail, uint64_t *cursor, uint32_t *placed, uint32_t *req_of_slot);

/*
 * O6: RDMA put descriptors for a symmetric heap, static or VMM.
 * Request i moves bytes[i] from heap offset src[i] to heap offset dst[i] of
 * PE pe[i]. chunk_shift == 0: static heap, one local key lkeys[0] and one
 * remote key rkeys[pe] per PE. Otherwise the heap is chunks of 2^chunk_shift
 * bytes (nchunks = heap_bytes >> chunk_shift), chunk k has local key lkeys[k]
 * and, on PE q, remote key rkeys[q * nchunks + k]. Each request is cut into
 * pieces: transfer = min(bytes left in the source chunk, bytes left in the
 * destination chunk, remaining, 2^31); each piece is a descriptor
 * {laddr = local_base + src + x, raddr = peer_base[pe] + dst + x, len, lkey,
 * rkey, req = i}. Descriptors of request i are desc[first[i] .. first[i] +
 * count[i]), first = running count over requests (refused ones included).
 * Status: EINVAL (zero bytes, pe >= npes), ERANGE (past the heap), ENOSPC
 * (first + count > desc_cap). *total = descriptors the batch needs.
 */
typedef struct {
    uint64_t laddr, raddr;
    uint32_t len, lkey, rkey, req;
} orc_put_desc;
void orc_build_put(const uint64_t *src, const uint64_t *dst, const uint64_t *bytes,
                   const uint32_t *pe, uint64_t n, uint64_t local_base, uint64_t heap_bytes,
                   unsigned chunk_shift, const uint32_t *lkeys, const uint64_t *peer_base,
                   const uint32_t *rkeys, uint32_t npes, orc_put_desc *desc, uint64_t desc_cap,
                   uint64_t *first, uint32_t *count, uint8_t *status, uint64_t *total);

/*
 * O7: one drain of a completion-queue mirror slot. src and dst are
 * u32[depth][4] (16-byte NVMe completion entries; the phase tag is bit 16 of
 * dword 3). If *gen is odd, entries are copied from src to dst starting at
 * *head while their phase equals *phase; *head advances (mod depth) and
 * *phase flips each time *head wraps to 0. If *gen is even, nothing is copied
 * and *ack becomes *gen - 1 (a queue detached before it was drained). Returns
 * the number of entries copied.
 */
uint64_t orc_cq_drain(const uint32_t *src, uint32_t *dst, uint32_t depth, uint32_t gen,
                      uint32_t *head, uint32_t *phase, uint32_t *ack);

/*
 * O4: host registration cache with reference counts ([NCCL-26]).
 * Handles are positive record ids, never reused; 0 is never a handle.
 */
typedef struct orc_registry orc_registry;
orc_registry *orc_reg_create(unsigned page_shift);
void orc_reg_destroy(orc_registry *g);
/* Returns the handle (> 0), or 0 for a zero-length or wrapping range. */
uint64_t orc_reg_register(orc_registry *g, uint64_t addr, uint64_t size);
/* Returns 0 on success, -1 for a handle that names no live record. */
int orc_reg_deregister(orc_registry *g, uint64_t handle);
/* Reference count of a live record, or -1. */
int64_t orc_reg_refs(const orc_registry *g, uint64_t handle);
uint64_t orc_reg_count(const orc_registry *g);
uint64_t orc_reg_capacity(const orc_registry *g);
/* Copies the live records in sorted order (start, end, handle); returns count. */
uint64_t orc_reg_export(const orc_registry *g, uint64_t *start, uint64_t *end,
                        uint64_t *handle, uint64_t max);

/*
 * O4b: batches for the registry, each item applied in order as O4 does,
 * against a caller capacity for the record table.
 * register: kind[i] = INVALID (handle 0: zero length or wrap), HIT (a record
 * that existed before the batch contains the range), NEW (this item inserted
 * a record), HIT_NEW (a record inserted earlier in the same batch contains it).
 * If the record count after the batch would exceed `capacity`, nothing is
 * applied, every kind is NOSPACE and every handle 0. Returns the capacity the
 * batch needs: `capacity` itself if it fits, else the capacity grown by O4's
 * rule (0 -> 32, then doubling) until the count fits.
 * deregister: status[i] = OK (count dropped), REMOVED (dropped to zero, record
 * freed) or STALE (no live record has that handle).
 */
enum { ORC_REG_INVALID = 0, ORC_REG_HIT = 1, ORC_REG_NEW = 2, ORC_REG_HIT_NEW = 3,
       ORC_REG_NOSPACE = 4 };
enum { ORC_DEREG_OK = 0, ORC_DEREG_REMOVED = 1, ORC_DEREG_STALE = 2 };
uint64_t orc_reg_next_id(const orc_registry *g);
uint64_t orc_reg_register_batch(orc_registry *g, uint64_t capacity,
                                const uint64_t *addr, const uint64_t *size, uint64_t n,
                                uint64_t *handle, uint8_t *kind);
void orc_reg_deregister_batch(orc_registry *g, const uint64_t *handle, uint64_t n,
                              uint8_t *status);

#ifdef __cplusplus
}
#endif

#endif /* DMADESC_ORACLE_H */

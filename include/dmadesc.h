/*
 * dmadesc.h - batched DMA-descriptor building on AMD Instinct MI355X (gfx950).
 *
 * Three data-parallel operations turn a batch of I/O requests against GPU
 * device memory into DMA descriptors:
 *
 *   dmadesc_mr_lookup          page-rounded containment lookup of each request
 *                              range in a table of registered memory regions
 *   dmadesc_build_prp          64 KiB GPU-page physical-address table -> 4 KiB
 *                              NVMe PRP1/PRP2 and chained PRP lists
 *   dmadesc_build_prp_packed   the same entries with the lists packed back to
 *                              back (qword-offset list pointers)
 *   dmadesc_partition_by_queue stable split of the requests by destination queue
 *   dmadesc_build_batch        all three in one call (one read of the requests)
 *
 * and one stage after them:
 *
 *   dmadesc_emit_sqe           64-byte NVMe submission entries in per-queue
 *                              rings, one window of the split per call
 *
 * a put-descriptor build for a symmetric heap:
 *
 *   dmadesc_build_put          RDMA put descriptors, one per chunk-bounded piece
 *                              (static heap or VMM heap with per-chunk keys)
 *
 * the completion side:
 *
 *   dmadesc_cq_mirror          copy NVMe completions from device-memory
 *                              completion queues to mirror queues as their
 *                              phase bit turns (one wave per queue)
 *
 * and the registration cache kept on the device:
 *
 *   dmadesc_reg_register       batch of registrations (page-rounded, refcounted)
 *   dmadesc_reg_deregister     batch of deregistrations
 *
 * Sources (web pages, cited by title and section):
 *   [NCCL-26] "NCCL 专家课程 26：GPUDirect RDMA、DMA-BUF、MR 与注册缓存",
 *             sections "IB Backend MR Cache" and
 *             "Communicator User Registration Cache".
 *   [UPCIE]   xNVMe "uPCIe CUDA" backend: introduction, "Memory Architecture",
 *             "Completions in device memory",
 *             "Choosing the GPU and Heap Sizes", "GPU-Resident Queue API",
 *             "Limitations".
 *   [MORI]    "mori通信库分析(一)——对称内存RDMA数据发送过程": the thread-scope
 *             put kernel (ballot / find-first-set / shuffle grouping of lanes by
 *             destination) and the warp-level WQE slot reservation.
 *   [CUFRAMES] "Синхронизация: stream sync, не CUDA events": data written on a
 *             stream is visible to others once that stream is synchronized.
 *   [NVMe]    NVM Express Base Specification: PRP rules, the common command
 *             format of a submission entry, queue sizes (not on the pages).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is caller-owned DEVICE memory on the current HIP
 *    device unless marked "host". The library allocates nothing, keeps no
 *    state between calls (apart from the test bound set by
 *    dmadesc_debug_wait_limit and the static per-device scratch of
 *    dmadesc_build_prp_packed_noalloc) and retains no pointer after
 *    returning.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    device's null stream). Outputs are valid once the caller synchronizes
 *    that stream or orders later work behind it on the same stream
 *    ([CUFRAMES]). Calls on distinct streams with distinct buffers may run
 *    concurrently; calls that share a workspace must be ordered.
 *  - Return value: 0 on success, or a negative errno value. On error nothing
 *    is launched and no output is touched:
 *      -EINVAL  null pointer where one is required, n >= 2^32, a parameter
 *               out of range (stated per call), workspace too small or not
 *               256-byte aligned;
 *      -EIO     the HIP runtime refused a kernel launch;
 *      -E2BIG   (dmadesc_build_prp_packed_noalloc only) a batch larger than
 *               its static scratch allows.
 *    Errors in individual requests are not call errors: they are reported
 *    per request in an output column (stated per call).
 *  - All arithmetic is exact unsigned 64-bit integer arithmetic; outputs are
 *    bit-for-bit deterministic (no atomics decide any output position).
 *  - `ws` is a caller-owned device workspace of at least
 *    dmadesc_workspace_bytes(op, n, param) bytes, 256-byte aligned (-EINVAL
 *    otherwise). Its contents on entry are ignored and on return are
 *    unspecified.
 */
#ifndef DMADESC_H
#define DMADESC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Lookup outcome per request (column `kind` of dmadesc_mr_lookup). */
enum dmadesc_kind {
    DMADESC_MISS = 0,      /* no region contains the rounded range               */
    DMADESC_EXACT = 1,     /* the rounded range equals a region                  */
    DMADESC_CONTAINED = 2, /* the rounded range lies inside a region             */
    DMADESC_INVALID = 3    /* zero length, or the range / rounded end wraps 2^64 */
};

/* PRP build status per request (column `status` of dmadesc_build_prp). */
enum dmadesc_prp_status {
    DMADESC_PRP_OK = 0,
    DMADESC_PRP_EINVAL = 1, /* len == 0, off not a multiple of 4, or off+len wraps */
    DMADESC_PRP_ERANGE = 2, /* off + len > lut_entries * 64 KiB (past the heap)     */
    DMADESC_PRP_ENOSPC = 3, /* the request's list pages pass pool_pages            */
    DMADESC_PRP_EBUSY = 4   /* the slot scan of the request's block did not finish:
                               a bounded wait expired (see dmadesc_debug_wait_limit);
                               nothing was written for the request              */
};

/* Default bound on the polls of one wait of the device-wide slot scan (the
 * decoupled look-back of dmadesc_build_prp, dmadesc_build_prp_packed and
 * dmadesc_build_put); a poll sleeps about 0.1 us, so the default is seconds. */
#define DMADESC_DEFAULT_WAIT_POLLS (1u << 22)

/* Operation codes for dmadesc_workspace_bytes. */
enum dmadesc_op {
    DMADESC_OP_MR_LOOKUP = 1,
    DMADESC_OP_BUILD_PRP = 2,
    DMADESC_OP_PARTITION = 3,
    DMADESC_OP_EMIT_SQE = 4,
    DMADESC_OP_REGISTRY = 5,
    DMADESC_OP_BUILD_PUT = 6
};

/* Largest nqueues dmadesc_partition_by_queue and dmadesc_emit_sqe accept. */
#define DMADESC_MAX_QUEUES 256u

/* Deepest submission ring (NVMe queue size limit); also the row stride of
 * dmadesc_emit_sqe's req_of_slot. */
#define DMADESC_SQ_MAX_DEPTH 65536u

/*
 * dmadesc_mr_lookup - page-rounded containment lookup.
 *
 * Defined by [NCCL-26] "IB Backend MR Cache": a range is widened to whole
 * pages (base = address with the in-page bits cleared; page count =
 * (address + size - base + page - 1) / page) and a registered region that
 * fully contains the widened range is a hit; a partial overlap is a miss.
 * "Communicator User Registration Cache" applies the same floor/cover
 * rounding before its containment test; exact and contained ranges reuse the
 * region's handle.
 *
 * Region table (device arrays, `nregions` entries, nregions < 2^31): sorted
 * by start, non-overlapping (end[r] <= start[r+1]), start[r] < end[r]; end is
 * exclusive. Abutting regions are allowed. A table that breaks these rules
 * gives unspecified (but memory-safe) results; dmadesc_mr_table_check tells
 * the two apart.
 *   reg_start  u64[nregions]   region start address
 *   reg_end    u64[nregions]   region end address (exclusive)
 *   reg_lkey   u32[nregions]   local key returned on a hit
 * Requests: absolute address a = va_base + off[i], length len[i].
 *   page_shift  log2 of the page size, 12..30 (12 = 4 KiB), else -EINVAL
 * Outputs (u = per request, n entries each):
 *   handle  i32  region index on a hit, -1 on MISS / INVALID
 *   lkey    u32  reg_lkey[handle] on a hit, 0 otherwise
 *   kind    u8   enum dmadesc_kind; EXACT iff both rounded bounds equal the
 *                region's bounds
 *   rbase   u64  rounded base (0 when INVALID)
 *   rend    u64  rounded end, exclusive (0 when INVALID)
 * Workspace (optional): for tables of more than 4,096 regions,
 *   dmadesc_workspace_bytes(DMADESC_OP_MR_LOOKUP, n, nregions) bytes
 *   (64 per run of 4 regions, 256-byte aligned) let the call copy the table
 *   into one record per run and answer each request from one cache line of
 *   it; the call overwrites the workspace. ws NULL takes the path without
 *   records (same results, slower on large tables); a workspace given too
 *   small or misaligned is -EINVAL. Smaller tables need none (0 bytes).
 */
int dmadesc_mr_lookup(const uint64_t *reg_start, const uint64_t *reg_end,
                      const uint32_t *reg_lkey, uint32_t nregions, uint32_t page_shift,
                      const uint64_t *off, const uint64_t *len, uint64_t n, uint64_t va_base,
                      int32_t *handle, uint32_t *lkey, uint8_t *kind,
                      uint64_t *rbase, uint64_t *rend,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * dmadesc_mr_table_check - validation of a region table (the debug mode of
 * dmadesc_mr_lookup).
 *
 * [NCCL-26] "IB Backend MR Cache" lets overlapping records stand side by side
 * after partial-overlap registrations, which leaves the containing record of
 * a range ambiguous; the lookup therefore takes sorted, non-overlapping,
 * page-aligned tables only. This call checks a table on the device: region r
 * is at fault when start[r] >= end[r], a bound is not a multiple of
 * 2^page_shift, or end[r] > start[r+1].
 *   scratch     device u64 the check writes (8-byte aligned)
 *   first_bad   host u64 or NULL: the smallest faulty index, UINT64_MAX when
 *               there is none
 * Returns 0 for a valid table, -EINVAL for a faulty one (or for bad
 * arguments: page_shift outside 12..30, nregions >= 2^31, null or unaligned
 * scratch, null arrays with nregions > 0), -EIO if the runtime fails. Unlike
 * every other call it synchronizes `stream` before it returns.
 */
int dmadesc_mr_table_check(const uint64_t *reg_start, const uint64_t *reg_end,
                           uint32_t nregions, uint32_t page_shift, uint64_t *scratch,
                           uint64_t *first_bad, void *stream);

/*
 * dmadesc_build_prp - GPU-page table -> NVMe PRP1/PRP2 and chained PRP lists.
 *
 * Defined by [UPCIE] introduction: one physical address per 64 KiB GPU page,
 * and PRP entries at 4 KiB granularity from the sub-page offsets inside each
 * 64 KiB entry; "Limitations": a list page holds 512 entries. Chaining follows
 * [NVMe]: the last entry of every non-final list page points to the next one.
 *
 *   lut          u64[lut_entries]  physical address of GPU page k (heap bytes
 *                [k*64 KiB, (k+1)*64 KiB)); lut_entries < 2^48, else -EINVAL.
 *                The physical address of heap byte x is lut[x>>16] + (x&0xFFFF).
 *   off, len     u64[n]            request heap offset and length in bytes
 *   list_bus_base                  bus address of list page 0; must be a
 *                                  multiple of 4096, else -EINVAL
 *   list_pool    u64[pool_pages][512], 16-byte aligned (else -EINVAL): list
 *                                  pages; page s has bus address
 *                                  list_bus_base + 4096*s. Entries the batch
 *                                  needs are written; after a request's last
 *                                  entry, words up to the next multiple of 8
 *                                  words of its final list page may be
 *                                  written (with 0; a controller never reads
 *                                  them); every other word, and every page
 *                                  >= *total_pages, is left untouched.
 *   prp1, prp2   u64[n]            PRP1: physical address of the first byte.
 *                                  PRP2: 0 for one 4 KiB page, the second
 *                                  page's address for two, else the bus
 *                                  address of the request's first list page.
 *   status       u8[n]             enum dmadesc_prp_status; any non-OK request
 *                                  gets prp1 = prp2 = 0 and no list entries.
 *   total_pages  u64 (device scalar) list pages the whole batch needs: the
 *                                  sum over requests not EINVAL/ERANGE. List
 *                                  pages are handed out in request order, so
 *                                  ENOSPC requests form a suffix of the
 *                                  list-using requests and a pool of
 *                                  *total_pages pages serves them all.
 * Per request, with pages p = ((off & 4095) + len + 4095) >> 12, entries
 * m = p - 1 and, for p >= 3, list pages L = ceil((m - 1) / 511).
 * Slot scan: list pages are handed out by a one-pass device-wide scan over
 * blocks of 1,024 requests (256 for batches of at most 2^16 requests, 512
 * for more than 2^16 and at most 2^19, 2,048 for more than 2^19 and at most
 * 2^22) whose waits are bounded. A block whose wait
 * expires (never at the default bound while blocks make progress) refuses
 * its list requests with DMADESC_PRP_EBUSY (prp1 = prp2 = 0, no list
 * entries); every other request is built exactly as above, and if the
 * batch's last block expired *total_pages is UINT64_MAX.
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_BUILD_PRP, n, 0); its
 * first 8 bytes hold, on return, a block counter (u32) and the count of
 * blocks whose wait expired (u32; read it after synchronizing: nonzero
 * means some requests carry DMADESC_PRP_EBUSY).
 */
int dmadesc_build_prp(const uint64_t *lut, uint64_t lut_entries,
                      const uint64_t *off, const uint64_t *len, uint64_t n,
                      uint64_t list_bus_base, uint64_t *list_pool, uint64_t pool_pages,
                      uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                      uint64_t *total_pages,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * dmadesc_build_prp_packed - dmadesc_build_prp with packed PRP lists.
 *
 * [NVMe] (not on the pages) lets the PRP list pointer carried in a command
 * (PRP2) name any qword of a page; the list then runs to the end of that page
 * and, when more than one entry is still needed there, the page's last entry
 * points to the start of the next list page. Lists are therefore laid back to
 * back: the pool is a run of list pages of 511 data slots each (words
 * 0..510); request i with m = pages - 1 >= 2 list entries takes data slots
 * [D, D + m), where D is the sum of m over all earlier list requests
 * (refused ones included), and slot d lies in pool word d + floor(d / 511).
 * Everything else is as in dmadesc_build_prp (same arguments, statuses,
 * PRP1, and PRP2 of one- and two-page requests), except:
 *   PRP2 (lists)   list_bus_base + 8 * word(D)
 *   word 511 of a list page: written by the request that owns the page's
 *                  last data slot -- the bus address of the next page when
 *                  two or more of its entries remain; its final entry when
 *                  exactly one remains (word 0 of the next page is then 0);
 *                  0 when its list ended in word 510
 *   ENOSPC         D + m > 511 * pool_pages (refused requests are a suffix)
 *   *total_pages   ceil(sum of m over all list requests / 511)
 *   padding        none: the library writes exactly the words of non-refused
 *                  lists and the zero words above, every other pool word stays
 *   extra check    (16 * lut_entries + 2) * n >= 2^62 -> -EINVAL
 * A batch's lists fill about (entries / 511) pages instead of one page or
 * more per list, and are written as one dense stream.
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_BUILD_PRP, n, 0), with the
 * same 8-byte header on return as dmadesc_build_prp (blocks, expired waits);
 * an expired wait refuses the block's list requests with DMADESC_PRP_EBUSY,
 * as in dmadesc_build_prp.
 */
int dmadesc_build_prp_packed(const uint64_t *lut, uint64_t lut_entries,
                             const uint64_t *off, const uint64_t *len, uint64_t n,
                             uint64_t list_bus_base, uint64_t *list_pool, uint64_t pool_pages,
                             uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                             uint64_t *total_pages,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * dmadesc_build_prp_packed_noalloc - dmadesc_build_prp_packed without a
 * caller workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Arguments,
 * outputs, statuses and errors are those of dmadesc_build_prp_packed; the
 * slot scan's workspace is instead a static device array of the library
 * (256 + 8 * DMADESC_NOALLOC_MAX_N / 1024 bytes, about 1 MiB) that every GPU
 * holds until the process ends; it is cleared by a kernel at the start of
 * each call. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). The first call on a device looks the array's device
 * address up once (hipGetSymbolAddress) with that device current.
 *   n > DMADESC_NOALLOC_MAX_N -> -E2BIG (nothing launched)
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams or from different threads) race and give
 * unspecified results; order them on one stream. The array's header (blocks,
 * expired waits) is not returned: refusals show as DMADESC_PRP_EBUSY.
 */
#define DMADESC_NOALLOC_MAX_N (1u << 27)
int dmadesc_build_prp_packed_noalloc(const uint64_t *lut, uint64_t lut_entries,
                                     const uint64_t *off, const uint64_t *len, uint64_t n,
                                     uint64_t list_bus_base, uint64_t *list_pool,
                                     uint64_t pool_pages, uint64_t *prp1, uint64_t *prp2,
                                     uint8_t *status, uint64_t *total_pages, void *stream);

/*
 * dmadesc_partition_by_queue - stable split of request indices by queue id.
 *
 * [MORI] groups a wave's lanes by destination with ballot / find-first-set /
 * shuffle and reserves queue slots once per group; here every queue's
 * requests are placed contiguously, in increasing request index.
 *   qid       u32[n]           destination queue of each request
 *   nqueues   1..DMADESC_MAX_QUEUES, else -EINVAL
 *   perm      u32[n]           request indices grouped by queue; queue q's
 *                              requests are perm[qoff[q] .. qoff[q+1]) in
 *                              increasing index order
 *   qoff      u64[nqueues + 2] bucket starts; bucket nqueues holds, in order,
 *                              the requests whose qid >= nqueues; qoff[nqueues+1] = n
 *   n_invalid u64 (device scalar) size of that overflow bucket
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_PARTITION, n, nqueues).
 */
int dmadesc_partition_by_queue(const uint32_t *qid, uint64_t n, uint32_t nqueues,
                               uint32_t *perm, uint64_t *qoff, uint64_t *n_invalid,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * dmadesc_build_batch - the whole path for one batch in one call: the
 * page-rounded region lookup, the PRP build and the stable split by queue,
 * reading off, len and qid once.
 *
 * The three steps belong to one request's way to the device:
 * [NCCL-26] "IB Backend MR Cache" (the containment lookup of the rounded
 * range, returning the region's handle and key), [UPCIE] introduction (PRP
 * entries from the GPU-page table when the command is built) and [MORI] the
 * thread-scope put (requests grouped by destination queue). Its outputs are
 * exactly those of dmadesc_mr_lookup, dmadesc_build_prp (flags 0) or
 * dmadesc_build_prp_packed (flags DMADESC_BATCH_PACKED) and
 * dmadesc_partition_by_queue called on the same arguments: the three column
 * groups are independent (a lookup miss still gets its PRPs and its queue
 * slot), and each keeps the errors, statuses and EBUSY refusals of its call.
 *   reg_start, reg_end, reg_lkey, nregions, page_shift, va_base
 *                 as dmadesc_mr_lookup; the lookup outputs handle, lkey,
 *                 kind, rbase, rend are either all given or all NULL (then
 *                 no lookup runs and the table arguments are ignored)
 *   lut, lut_entries, list_bus_base, list_pool, pool_pages, prp1, prp2,
 *   status, total_pages   as dmadesc_build_prp
 *   qid, nqueues, perm, qoff, n_invalid   as dmadesc_partition_by_queue
 *   off, len, n   the requests, shared by all three
 *   flags         DMADESC_BATCH_PACKED or 0; other bits -EINVAL
 * Workspace: dmadesc_batch_workspace_bytes(n, nqueues, nregions) bytes
 * (nregions 0 when no lookup runs); its first 8 bytes hold, on return, the
 * slot scan's block counter and count of expired waits, as in
 * dmadesc_build_prp.
 */
#define DMADESC_BATCH_PACKED 1u
int dmadesc_build_batch(const uint64_t *reg_start, const uint64_t *reg_end,
                        const uint32_t *reg_lkey, uint32_t nregions, uint32_t page_shift,
                        uint64_t va_base, const uint64_t *lut, uint64_t lut_entries,
                        const uint64_t *off, const uint64_t *len, const uint32_t *qid,
                        uint64_t n, uint32_t nqueues, uint64_t list_bus_base,
                        uint64_t *list_pool, uint64_t pool_pages, uint32_t flags,
                        int32_t *handle, uint32_t *lkey, uint8_t *kind, uint64_t *rbase,
                        uint64_t *rend, uint64_t *prp1, uint64_t *prp2, uint8_t *status,
                        uint64_t *total_pages, uint32_t *perm, uint64_t *qoff,
                        uint64_t *n_invalid, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of dmadesc_build_batch (0 for nqueues outside
 * 1..DMADESC_MAX_QUEUES, n >= 2^32 or nregions >= 2^31). Host-only. */
size_t dmadesc_batch_workspace_bytes(uint64_t n, uint32_t nqueues, uint32_t nregions);

/*
 * dmadesc_emit_sqe - NVMe submission entries per queue, one window per call.
 *
 * [UPCIE] "GPU-Resident Queue API": a kernel fills the submission queue with
 * 64-byte entries, each written as four 16-byte stores that the L2 merges
 * before they leave the GPU. [MORI] warp-level WQE reservation: the requests
 * bound for one queue take consecutive slots from its tail, which then moves
 * on by their number. Entry layout [NVMe]: dword 0 = opcode | command id << 16
 * (fused and PRP/SGL bits 0), dword 1 = nsid, dwords 2-5 = 0, dwords 6-9 =
 * PRP1, PRP2, dwords 10-11 = starting LBA, dword 12 = blocks - 1 (bits 15:0),
 * dwords 13-15 = 0. The command id is the ring slot.
 *
 * Inputs (device unless noted):
 *   perm, qoff   the output of dmadesc_partition_by_queue for these n
 *                requests with the same nqueues (qoff: nqueues + 2 entries)
 *   status       u8[n]  dmadesc_build_prp's status
 *   len, slba    u64[n] byte length (as given to dmadesc_build_prp) and
 *                starting logical block of each request
 *   prp1, prp2   u64[n] dmadesc_build_prp's outputs
 *   opcode       0..255 (host), e.g. 0x02 read, 0x01 write, else -EINVAL
 *   nsid         namespace id (host)
 *   lba_shift    log2 of the logical block size, 9..16 (host), else -EINVAL
 *   ring         u64[nqueues] device address of queue q's ring of depth[q]
 *                64-byte entries
 *   depth        u32[nqueues] ring size in entries
 *   free_slots   u32[nqueues] slots the caller allows this call to fill
 * In/out:
 *   tail         u32[nqueues] next slot to fill; advanced mod depth[q]
 *   cursor       u64[nqueues] entries of bucket q consumed by earlier calls;
 *                advanced by this call's window
 * Outputs:
 *   placed       u32[nqueues] entries written into ring q by this call
 *   req_of_slot  u32[nqueues * DMADESC_SQ_MAX_DEPTH] or NULL: for every slot s
 *                this call fills in ring q, entry q * 65536 + s receives the
 *                request index (to map a completion's command id back)
 * Per queue q: the queue is refused (nothing read, consumed or written, tail
 * and cursor unchanged, placed[q] = 0) when ring[q] is 0 or not 64-byte
 * aligned, depth[q] is outside [2, 65536] or tail[q] >= depth[q]. Otherwise
 * the call consumes W = min(free_slots[q], depth[q] - 1, bucket size -
 * cursor[q]) entries of bucket q after the first cursor[q]; in that order,
 * every consumed request that is placeable -- status OK and len a positive
 * multiple of 2^lba_shift of at most 65536 blocks -- gets the next slot from
 * tail[q]; the others are consumed without a slot, so the ring holds no hole.
 * Calls with cursor carried over drain a batch larger than the rings. The
 * overflow bucket (qid >= nqueues) is never consumed. Slots outside the ones
 * filled, and req_of_slot entries for them, are not written. Outputs must not
 * overlap inputs (tail and cursor are updated in place). Memory safety needs
 * perm/qoff to come from the split of these n requests and each ring and
 * req_of_slot to have the stated size.
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_EMIT_SQE, n, nqueues):
 * 2,196 bytes per queue and 1,024-entry tile of a window (64 tiles per
 * queue) plus 16 per queue, about 9 MB for 64 queues; independent of n.
 */
int dmadesc_emit_sqe(const uint32_t *perm, const uint64_t *qoff, uint32_t nqueues,
                     const uint8_t *status, const uint64_t *len, const uint64_t *slba,
                     const uint64_t *prp1, const uint64_t *prp2, uint64_t n,
                     uint32_t opcode, uint32_t nsid, uint32_t lba_shift,
                     const uint64_t *ring, const uint32_t *depth, const uint32_t *free_slots,
                     uint32_t *tail, uint64_t *cursor, uint32_t *placed,
                     uint32_t *req_of_slot, void *ws, size_t ws_bytes, void *stream);

/* One RDMA put descriptor (32 bytes, little endian). */
typedef struct dmadesc_put_desc {
    uint64_t laddr;   /* local address: local_base + src + x      */
    uint64_t raddr;   /* remote address: peer_base[pe] + dst + x  */
    uint32_t len;     /* bytes of this piece (1 .. 2^31)          */
    uint32_t lkey;    /* key of the source chunk                  */
    uint32_t rkey;    /* key of the destination chunk on pe       */
    uint32_t req;     /* request index                            */
} dmadesc_put_desc;

/*
 * dmadesc_build_put - RDMA put descriptors for a symmetric heap.
 *
 * [MORI] thread-scope put and QueryRemoteAddr: the remote address of a heap
 * offset is the peer's heap base plus the same offset. Static heap
 * (chunk_shift == 0): one local key lkeys[0] and one remote key rkeys[pe] per
 * peer; a put is one transfer. VMM heap (chunk_shift 12..31): the heap is
 * chunks of 2^chunk_shift bytes with their own keys (lkeys[k]; on PE q,
 * rkeys[q * nchunks + k], nchunks = heap_bytes >> chunk_shift); each transfer
 * is min(bytes left in the source chunk, bytes left in the destination chunk,
 * remaining), so every piece lies in one chunk on both sides. No piece exceeds
 * 2^31 bytes (the RDMA message limit; it binds only for a static heap).
 *   src, dst, bytes u64[n]  heap offsets (local source, remote destination)
 *                           and length of each put
 *   pe              u32[n]  destination PE (< npes, 1..65536)
 *   local_base, peer_base[npes]  heap base addresses (host value / device)
 *   heap_bytes      heap size; with VMM a multiple of the chunk size with
 *                   fewer than 2^30 chunks
 *   desc            dmadesc_put_desc[desc_cap] (16-byte aligned)
 * Outputs: first u64[n] (slot of the first descriptor of put i: a running
 * count over all puts, refused ones included), count u32[n] (its pieces; 0
 * for EINVAL/ERANGE), status u8[n] (enum dmadesc_prp_status: EINVAL zero bytes
 * or pe >= npes, ERANGE past the heap on either side, ENOSPC first + count >
 * desc_cap, refused puts are a suffix; EBUSY: the slot scan of the put's
 * block did not finish, first = UINT64_MAX), *total (device u64: descriptors
 * the batch needs; UINT64_MAX if the last block's scan did not finish).
 * Descriptors of refused puts are not written; no other descriptor slot is
 * written. Extra check: n * (most pieces per put) >= 2^62 -> -EINVAL.
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_BUILD_PUT, n, 0); as for
 * dmadesc_build_prp, its first 8 bytes hold on return a block counter and
 * the count of blocks whose bounded wait expired (0 when blocks make
 * progress; nonzero means some puts carry DMADESC_PRP_EBUSY).
 */
int dmadesc_build_put(const uint64_t *src, const uint64_t *dst, const uint64_t *bytes,
                      const uint32_t *pe, uint64_t n, uint64_t local_base, uint64_t heap_bytes,
                      uint32_t chunk_shift, const uint32_t *lkeys, const uint64_t *peer_base,
                      const uint32_t *rkeys, uint32_t npes, dmadesc_put_desc *desc,
                      uint64_t desc_cap, uint64_t *first, uint32_t *count, uint8_t *status,
                      uint64_t *total, void *ws, size_t ws_bytes, void *stream);

/* One mirrored completion queue (shared by host and device; 48 bytes). */
#define DMADESC_CQ_MAX_SLOTS 64u
#define DMADESC_CQ_MAX_DEPTH 65536u
typedef struct dmadesc_cq_slot {
    uint64_t src;          /* device address of the device-memory queue (16-byte aligned) */
    uint64_t dst;          /* device-visible address of the mirror queue (16-byte aligned) */
    uint32_t depth;        /* entries of 16 bytes, 2 .. 65536                          */
    uint32_t generation;   /* host: odd while the queue is attached                    */
    uint32_t ack;          /* mirror: generation it has finished with                  */
    uint32_t head;         /* mirror state: next entry to copy (host sets 0 to attach)  */
    uint32_t phase;        /* mirror state: phase the next entry carries (host sets 1)  */
    uint32_t reserved;
    uint64_t copied;       /* mirror: entries copied under the current attachment       */
} dmadesc_cq_slot;

/*
 * dmadesc_cq_mirror - completion-queue mirror.
 *
 * [UPCIE] "Completions in device memory": one kernel serves every mirrored queue (up to
 * 64) with one wave each and copies completions from the device-memory queue
 * into the mirror queue as their phase bit turns (NVMe: phase tag = bit 16 of
 * dword 3, 1 on the controller's first pass, inverted on each later pass).
 * The host fills a slot (addresses, depth, head 0, phase 1, copied 0) and then
 * raises its generation to an odd value; the wave copies until the generation
 * changes, then writes the value it worked under to `ack`; a wave finding an
 * even generation writes generation - 1. The host frees nothing of a queue
 * before it sees that acknowledgement. A copied entry is first written whole
 * with its old phase bit and only then, after a release, given dword 3 with
 * the new one, so a consumer polling the mirror's phase bits never reads a
 * partial entry; each poll's copies are released before the next poll.
 *   slots       dmadesc_cq_slot[nslots] (device or host-mapped memory),
 *               nslots 1..DMADESC_CQ_MAX_SLOTS
 *   stop        u32 (device or host-mapped): nonzero asks the waves to leave
 *               after one more drain
 *   idle_polls  1..2^24: a wave also leaves after this many polls in a row
 *               that copied nothing (a poll sleeps ~0.2 µs when idle)
 * The call is one launch on `stream` that stays resident until every wave has
 * left (at most 2^22 polls each); slots keep head, phase and copied, so the
 * next call continues. A slot with an unusable description (depth, null or
 * unaligned address, head >= depth) copies nothing and acknowledges nothing.
 * Run it on a stream of its own: work on that stream waits for it, and so may
 * work on a stream that shares its hardware queue. Errors: -EINVAL for a
 * null or non-8-byte-aligned `slots`, a null `stop`, nslots or idle_polls out
 * of range; -EIO if the launch fails.
 */
int dmadesc_cq_mirror(dmadesc_cq_slot *slots, uint32_t nslots, const uint32_t *stop,
                      uint32_t idle_polls, void *stream);

/* Registration cache limits and per-call outcomes. */
#define DMADESC_REG_MAX_BATCH 65536u          /* calls per batch                  */
#define DMADESC_REG_MAX_CAPACITY (1u << 24)   /* records a table may hold         */
enum dmadesc_reg_kind {
    DMADESC_REG_INVALID = 0,  /* zero length, or the range or its rounded end wraps  */
    DMADESC_REG_HIT = 1,      /* a record present before the batch contains it       */
    DMADESC_REG_NEW = 2,      /* this call inserted a record                          */
    DMADESC_REG_HIT_NEW = 3,  /* a record inserted earlier in this batch contains it  */
    DMADESC_REG_NOSPACE = 4   /* the batch did not fit the capacity; nothing applied  */
};
enum dmadesc_dereg_status {
    DMADESC_DEREG_OK = 0,      /* one reference dropped                                */
    DMADESC_DEREG_REMOVED = 1, /* the last reference dropped; the record is freed      */
    DMADESC_DEREG_STALE = 2    /* no live record holds the handle (an error)           */
};

/*
 * dmadesc_reg_register / dmadesc_reg_deregister - the registration cache.
 *
 * [NCCL-26] "Communicator User Registration Cache": a registration widens the
 * range [addr, addr + size) to whole pages (floor of the start, ceiling of the
 * end); if a record fully contains the widened range, that record gains a
 * reference and its handle is returned, else a new record is inserted in
 * start order. "IB Backend MR Cache": a deregistration drops a reference and
 * frees the record at zero; a handle not in the cache is an error; the record
 * array grows from 0 to 32 and then doubles. A batch means exactly what its
 * calls made one after another, in index order, mean; among several records
 * containing a range the first in start order is used, and a new record goes
 * after the records with the same start.
 *
 * Table (caller-owned device memory; `capacity` <= DMADESC_REG_MAX_CAPACITY):
 *   start, end  u64[capacity]  widened range of each record (end exclusive)
 *   id          u64[capacity]  handle of each record (> 0, never reused)
 *   refs        u32[capacity]  reference count
 *     slots 0 .. count-1 hold the live records in increasing handle order
 *   by_start    u32[capacity]  slots of the live records in (start, handle)
 *                              order
 *   state       u64[2]         count of live records, next handle; a new
 *                              table is state = {0, 1}
 * register: addr, size u64[n] (n <= DMADESC_REG_MAX_BATCH); page_shift 12..30.
 *   Outputs handle u64[n] (0 for INVALID and NOSPACE), kind u8[n] (enum
 *   dmadesc_reg_kind) and *needed (device u64): the capacity the batch needs,
 *   equal to `capacity` when it fits, else `capacity` grown 0 -> 32 -> 64 ...
 *   until it fits. A batch that does not fit changes nothing: the caller
 *   copies the table into arrays of *needed entries and calls again.
 * deregister: handle u64[n]; output status u8[n] (enum dmadesc_dereg_status).
 *   Freed records leave the table; the others keep their order.
 * Both: the table is updated in place; calls on one table must be ordered.
 * Workspace: dmadesc_workspace_bytes(DMADESC_OP_REGISTRY, n, capacity).
 */
int dmadesc_reg_register(uint64_t *start, uint64_t *end, uint64_t *id, uint32_t *refs,
                         uint32_t *by_start, uint64_t *state, uint64_t capacity,
                         uint32_t page_shift, const uint64_t *addr, const uint64_t *size,
                         uint64_t n, uint64_t *handle, uint8_t *kind, uint64_t *needed,
                         void *ws, size_t ws_bytes, void *stream);
int dmadesc_reg_deregister(uint64_t *start, uint64_t *end, uint64_t *id, uint32_t *refs,
                           uint32_t *by_start, uint64_t *state, uint64_t capacity,
                           const uint64_t *handle, uint64_t n, uint8_t *status,
                           void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes needed by `op` for n requests (`param` = nqueues for
 * DMADESC_OP_PARTITION and DMADESC_OP_EMIT_SQE, the table capacity for
 * DMADESC_OP_REGISTRY, nregions for DMADESC_OP_MR_LOOKUP (its optional
 * record workspace), ignored otherwise). Returns 0 for an unknown op or
 * for an op that needs none. Host-only; launches nothing. */
size_t dmadesc_workspace_bytes(int op, uint64_t n, uint32_t param);

/* Static description of a return code (host-only). */
const char *dmadesc_strerror(int err);

/* Library ABI version (host-only). */
int dmadesc_version(void);

/* Sets the process-wide bound on the polls of one wait of the slot scan
 * (DMADESC_DEFAULT_WAIT_POLLS at load; 0 makes a wait give up at the first
 * poll that finds a predecessor not yet published) for calls launched
 * afterwards, and returns the previous bound. For tests of the refusal path
 * (DMADESC_PRP_EBUSY): every kernel still ends normally at any bound. */
uint32_t dmadesc_debug_wait_limit(uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* DMADESC_H */

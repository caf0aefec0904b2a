/*
 * oracle.c - plain, single-threaded CPU reference (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library. It shares nothing with the GPU library. Each function
 * follows the steps of the passage it cites, in that order, with no blocking,
 * fusion or reordering; exact 128-bit arithmetic is used wherever a 64-bit
 * intermediate could wrap, so that a reader can check it by eye.
 *
 * Parity status of each function is recorded beside it ("pinned by ...").
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

/* ------------------------------------------------------------------------
 * O1  Page-rounded containment lookup.
 *
 * [NCCL-26] "IB Backend MR Cache": a range is first widened to whole system
 * pages -- the base is the address with the in-page bits cleared, and the page
 * count is (address + size - base + page - 1) / page -- and the cache is then
 * searched by address; an existing region that fully contains the widened
 * range is a hit and is reused, a partial overlap is not a hit. The
 * "Communicator User Registration Cache" section applies the same floor/cover
 * rounding before its containment test.
 *
 * Readings: the region id in the sorted table is the handle (-1 = miss); the
 * exact/contained distinction is made on the rounded bounds; a zero-length
 * range, or one whose end or rounded end does not fit in 64 bits, is INVALID.
 *
 * Pinned by: the four-row rounding table printed in "IB Backend MR Cache"; the
 * register sequence of "真实 ncclCommRegister 语义实验" replayed on O4 and
 * looked up here; brute-force containment scans over every region.
 * ------------------------------------------------------------------------ */
void orc_mr_lookup(const uint64_t *start, const uint64_t *end, const uint32_t *lkey,
                   uint64_t nregions, unsigned page_shift,
                   const uint64_t *off, const uint64_t *len, uint64_t n, uint64_t va_base,
                   int32_t *handle, uint32_t *lkey_out, uint8_t *kind,
                   uint64_t *rbase, uint64_t *rend)
{
    const uint64_t page = 1ull << page_shift;
    for (uint64_t i = 0; i < n; ++i) {
        handle[i] = -1;
        lkey_out[i] = 0;
        kind[i] = ORC_MISS;
        rbase[i] = 0;
        rend[i] = 0;

        /* Absolute address of the range, and validity. */
        u128 a_wide = (u128)va_base + off[i];
        uint64_t size = len[i];
        if (size == 0 || a_wide + size > (u128)UINT64_MAX) {
            kind[i] = ORC_INVALID;
            continue;
        }
        uint64_t a = (uint64_t)a_wide;

        /* Round down the base, count the covering pages, round up the end. */
        uint64_t base = a & ~(page - 1);
        u128 pages = ((u128)a + size - base + page - 1) / page;
        u128 end_wide = (u128)base + pages * page;
        if (end_wide > (u128)UINT64_MAX) {
            kind[i] = ORC_INVALID;
            continue;
        }
        uint64_t top = (uint64_t)end_wide;
        rbase[i] = base;
        rend[i] = top;

        /* The only region that can contain [base, top) in a sorted,
         * non-overlapping table is the last one starting at or below base:
         * binary search for the count of starts <= base. */
        uint64_t lo = 0, hi = nregions;
        while (lo < hi) {
            uint64_t mid = lo + (hi - lo) / 2;
            if (start[mid] <= base) lo = mid + 1;
            else hi = mid;
        }
        if (lo == 0) continue;                 /* no region starts at or below */
        uint64_t r = lo - 1;
        if (top <= end[r]) {                   /* full containment: a hit */
            handle[i] = (int32_t)r;
            lkey_out[i] = lkey[r];
            kind[i] = (base == start[r] && top == end[r]) ? ORC_EXACT : ORC_CONTAINED;
        }                                      /* partial overlap or disjoint: miss */
    }
}

/* ------------------------------------------------------------------------
 * O2  GPU-page table -> NVMe PRP entries and chained PRP lists.
 *
 * [UPCIE] introduction: GPU memory is resolved once into a table holding one
 * physical address per 64 KiB GPU page; at submission PRP entries are formed
 * at 4 KiB granularity from the 4 KiB sub-page offsets inside each 64 KiB
 * entry. "Limitations": one list page holds 512 entries, so PRP1 plus one
 * list page reaches 513 x 4 KiB; that backend does not chain.
 * [NVMe] PRP rules (not on the pages): PRP1 is the first page's address with
 * the byte offset; PRP2 is 0 for a one-page transfer, the second page's
 * address for two pages, and otherwise the bus address of a PRP list; when a
 * list needs more entries than a page holds, the last entry of each
 * non-final list page points to the next list page.
 *
 * Readings: the physical address of heap byte x is table[x >> 16] plus
 * (x & 0xFFFF); list pages are handed out in request order from a running
 * counter (an exclusive prefix of the per-request page counts); a request
 * refused for lack of pool pages still advances the counter, so the refused
 * set is a suffix and *total is the capacity the batch needs; a request with
 * zero length, an offset that is not a multiple of 4 (PRP1 must be dword
 * aligned), or an end that wraps is EINVAL; one that ends past the heap is
 * ERANGE. Refused requests get PRP1 = PRP2 = 0 and write no list entries.
 *
 * Pinned by: a byte-walk brute force over tiny heaps (every 4 KiB physical
 * page the bytes of the request touch, in order, against PRP1/PRP2/list
 * chain), the identity-table special case (the textbook contiguous PRP list),
 * the 513-page single-list limit from "Limitations", and chain-walk checks of
 * list sizes around every multiple of 511. Chaining itself follows [NVMe];
 * no page prints a chained example.
 * ------------------------------------------------------------------------ */
static uint64_t phys_of(const uint64_t *lut, uint64_t x)
{
    return lut[x >> 16] + (x & 0xFFFFull);
}

void orc_build_prp(const uint64_t *lut, uint64_t lut_entries,
                   const uint64_t *off, const uint64_t *len, uint64_t n,
                   uint64_t list_bus_base, uint64_t *pool, uint64_t pool_pages,
                   uint64_t *prp1, uint64_t *prp2, uint8_t *status, uint64_t *total)
{
    const u128 heap = (u128)lut_entries << 16;
    uint64_t next_slot = 0;                       /* running list-page counter */

    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t o = off[i], size = len[i];
        prp1[i] = 0;
        prp2[i] = 0;
        status[i] = ORC_OK;

        /* 1. Validate. */
        if (size == 0 || (o % 4) != 0 || (u128)o + size > (u128)UINT64_MAX) {
            status[i] = ORC_EINVAL;
            continue;
        }
        if ((u128)o + size > heap) {
            status[i] = ORC_ERANGE;
            continue;
        }

        /* 2. Number of 4 KiB pages the byte range touches. */
        uint64_t npages = (uint64_t)(((u128)(o & 4095) + size + 4095) >> 12);
        uint64_t page0 = o & ~4095ull;            /* heap offset of page 0 */

        /* 3./5. PRP1, then PRP2 by page count. */
        if (npages == 1) {
            prp1[i] = phys_of(lut, o);
            prp2[i] = 0;
            continue;
        }
        if (npages == 2) {
            prp1[i] = phys_of(lut, o);
            prp2[i] = phys_of(lut, page0 + 4096);
            continue;
        }
        uint64_t entries = npages - 1;                    /* pages 1 .. n-1 */
        uint64_t lpages = (entries - 1 + 510) / 511;      /* ceil((entries-1)/511) */
        uint64_t slot = next_slot;
        next_slot += lpages;                              /* 7. advance, refused or not */
        if ((u128)slot + lpages > pool_pages) {
            status[i] = ORC_ENOSPC;
            continue;
        }
        prp1[i] = phys_of(lut, o);
        prp2[i] = list_bus_base + slot * 4096;

        /* 4./6. Fill the list pages in order; a full non-final page gets a
         * pointer to the next page in its last entry. */
        if (pool) {
            uint64_t t = 0, pos = 0;
            for (uint64_t k = 1; k < npages; ++k) {
                if (pos == 511 && t + 1 < lpages) {
                    pool[(slot + t) * 512 + 511] = list_bus_base + (slot + t + 1) * 4096;
                    ++t;
                    pos = 0;
                }
                pool[(slot + t) * 512 + pos] = phys_of(lut, page0 + 4096 * k);
                ++pos;
            }
        }
    }
    *total = next_slot;
}

/* ------------------------------------------------------------------------
 * O2p  The same PRP entries with packed lists.
 *
 * [NVMe] (not on the pages): the PRP list pointer carried in a command may
 * name any qword of a page, not only its start; a list then runs to the end
 * of that page, and when more than one entry is still needed there, the
 * page's last entry points to the start of the next list page. Everything
 * else -- which entries a request needs, PRP1, and PRP2 for one- and
 * two-page requests -- is O2 unchanged.
 *
 * Readings: lists are laid back to back in request order in "data slots",
 * 511 to a page (words 0..510), so a request's list starts where the
 * previous one ended; word 511 of a page belongs to the request that owns the
 * page's last data slot and holds a pointer, that request's final entry (when
 * exactly one remains; the slot that entry would have taken, word 0 of the
 * next page, is then 0) or 0 (its list ended in word 510). A refused request
 * writes nothing.
 *
 * Pinned by: NVMe chain walks from each PRP2 (with its offset) against the
 * byte walk of the request, disjointness of all requests' words, the dense
 * page count, and hand-built layouts around page ends.
 * ------------------------------------------------------------------------ */
static uint64_t slot_word(u128 d)
{
    return (uint64_t)(d + d / 511);
}

void orc_build_prp_packed(const uint64_t *lut, uint64_t lut_entries,
                          const uint64_t *off, const uint64_t *len, uint64_t n,
                          uint64_t list_bus_base, uint64_t *pool, uint64_t pool_pages,
                          uint64_t *prp1, uint64_t *prp2, uint8_t *status, uint64_t *total)
{
    const u128 heap = (u128)lut_entries << 16;
    const u128 capacity = (u128)pool_pages * 511;   /* data slots in the pool */
    u128 next = 0;                                  /* running data-slot counter */

    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t o = off[i], size = len[i];
        prp1[i] = 0;
        prp2[i] = 0;
        status[i] = ORC_OK;

        /* Validation, page count, PRP1 and short PRP2: as in O2. */
        if (size == 0 || (o % 4) != 0 || (u128)o + size > (u128)UINT64_MAX) {
            status[i] = ORC_EINVAL;
            continue;
        }
        if ((u128)o + size > heap) {
            status[i] = ORC_ERANGE;
            continue;
        }
        uint64_t npages = (uint64_t)(((u128)(o & 4095) + size + 4095) >> 12);
        uint64_t page0 = o & ~4095ull;
        if (npages == 1) {
            prp1[i] = phys_of(lut, o);
            continue;
        }
        if (npages == 2) {
            prp1[i] = phys_of(lut, o);
            prp2[i] = phys_of(lut, page0 + 4096);
            continue;
        }

        /* Data slots of this request's entries. */
        const uint64_t m = npages - 1;
        const u128 first = next;
        next += m;
        if (first + m > capacity) {
            status[i] = ORC_ENOSPC;
            continue;
        }
        prp1[i] = phys_of(lut, o);
        prp2[i] = list_bus_base + 8 * slot_word(first);
        if (pool == NULL) continue;

        for (uint64_t k = 0; k < m; ++k) {
            const u128 d = first + k;
            const uint64_t entry = phys_of(lut, page0 + 4096 * (k + 1));
            if (k >= 1 && d % 511 == 0) {
                /* The list enters a new page at entry k: the last word of the
                 * page before is a pointer, or this final entry itself. */
                const uint64_t last = slot_word(d) - 1;              /* word 511 */
                if (k == m - 1) {
                    pool[last] = entry;
                    pool[slot_word(d)] = 0;
                    continue;
                }
                pool[last] = list_bus_base + 4096 * (uint64_t)(d / 511);
            }
            pool[slot_word(d)] = entry;
        }
        const u128 end = first + m - 1;
        if (end % 511 == 510) pool[slot_word(end) + 1] = 0;          /* word 511 unused */
    }
    *total = (uint64_t)((next + 510) / 511);
}

/* ------------------------------------------------------------------------
 * O3  Stable split of requests by destination queue.
 *
 * A plain counting split: count each bucket, take the exclusive prefix as the
 * bucket starts, then place the request indices in increasing order behind a
 * per-bucket cursor, so that equal queue ids keep their original order.
 * [MORI] groups a wave's lanes by destination before issuing and reserves
 * queue slots per group; the order of equal keys is not stated there, and the
 * reading here is stable (ties by original index). Queue ids >= nqueues go to
 * an overflow bucket after the valid ones.
 *
 * Pinned by: a library stable sort of the indices by queue id.
 * ------------------------------------------------------------------------ */
void orc_partition(const uint32_t *qid, uint64_t n, uint32_t nqueues,
                   uint32_t *perm, uint64_t *qoff, uint64_t *n_invalid)
{
    const uint64_t nb = (uint64_t)nqueues + 1;
    uint64_t *cursor = (uint64_t *)calloc(nb, sizeof(uint64_t));
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t b = qid[i] < nqueues ? qid[i] : nqueues;
        cursor[b]++;
    }
    qoff[0] = 0;
    for (uint64_t b = 0; b < nb; ++b) qoff[b + 1] = qoff[b] + cursor[b];
    *n_invalid = cursor[nqueues];
    for (uint64_t b = 0; b < nb; ++b) cursor[b] = qoff[b];
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t b = qid[i] < nqueues ? qid[i] : nqueues;
        perm[cursor[b]++] = (uint32_t)i;
    }
    free(cursor);
}

/* ------------------------------------------------------------------------
 * O5  NVMe submission entries per queue.
 *
 * [UPCIE] "GPU-Resident Queue API": a kernel on the GPU fills the submission
 * queue itself, one 64-byte entry per command, written as four 16-byte stores.
 * [MORI] warp-level WQE reservation: the lanes bound for one queue take
 * consecutive slots starting at that queue's tail, and the tail then moves on
 * by their number. The entry layout is the NVMe common command format [NVMe]
 * (not on the pages): dword 0 = opcode (bits 7:0), fused operation and PRP
 * data transfer (bits 15:8, zero), command identifier (bits 31:16); dword 1 =
 * namespace id; dwords 2-5 = 0 (no metadata pointer); dwords 6-7 = PRP1;
 * dwords 8-9 = PRP2; dwords 10-11 = starting LBA; dword 12 bits 15:0 = number
 * of logical blocks minus one; dwords 13-15 = 0. A queue of depth D holds at
 * most D - 1 entries, and D is at most 65536.
 *
 * Readings: a queue's entries follow the stable split order (request order);
 * the command identifier is the ring slot; a call consumes a window of each
 * bucket no longer than the free slots, so a batch larger than the rings
 * drains over several calls; a consumed request that cannot be expressed
 * (PRP not OK, length not a whole number of blocks, more than 65536 blocks) is
 * skipped without a slot, so the ring never holds a hole; the request index
 * of every filled slot is recorded beside the ring, which is what turns a
 * completion's command identifier back into a request.
 *
 * Pinned by: entries rebuilt field by field with Python's struct module from
 * the NVMe field table, and a replay of every queue as a Python deque fed
 * from a NumPy stable sort, over several calls that drain a batch.
 * ------------------------------------------------------------------------ */
static void put_le32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static void put_le64(uint8_t *p, uint64_t v)
{
    put_le32(p, (uint32_t)v);
    put_le32(p + 4, (uint32_t)(v >> 32));
}

void orc_emit_sqe(const uint32_t *perm, const uint64_t *qoff, uint32_t nqueues,
                  const uint8_t *status, const uint64_t *len, const uint64_t *slba,
                  const uint64_t *prp1, const uint64_t *prp2, uint64_t n,
                  uint8_t opcode, uint32_t nsid, unsigned lba_shift,
                  uint8_t *const *ring, const uint32_t *depth, const uint32_t *free_slots,
                  uint32_t *tail, uint64_t *cursor, uint32_t *placed, uint32_t *req_of_slot)
{
    const uint64_t block = 1ull << lba_shift;
    for (uint32_t q = 0; q < nqueues; ++q) {
        placed[q] = 0;
        const uint32_t d = depth[q];
        if (ring[q] == NULL || d < 2 || d > 65536 || tail[q] >= d) continue;   /* refused */

        /* The window: the next entries of bucket q, no more than the ring takes. */
        const uint64_t size = qoff[q + 1] - qoff[q];
        const uint64_t left = cursor[q] < size ? size - cursor[q] : 0;
        uint64_t room = free_slots[q] < d - 1 ? free_slots[q] : d - 1;
        const uint64_t w = room < left ? room : left;

        uint32_t k = 0;
        for (uint64_t j = 0; j < w; ++j) {
            const uint32_t i = perm[qoff[q] + cursor[q] + j];
            if (i >= n) continue;                 /* not a request of this batch */
            const uint64_t blocks = len[i] / block;
            const int placeable = status[i] == ORC_OK && len[i] % block == 0 &&
                                  blocks >= 1 && blocks <= 65536;
            if (!placeable) continue;
            const uint32_t s = (tail[q] + k) % d;
            ++k;
            if (req_of_slot) req_of_slot[(uint64_t)q * 65536 + s] = i;
            uint8_t *e = ring[q] + (uint64_t)s * 64;
            memset(e, 0, 64);
            put_le32(e + 0, (uint32_t)opcode | (s << 16));
            put_le32(e + 4, nsid);
            put_le64(e + 24, prp1[i]);
            put_le64(e + 32, prp2[i]);
            put_le64(e + 40, slba[i]);
            put_le32(e + 48, (uint32_t)(blocks - 1));
        }
        placed[q] = k;
        tail[q] = (tail[q] + k) % d;
        cursor[q] += w;
    }
}

/* ------------------------------------------------------------------------
 * O6  RDMA put descriptors for a symmetric heap.
 *
 * [MORI] thread-scope put: the remote address of a heap address is the peer's
 * heap base plus the same offset. In a static heap one local key and one
 * remote key per peer cover the whole heap and the whole remainder is sent at
 * once. In a VMM heap each chunk has its own keys; every round the source
 * chunk and the destination chunk are looked up, each giving the bytes left in
 * that chunk and its key, and the round sends min(source chunk left,
 * destination chunk left, remaining), so a key is always valid for what it
 * covers.
 *
 * Readings: chunks are 2^chunk_shift bytes everywhere in the heap and on
 * every PE; a piece never exceeds 2^31 bytes (the RDMA message limit; it only
 * matters for a static heap); descriptors are laid out request after request
 * from a running count that refused requests also advance.
 *
 * Pinned by: the closed-form piece count 1 + (source boundaries crossed) +
 * (destination boundaries crossed) - (shared ones); a byte walk on tiny chunks
 * (pieces are the maximal runs of bytes with one source chunk and one
 * destination chunk); sum of lengths, contiguity, keys and addresses.
 * ------------------------------------------------------------------------ */
#define ORC_PUT_MAX_MSG (1ull << 31)

void orc_build_put(const uint64_t *src, const uint64_t *dst, const uint64_t *bytes,
                   const uint32_t *pe, uint64_t n, uint64_t local_base, uint64_t heap_bytes,
                   unsigned chunk_shift, const uint32_t *lkeys, const uint64_t *peer_base,
                   const uint32_t *rkeys, uint32_t npes, orc_put_desc *desc, uint64_t desc_cap,
                   uint64_t *first, uint32_t *count, uint8_t *status, uint64_t *total)
{
    const int vmm = chunk_shift != 0;
    const uint64_t chunk = vmm ? 1ull << chunk_shift : 0;
    const uint64_t nchunks = vmm ? heap_bytes >> chunk_shift : 1;
    uint64_t next = 0;
    for (uint64_t i = 0; i < n; ++i) {
        first[i] = next;
        count[i] = 0;
        status[i] = ORC_OK;
        if (bytes[i] == 0 || pe[i] >= npes) {
            status[i] = ORC_EINVAL;
            continue;
        }
        if ((u128)src[i] + bytes[i] > heap_bytes || (u128)dst[i] + bytes[i] > heap_bytes) {
            status[i] = ORC_ERANGE;
            continue;
        }
        /* The rounds of the put loop, first only counted. */
        uint64_t pieces = 0;
        for (uint64_t x = 0; x < bytes[i];) {
            uint64_t t = bytes[i] - x;
            if (vmm) {
                const uint64_t src_left = chunk - (src[i] + x) % chunk;
                const uint64_t dst_left = chunk - (dst[i] + x) % chunk;
                if (src_left < t) t = src_left;
                if (dst_left < t) t = dst_left;
            }
            if (t > ORC_PUT_MAX_MSG) t = ORC_PUT_MAX_MSG;
            x += t;
            ++pieces;
        }
        count[i] = (uint32_t)pieces;
        next += pieces;
        if (first[i] + pieces > desc_cap) {
            status[i] = ORC_ENOSPC;
            continue;
        }
        if (desc == NULL) continue;
        /* The same rounds, now writing one descriptor each. */
        uint64_t k = first[i];
        for (uint64_t x = 0; x < bytes[i];) {
            uint64_t t = bytes[i] - x;
            uint32_t lkey = lkeys[0], rkey = rkeys[pe[i]];
            if (vmm) {
                const uint64_t sc = (src[i] + x) >> chunk_shift, dc = (dst[i] + x) >> chunk_shift;
                const uint64_t src_left = chunk - (src[i] + x) % chunk;
                const uint64_t dst_left = chunk - (dst[i] + x) % chunk;
                if (src_left < t) t = src_left;
                if (dst_left < t) t = dst_left;
                lkey = lkeys[sc];
                rkey = rkeys[(uint64_t)pe[i] * nchunks + dc];
            }
            if (t > ORC_PUT_MAX_MSG) t = ORC_PUT_MAX_MSG;
            desc[k].laddr = local_base + src[i] + x;
            desc[k].raddr = peer_base[pe[i]] + dst[i] + x;
            desc[k].len = (uint32_t)t;
            desc[k].lkey = lkey;
            desc[k].rkey = rkey;
            desc[k].req = (uint32_t)i;
            ++k;
            x += t;
        }
    }
    *total = next;
}

/* ------------------------------------------------------------------------
 * O7  Completion-queue mirror, one drain.
 *
 * [UPCIE] "Completions in device memory": a resident kernel watches
 * each device-memory completion queue and copies completions into the host
 * queue as their phase bit turns; per queue the host and the kernel share the
 * two queue addresses, the depth, a generation (odd while attached) and an
 * acknowledgement; a queue found with an even generation is acknowledged with
 * the odd value before it. [NVMe] (not on the pages): a completion entry is 16
 * bytes with the phase tag in bit 16 of its fourth dword; the controller
 * writes the tag as 1 on its first pass through the queue and inverts it on
 * every later pass.
 *
 * Readings: a drain copies every entry that carries the expected phase, in
 * queue order, and stops at the first that does not; the slot keeps the next
 * position and the expected phase across drains.
 *
 * Pinned by: a controller model that writes completions in passes with the
 * phase inverted each pass; everything it wrote comes out once, in order.
 * ------------------------------------------------------------------------ */
uint64_t orc_cq_drain(const uint32_t *src, uint32_t *dst, uint32_t depth, uint32_t gen,
                      uint32_t *head, uint32_t *phase, uint32_t *ack)
{
    if ((gen & 1u) == 0) {
        *ack = gen - 1;
        return 0;
    }
    uint64_t copied = 0;
    while (((src[(uint64_t)*head * 4 + 3] >> 16) & 1u) == *phase) {
        memcpy(&dst[(uint64_t)*head * 4], &src[(uint64_t)*head * 4], 16);
        ++copied;
        if (++*head == depth) {
            *head = 0;
            *phase ^= 1u;
        }
    }
    return copied;
}

/* ------------------------------------------------------------------------
 * O4  Registration cache with reference counts.
 *
 * [NCCL-26] "Communicator User Registration Cache": register rounds the range
 * to whole pages; if an existing record fully contains it, its count goes up
 * and its handle is returned; otherwise a new record is inserted in sorted
 * position. "IB Backend MR Cache": deregister drops the count and frees the
 * record at zero; a handle not in the cache is an error; the record array
 * grows from 0 to 32 and then doubles (32 -> 64 -> 128).
 *
 * Readings: a handle is a record id that is never reused (so a stale handle
 * is always detected); records are kept sorted by start, a new record goes
 * after existing records with the same start; when several records contain a
 * range, the first in sorted order is reused.
 *
 * Pinned by: the 8 MiB register/deregister sequence of
 * "真实 ncclCommRegister 语义实验" and the capacity growth sequence.
 * ------------------------------------------------------------------------ */
typedef struct {
    uint64_t start, end, id;
    int64_t refs;
} orc_record;

struct orc_registry {
    uint64_t page;
    uint64_t count, capacity, next_id;
    orc_record *rec;
};

orc_registry *orc_reg_create(unsigned page_shift)
{
    orc_registry *g = (orc_registry *)calloc(1, sizeof(*g));
    g->page = 1ull << page_shift;
    g->next_id = 1;
    return g;
}

void orc_reg_destroy(orc_registry *g)
{
    if (!g) return;
    free(g->rec);
    free(g);
}

uint64_t orc_reg_register(orc_registry *g, uint64_t addr, uint64_t size)
{
    if (size == 0 || (u128)addr + size > (u128)UINT64_MAX) return 0;
    uint64_t base = addr & ~(g->page - 1);
    u128 pages = ((u128)addr + size - base + g->page - 1) / g->page;
    u128 top_wide = (u128)base + pages * g->page;
    if (top_wide > (u128)UINT64_MAX) return 0;
    uint64_t top = (uint64_t)top_wide;

    for (uint64_t k = 0; k < g->count; ++k) {
        if (g->rec[k].start <= base && top <= g->rec[k].end) {
            g->rec[k].refs++;
            return g->rec[k].id;
        }
    }
    if (g->count == g->capacity) {
        uint64_t cap = g->capacity == 0 ? 32 : 2 * g->capacity;
        g->rec = (orc_record *)realloc(g->rec, cap * sizeof(orc_record));
        g->capacity = cap;
    }
    uint64_t pos = 0;
    while (pos < g->count && g->rec[pos].start <= base) ++pos;
    memmove(&g->rec[pos + 1], &g->rec[pos], (g->count - pos) * sizeof(orc_record));
    g->rec[pos].start = base;
    g->rec[pos].end = top;
    g->rec[pos].id = g->next_id++;
    g->rec[pos].refs = 1;
    g->count++;
    return g->rec[pos].id;
}

static int64_t find_record(const orc_registry *g, uint64_t handle)
{
    for (uint64_t k = 0; k < g->count; ++k)
        if (g->rec[k].id == handle) return (int64_t)k;
    return -1;
}

int orc_reg_deregister(orc_registry *g, uint64_t handle)
{
    int64_t k = find_record(g, handle);
    if (k < 0) return -1;
    if (--g->rec[k].refs == 0) {
        memmove(&g->rec[k], &g->rec[k + 1], (g->count - (uint64_t)k - 1) * sizeof(orc_record));
        g->count--;
    }
    return 0;
}

int64_t orc_reg_refs(const orc_registry *g, uint64_t handle)
{
    int64_t k = find_record(g, handle);
    return k < 0 ? -1 : g->rec[k].refs;
}

uint64_t orc_reg_count(const orc_registry *g) { return g->count; }
uint64_t orc_reg_capacity(const orc_registry *g) { return g->capacity; }

uint64_t orc_reg_export(const orc_registry *g, uint64_t *start, uint64_t *end,
                        uint64_t *handle, uint64_t max)
{
    uint64_t k = 0;
    for (; k < g->count && k < max; ++k) {
        start[k] = g->rec[k].start;
        end[k] = g->rec[k].end;
        handle[k] = g->rec[k].id;
    }
    return k;
}

/* ------------------------------------------------------------------------
 * O4b  Registry batches.
 *
 * Each item is applied in order with O4's register/deregister, so a batch
 * means exactly what the same calls made one after another mean ([NCCL-26]
 * "Communicator User Registration Cache" and "IB Backend MR Cache"). The
 * record table's room is the caller's: a register batch that would leave more
 * records than the capacity is applied to a copy, found too large, and
 * dropped, and the call reports the capacity O4's growth rule (0 -> 32, then
 * doubling) reaches from the caller's.
 *
 * Pinned by: the register experiment of "真实 ncclCommRegister 语义实验" as
 * one batch and as a deregister batch (the fourth deregister is stale), the
 * 0 -> 32 -> 64 -> 128 growth, and a record-list model in Python replayed
 * over random batches.
 * ------------------------------------------------------------------------ */
uint64_t orc_reg_next_id(const orc_registry *g) { return g->next_id; }

static orc_registry *reg_clone(const orc_registry *g)
{
    orc_registry *c = (orc_registry *)calloc(1, sizeof(*c));
    *c = *g;
    c->rec = NULL;
    if (g->capacity) {
        c->rec = (orc_record *)malloc(g->capacity * sizeof(orc_record));
        memcpy(c->rec, g->rec, g->count * sizeof(orc_record));
    }
    return c;
}

uint64_t orc_reg_register_batch(orc_registry *g, uint64_t capacity,
                                const uint64_t *addr, const uint64_t *size, uint64_t n,
                                uint64_t *handle, uint8_t *kind)
{
    orc_registry *c = reg_clone(g);
    const uint64_t first_new = c->next_id;
    for (uint64_t i = 0; i < n; ++i) {
        const uint64_t before = c->count;
        const uint64_t h = orc_reg_register(c, addr[i], size[i]);
        handle[i] = h;
        if (h == 0) kind[i] = ORC_REG_INVALID;
        else if (h < first_new) kind[i] = ORC_REG_HIT;
        else if (c->count > before) kind[i] = ORC_REG_NEW;
        else kind[i] = ORC_REG_HIT_NEW;
    }
    uint64_t need = capacity;
    while (need < c->count) need = need == 0 ? 32 : 2 * need;
    if (c->count > capacity) {                      /* refused: keep g as it was */
        for (uint64_t i = 0; i < n; ++i) {
            handle[i] = 0;
            kind[i] = ORC_REG_NOSPACE;
        }
        orc_reg_destroy(c);
        return need;
    }
    free(g->rec);
    *g = *c;                                        /* take the copy's records */
    free(c);
    return need;
}

void orc_reg_deregister_batch(orc_registry *g, const uint64_t *handle, uint64_t n,
                              uint8_t *status)
{
    for (uint64_t i = 0; i < n; ++i) {
        const int64_t refs = orc_reg_refs(g, handle[i]);
        if (refs < 0) {
            status[i] = ORC_DEREG_STALE;
            continue;
        }
        orc_reg_deregister(g, handle[i]);
        status[i] = refs == 1 ? ORC_DEREG_REMOVED : ORC_DEREG_OK;
    }
}

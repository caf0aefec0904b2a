/*
 * synth.h - seeded synthetic workloads for the batched DMA-descriptor path.
 *
 * This module only draws random numbers and lays them out as plain arrays
 * (a GPU-page physical-address table, a registered-region table, and a
 * structure-of-arrays request batch). It contains none of the method's
 * arithmetic: no page rounding, no region search, no PRP construction, no
 * queue split. Both the CPU oracle and the GPU library consume its output.
 *
 * Random source: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), written from its published
 * definition. One stream per workload; draw order is the GPU-page table
 * permutation, then the regions, then the requests in index order, so the
 * first k requests of a batch of n are the same as a batch of k.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum synth_workload {
    SYNTH_TINY = 1,     /* 1 GiB heap, 64 regions, 4096 requests, 1 queue          */
    SYNTH_SMALL = 2,    /* 8 GiB heap, 1024 x 8 MiB regions, 1 Mi requests, 64 q    */
    SYNTH_LARGE = 3,    /* 8 GiB heap, no regions, 256 Ki requests 128 KiB-8 MiB    */
    SYNTH_MRHEAVY = 4,  /* no heap, 64 Ki regions, 16 Mi lookup ranges              */
    SYNTH_MIXED = 5     /* 256 GiB heap, 4096 regions, 16 Mi requests, Zipf queues  */
};

typedef struct synth_shape {
    uint64_t n;             /* default request count                                  */
    uint64_t lut_entries;   /* GPU-page table length (64 KiB pages); 0 = no heap      */
    uint64_t regions;       /* registered-region count; 0 = no lookup                 */
    uint32_t nqueues;       /* destination queues; 0 = no split                       */
    uint32_t page_shift;    /* region page size used by the lookup (log2 bytes)       */
    uint64_t va_base;       /* virtual address of heap offset 0 for the lookup        */
    uint64_t list_bus_base; /* bus address of PRP-list pool slot 0                    */
    uint64_t default_seed;  /* seed of the workload's stream                          */
} synth_shape;

/* Fixed address-space constants (high bits set on purpose to expose any
 * 32-bit truncation). */
#define SYNTH_HEAP_VA_BASE   0x0000700000000000ull
#define SYNTH_PHYS_BASE      0x0000200000000000ull
#define SYNTH_LIST_BUS_BASE  0x0000100000000000ull

/* Returns 0 and fills *out, or -1 for an unknown workload. */
int synth_shape_of(int workload, synth_shape *out);

/* Raw SplitMix64: writes k consecutive outputs of the stream seeded with
 * `seed` (used by tests to pin the generator to its published definition). */
void synth_splitmix64(uint64_t seed, uint64_t k, uint64_t *out);

/*
 * Fills caller-allocated host arrays for `workload` with `n` requests
 * (any n; the distribution is the workload's). seed == 0 selects the
 * workload's default seed. Arrays whose count in synth_shape is 0 may be
 * NULL. qid may be NULL for workloads with no queues. Returns 0, or -1 for
 * an unknown workload.
 *   lut     u64[lut_entries]       physical address of each 64 KiB GPU page
 *   rstart  u64[regions]           region start (VA, 4 KiB aligned, sorted)
 *   rend    u64[regions]           region end (exclusive, 4 KiB aligned)
 *   rlkey   u32[regions]           nonzero local key per region
 *   off     u64[n]                 request byte offset (heap offset, or VA
 *                                  for the lookup-only workload)
 *   len     u64[n]                 request length in bytes
 *   qid     u32[n]                 destination queue id
 */
int synth_fill(int workload, uint64_t seed, uint64_t n,
               uint64_t *lut, uint64_t *rstart, uint64_t *rend, uint32_t *rlkey,
               uint64_t *off, uint64_t *len, uint32_t *qid);

/*
 * Starting logical block of each request for the submission-entry stage:
 * uniform over a namespace of SYNTH_NS_BLOCKS blocks, leaving room for the
 * largest command (65536 blocks). Drawn from a stream of its own (the
 * workload's seed xor SYNTH_SLBA_STREAM), so it does not disturb the arrays of
 * synth_fill. Returns 0, or -1 for an unknown workload.
 */
#define SYNTH_NS_BLOCKS     (1ull << 40)
#define SYNTH_SLBA_STREAM   0x51BA51BA51BA51BAull
int synth_fill_slba(int workload, uint64_t seed, uint64_t n, uint64_t *slba);

#ifdef __cplusplus
}
#endif

#endif /* SYNTH_H */

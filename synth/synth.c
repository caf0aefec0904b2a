/*
 * synth.c - seeded synthetic workloads (see synth.h). Draws and lays out
 * random inputs only; holds none of the descriptor-building arithmetic.
 */
#include "synth.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#define KiB 1024ull
#define MiB (1024ull * KiB)
#define GiB (1024ull * MiB)

typedef struct { uint64_t s; } rng_t;

/* SplitMix64 step: advance the Weyl state by the golden-ratio increment,
 * then apply the two xor-shift-multiply finalisation rounds. */
static uint64_t next64(rng_t *r)
{
    uint64_t z = (r->s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Uniform integer in [0, k) by the 128-bit multiply-high map. */
static uint64_t below(rng_t *r, uint64_t k)
{
    return (uint64_t)(((unsigned __int128)next64(r) * k) >> 64);
}

/* Uniform double in [0, 1) from the top 53 bits. */
static double unit(rng_t *r)
{
    return (double)(next64(r) >> 11) * (1.0 / 9007199254740992.0);
}

static uint32_t nonzero32(rng_t *r)
{
    uint32_t v;
    do { v = (uint32_t)(next64(r) >> 32); } while (v == 0);
    return v;
}

void synth_splitmix64(uint64_t seed, uint64_t k, uint64_t *out)
{
    rng_t r = { seed };
    for (uint64_t i = 0; i < k; ++i) out[i] = next64(&r);
}

int synth_shape_of(int w, synth_shape *o)
{
    o->page_shift = 12;
    o->list_bus_base = SYNTH_LIST_BUS_BASE;
    o->va_base = SYNTH_HEAP_VA_BASE;
    o->default_seed = 0xD3A5C0DE00000000ull + (uint64_t)w;
    switch (w) {
    case SYNTH_TINY:
        o->n = 4096; o->lut_entries = (1 * GiB) >> 16; o->regions = 64; o->nqueues = 1;
        return 0;
    case SYNTH_SMALL:
        o->n = 1048576; o->lut_entries = (8 * GiB) >> 16; o->regions = 1024; o->nqueues = 64;
        return 0;
    case SYNTH_LARGE:
        o->n = 262144; o->lut_entries = (8 * GiB) >> 16; o->regions = 0; o->nqueues = 16;
        return 0;
    case SYNTH_MRHEAVY:
        o->n = 16777216; o->lut_entries = 0; o->regions = 65536; o->nqueues = 0;
        o->va_base = 0;   /* request offsets are virtual addresses */
        return 0;
    case SYNTH_MIXED:
        o->n = 16777216; o->lut_entries = (256 * GiB) >> 16; o->regions = 4096; o->nqueues = 64;
        return 0;
    default:
        return -1;
    }
}

/* GPU-page table: a Fisher-Yates permutation of distinct 64 KiB frames
 * above a high physical base. */
static void fill_lut(rng_t *r, uint64_t *lut, uint64_t p)
{
    for (uint64_t i = 0; i < p; ++i) lut[i] = i;
    for (uint64_t i = p; i > 1; --i) {
        uint64_t j = below(r, i);
        uint64_t t = lut[i - 1]; lut[i - 1] = lut[j]; lut[j] = t;
    }
    for (uint64_t i = 0; i < p; ++i) lut[i] = SYNTH_PHYS_BASE + (lut[i] << 16);
}

static uint64_t floor4k(double x) { return ((uint64_t)x) & ~4095ull; }

/* Zipf(s) over q queues, queue 0 most popular: P(k) proportional to (k+1)^-s.
 * Inverse CDF over a precomputed cumulative table. */
static uint32_t zipf_draw(rng_t *r, const double *cdf, uint32_t q)
{
    double u = unit(r);
    for (uint32_t k = 0; k < q; ++k)
        if (u < cdf[k]) return k;
    return q - 1;
}

int synth_fill(int w, uint64_t seed, uint64_t n,
               uint64_t *lut, uint64_t *rstart, uint64_t *rend, uint32_t *rlkey,
               uint64_t *off, uint64_t *len, uint32_t *qid)
{
    synth_shape sh;
    if (synth_shape_of(w, &sh) != 0) return -1;
    rng_t r = { seed ? seed : sh.default_seed };
    const uint64_t P = sh.lut_entries, R = sh.regions;
    const uint64_t heap = P << 16;
    const uint64_t vb = SYNTH_HEAP_VA_BASE;

    if (P) fill_lut(&r, lut, P);

    /* ---- registered regions (sorted, non-overlapping, 4 KiB aligned) ---- */
    if (w == SYNTH_TINY) {
        uint64_t cur = vb;
        for (uint64_t k = 0; k < R; ++k) {
            cur += 64 * KiB * below(&r, 17);           /* gap 0..16 x 64 KiB (0 = abutting) */
            uint64_t size = MiB * (1 + below(&r, 64));  /* 1..64 MiB */
            rstart[k] = cur; rend[k] = cur + size; cur += size;
            rlkey[k] = nonzero32(&r);
        }
    } else if (w == SYNTH_SMALL) {
        for (uint64_t k = 0; k < R; ++k) {             /* 8 MiB regions tiling the heap */
            rstart[k] = vb + k * 8 * MiB; rend[k] = rstart[k] + 8 * MiB;
            rlkey[k] = nonzero32(&r);
        }
    } else if (w == SYNTH_MRHEAVY) {
        uint64_t cur = vb;
        for (uint64_t k = 0; k < R; ++k) {
            cur += floor4k(4.0 * KiB * pow(256.0, unit(&r)));        /* gap 4 KiB..1 MiB  */
            uint64_t size = floor4k(64.0 * KiB * pow(1024.0, unit(&r))); /* 64 KiB..64 MiB */
            rstart[k] = cur; rend[k] = cur + size; cur += size;
            rlkey[k] = nonzero32(&r);
        }
    } else if (w == SYNTH_MIXED) {
        for (uint64_t k = 0; k < R; ++k) {             /* one region per 64 MiB slot */
            uint64_t slot = vb + k * 64 * MiB;
            rstart[k] = slot + 64 * KiB * below(&r, 256);
            rend[k] = slot + 64 * MiB - 64 * KiB * below(&r, 256);
            rlkey[k] = nonzero32(&r);
        }
    }

    /* ---- requests ---- */
    double zcdf[64];
    if (w == SYNTH_MIXED) {
        double acc = 0.0, tot = 0.0;
        for (int k = 0; k < 64; ++k) tot += pow((double)(k + 1), -1.1);
        for (int k = 0; k < 64; ++k) { acc += pow((double)(k + 1), -1.1); zcdf[k] = acc / tot; }
    }
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t o = 0, l = 0; uint32_t q = 0;
        switch (w) {
        case SYNTH_TINY:
            o = 512 * below(&r, heap / 512);
            l = 512 * (1 + below(&r, 256));
            if (l > heap - o) l = heap - o;
            q = 0;
            break;
        case SYNTH_SMALL: {
            l = below(&r, 10) < 9 ? 4096 : 512;
            uint64_t gran = below(&r, 10) < 9 ? 4096 : 512;
            o = gran * below(&r, (heap - l) / gran + 1);
            q = (uint32_t)below(&r, 64);
            break;
        }
        case SYNTH_LARGE:
            l = 4096 * (32 + below(&r, 2017));           /* 128 KiB .. 8 MiB */
            o = 4 * below(&r, (heap - l) / 4 + 1);
            q = (uint32_t)below(&r, 16);
            break;
        case SYNTH_MIXED: {
            double x = floor(pow(2049.0, unit(&r)));     /* log-uniform 1..2048 */
            uint64_t k = x < 1.0 ? 1 : (x > 2048.0 ? 2048 : (uint64_t)x);
            l = 512 * k;
            o = 4 * below(&r, (heap - l) / 4 + 1);
            q = zipf_draw(&r, zcdf, 64);
            break;
        }
        case SYNTH_MRHEAVY: {
            uint64_t cls = below(&r, 10);
            uint64_t k = below(&r, R);
            uint64_t s = rstart[k], e = rend[k];
            if (cls < 3) {                               /* 30%: exact region */
                o = s; l = e - s;
            } else if (cls < 8) {                        /* 50%: strictly inside */
                do {
                    o = s + below(&r, e - s);
                    l = 1 + below(&r, e - o);
                } while (o == s && l == e - s);
            } else if (cls < 9) {                        /* 10%: inside the following gap */
                uint64_t g = (k + 1 < R) ? rstart[k + 1] - e : 1 * MiB;
                o = e + below(&r, g);
                l = 1 + below(&r, e + g - o);
            } else {                                     /* 10%: across a region edge */
                uint64_t edge = below(&r, 2) ? e : s;
                uint64_t d1 = 1 + below(&r, 4096), d2 = 1 + below(&r, 4096);
                o = edge - d1; l = d1 + d2;
            }
            break;
        }
        }
        off[i] = o; len[i] = l;
        if (qid) qid[i] = q;
    }
    return 0;
}

int synth_fill_slba(int w, uint64_t seed, uint64_t n, uint64_t *slba)
{
    synth_shape sh;
    if (synth_shape_of(w, &sh) != 0) return -1;
    rng_t r = { (seed ? seed : sh.default_seed) ^ SYNTH_SLBA_STREAM };
    for (uint64_t i = 0; i < n; ++i) slba[i] = below(&r, SYNTH_NS_BLOCKS - 65536 + 1);
    return 0;
}

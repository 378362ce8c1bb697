/*
 * gen.c -- seeded synthetic inputs for the histogram workloads.
 *
 * This file only draws random bin indices. It holds none of the histogram's
 * arithmetic: both the HIP path and the CPU oracle consume the same bytes
 * that it writes.
 *
 * Random numbers
 * --------------
 * SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used in its counter form: element i
 * (0-based) of the stream with key k is mix(k + (i + 1) * GAMMA). This is the
 * value the sequential generator returns on its (i+1)-th call when started
 * from state k, so a stream can be filled in parallel and stays identical to
 * a sequential fill. Independent sub-streams use key = mix(seed ^ tag) with
 * one fixed tag per purpose.
 *
 * Distributions
 * -------------
 *  uniform   [0, R): the top log2(R) bits of a draw when R is a power of
 *            two (exact), else the high word of draw * R.
 *  zipf      finite Zipf with exponent s over ranks 1..K, P(k) ~ k^-s,
 *            sampled by inverse CDF (smallest k with CDF(k) > u * CDF(K));
 *            rank k maps to bin perm[k-1], perm a Fisher-Yates permutation.
 *  gaussian  Box-Muller (G. Box, M. Muller, 1958): z = sqrt(-2 ln u1)
 *            cos(2 pi u2), value = nearbyint(mu + sigma z), then clamped.
 *  shuffle   Fisher-Yates (Durstenfeld) with bounded draws by D. Lemire,
 *            "Fast random integer generation in an interval" (2019),
 *            multiply-shift with rejection.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

#define TAG_UNIFORM 0x554e49464f524d31ULL
#define TAG_ZIPF    0x5a4950462d52414eULL
#define TAG_PERM    0x5045524d2d5a4950ULL
#define TAG_GAUSS   0x4741555353494e31ULL
#define TAG_SHUFFLE 0x53485546464c4531ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

uint64_t gen_key(uint64_t seed, uint64_t tag) { return mix64(seed ^ tag); }

void gen_stream(uint64_t key, uint64_t first, uint64_t count, uint64_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)count; ++i) out[i] = draw(key, first + (uint64_t)i);
}

static inline int is_pow2(uint64_t r) { return r && !(r & (r - 1)); }

static inline uint32_t bounded_fast(uint64_t v, uint32_t range)
{
    if (is_pow2(range)) {
        unsigned bits = (unsigned)__builtin_ctzll(range);
        return bits ? (uint32_t)(v >> (64 - bits)) : 0u;
    }
    return (uint32_t)(((unsigned __int128)v * range) >> 64);
}

/* out[i] = lo + uniform draw in [0, range) from element (first + i). */
void gen_uniform(uint64_t key, uint64_t first, int32_t *out, uint64_t n, int32_t lo,
                 uint32_t range)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i)
        out[i] = lo + (int32_t)bounded_fast(draw(key, first + (uint64_t)i), range);
}

/* Sequential source of bounded draws for Fisher-Yates. */
typedef struct { uint64_t key, ctr; } seq_rng;

static inline uint64_t seq_next(seq_rng *r) { return draw(r->key, r->ctr++); }

static inline uint64_t seq_bounded(seq_rng *r, uint64_t range)
{
    uint64_t x = seq_next(r);
    unsigned __int128 m = (unsigned __int128)x * range;
    uint64_t l = (uint64_t)m;
    if (l < range) {
        uint64_t t = (0 - range) % range;
        while (l < t) {
            x = seq_next(r);
            m = (unsigned __int128)x * range;
            l = (uint64_t)m;
        }
    }
    return (uint64_t)(m >> 64);
}

/* In-place Fisher-Yates. The draws are independent of the data, so the swap
 * targets are produced a few steps ahead and their cache lines prefetched;
 * the sequence of swaps is exactly the textbook one. */
#define SHUFFLE_AHEAD 32
void gen_shuffle(uint64_t key, int32_t *a, uint64_t n)
{
    if (n < 2) return;
    seq_rng r = {key, 0};
    uint64_t ring[SHUFFLE_AHEAD];
    uint64_t i = n - 1, produced = n - 1; /* next i to produce a target for */
    unsigned head = 0, fill = 0;
    while (fill < SHUFFLE_AHEAD && produced >= 1) {
        uint64_t j = seq_bounded(&r, produced + 1);
        __builtin_prefetch(&a[j], 1, 0);
        ring[(head + fill) % SHUFFLE_AHEAD] = j;
        ++fill;
        --produced;
    }
    for (; i >= 1; --i) {
        uint64_t j = ring[head];
        head = (head + 1) % SHUFFLE_AHEAD;
        --fill;
        if (produced >= 1) {
            uint64_t jn = seq_bounded(&r, produced + 1);
            __builtin_prefetch(&a[jn], 1, 0);
            ring[(head + fill) % SHUFFLE_AHEAD] = jn;
            ++fill;
            --produced;
        }
        int32_t t = a[i];
        a[i] = a[j];
        a[j] = t;
    }
}

/* Fisher-Yates permutation of [0, k). */
void gen_permutation(uint64_t key, int32_t *perm, uint32_t k)
{
    for (uint32_t i = 0; i < k; ++i) perm[i] = (int32_t)i;
    gen_shuffle(key, perm, k);
}

/* Finite Zipf(s) over ranks 1..k, ranks mapped to bins through a random
 * permutation drawn from the seed's "perm" stream. Returns 0 on success. */
int gen_zipf(uint64_t seed, int32_t *out, uint64_t n, uint32_t k, double s)
{
    if (k == 0) return 1;
    double *cdf = (double *)malloc((size_t)k * sizeof(double));
    int32_t *perm = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    if (!cdf || !perm) { free(cdf); free(perm); return 2; }
    double acc = 0.0;
    for (uint32_t r = 1; r <= k; ++r) {
        acc += pow((double)r, -s);
        cdf[r - 1] = acc;
    }
    gen_permutation(gen_key(seed, TAG_PERM), perm, k);
    const uint64_t key = gen_key(seed, TAG_ZIPF);
    const double total = cdf[k - 1];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        double u = (double)(draw(key, (uint64_t)i) >> 11) * 0x1.0p-53;
        double target = u * total;
        uint32_t lo = 0, hi = k - 1; /* smallest index with cdf > target */
        while (lo < hi) {
            uint32_t mid = lo + (hi - lo) / 2;
            if (cdf[mid] > target) hi = mid; else lo = mid + 1;
        }
        out[i] = perm[lo];
    }
    free(cdf);
    free(perm);
    return 0;
}

/* Rounded, clamped Gaussian draws, Box-Muller with one output per pair. */
void gen_gauss(uint64_t key, int32_t *out, uint64_t n, double mu, double sigma, int32_t lo,
               int32_t hi)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t a = draw(key, 2 * (uint64_t)i), b = draw(key, 2 * (uint64_t)i + 1);
        double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
        double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
        double z = sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
        double v = nearbyint(mu + sigma * z);
        if (v < (double)lo) v = (double)lo;
        if (v > (double)hi) v = (double)hi;
        out[i] = (int32_t)v;
    }
}

static uint64_t count_equal(const int32_t *a, uint64_t n, int32_t v)
{
    uint64_t c = 0;
#pragma omp parallel for reduction(+ : c) schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) c += (a[i] == v);
    return c;
}

/*
 * The five benchmark workloads, at any length n (the recipe scales; the
 * published sizes are the defaults in the Python wrapper).
 *   1: uniform [0, 8192), seed 0
 *   2: uniform [0, 65536), seed 1
 *   3: Zipf s = 1.1 over 262144 ranks, ranks permuted to bins, seed 2
 *   4: floor(n/10) copies of bin 524287, the rest uniform [0, 2^20),
 *      shuffled, seed 3.  aux[0] = uniform draws that also hit 524287.
 *   5: floor(n/2) uniform [0, 2^19), the rest rounded Gaussian
 *      (262144, 1000^2) clamped to [0, 2^19 - 1], shuffled, seed 4.
 *      aux[0] = Gaussian draws >= 262144.
 * Returns 0 on success, nonzero for an unknown config or allocation failure.
 */
int gen_config(int cfg, int32_t *out, uint64_t n, uint64_t *aux)
{
    if (aux) aux[0] = 0;
    switch (cfg) {
    case 1:
        gen_uniform(gen_key(0, TAG_UNIFORM), 0, out, n, 0, 8192u);
        return 0;
    case 2:
        gen_uniform(gen_key(1, TAG_UNIFORM), 0, out, n, 0, 65536u);
        return 0;
    case 3:
        return gen_zipf(2, out, n, 262144u, 1.1);
    case 4: {
        const uint64_t hot = n / 10;
        const int32_t hot_bin = 524287;
        for (uint64_t i = 0; i < hot; ++i) out[i] = hot_bin;
        gen_uniform(gen_key(3, TAG_UNIFORM), 0, out + hot, n - hot, 0, 1u << 20);
        if (aux) aux[0] = count_equal(out + hot, n - hot, hot_bin);
        gen_shuffle(gen_key(3, TAG_SHUFFLE), out, n);
        return 0;
    }
    case 5: {
        const uint64_t nu = n / 2;
        gen_uniform(gen_key(4, TAG_UNIFORM), 0, out, nu, 0, 1u << 19);
        gen_gauss(gen_key(4, TAG_GAUSS), out + nu, n - nu, 262144.0, 1000.0, 0,
                  (1 << 19) - 1);
        if (aux) {
            uint64_t c = 0;
            for (uint64_t i = nu; i < n; ++i) c += (out[i] >= 262144);
            aux[0] = c;
        }
        gen_shuffle(gen_key(4, TAG_SHUFFLE), out, n);
        return 0;
    }
    default:
        return 1;
    }
}

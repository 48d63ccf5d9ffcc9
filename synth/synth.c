/*
 * synth.c -- seeded, counter-based synthetic input generator.
 *
 * This module produces the input bytes that both the CPU oracle and the HIP
 * path consume. It holds none of the combine's arithmetic: it only draws
 * random numbers and rounds them to the storage formats (fp32, bf16, fp16).
 *
 * Random stream. Element i of stream `key` is splitmix64(key + (i+1)*GAMMA),
 * where splitmix64 is the output finaliser of Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators" (OOPSLA 2014), with the
 * constants of Vigna's public-domain splitmix64.c. Because every element is a
 * pure function of (key, i), the result does not depend on how the work is
 * split across threads.
 *
 * Uniforms take the top 53 bits of the hash: u = (h >> 11) * 2^-53 in [0,1).
 * Normals use the Box-Muller transform on the pair (2k, 2k+1):
 *   r = sqrt(-2 ln(1 - u0)), z0 = r cos(2 pi u1), z1 = r sin(2 pi u1).
 * Values are computed in fp64, rounded to fp32 by the C cast (round to
 * nearest even), then to bf16 / fp16 by round-to-nearest-even on the bits.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Stream key for (seed, config id, tensor id, sub-stream). */
uint64_t synth_key(uint64_t seed, uint32_t cfg, uint32_t tensor, uint32_t sub) {
    uint64_t tag = ((uint64_t)cfg << 40) ^ ((uint64_t)tensor << 20) ^ (uint64_t)sub;
    return mix64(mix64(seed + GAMMA) ^ mix64(tag + 2 * GAMMA));
}

uint64_t synth_hash(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double u01(uint64_t key, uint64_t i) {
    return (double)(synth_hash(key, i) >> 11) * 0x1.0p-53;
}

/* ---- storage rounding (round to nearest, ties to even) ---- */

static inline uint32_t f32_bits(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    return x;
}

uint16_t synth_f32_to_bf16(float f) {
    uint32_t x = f32_bits(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((x >> 16) & 0x8000u) | 0x7fc0u);
    x += 0x7fffu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

uint16_t synth_f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return (uint16_t)(sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u));
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 rounds to inf */
    if (ax < 0x38800000u) {                                   /* below 2^-14: subnormal */
        int e = (int)(ax >> 23);
        if (e < 102) return (uint16_t)sign; /* < 2^-25 rounds to zero */
        uint32_t m = (ax & 0x7fffffu) | 0x800000u;
        int shift = 126 - e; /* value / 2^-24 = m * 2^(e-126) */
        uint32_t q = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) q++;
        return (uint16_t)(sign | q);
    }
    uint32_t r = ax - 0x38000000u; /* rebias exponent 127 -> 15 */
    r += 0xfffu + ((r >> 13) & 1u);
    return (uint16_t)(sign | (r >> 13));
}

/* ---- fill ---- */

enum { DIST_UNIFORM = 0, DIST_NORMAL = 1 };
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_F16 = 3 };

typedef struct {
    uint64_t key;
    int64_t off;
    int64_t lo_i, hi_i, n;
    int dist, out;
    double a, b;
    void* dst;
} job_t;

static inline double draw(const job_t* j, int64_t i) {
    i += j->off; /* position in the stream */
    if (j->dist == DIST_UNIFORM) return j->a + (j->b - j->a) * u01(j->key, (uint64_t)i);
    int64_t k = i >> 1;
    double u0 = u01(j->key, (uint64_t)(2 * k));
    double u1 = u01(j->key, (uint64_t)(2 * k + 1));
    double r = sqrt(-2.0 * log(1.0 - u0));
    double t = 6.283185307179586476925286766559 * u1;
    double z = (i & 1) ? r * sin(t) : r * cos(t);
    return j->a + j->b * z;
}

static void* run(void* p) {
    const job_t* j = (const job_t*)p;
    for (int64_t i = j->lo_i; i < j->hi_i; ++i) {
        double v = draw(j, i);
        switch (j->out) {
            case OUT_F64: ((double*)j->dst)[i] = v; break;
            case OUT_F32: ((float*)j->dst)[i] = (float)v; break;
            case OUT_BF16: ((uint16_t*)j->dst)[i] = synth_f32_to_bf16((float)v); break;
            default: ((uint16_t*)j->dst)[i] = synth_f32_to_f16((float)v); break;
        }
    }
    return 0;
}

/*
 * Fill dst[0..n) with stream elements off .. off+n-1 of stream `key`.
 * dist: 0 = U[a,b), 1 = N(mean=a, std=b).
 * out: 0 = fp64, 1 = fp32, 2 = bf16 bits, 3 = fp16 bits. nthreads >= 1.
 */
int synth_fill(uint64_t key, int64_t off, int64_t n, int dist, double a, double b, int out,
               void* dst, int nthreads) {
    if (n < 0 || off < 0 || !dst || dist < 0 || dist > 1 || out < 0 || out > 3) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < (1 << 16)) nthreads = 1;
    pthread_t th[64];
    int joined[64];
    job_t jobs[64];
    int64_t per = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        job_t* j = &jobs[t];
        j->key = key;
        j->off = off;
        j->n = n;
        j->dist = dist;
        j->out = out;
        j->a = a;
        j->b = b;
        j->dst = dst;
        j->lo_i = (int64_t)t * per < n ? (int64_t)t * per : n;
        j->hi_i = j->lo_i + per < n ? j->lo_i + per : n;
        joined[t] = 0;
        if (t > 0 && j->lo_i < j->hi_i && pthread_create(&th[t], 0, run, j) == 0) joined[t] = 1;
        else if (t > 0) run(j);
    }
    run(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (joined[t]) pthread_join(th[t], 0);
    return 0;
}

/* Raw uniforms in [0,1) as fp64 (used to place special entries). */
int synth_u01(uint64_t key, int64_t off, int64_t n, double* dst, int nthreads) {
    return synth_fill(key, off, n, DIST_UNIFORM, 0.0, 1.0, OUT_F64, dst, nthreads);
}

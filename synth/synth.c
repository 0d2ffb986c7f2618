/*
 * Seeded synthetic inputs shared by the oracle side and the HIP side of the
 * test and bench harness. This file holds no step of the forward pass: it only
 * draws numbers and encodes them in the storage formats of a GGUF tensor set
 * (F32, F16, and Q8_0 blocks of {fp16 d, int8 qs[32]}).
 *
 * Random numbers come from a counter-based SplitMix64 (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014): draw i of a
 * stream is the SplitMix64 finaliser applied to key + (i + 1) * golden, which is
 * exactly the i-th output of a SplitMix64 generator seeded with `key`. The key of
 * a stream is mix(seed ^ mix(stream_id)), where stream_id is the FNV-1a 64-bit
 * hash of the tensor name. Normal variates come from the Box-Muller transform,
 * one pair per two uniform draws. Because every value depends only on
 * (seed, stream, index), the output is independent of the thread count.
 *
 * The binary16 encoder below is this module's own (round to nearest even,
 * subnormals kept, overflow to infinity), written from IEEE 754-2008.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_fnv1a64(const char* s) {
    uint64_t h = 0xcbf29ce484222325ULL;
    for (; *s; ++s) {
        h ^= (uint8_t)*s;
        h *= 0x100000001b3ULL;
    }
    return h;
}

static uint64_t stream_key(uint64_t seed, uint64_t stream) { return mix64(seed ^ mix64(stream)); }

/* Draw i of the stream (i >= 0). */
uint64_t synth_draw(uint64_t seed, uint64_t stream, int64_t i) {
    return mix64(stream_key(seed, stream) + (uint64_t)(i + 1) * GOLDEN);
}

/* 53-bit uniform in (0, 1] and [0, 1). */
static double u_open0(uint64_t z) { return ((double)(z >> 11) + 1.0) * (1.0 / 9007199254740992.0); }
static double u_closed0(uint64_t z) { return (double)(z >> 11) * (1.0 / 9007199254740992.0); }

/* Standard normal number j of the stream: pair j/2 uses draws 2*(j/2), 2*(j/2)+1. */
static double normal_at(uint64_t key, int64_t j) {
    int64_t p = j >> 1;
    double u1 = u_open0(mix64(key + (uint64_t)(2 * p + 1) * GOLDEN));
    double u2 = u_closed0(mix64(key + (uint64_t)(2 * p + 2) * GOLDEN));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (j & 1) ? r * sin(a) : r * cos(a);
}

static uint16_t enc_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) return sign | (ax > 0x7f800000u ? 0x7e00u : 0x7c00u);
    int e = (int)(ax >> 23) - 127;
    uint32_t full = (ax & 0x7fffffu) | 0x800000u;
    if (e >= -14) {
        /* normal range of binary16: keep 10 fraction bits */
        uint32_t h = ((uint32_t)(e + 15) << 10) | ((full & 0x7fffffu) >> 13);
        uint32_t rem = full & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may reach the exponent */
        if (h >= 0x7c00u) h = 0x7c00u;
        return sign | (uint16_t)h;
    }
    if (ax == 0) return sign;
    int shift = -1 - e; /* subnormal: units of 2^-24 */
    if (shift >= 25) return sign;
    uint32_t q = full >> shift, rem = full & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return sign | (uint16_t)q;
}

uint16_t synth_f16_bits(float f) { return enc_f16(f); }

/* out[i] = mean + std * N_i, stored as float. */
void synth_normal_f32(uint64_t seed, uint64_t stream, double mean, double std, int64_t n, float* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(mean + std * normal_at(key, i));
}

/* Same values as synth_normal_f32, rounded once more to binary16. */
void synth_normal_f16(uint64_t seed, uint64_t stream, double mean, double std, int64_t n, uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = enc_f16((float)(mean + std * normal_at(key, i)));
}

/*
 * Q8_0 blocks drawn directly in the storage format: per block b, the scale is
 * fp16(|N(0, scale_std)|) from normal number b of the stream, and quant j is an
 * integer uniform over [-127, 127] from draw (n_blocks + 32*b + j), taken by the
 * multiply-shift reduction (draw >> 32) * 255 >> 32.
 */
void synth_q8_0(uint64_t seed, uint64_t stream, double scale_std, int64_t n_blocks, uint8_t* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < n_blocks; b++) {
        uint8_t* blk = out + 34 * b;
        uint16_t d = enc_f16((float)fabs(scale_std * normal_at(key, b)));
        blk[0] = (uint8_t)(d & 0xff);
        blk[1] = (uint8_t)(d >> 8);
        for (int j = 0; j < 32; j++) {
            uint64_t z = mix64(key + (uint64_t)(2 * n_blocks + 32 * b + j + 1) * GOLDEN);
            int q = (int)(((z >> 32) * 255u) >> 32) - 127;
            blk[2 + j] = (uint8_t)(int8_t)q;
        }
    }
}

/* Token ids uniform over [0, vocab). */
void synth_uniform_ids(uint64_t seed, uint64_t stream, int32_t vocab, int64_t n, int32_t* out) {
    uint64_t key = stream_key(seed, stream);
    for (int64_t i = 0; i < n; i++) {
        uint64_t z = mix64(key + (uint64_t)(i + 1) * GOLDEN);
        out[i] = (int32_t)(((z >> 32) * (uint64_t)vocab) >> 32);
    }
}

/* Floats uniform over [lo, hi). */
void synth_uniform_f32(uint64_t seed, uint64_t stream, double lo, double hi, int64_t n, float* out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(lo + (hi - lo) * u_closed0(mix64(key + (uint64_t)(i + 1) * GOLDEN)));
}

/*
 * Seeded, counter-based input generator for the quantized MoE FFN layer.
 *
 * This file holds no arithmetic of the method itself: it only draws random
 * words, uniforms and normals and rounds them to bf16 bit patterns.  Both
 * the CPU oracle and the GPU path are fed from it; neither includes it.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Draw i of a stream with
 * key K is mix64(K + (i + 1) * GAMMA), so any element can be produced
 * without producing the ones before it.  A stream key is derived from the
 * (seed, stream id) pair with the same mixing function.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64(stream + SYNTH_GAMMA));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * SYNTH_GAMMA);
}

/* float -> bf16 bit pattern, round to nearest even (finite inputs only). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* 32-bit words first .. first+n-1 of a stream: word w is the low (w even)
 * or high (w odd) half of draw w/2. */
void synth_u32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, uint32_t* out) {
    uint64_t key = stream_key(seed, stream);
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t w = first + j;
        uint64_t d = draw(key, w >> 1);
        out[j] = (w & 1) ? (uint32_t)(d >> 32) : (uint32_t)d;
    }
}

/* Raw 64-bit draws first .. first+n-1. */
void synth_u64(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, uint64_t* out) {
    uint64_t key = stream_key(seed, stream);
    for (uint64_t j = 0; j < n; ++j) out[j] = draw(key, first + j);
}

/* bf16(lo + (hi - lo) * u), u = top 24 bits of draw i scaled to [0, 1),
 * computed in fp32 and rounded to bf16 (nearest even). */
void synth_uniform_bf16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                        float lo, float hi, uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t d = draw(key, first + j);
        float u = (float)(d >> 40) * (1.0f / 16777216.0f);
        out[j] = f32_to_bf16_rne(lo + (hi - lo) * u);
    }
}

/* bf16 of a standard normal by Box-Muller on draws 2i and 2i+1:
 * z = sqrt(-2 ln u1) cos(2 pi u2), u1 in (0, 1], u2 in [0, 1), computed in
 * double, then rounded to fp32 and to bf16 (nearest even). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, uint16_t* out) {
    uint64_t key = stream_key(seed, stream);
    const double two_pi = 6.283185307179586476925286766559;
    for (uint64_t j = 0; j < n; ++j) {
        uint64_t i = first + j;
        uint64_t d1 = draw(key, 2 * i), d2 = draw(key, 2 * i + 1);
        double u1 = ((double)(d1 >> 11) + 1.0) * (1.0 / 9007199254740992.0);
        double u2 = (double)(d2 >> 11) * (1.0 / 9007199254740992.0);
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[j] = f32_to_bf16_rne((float)z);
    }
}

/* Bias bit patterns -mid * scale for bf16 scales, mid a power of two:
 * the product is exact in bf16, so this is an exponent shift of each scale. */
void synth_neg_mul_bf16(const uint16_t* scales, uint64_t n, float mid, uint16_t* out) {
    for (uint64_t j = 0; j < n; ++j) {
        uint32_t u = (uint32_t)scales[j] << 16;
        float s;
        memcpy(&s, &u, 4);
        out[j] = f32_to_bf16_rne(-mid * s);
    }
}

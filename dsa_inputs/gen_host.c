/*
 * gen_host.c -- seeded, counter-based synthetic inputs (host twin).
 *
 * This module holds no arithmetic of the attention method; it only produces
 * random tensors.  The device twin (gen_device.hip) implements the same
 * definition and produces bit-identical values.
 *
 * Definition (SplitMix64, Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014):
 *   G        = 0x9E3779B97F4A7C15
 *   mix(z)   : z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   sm(x)    = mix(x + G)                      (all arithmetic mod 2^64)
 *   key      = sm(sm(seed) ^ tensor_id)
 *   draw(i,j)= sm(key + G * (4*i + j))          j in {0,1,2}
 *   normal(i): S = sum of the twelve 16-bit fields of draw(i,0..2);
 *              N = (S - 393210) / 65536  (exact in fp32; mean 0, variance 1 - 2^-32,
 *              Irwin-Hall approximation with tails cut at +-6), then rounded to bf16 (RNE).
 *   uniform(i) = (draw(i,0) >> 40) / 2^24     (exact fp32 in [0,1))
 */
#include <stdint.h>
#include <string.h>

#define G 0x9E3779B97F4A7C15ULL

static uint64_t mix(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static uint64_t sm(uint64_t x) { return mix(x + G); }

uint64_t gen_key(uint64_t seed, uint64_t tensor_id) { return sm(sm(seed) ^ tensor_id); }

uint64_t gen_draw(uint64_t key, uint64_t i, uint64_t j) { return sm(key + G * (4 * i + j)); }

static float normal_f32(uint64_t key, uint64_t i) {
    int64_t s = 0;
    int j, f;
    for (j = 0; j < 3; j++) {
        uint64_t x = gen_draw(key, i, (uint64_t)j);
        for (f = 0; f < 4; f++) s += (int64_t)((x >> (16 * f)) & 0xFFFF);
    }
    return (float)(s - 393210) / 65536.0f;   /* |s-393210| < 2^19: exact */
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFF + ((u >> 16) & 1);           /* inputs are finite */
    return (uint16_t)(u >> 16);
}

/* out[t] = bf16(normal(start + t)), t < n */
void gen_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t n, uint16_t* out) {
    uint64_t key = gen_key(seed, tensor_id);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) out[t] = f32_to_bf16_rne(normal_f32(key, start + (uint64_t)t));
}

/* Gather form: out[t] = bf16(normal(index[t])). */
void gen_normal_bf16_at(uint64_t seed, uint64_t tensor_id, const int64_t* index, int64_t n, uint16_t* out) {
    uint64_t key = gen_key(seed, tensor_id);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) out[t] = f32_to_bf16_rne(normal_f32(key, (uint64_t)index[t]));
}

/* out[t] = uniform(start + t) * mul, the product evaluated in double and rounded to fp32. */
void gen_uniform_f32(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t n, double mul, float* out) {
    uint64_t key = gen_key(seed, tensor_id);
    int64_t t;
    for (t = 0; t < n; t++) {
        double u = (double)(gen_draw(key, start + (uint64_t)t, 0) >> 40) / 16777216.0;
        out[t] = (float)(u * mul);
    }
}

/* Raw 64-bit draws (sub-index 0), for permutations and integer choices. */
void gen_u64(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t n, uint64_t* out) {
    uint64_t key = gen_key(seed, tensor_id);
    int64_t t;
    for (t = 0; t < n; t++) out[t] = gen_draw(key, start + (uint64_t)t, 0);
}

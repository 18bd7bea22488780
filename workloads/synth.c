/*
 * Seeded synthetic inputs for the sparse-MoE layer workloads.
 *
 * This file holds no part of the layer's arithmetic: it only draws numbers.
 * Both the GPU path's tests and the CPU oracle receive tensors made here.
 *
 * Generator (counter-based, so every element is independent of thread count
 * and of the tensor's total length):
 *   key(seed, tag) = mix(mix(seed) ^ tag)
 *   word(i)        = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
 * where mix() is the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Elements 2p and 2p+1 share word(p): its high and low 32 bits give u1, u2 in
 * (0,1), and the Box-Muller transform gives the pair
 *   z(2p) = sqrt(-2 ln u1) * cos(2 pi u2),  z(2p+1) = sqrt(-2 ln u1) * sin(2 pi u2),
 * two independent standard normals.
 * value = fp32(z * std) rounded to nearest even, then to bfloat16 (RNE).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16); /* inf/nan: never drawn */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t tag) { return mix64(mix64(seed) ^ tag); }

static void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  uint64_t w = mix64(key + (p + 1) * 0x9E3779B97F4A7C15ULL);
  double u1 = ((double)(w >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(w & 0xFFFFFFFFu) + 0.5) * (1.0 / 4294967296.0);
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(th);
  *z1 = r * sin(th);
}

/* calls emit(j, z) for every element index j in [start, start + n) */
#define FOR_EACH_NORMAL(key, start, n, BODY)                                     \
  do {                                                                           \
    uint64_t p0 = (start) >> 1, p1 = ((start) + (uint64_t)(n) + 1) >> 1;         \
    _Pragma("omp parallel for schedule(static)")                                 \
    for (int64_t pp = (int64_t)p0; pp < (int64_t)p1; ++pp) {                     \
      double zz[2];                                                              \
      normal_pair((key), (uint64_t)pp, &zz[0], &zz[1]);                          \
      for (int h = 0; h < 2; ++h) {                                              \
        uint64_t i = 2 * (uint64_t)pp + (uint64_t)h;                             \
        if (i < (start) || i >= (start) + (uint64_t)(n)) continue;              \
        int64_t j = (int64_t)(i - (start));                                      \
        double z = zz[h];                                                        \
        BODY;                                                                    \
      }                                                                          \
    }                                                                            \
  } while (0)

/* out[j] = bf16(fp32(normal(key, start + j) * std)), j in [0, n) */
void synth_normal_bf16(uint64_t key, uint64_t start, int64_t n, double std, uint16_t* out) {
  FOR_EACH_NORMAL(key, start, n, out[j] = f32_to_bf16_rne((float)(z * std)));
}

/* Same draw, kept in fp32 (used for checks of the generator itself). */
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, double std, float* out) {
  FOR_EACH_NORMAL(key, start, n, out[j] = (float)(z * std));
}

/* Integer-valued draw: multiples of 2^-3 in [-2, 2] (exactly representable in bf16),
 * used where a test needs every dot product to be exact. */
void synth_grid_bf16(uint64_t key, uint64_t start, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint64_t w = mix64(key + (start + (uint64_t)j + 1) * 0x9E3779B97F4A7C15ULL);
    int v = (int)(w % 33u) - 16;               /* -16..16 */
    out[j] = f32_to_bf16_rne((float)v * 0.125f);
  }
}

/*
 * Seeded synthetic inputs for the dense-decoder workloads: weights, prompts,
 * 4-bit affine codes and uniform draws.  This file holds no part of the
 * decoder's arithmetic; both the CPU oracle and the GPU library consume the
 * host arrays it writes.
 *
 * Generator (counter based, so any element can be produced independently and
 * the result does not depend on the thread count):
 *   SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
 *   pseudorandom number generators", OOPSLA 2014) applied to the state
 *       s = key + (ctr + 1) * 0x9E3779B97F4A7C15
 *   u = ((z >> 11) + 1) * 2^-53              in (0, 1]
 *   normal: Box-Muller cosine branch, element i uses counters 2i and 2i+1
 *       n = sqrt(-2 ln u1) * cos(2 pi u2)
 *   bf16: value -> fp32 (round to nearest even) -> bf16 (round to nearest even)
 *   key  = seed XOR FNV-1a-64(tensor tag)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t splitmix64_at(uint64_t key, uint64_t ctr) {
  uint64_t z = key + (ctr + 1ULL) * GOLDEN_GAMMA;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double unit_open0(uint64_t z) {
  return (double)((z >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unit_open0(splitmix64_at(key, 2 * i));
  double u2 = unit_open0(splitmix64_at(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

uint64_t synth_fnv1a64(const char* s) {
  uint64_t h = 0xcbf29ce484222325ULL;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001b3ULL;
  }
  return h;
}

uint64_t synth_splitmix64(uint64_t key, uint64_t ctr) { return splitmix64_at(key, ctr); }

/* out[i] = bf16(std * N(0,1)), optionally |.| when absval != 0 */
void synth_normal_bf16(uint64_t key, int64_t n, double std, int absval, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v = std * normal_at(key, (uint64_t)i);
    if (absval) v = fabs(v);
    out[i] = f32_to_bf16_rne((float)v);
  }
}

void synth_normal_f32(uint64_t key, int64_t n, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(std * normal_at(key, (uint64_t)i));
}

void synth_normal_f64(uint64_t key, int64_t n, double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = std * normal_at(key, (uint64_t)i);
}

/* uniform integers in [0, range): multiply-shift of the high 32 bits */
void synth_uniform_int(uint64_t key, int64_t n, int32_t range, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t z = splitmix64_at(key, (uint64_t)i);
    out[i] = (int32_t)(((z >> 32) * (uint64_t)(uint32_t)range) >> 32);
  }
}

/* uniform doubles in (0, 1] */
void synth_uniform_f64(uint64_t key, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unit_open0(splitmix64_at(key, (uint64_t)i));
}

/* 4-bit codes: code of element e = top 4 bits of draw e; eight codes per
 * uint32 word, element 8w+j in bits 4j..4j+3 of word w (least significant
 * nibble first).  n_elems must be a multiple of 8. */
void synth_q4_codes(uint64_t key, int64_t n_elems, uint32_t* out) {
  int64_t n_words = n_elems / 8;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < n_words; ++w) {
    uint32_t word = 0;
    for (int j = 0; j < 8; ++j) {
      uint64_t z = splitmix64_at(key, (uint64_t)(8 * w + j));
      word |= (uint32_t)(z >> 60) << (4 * j);
    }
    out[w] = word;
  }
}

/* Fill one fp32 tensor with a constant (norm gains). */
void synth_fill_f32(int64_t n, float v, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = v;
}

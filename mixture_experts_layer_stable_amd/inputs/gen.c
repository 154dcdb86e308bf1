/*
 * Seeded synthetic inputs for the MoE layer workloads.
 *
 * This file holds no arithmetic of the MoE layer itself: it only turns a
 * (seed, stream, index) triple into numbers. It is shared by the test and
 * benchmark harness, which hands the same arrays to the oracle and to the GPU
 * library.
 *
 * Generator: a counter-based stream built on the SplitMix64 finaliser
 * (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014). Word w of stream s is mix64(key_s + (w+1)*gamma).
 *
 * Normal deviates: the textbook "sum of twelve uniforms minus six"
 * (Irwin-Hall, n = 12) approximation of N(0,1), done in exact integer
 * arithmetic on 16-bit uniforms, so every platform produces the same bits:
 *   z = (sum_{q<12} u_q - 6*65535) / 65536,  u_q uniform on {0..65535}.
 * z has mean 0 and variance 1 - 2^-32. The float product z*scale is a single
 * IEEE multiply and the bf16 conversion is round-to-nearest-even on the bits.
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 0x8CB92BA72F3D8DD7ULL));
}

static inline uint64_t word_at(uint64_t key, uint64_t w) { return mix64(key + (w + 1) * GAMMA); }

static inline float normal_at(uint64_t key, uint64_t i) {
  int64_t s = 0;
  for (int q = 0; q < 3; ++q) {
    uint64_t w = word_at(key, 3 * i + (uint64_t)q);
    s += (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) + (int64_t)((w >> 32) & 0xFFFF) +
         (int64_t)(w >> 48);
  }
  s -= 6 * 65535;                      /* |s| <= 393210 < 2^19: exact in float */
  return (float)s * (1.0f / 65536.0f); /* power-of-two scale: exact */
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40); /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* n normal deviates of stream (seed, stream) starting at element `offset`,
 * times `scale`. out_kind 0: float32 array; 1: bf16 bit patterns (uint16). */
void mok_gen_normal(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, float scale, int out_kind,
                    void* out) {
  const uint64_t key = stream_key(seed, stream);
  if (out_kind == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) o[i] = normal_at(key, offset + (uint64_t)i) * scale;
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) o[i] = f32_to_bf16_rne(normal_at(key, offset + (uint64_t)i) * scale);
  }
}

/* n raw 64-bit words of stream (seed, stream) starting at word `offset`. */
void mok_gen_words(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, uint64_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = word_at(key, offset + (uint64_t)i);
}

/*
 * Seeded synthetic inputs for the NVFP4 fused-MoE workloads.
 *
 * This module is shared by the CPU oracle side and the GPU side of every test
 * and benchmark. It draws random numbers and nothing else: it holds none of
 * the MoE method's arithmetic (no routing, no NVFP4 encoding, no GEMM).
 *
 * Generator (counter-based, stateless, thread-order independent):
 *   splitmix64 finaliser  sm(z) = mix(z + 0x9E3779B97F4A7C15)
 *   bits(seed, stream, i) = sm(sm(sm(seed) ^ stream) ^ i)
 *   uniform(seed, stream, i) = ((bits >> 11) + 0.5) * 2^-53      in (0, 1)
 *   normal(seed, stream, i)  = sqrt(-2 ln u1) * cos(2 pi u2)       (Box-Muller, fp64)
 *                              u1 = uniform(.., 2i), u2 = uniform(.., 2i+1)
 * A value drawn at index i depends only on (seed, stream, i), so any slice of
 * a tensor can be regenerated on its own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t i) {
  return sm_mix(sm_mix(sm_mix(seed) ^ stream) ^ i);
}

static inline double synth_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
  return ((double)(synth_bits(seed, stream, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = synth_uniform(seed, stream, 2 * i);
  double u2 = synth_uniform(seed, stream, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* out[j] = (float)(mean + sigma * normal(seed, stream, offset + j)), j < n */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      double mean, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = (float)(mean + sigma * synth_normal(seed, stream, offset + (uint64_t)j));
}

/* Round a binary32 value to bfloat16 (round to nearest, ties to even). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[j] = bf16((float)(sigma * normal(seed, stream, offset + j))), j < n */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = f32_to_bf16_rne((float)(sigma * synth_normal(seed, stream, offset + (uint64_t)j)));
}

/* A seeded permutation of 1..n (Fisher-Yates driven by synth_bits). */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i + 1;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(synth_bits(seed, stream, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* logits[t][e] = (float)(normal(seed, stream, offset + t*E + e) + bias[e]) */
void synth_logits(uint64_t seed, uint64_t stream, uint64_t offset, int32_t T, int32_t E,
                  const double* bias, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)T * E; ++i) {
    double b = bias ? bias[i % E] : 0.0;
    out[i] = (float)(synth_normal(seed, stream, offset + (uint64_t)i) + b);
  }
}

/* n bytes: byte i = lo + (b_i mod span) (span in 1..256), b_i = byte (i mod 8) of
 * bits(seed, stream, i / 8) (little-endian), i counted from offset. */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, uint32_t lo, uint32_t span,
                 uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t j = offset + (uint64_t)i;
    const uint32_t b = (uint32_t)(synth_bits(seed, stream, j >> 3) >> (8 * (j & 7))) & 0xFFu;
    out[i] = (uint8_t)(lo + b % span);
  }
}

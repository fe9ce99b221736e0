// Device helpers of the row quantisers shared by the quantiser kernels and the routing
// kernels (which quantise the activation rows of small batches beside the routing work).
// The steps are comparisons, maxima, exact power-of-two scalings, roundings, and the
// binary32 products and quotients of the NVFP4 rule (6 gs, E4M3(s) gs, |v| / d); no product
// feeds an addition, so FP contraction cannot fuse anything and change a byte.
#pragma once
#include "common.hpp"

namespace nvmoe {

__device__ __forceinline__ void load16(const uint16_t* p, float* v) {
  const u32x4 a = *(const u32x4*)p;
  const u32x4 b = *(const u32x4*)(p + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load16(const float* p, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 a = *(const f32x4*)(p + 4 * i);
    v[4 * i] = a.x;
    v[4 * i + 1] = a.y;
    v[4 * i + 2] = a.z;
    v[4 * i + 3] = a.w;
  }
}

// Nearest E2M1 magnitude code to r >= 0 (ties to the even code), saturating at 6.
// Signed E2M1 value of a code (sign in bit 3): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;   // m >= 2: (1 or 1.5) 2^(m/2 - 1); m = 1: 0.5; m = 0: 0
  const float v = m < 2u ? 0.5f * (float)m : __builtin_ldexpf((m & 1u) ? 1.5f : 1.0f, (int)(m >> 1) - 1);
  return (c & 8u) ? -v : v;
}

__device__ __forceinline__ uint32_t e2m1_encode_rne_sat(float r) {
  return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) + (uint32_t)(r >= 1.75f) +
         (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) + (uint32_t)(r > 5.0f);
}

// Quantise one 16-element block with global scale gs; writes 8 code bytes and 1 scale byte,
// and with x16 != nullptr the 16 decoded values without the global scale, E2M1(code) x
// E4M3(s), as fp16 (at most 6 significant bits in [2^-10, 2688]: exact), the operands of the
// fp16 MFMAs of the prefill GEMMs, whose epilogue applies gs.
__device__ __forceinline__ void quant_block(const float* v, float gs, uint8_t* packed, uint8_t* scale,
                                            uint16_t* x16 = nullptr) {
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
  uint32_t s = 0u;
  if (gs != 0.0f) {
    const float six_gs = 6.0f * gs;
    s = e4m3_encode_rne_sat(ab / six_gs);
  }
  const float d = e4m3_to_f32(s) * gs;
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t code = (__float_as_uint(v[i]) >> 31) << 3;
    if (d != 0.0f) code |= e2m1_encode_rne_sat(fabsf(v[i]) / d);
    if (i < 8)
      lo |= code << (4 * i);
    else
      hi |= code << (4 * (i - 8));
  }
  *(u32x2*)packed = u32x2{lo, hi};
  *scale = (uint8_t)s;
  if (x16) {
    const float sv = e4m3_to_f32(s);
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const uint32_t c0 = ((i < 8 ? lo : hi) >> (4 * (i & 7))) & 15u, c1 = ((i < 8 ? lo : hi) >> (4 * ((i + 1) & 7))) & 15u;
      const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(e2m1_value(c0) * sv));
      const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(e2m1_value(c1) * sv));
      q[i / 2] = h0 | (h1 << 16);
    }
    *(u32x4*)x16 = u32x4{q[0], q[1], q[2], q[3]};
    *(u32x4*)(x16 + 8) = u32x4{q[4], q[5], q[6], q[7]};
  }
}

template <typename T>
__device__ __forceinline__ float wave_row_absmax(const T* row, int K) {
  const int lane = threadIdx.x & (WAVE - 1);
  float m = 0.0f;
  for (int b = lane; b < K / 16; b += WAVE) {
    float v[16];
    load16(row + (size_t)b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
  return m;
}

template <typename T>
__device__ __forceinline__ void wave_quant_row(const T* row, int K, float gs, uint8_t* packed, uint8_t* scales,
                                               uint16_t* x16) {
  const int lane = threadIdx.x & (WAVE - 1);
  for (int b = lane; b < K / 16; b += WAVE) {
    float v[16];
    load16(row + (size_t)b * 16, v);
    quant_block(v, gs, packed + (size_t)b * 8, scales + b, x16 ? x16 + (size_t)b * 16 : nullptr);
  }
}

// One wave quantises one row: its global scale gs = max|x| / 2688 (written to *gs_out by
// lane 0), then its 16-column blocks (and, with x16, their decoded fp16 values).
template <typename T>
__device__ __forceinline__ void nvfp4_row_wave(const T* row, int K, uint8_t* packed, uint8_t* scales, float* gs_out,
                                               uint16_t* x16 = nullptr) {
  const float g = wave_row_absmax(row, K) / 2688.0f;
  if ((threadIdx.x & (WAVE - 1)) == 0) *gs_out = g;
  wave_quant_row(row, K, g, packed, scales, x16);
}

// MXFP8 rows (the W4A8 profile's activations): per 32 consecutive k one E8M0 scale 2^X with
// X = floor(log2 max|x|) - 8 (8 = the exponent of E4M3's largest normal, 448 = 1.75 2^8),
// clamped to [-127, 127] (-127 for a zero block or one below 2^-118), and E4M3 codes of
// |x| 2^-X (exact power-of-two scaling, round to nearest even, saturating at 448) with the
// sign of x. One wave per row, a lane per 32-column block.
template <typename T>
__device__ __forceinline__ void mxfp8_row_wave(const T* row, int K, uint8_t* codes, uint8_t* scales, int lane) {
  for (int b = lane; b < K / 32; b += WAVE) {
    float v[32];
    load16(row + (size_t)b * 32, v);
    load16(row + (size_t)b * 32 + 16, v + 16);
    float A = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) A = fmaxf(A, fabsf(v[i]));
    // A = f 2^E with f in [0.5, 1): floor(log2 A) = E - 1; below 2^-118 the clamp decides
    int X = A < 0x1p-118f ? -127 : min(__builtin_amdgcn_frexp_expf(A) - 1 - 8, 127);
    scales[b] = (uint8_t)(X + 127);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t word = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = v[4 * q + i];
        const uint32_t code = ((__float_as_uint(e) >> 31) << 7) | e4m3_encode_rne_sat(__builtin_ldexpf(fabsf(e), -X));
        word |= code << (8 * i);
      }
      w[q] = word;
    }
    uint8_t* dst = codes + (size_t)b * 32;
    *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
    *(u32x4*)(dst + 16) = u32x4{w[4], w[5], w[6], w[7]};
  }
}

// FP8 rows with one scale per row (the W4A8 path on NVFP4 weights): s = max|x| / 448 in
// binary32 (448 = E4M3's largest value), codes sign << 7 | E4M3_rne_sat(|x| / s) (binary32
// division; 0 where s is 0). One wave per row, a lane per 16-column block; writes the scale
// (lane 0), the codes when `codes` is set and, when `x16` is set, their exact fp16 decode
// E4M3(code) without the scale (E4M3 is a subset of fp16), the operands of the fp16 MFMAs,
// whose epilogue applies s.
template <typename T>
__device__ __forceinline__ void fp8_row_wave(const T* row, int K, uint8_t* codes, float* s_out, uint16_t* x16,
                                             int lane) {
  const float s = wave_row_absmax(row, K) / 448.0f;
  if (lane == 0) *s_out = s;
  for (int b = lane; b < K / 16; b += WAVE) {
    float v[16];
    load16(row + (size_t)b * 16, v);
    uint32_t w[4] = {0u, 0u, 0u, 0u}, h[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t sign = (__float_as_uint(v[i]) >> 31) << 7;
      const uint32_t code = sign | (s != 0.0f ? e4m3_encode_rne_sat(fabsf(v[i]) / s) : 0u);
      w[i >> 2] |= code << (8 * (i & 3));
      const uint32_t f = __builtin_bit_cast(uint16_t, (_Float16)e4m3_to_f32(code));
      if (i & 1)
        h[i >> 1] |= f << 16;
      else
        h[i >> 1] = f;
    }
    if (codes) *(u32x4*)(codes + (size_t)b * 16) = u32x4{w[0], w[1], w[2], w[3]};
    if (x16) {
      *(u32x4*)(x16 + (size_t)b * 16) = u32x4{h[0], h[1], h[2], h[3]};
      *(u32x4*)(x16 + (size_t)b * 16 + 8) = u32x4{h[4], h[5], h[6], h[7]};
    }
  }
}

__device__ __forceinline__ float bf16x8_absmax(const u32x4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
  return m;
}
__device__ __forceinline__ u32x4 bf16x8_to_f16(const u32x4& v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = (_Float16)(__uint_as_float(w[i] << 16) * scale);
    const _Float16 hi = (_Float16)(__uint_as_float(w[i] & 0xFFFF0000u) * scale);
    o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}
// NV 16-byte pieces per lane per pass, all loaded before any is used (indices clamped to the
// last piece, so no load is conditional and the repeats change no maximum); a row of at most
// 64 NV pieces is converted from the registers of its first read.
template <int NV>
__device__ __forceinline__ void f16_row_wave_nv(const uint16_t* row, int npc, uint16_t* out, float* xf_out, int lane) {
  u32x4 v[NV];
  float m = 0.0f;
  for (int c0 = 0; c0 < npc; c0 += WAVE * NV) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = *(const u32x4*)(row + (size_t)min(c0 + lane + WAVE * i, npc - 1) * 8);
#pragma unroll
    for (int i = 0; i < NV; ++i) m = fmaxf(m, bf16x8_absmax(v[i]));
  }
#pragma unroll
  for (int off = WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
  int p = 0;
  if (m > 0.0f) p = 14 - ((int)((__float_as_uint(m) >> 23) & 0xFFu) - 127);
  p = p < -126 ? -126 : (p > 126 ? 126 : p);
  const float scale = __uint_as_float((uint32_t)(p + 127) << 23);
  if (lane == 0) *xf_out = __uint_as_float((uint32_t)(127 - p) << 23);
  const bool held = npc <= WAVE * NV;
  for (int c0 = 0; c0 < npc; c0 += WAVE * NV) {
    if (!held) {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = *(const u32x4*)(row + (size_t)min(c0 + lane + WAVE * i, npc - 1) * 8);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = c0 + lane + WAVE * i;
      if (c < npc) *(u32x4*)(out + (size_t)c * 8) = bf16x8_to_f16(v[i], scale);
    }
  }
}
// bf16 activation rows -> fp16 for the gate_up MFMA: every row is multiplied by the power
// of two 2^p that puts its max |x| in [2^14, 2^15) (p clamped to [-126, 126]), which is exact
// for every element whose scaled magnitude is a normal fp16 (>= 2^-14, i.e. >= 2^-28 of the
// row maximum; smaller ones round to the fp16 subnormal grid). The epilogue multiplies by
// xf[r] = 2^-p. One wave per row; xf_out is the row's factor.
__device__ __forceinline__ void f16_row_wave(const uint16_t* row, int K, uint16_t* out, float* xf_out, int lane) {
  const int npc = K / 8;
  if (npc <= WAVE * 2)
    f16_row_wave_nv<2>(row, npc, out, xf_out, lane);
  else if (npc <= WAVE * 4)
    f16_row_wave_nv<4>(row, npc, out, xf_out, lane);
  else
    f16_row_wave_nv<8>(row, npc, out, xf_out, lane);
}

}  // namespace nvmoe

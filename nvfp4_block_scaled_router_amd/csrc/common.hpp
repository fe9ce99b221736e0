// Device-side helpers shared by the HIP kernels of libnvfp4moe.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int KCHUNK = 128;        // K elements per pipeline chunk (64 bytes of E2M1 per row)
constexpr int SCALE_GROUP = 8;     // K chunks whose block scales one lane loads at once (16 bytes)

// ------------------------------------------------------------------ packed layout
// One NVFP4 projection of G experts, N rows, K columns, after moe_pack_weights:
//   fp4 tiles   [G][N/16][K/128][64 lanes][16 B]  lane l of a 16-row tile holds row
//               (l % 16), columns 32*(l/16) .. +31 of the 128-column chunk
//   scale tiles [G][N/16][ceil(K/1024)][64 lanes][16 B]  byte 2c+h of lane l holds the
//               block scale of row (l % 16), block 8*(8*sg + c) + 2*(l/16) + h
//   global      [G] f32
// For gate_up the 16-row tiles alternate gate and up: tile 2q is gate rows 16q..16q+15,
// tile 2q+1 is up rows 16q..16q+15 (boundary rows I+16q..), so one wave holds the gate
// and up accumulators of the same output columns.
struct ProjLayout {
  int N, K, KC, KSG;               // rows, columns, K chunks, scale groups
  size_t fp4_expert, sc_expert;    // bytes per expert
};

// Raw buffer resource (base, byte range; stride 0, 32-bit data format) for buffer loads with
// a 32-bit per-lane offset and a scalar offset: the base stays in SGPRs, and an access at or
// past `bytes` reads 0 instead of memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__host__ __device__ inline ProjLayout proj_layout(int N, int K) {
  ProjLayout p;
  p.N = N;
  p.K = K;
  p.KC = K / KCHUNK;
  p.KSG = (p.KC + SCALE_GROUP - 1) / SCALE_GROUP;
  p.fp4_expert = (size_t)(N / 16) * p.KC * WAVE * 16;
  p.sc_expert = (size_t)(N / 16) * p.KSG * WAVE * 16;
  return p;
}

// ------------------------------------------------------------------ number formats

// E4M3fn byte -> fp32 (exact). 0x7F/0xFF (NaN) are rejected by host validation. The
// subnormal path is a branch that whole waves skip in practice; this form measured about
// 10% faster in the decode GEMMs than a select between both paths or the hardware fp8
// convert.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -v : v;
}

// Two E4M3fn bytes (bits 0..15) -> two fp16 values, by the hardware fp8 convert (scale
// operand 1). Every E4M3 value, subnormals included, is exact in fp16.
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t b2) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b2, 1.0f, false);
}

// Eight E2M1 codes times one E4M3 block scale s (given as the fp16 pair {s, s}) as fp16:
// the fp4 convert, then one packed fp16 multiply. q * s has at most 6 significant bits and
// lies in [2^-10, 2688], inside fp16's normal range, so the product is exact.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s) {
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s);
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s);
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s);
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s);
  return __builtin_bit_cast(f16x8, o);
}

// Nearest E4M3fn code to v >= 0, ties to even, v >= 448 saturates to 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);  // subnormals: multiples of 2^-9
  const int e = (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;     // v in [2^e, 2^(e+1))
  const float scale = __uint_as_float((uint32_t)(3 - e + 127) << 23); // exact 2^(3-e)
  uint32_t m = (uint32_t)__builtin_rintf(v * scale);                 // 8..16
  int ee = e;
  if (m == 16u) {
    m = 8u;
    ++ee;
  }
  return ((uint32_t)(ee + 7) << 3) | (m - 8u);
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// silu(g) * u with the hardware reciprocal (about 1 ulp); exp(-g) = inf gives -0.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace nvmoe

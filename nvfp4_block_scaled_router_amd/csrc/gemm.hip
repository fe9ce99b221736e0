// Grouped NVFP4 GEMMs of the MoE layer on gfx950 MFMA, and the weighted combine.
//
//   gate_up: [g|u][row] = W1_e . x_row  (W1_e = E2M1 x E4M3(per 16 along H) x gs_e),
//            epilogue h = silu(g*sc) * (u*sc), sc = gs_e (x the row's activation factor),
//            stored as fp16 scaled by 2^e per 16-column block (e puts the block's largest
//            |h| in [2^14, 2^15)), or as fp32 for the row quantiser when the down GEMM
//            takes NVFP4 activations;
//   down:    y[row] = W2_e . h_row * gs_e, h brought to one scale per row (h16) or decoded
//            from its NVFP4 row (codes x E4M3 block scales, the row's global scale in the
//            epilogue); y stored as fp16 scaled per 16-column block like h;
//   combine: out[t] = bf16(sum_j w_j y[inv[t][j]] (+ shared)), fp32.
// ([megamoe] README "MoE kernel": grouped GEMM with the global scale, SwiGLU and
// clamping applied in registers in the epilogue; [vllm.cpp] "Device-resident decode
// campaign": grouped kernels with a per-group weight-row index, then MoeCombineKernel.)
//
// Dequant route: the per-16 E4M3 block scale is not a power of two and covers half
// an E8M0 block of the scaled MFMA, so each weight q*s (at most 6 significant bits) is
// rebuilt exactly in registers as fp16 and fed to the fp16 MFMA (V_MFMA_F32_16X16X32_F16)
// with fp32 accumulation: the convert applies the power of two of s (its scale operand is
// exponent-only), one packed fp16 multiply the significand, 1 VALU op per weight.
// Activations are fp16 too: bf16 rows rescaled exactly by a power of two into fp16 range
// (undone in the epilogue), NVFP4 and FP8 rows decoded exactly, h16 as stored. (A bf16 route
// for small decode batches, bf16 rows straight into a bf16 MFMA at 2 VALU ops per weight,
// measured slower once the rescale rode on the routing launch.) Every product q*s*x is
// formed exactly. Global scales (per expert, per activation row) are constant over K and
// are applied once in the epilogue.
//
// Operand roles: MFMA A = 16 weight rows x 32 k (one lane: row l%16, 8 consecutive
// k of a 32-wide lane group), MFMA B = 32 k x 16 tokens (lane: token l%16, the same
// 8 k). Inside a 128-column chunk, lane group g = l/16 owns columns 32g..32g+31 and
// feeds 8 of them to each of the chunk's 4 MFMAs; A and B use the same k order, so
// the dot products are unchanged. D: lane l holds rows 4*(l/16)+r, r < 4, of token
// l%16, i.e. 4 consecutive output features of one token.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nvmoe {

// ----------------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t pick_dword(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The two raw block-scale bytes of chunk c of this lane.
__device__ __forceinline__ uint32_t chunk_scale_bytes(const u32x4& sg, int c) {
  return (pick_dword(sg, c >> 1) >> (16 * (c & 1))) & 0xFFFFu;
}

// h column f is stored at h_pos(f): inside each 128-column chunk, the 8-column piece for
// (lane group g, MFMA step j) -- columns 32g + 8j .. +7, see the operand roles above -- sits
// at piece 4j + g, so the 4 lane groups' loads for one MFMA step read 64 contiguous bytes
// of a row (half the cache lines of the unpermuted order).
__device__ __forceinline__ int h_pos(int f) {
  return (f & ~127) | (((f >> 3) & 3) << 5) | (((f >> 5) & 3) << 3) | (f & 7);
}
// 16-byte piece index inside a chunk: stored piece p holds k-piece h_piece(p).
__device__ __forceinline__ int h_piece(int p) { return ((p & 3) << 2) | (p >> 2); }

// Dequantised fp16 MFMA operands of one 16-row NVFP4 tile for one 128-column chunk (j-th
// operand = columns 32*(l/16) + 8j .. +7 of the lane).
struct WOps {
  f16x8 v[4];
  __device__ __forceinline__ void make(const u32x4& w, uint32_t sb) {
    const f16x2 s = e4m3x2_to_f16x2(sb);
    const f16x2 sa = {s.x, s.x}, sc = {s.y, s.y};
    v[0] = dequant8_f16(w.x, sa);
    v[1] = dequant8_f16(w.y, sa);
    v[2] = dequant8_f16(w.z, sc);
    v[3] = dequant8_f16(w.w, sc);
  }
};

// Operand j (columns 32 (l / 16) + 8j .. +7 of the lane) of one weight tile alone, for loops
// that dequantise right before each MFMA step: sb holds the chunk's two block-scale bytes.
__device__ __forceinline__ f16x8 wop_j(const u32x4& w, uint32_t sb, int j) {
  const f16x2 s = e4m3x2_to_f16x2(sb);
  return dequant8_f16(pick_dword(w, j), j < 2 ? f16x2{s.x, s.x} : f16x2{s.y, s.y});
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One scaled MFMA 16x16x128 on raw MX codes: A = 16 weight rows of E2M1 (lane l: row l%16,
// k 32(l/16) .. +31, low nibble first; its E8M0 scale sa in the low byte), B = 16 token rows
// of E4M3 (lane l: row l%16, k 16(l/16) .. +15 in its first 16 bytes and 64 + 16(l/16) .. +15
// in the next 16; E8M0 scale sb of the token's block l/16). This pairing of the two operands'
// k with the scale blocks was measured on gfx950 with one-hot inputs.
__device__ __forceinline__ f32x4 mfma_mx(const u32x4& a, uint32_t sa, const u32x4& b0, const u32x4& b1, uint32_t sb,
                                         f32x4 c) {
  const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8 bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const u32x4& b, f32x4 c) {
  return mfma16x16x32_f16(a, __builtin_bit_cast(f16x8, b), c);
}

__device__ __forceinline__ const u32x4* fp4_tile(const GemmArgs& a, const ProjLayout& L, int g, int q, int kc) {
  const size_t tile = ((size_t)g * (L.N / 16) + q) * L.KC + kc;
  return (const u32x4*)(a.wfp4 + tile * (WAVE * 16)) + (threadIdx.x & (WAVE - 1));
}

__device__ __forceinline__ const u32x4* sc_tile(const GemmArgs& a, const ProjLayout& L, int g, int q, int sg) {
  const size_t tile = ((size_t)g * (L.N / 16) + q) * L.KSG + sg;
  return (const u32x4*)(a.wsc + tile * (WAVE * 16)) + (threadIdx.x & (WAVE - 1));
}

// The maximum / minimum over lanes l, l ^ 16, l ^ 32 and l ^ 48: the four lanes that hold one
// token row's 16 columns of a D tile. Cross-row lane swaps (v_permlane16_swap, then
// v_permlane32_swap, each with both operands the value: the pair then holds the values of
// lanes l and l ^ 16, resp. l and l ^ 32), no LDS traffic.
__device__ __forceinline__ float max_row4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int min_row4(int v) {
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  const int m = min((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)m, (uint32_t)m, false, false);
  return min((int)b[0], (int)b[1]);
}

// Epilogue for one 16-feature x 16-token D tile pair (gate, up) of gate_up: h = silu(g) u,
// or with a finite limit L the clamped silu(min(g, L)) min(max(u, -L), L) (L = +inf leaves
// g and u as they are), for the 16 h columns hs*16 .. +15 of token row `row` (lane: 4 of
// them), stored as fp16
// scaled by 2^e with e chosen on the block's largest |h| (the 4 lanes of the row share it
// through two lane swaps) and recorded in hexp. All 4 lanes of a row must be active
// together (they are: they hold the same token).
// The 4 h values of this lane for a gate/up D tile pair (see epilogue_pair).
// CLAMP false: the limit is +inf (no min / max: the same values for finite g and u).
template <bool CLAMP = true>
__device__ __forceinline__ f32x4 h_pair(const f32x4& gacc, const f32x4& uacc, float sc, float lim) {
  auto act = [&](float g, float u) {
    return CLAMP ? silu_mul(fminf(g * sc, lim), fminf(fmaxf(u * sc, -lim), lim)) : silu_mul(g * sc, u * sc);
  };
  return f32x4{act(gacc.x, uacc.x), act(gacc.y, uacc.y), act(gacc.z, uacc.z), act(gacc.w, uacc.w)};
}
// Four fp32 values times 2^e (exact) as packed fp16, two per packed convert.
__device__ __forceinline__ u32x2 pack_f16x4(float a, float b, float c, float d, int e) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const f2 lo = {__builtin_ldexpf(a, e), __builtin_ldexpf(b, e)}, hi = {__builtin_ldexpf(c, e), __builtin_ldexpf(d, e)};
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, h2)),
               __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, h2))};
}
// The fp16 form of 4 h values of a 16-column block: scaled by 2^e, e putting the block's
// largest |h| (over the row's 4 lanes) in [2^14, 2^15). Returns e.
__device__ __forceinline__ int h16_tile(const f32x4& h, u32x2& packed) {
  const float mx = max_row4(fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
  // mx = f 2^x with f in [0.5, 1): mx 2^(15 - x) lies in [2^14, 2^15)
  const int e = min(max(15 - __builtin_amdgcn_frexp_expf(mx), -H_EXP_MAX), H_EXP_MAX);
  packed = pack_f16x4(h.x, h.y, h.z, h.w, e);
  return e;
}

template <int MODE>
__device__ __forceinline__ void epilogue_pair(const GemmArgs& a, const f32x4& gacc, const f32x4& uacc, float sc,
                                              int row, int hs, float lim) {
  const int lg = (threadIdx.x & (WAVE - 1)) >> 4;
  const int NO = a.N / 2;
  const int col = hs * 16 + 4 * lg;
  const size_t off = (size_t)row * NO + (a.h_natural ? col : h_pos(col));   // 4 columns stay contiguous
  const f32x4 hv = lim == INFINITY ? h_pair<false>(gacc, uacc, sc, lim) : h_pair<true>(gacc, uacc, sc, lim);
  if (a.hf) {   // fp32 h in column order for the row quantiser (NVFP4 down GEMM)
    *(f32x4*)(a.hf + (size_t)row * NO + hs * 16 + 4 * lg) = hv;
    return;
  }
  const float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float mx = max_row4(fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3]))));
  // mx = f 2^x with f in [0.5, 1): mx 2^(15 - x) lies in [2^14, 2^15)
  const int e = min(max(15 - __builtin_amdgcn_frexp_expf(mx), -H_EXP_MAX), H_EXP_MAX);
  *(u32x2*)(a.out + off) = pack_f16x4(h[0], h[1], h[2], h[3], e);
  if (lg == 0) {
    a.hexp[(size_t)row * (NO / 16) + hs] = (int8_t)e;
    if (a.hmin) atomicMin(&a.hmin[row], e);
  }
}

// MX8 gate_up epilogue for the two gate/up tile pairs of one aligned 32-column h block
// (columns 32 blk .. +31; lane: 4 columns of each 16-column half) of token row `row`: h as in
// epilogue_pair, then MXFP8 in registers: the block's E8M0 scale 2^X with X = floor(log2
// max|h|) - 8 (clamped to [-127, 127], -127 below 2^-118; the 4 lanes of the row share the max
// through two lane swaps) and E4M3 codes of |h| 2^-X (nearest even, saturating at 448) with
// the sign. All 4 lanes of a row must be active together.
__device__ __forceinline__ void epilogue_mx8(const GemmArgs& a, const f32x4& g0, const f32x4& u0, const f32x4& g1,
                                             const f32x4& u1, int row, int blk, float lim) {
  const int lg = (threadIdx.x & (WAVE - 1)) >> 4;
  const int NO = a.N / 2;
  auto act = [&](float g, float u) { return silu_mul(fminf(g, lim), fminf(fmaxf(u, -lim), lim)); };
  const float h[8] = {act(g0.x, u0.x), act(g0.y, u0.y), act(g0.z, u0.z), act(g0.w, u0.w),
                      act(g1.x, u1.x), act(g1.y, u1.y), act(g1.z, u1.z), act(g1.w, u1.w)};
  float A = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) A = fmaxf(A, fabsf(h[i]));
  A = max_row4(A);
  const int X = A < 0x1p-118f ? -127 : min(__builtin_amdgcn_frexp_expf(A) - 1 - 8, 127);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = ((__float_as_uint(h[i]) >> 31) << 7) | e4m3_encode_rne_sat(__builtin_ldexpf(fabsf(h[i]), -X));
    w[i >> 2] |= code << (8 * (i & 3));
  }
  uint8_t* dst = a.hq8 + (size_t)row * NO + 32 * blk + 4 * lg;
  *(uint32_t*)dst = w[0];
  *(uint32_t*)(dst + 16) = w[1];
  if (lg == 0) a.hs8[(size_t)row * (NO / 32) + blk] = (uint8_t)(X + 127);
}

// Smallest h block exponent of a row (nblk bytes, nblk a multiple of 8), read as 8-byte
// words split over the row's 4 lanes l16 + 16 lg and combined through two lane swaps. Up to
// four words per lane are loaded together (indices clamped to the row: a repeated word leaves
// the minimum as it is), so a row of up to 128 blocks takes one memory round trip.
__device__ __forceinline__ int row_exp_min4(const int8_t* erow, int nblk, int lg) {
  const int nw = nblk / 8;
  int m = H_EXP_INIT;
  for (int w0 = lg; w0 < nw; w0 += 16) {
    u32x2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *(const u32x2*)(erow + 8 * min(w0 + 4 * u, nw - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        m = min(m, (int)(int8_t)(v[u].x >> (8 * b)));
        m = min(m, (int)(int8_t)(v[u].y >> (8 * b)));
      }
  }
  return min_row4(m);
}

// 2^d for d <= 0 as fp16 (0 below the fp16 range): the per-block factor that brings h16
// of a block with exponent e to the row's common scale 2^P, d = P - e.
__device__ __forceinline__ _Float16 h_factor(int d) { return (_Float16)__builtin_ldexpf(1.0f, d); }

// Down epilogue for one 16-feature x 16-token D tile: y = acc * sc for the features
// q*16 .. +15 of token row `row` (lane: 4 of them), stored as fp16 scaled by 2^e with e
// chosen on the block's largest |y| (shared by the row's 4 lanes, as for h) and recorded in
// yexp; half the bytes of fp32 y for the combine to read, with an 11-bit significand. sc >= 0
// (or NaN), so max|acc * sc| = max|acc| * sc (rounding is monotone), and acc * (sc 2^e) is
// acc * sc scaled by 2^e rounded once: the same fp16 values as scaling the rounded product
// (fp32 underflow aside), for one multiply per value. e is also capped so that sc 2^e stays
// finite: the cap binds only where max|acc| is below about 2^-112 (never for fp16 products,
// whose sums are multiples of 2^-48), and then the stored values sit that many binades lower
// in fp16's range. All 4 lanes of a row must be active together.
__device__ __forceinline__ int y16_tile(const f32x4& acc, float sc, u32x2& packed) {
  const float mx = max_row4(fmaxf(fmaxf(fabsf(acc.x), fabsf(acc.y)), fmaxf(fabsf(acc.z), fabsf(acc.w))) * sc);
  const int e = min(max(15 - __builtin_amdgcn_frexp_expf(mx), -H_EXP_MAX),
                    min(H_EXP_MAX, 127 - __builtin_amdgcn_frexp_expf(sc)));
  const float f = __builtin_ldexpf(sc, e);
  const uint32_t q0 = __builtin_bit_cast(uint16_t, (_Float16)(acc.x * f));
  const uint32_t q1 = __builtin_bit_cast(uint16_t, (_Float16)(acc.y * f));
  const uint32_t q2 = __builtin_bit_cast(uint16_t, (_Float16)(acc.z * f));
  const uint32_t q3 = __builtin_bit_cast(uint16_t, (_Float16)(acc.w * f));
  packed = u32x2{q0 | (q1 << 16), q2 | (q3 << 16)};
  return e;
}
__device__ __forceinline__ void epilogue_single(const GemmArgs& a, const f32x4& acc, float sc, int row, int q) {
  const int lg = (threadIdx.x & (WAVE - 1)) >> 4;
  u32x2 p;
  const int e = y16_tile(acc, sc, p);
  *(u32x2*)(a.yout + (size_t)row * a.N + q * 16 + 4 * lg) = p;
  if (lg == 0) a.yexp[(size_t)row * (a.N / 16) + q] = (int8_t)e;
}

// ------------------------------------------------------------------ decode GEMM
// Small row counts per expert (<= 16 rows per tile): weight streaming bound. A
// workgroup owns NSUB 16-row weight tiles of one expert and one 16-row token tile; its
// NW <= MAXW waves split K into contiguous chunk ranges (a wider split, up to one chunk per
// wave, measured slower: fewer workgroups fit a CU; and no faster on the smallest grids, a
// single token's 8 experts). Partial tiles are reduced through
// LDS in wave order (deterministic). Token operands come straight from global memory
// (tiny, shared through L2); each lane's token-operand load is reused by NSUB tiles.
constexpr int DEC_MAX_WAVES = 4;   // measured best of 4 / 8 / 16 on the decode workloads

// MAXW: the wave count the launch may use (8 for the MX8 gate_up of small batches: its epilogue
// needs 4 tiles per workgroup, so a small grid has half the workgroups of the 2-tile split and
// splits K wider instead; the 8-wave instance is kept apart because its reduction buffer halves
// the workgroups a CU holds).
// The decode GEMM's work for one workgroup: slot `slot` of its tile list, weight tiles
// bx * NSUB .. +NSUB-1, the workgroup's waves splitting K; `red` holds MAXW x NSUB x 64 f32x4
// of LDS for the reduction.
template <int MODE, int NSUB, int MAXW>
__device__ __forceinline__ void decode_body(const GemmArgs& a, int bx, int slot, f32x4* red_lds) {
  constexpr bool MX8 = MODE == GEMM_GATEUP_MX8 || MODE == GEMM_DOWN_MX8;   // scaled MFMA on MX codes
  constexpr bool DOWNM = MODE == GEMM_DOWN || MODE == GEMM_DOWN_FP4 || MODE == GEMM_DOWN_MX8;
  // the slot's entries are read together with the count (slots past it hold stale values
  // that are never used; the tile arrays have room for any grid), saving one dependent
  // round trip before the weight loads; a second-list launch starts after the first list
  const int first = a.tile_first ? a.tile_first[0] : 0;
  const int ntiles = a.tile_count[0];
  // the slot's group and first row are the same for the whole workgroup (readfirstlane tells
  // the compiler, which keeps them in SGPRs for the buffer resources and addresses)
  const int g = __builtin_amdgcn_readfirstlane(a.tile_group[first + slot]);
  const int row0 = __builtin_amdgcn_readfirstlane(a.tile_row0[first + slot]);
  if (slot >= ntiles) return;
  const ProjLayout L = proj_layout(a.N, a.K);
  const int NW = blockDim.x >> 6;
  const int q0 = bx * NSUB;
  const float wgs = a.wgs[g];
  const int nvalid = min(DECODE_TILE_ROWS, a.offsets[g + 1] - row0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const int row = row0 + min(l16, nvalid - 1);            // clamp: extra columns are never stored
  const int kc0 = (wave * L.KC) / NW, kc1 = ((wave + 1) * L.KC) / NW;

  const uint16_t* xrow = nullptr;                          // 16-bit token rows (fp16 x, h16)
  const int8_t* erow = nullptr;                            // h block exponents of the row
  const uint8_t* qrow = nullptr;
  const uint8_t* srow = nullptr;
  float sc = wgs;                                          // epilogue factor, loaded before the loop
  int hm = 0;                                              // the row's common h exponent
  if (MODE == GEMM_DOWN) {
    xrow = a.x + (size_t)row * L.K;
    if (a.hexp) {                                          // permuted h16 with block exponents
      erow = a.hexp + (size_t)row * (L.K / 16);
      hm = a.hmin ? a.hmin[row] : row_exp_min4(erow, L.K / 16, lg);
      sc = __builtin_ldexpf(wgs, -hm);
    } else {                                               // plain rows with one factor each
      sc *= a.xg[row];
    }
  } else if (MODE == GEMM_DOWN_FP4) {                       // NVFP4 h rows, addressed by row
    qrow = a.xq + (size_t)row * (L.K / 2);
    srow = a.xs + (size_t)row * (L.K / 16);
    sc *= a.xg[row];
  } else if (MX8) {                                          // MXFP8 rows: codes and E8M0 scales
    const int t = MODE == GEMM_DOWN_MX8 ? row : a.tok[row];
    qrow = a.xq + (size_t)t * L.K;
    srow = a.xs + (size_t)t * (L.K / 32);
  } else {
    const int t = a.tok[row];
    if (MODE == GEMM_GATEUP_FP4) {
      qrow = a.xq + (size_t)t * (L.K / 2);
      srow = a.xs + (size_t)t * (L.K / 16);
    } else {
      xrow = a.x + (size_t)t * L.K;
    }
    sc *= a.xg[t];
  }

  f32x4 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight and block-scale tiles through buffer resources of the group (base in SGPRs; tile
  // (q, kc) at (q KC + kc) 1 KiB, scale tile (q, kc / 8) at (q KSG + kc / 8) 1 KiB)
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.wfp4 + (size_t)g * L.fp4_expert, (uint32_t)L.fp4_expert);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(a.wsc + (size_t)g * L.sc_expert, (uint32_t)L.sc_expert);
  const uint32_t lane_off = (uint32_t)lane * 16;
  u32x4 sgv[NSUB];
  int sg_loaded = -1;
  for (int kc = kc0; kc < kc1; ++kc) {
    if ((kc >> 3) != sg_loaded) {
      sg_loaded = kc >> 3;
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        sgv[s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, lane_off, (uint32_t)((q0 + s) * L.KSG + sg_loaded) * 1024u, 0));
    }
    u32x4 wv[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
      wv[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane_off, (uint32_t)((q0 + s) * L.KC + kc) * 1024u, 0));
    if constexpr (MX8) {
      const u32x4 b0 = *(const u32x4*)(qrow + (size_t)kc * KCHUNK + 16 * lg);
      const u32x4 b1 = *(const u32x4*)(qrow + (size_t)kc * KCHUNK + 64 + 16 * lg);
      const uint32_t sb = srow[kc * 4 + lg];
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        acc[s] = mfma_mx(wv[s], chunk_scale_bytes(sgv[s], kc & 7) & 0xFFu, b0, b1, sb, acc[s]);
      continue;
    }
    u32x4 bop[4];
    if (MODE == GEMM_GATEUP_FP4 || MODE == GEMM_DOWN_FP4) {
      const u32x4 xv = *(const u32x4*)(qrow + (size_t)kc * 64 + lg * 16);
      const uint32_t sp = *(const uint16_t*)(srow + (size_t)kc * 8 + 2 * lg);
      WOps xo;
      xo.make(xv, sp);
#pragma unroll
      for (int j = 0; j < 4; ++j) bop[j] = __builtin_bit_cast(u32x4, xo.v[j]);
    } else if (MODE == GEMM_DOWN && erow) {   // h16: piece (g, j) at 4j + g; blocks 2g (j < 2), 2g + 1
      const uint16_t* src = xrow + (size_t)kc * KCHUNK + lg * 8;
      const uint32_t eb = *(const uint16_t*)(erow + kc * 8 + 2 * lg);
      const _Float16 f0 = h_factor(hm - (int)(int8_t)(eb & 0xFFu)), f1 = h_factor(hm - (int)(int8_t)(eb >> 8));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x8 v = *(const f16x8*)(src + 32 * j);
        bop[j] = __builtin_bit_cast(u32x4, v * (j < 2 ? f0 : f1));
      }
    } else {
      const u32x4* src = (const u32x4*)(xrow + (size_t)kc * KCHUNK + lg * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) bop[j] = src[j];
    }
    // step j's weight operands only are dequantised right before its MFMAs (8 live operand
    // registers per tile, not 32)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        acc[s] = mfma_f16(wop_j(wv[s], chunk_scale_bytes(sgv[s], kc & 7), j), bop[j], acc[s]);
  }

  f32x4 (*red)[NSUB][WAVE] = (f32x4 (*)[NSUB][WAVE])red_lds;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) red[wave][s][lane] = acc[s];
  __syncthreads();
  // wave w finishes tiles w, w + NW, ...: fixed-order sum over the K ranges
  if (l16 >= nvalid) return;
  const int orow = row0 + l16;                             // == row on the lanes that remain
  if (DOWNM) {
    for (int s = wave; s < NSUB; s += NW) {
      f32x4 sum = red[0][s][lane];
      for (int w = 1; w < NW; ++w) sum += red[w][s][lane];
      epilogue_single(a, sum, sc, orow, q0 + s);
    }
  } else {
    const float lim = g < a.clamp_groups ? a.swiglu_limit : INFINITY;
    if constexpr (MODE == GEMM_GATEUP_MX8 && NSUB == 4) {
      if (a.hq8) {   // one wave quantises the 32-column block of both pairs (sc = 1: MX has no global scale)
        if (wave == 0) {
          f32x4 t[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            t[s] = red[0][s][lane];
            for (int w = 1; w < NW; ++w) t[s] += red[w][s][lane];
          }
          epilogue_mx8(a, t[0], t[1], t[2], t[3], orow, bx, lim);
        }
        return;
      }
    }
    // gate (even tile) and up (odd tile) of the same columns are finished together
    for (int s = 2 * wave; s < NSUB; s += 2 * NW) {
      f32x4 gsum = red[0][s][lane], usum = red[0][s + 1][lane];
      for (int w = 1; w < NW; ++w) {
        gsum += red[w][s][lane];
        usum += red[w][s + 1][lane];
      }
      epilogue_pair<MODE>(a, gsum, usum, sc, orow, (q0 + s) >> 1, lim);
    }
  }
}

template <int MODE, int NSUB, int MAXW = DEC_MAX_WAVES>
__global__ __launch_bounds__(64 * MAXW) void gemm_decode_kernel(GemmArgs a) {
  __shared__ f32x4 red[MAXW * NSUB * WAVE];
  decode_body<MODE, NSUB, MAXW>(a, blockIdx.x, blockIdx.y, red);
}

// XCD-aware work order of the prefill GEMMs. Workgroups are handed to the 8 XCDs (each
// with its own L2) round-robin by linear id, so consecutive ids never share an L2. The
// grid is (n-blocks) x (slot bound rounded up to 8); workgroup id i runs on XCD i % 8 and
// is given the (i / 8)-th item of that XCD's list: a contiguous run of ceil(ntiles / 8)
// tile slots, each with all its n-blocks. The n-blocks of one token tile then share its
// rows in one L2, and consecutive slots (mostly of one expert) share its weight tiles.
struct PrefillItem {
  int slot, nb;
};
__device__ __forceinline__ PrefillItem prefill_item(int ntiles, int lin, int NB) {
  const int xcd = lin & 7, j = lin >> 3;
  const int per_xcd = (ntiles + 7) >> 3;
  PrefillItem it;
  const int k = j / NB;
  it.nb = j - k * NB;
  it.slot = k < per_xcd ? xcd * per_xcd + k : ntiles;   // past the list: no work
  return it;
}

// LDS slot swizzle of the prefill token tiles: piece c of row r sits at slot c ^ lds_swz(r).
// An MFMA operand read has lane (l%16, l/16) fetch row 16t + l%16, piece 4(l/16) + j. With
// lds_swz(r) = G((r >> 1) & 7) ^ 4 (r & 1), G(q) = (q & 3) | 2 (q & 4), these 16-byte reads
// measured free of bank conflicts on gfx950 (SQ_LDS_BANK_CONFLICT = 0, the speed of a
// linear read), where the plain c ^ (r % 16) costs 4 conflict cycles per read.
__device__ __forceinline__ int lds_swz(int r) {
  const int q = (r >> 1) & 7;
  return ((q & 3) | ((q & 4) << 1)) ^ ((r & 1) << 2);
}

// ----------------------------------------------------------------- prefill GEMM
// Tiles of TSUB*16 token rows of one expert x (WAVES x NSUB) 16-row weight tiles. The
// token tile of each 128-column chunk sits in LDS (rows of 256 bytes: one chunk of 16-bit
// values, 16-byte piece c of row r at slot c ^ lds_swz(r)), shared by the waves; each
// wave streams its own weight tiles straight into registers (two alternating register
// sets, one chunk ahead) and dequantises them there. Token tiles arrive by
//  - LDS DMA (fp16 rows: the rescaled activations of GATEUP_F16 gathered through the
//    row -> token map, or DOWN's own h16 rows, already at each row's common scale 2^P):
//    global_load_lds_dwordx4 straight into an NBUF-deep ring of stages, no staging
//    registers, chunk kc + NBUF - 1 in flight while chunk kc is consumed. One DMA instruction
//    writes 64 consecutive 16-byte slots (lane i -> slot i), so the swizzle is applied on the
//    global side: the lane that fills slot (r, c) fetches piece c ^ lds_swz(r) of row r;
//  NVFP4 rows (x of W4A4, h of W4A4 down) arrive the same way as their exact fp16 decode,
//  written by the row quantiser beside the codes, with the row's global scale applied in
//  the epilogue.
// Issue order inside a chunk is pinned with scheduling barriers (the wait counts rely on it).
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}
// The same through a buffer resource: byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds_dst, 16, (int)voff,
                                           (int)soff, 0, 0);
}

template <int V> struct IntC { static constexpr int value = V; };


// The K loop of the three-stage pipelines: step(kc, set kc % 3, kind) for kc = 0 .. KC - 1, the
// set and the kind as compile-time constants. Every chunk but the last two issues the loads of
// chunk kc + 2 (STEP_FULL); chunk KC - 2 issues nothing and may leave chunk KC - 1's loads in
// flight (STEP_NEXT_TO_LAST); chunk KC - 1 waits for everything (STEP_LAST). The steady state
// runs in groups of three with no branch; the remaining 1 to 4 chunks are spelled out.
constexpr int STEP_FULL = 0, STEP_NEXT_TO_LAST = 1, STEP_LAST = 2;
template <typename F>
__device__ __forceinline__ void run_chunks(int KC, F&& step) {
  int kc = 0;
  for (; kc + 5 <= KC; kc += 3) {
    step(kc, IntC<0>(), IntC<STEP_FULL>());
    step(kc + 1, IntC<1>(), IntC<STEP_FULL>());
    step(kc + 2, IntC<2>(), IntC<STEP_FULL>());
  }
  switch (KC - kc) {   // kc is a multiple of 3 here
    case 4:
      step(kc, IntC<0>(), IntC<STEP_FULL>());
      step(kc + 1, IntC<1>(), IntC<STEP_FULL>());
      step(kc + 2, IntC<2>(), IntC<STEP_NEXT_TO_LAST>());
      step(kc + 3, IntC<0>(), IntC<STEP_LAST>());
      break;
    case 3:
      step(kc, IntC<0>(), IntC<STEP_FULL>());
      step(kc + 1, IntC<1>(), IntC<STEP_NEXT_TO_LAST>());
      step(kc + 2, IntC<2>(), IntC<STEP_LAST>());
      break;
    case 2:
      step(kc, IntC<0>(), IntC<STEP_NEXT_TO_LAST>());
      step(kc + 1, IntC<1>(), IntC<STEP_LAST>());
      break;
    default:
      step(kc, IntC<0>(), IntC<STEP_LAST>());
      break;
  }
}

// s_waitcnt immediate: vmcnt(vm) lgkmcnt(lgkm), expcnt not waited.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// The prefill GEMM's work for the workgroup of linear id `lin` in a grid of NB n-blocks per
// row of slots (see prefill_item); `tile` is NBUF x TSUB*16*16 16-byte slots of LDS.
template <int MODE, int NSUB, int TSUB, int NBUF, int WAVES>
__device__ __forceinline__ void prefill_body(const GemmArgs& a, int lin, int NB, u32x4* tile) {
  static_assert(MODE == GEMM_GATEUP_F16 || MODE == GEMM_DOWN, "prefill modes: fp16 rows by LDS DMA");
  constexpr bool DOWNM = MODE == GEMM_DOWN;           // rows addressed directly (gate_up gathers tokens)
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  static_assert(NBUF == 2 || NBUF == 3, "LDS ring depth");
  constexpr int M = TSUB * 16;
  constexpr int STAGE = M * 16;                       // 16-byte slots per stage
  constexpr int NT = 64 * WAVES;                      // threads
  constexpr int D = STAGE / NT;                       // DMA instructions per lane per chunk
  static_assert(D >= 1 && STAGE % NT == 0, "tile size");

  const int ntiles = a.tile_count[0];
  const PrefillItem item = prefill_item(ntiles, lin, NB);
  const int slot = item.slot;
  if (slot >= ntiles) return;
  const int g = __builtin_amdgcn_readfirstlane(a.tile_group[slot]);      // uniform: kept in SGPRs
  const int row0 = __builtin_amdgcn_readfirstlane(a.tile_row0[slot]);
  const ProjLayout L = proj_layout(a.N, a.K);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (WAVE - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const int q0 = (item.nb * WAVES + wave) * NSUB;         // the launch covers N exactly
  const int nvalid = min(M, a.offsets[g + 1] - row0);
  const float wgs = a.wgs[g];                             // read with the tile entry, not after the K loop

  // Every load goes through a buffer resource (base and range in SGPRs, a 32-bit offset per
  // lane, the chunk's offset as the scalar offset): no 64-bit address registers, and no
  // address arithmetic per chunk.
  // ---- token-tile DMA. Instruction i of this wave fills slots (WAVES i + wave) * 64 .. +63:
  // row r = 4 (WAVES i + wave) + lane / 16, slot column lane % 16. The gate_up gathers token
  // rows from the activation base (T K 2 <= 2^31 bytes), the down GEMM reads its own rows from
  // the tile's first row (a 64-bit base; offsets within the tile's nvalid rows).
  uint32_t src_off[D];
  const __amdgpu_buffer_rsrc_t xr =
      DOWNM ? buffer_rsrc(a.x + (size_t)row0 * L.K, (uint32_t)nvalid * L.K * 2) : buffer_rsrc(a.x, 0xFFFFFFFFu);
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int r = 4 * (WAVES * i + wave) + lg;
    const int rl = min(r, nvalid - 1);                   // rows past the group repeat its last row
    const int kp = l16 ^ lds_swz(r);                     // k-order piece this slot holds
    const uint32_t src = DOWNM ? (uint32_t)rl : (uint32_t)a.tok[row0 + rl];
    src_off[i] = (src * (uint32_t)L.K + kp * 8) * 2;
  }
  auto dma = [&](int kc, int st) {
#pragma unroll
    for (int i = 0; i < D; ++i)
      dma16(xr, src_off[i], (uint32_t)kc * (KCHUNK * 2), &tile[st * STAGE + (WAVES * i + wave) * 64]);
  };

  // ---- weights of this wave: fp4 16 B per lane per chunk; the chunk's two block-scale
  // bytes come from the dword holding them (a 16-bit load would be zero-extended right
  // after it, which makes the compiler wait for the load at once). Tile (q, kc) of the group
  // sits at (q KC + kc) 1 KiB, its scale tile (q, kc / 8) at (q KSG + kc / 8) 1 KiB.
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.wfp4 + (size_t)g * L.fp4_expert, (uint32_t)L.fp4_expert);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(a.wsc + (size_t)g * L.sc_expert, (uint32_t)L.sc_expert);
  const uint32_t lane_off = (uint32_t)lane * 16;
  auto load_w = [&](int kc, u32x4 (&w)[NSUB], uint32_t (&sb)[NSUB]) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      w[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane_off, (uint32_t)((q0 + s) * L.KC + kc) * 1024u, 0));
      sb[s] = __builtin_amdgcn_raw_buffer_load_b32(
          sr, lane_off, (uint32_t)((q0 + s) * L.KSG + (kc >> 3)) * 1024u + (uint32_t)(kc & 6) * 2u, 0);
    }
  };

  // The MFMAs (and their LDS reads) cover only the 16-row slices up to the tile's last valid
  // row, in steps of 2 slices: an expert's last tile is partly empty (about half a tile per
  // expert on average), and the staging above still moves whole tiles so that every
  // workgroup issues the same loads and waits.
  static_assert(TSUB == 8 || TSUB == 6 || TSUB == 4, "row tiers assume 4, 6 or 8 slices");
  auto body = [&](auto tvc) {
    constexpr int TV = decltype(tvc)::value;
    f32x4 acc[NSUB][TV];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int t = 0; t < TV; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA step j of the chunk in LDS stage st: the weight operands of step j only are dequantised here (raw
    // dword j of each tile times its block scale), which keeps 8 fp16 operand registers live
    // per tile instead of the chunk's 32
    auto mma = [&](int st, int j, const u32x4 (&rc)[NSUB], const f16x2 (&s2)[NSUB]) {
      const u32x4* T0 = &tile[st * STAGE];
      const int c = (lg * 4 + j) ^ lds_swz(l16);
      u32x4 bop[TV];
#pragma unroll
      for (int t = 0; t < TV; ++t) bop[t] = T0[(t * 16 + l16) * 16 + c];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const f16x2 sj = j < 2 ? f16x2{s2[s].x, s2[s].x} : f16x2{s2[s].y, s2[s].y};
        const f16x8 w = dequant8_f16(pick_dword(rc[s], j), sj);
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[s][t] = mfma16x16x32_f16(w, __builtin_bit_cast(f16x8, bop[t]), acc[s][t]);
      }
    };
    {
      // fp16 rows by LDS DMA into an NBUF-deep ring; raw weights one chunk ahead in two
      // register sets (chunk parity), dequantised right before the chunk's MFMAs. Chunk kc:
      // wait for chunk kc in LDS and its weights (older loads complete, the newest NBUF - 2
      // chunks' DMA may stay in flight), barrier, issue the raw weights of kc + 1 and the DMA
      // of kc + NBUF - 1 (both clamped to the last chunk near the end, so every chunk issues
      // the same loads and one wait count fits all; the clamped loads at the end feed no later
      // wait), consume chunk kc. Issue order is pinned with scheduling barriers: the wait count
      // covers the LDS stages written by DMA, which the compiler does not track.
      u32x4 rA[NSUB], rB[NSUB];
      uint32_t sA[NSUB], sB[NSUB];
      load_w(0, rA, sA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NBUF - 1; ++c) dma(min(c, L.KC - 1), c);
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](int kc, const u32x4 (&rc)[NSUB], const uint32_t (&sc)[NSUB], u32x4 (&rf)[NSUB],
                      uint32_t (&sf)[NSUB]) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(D * (NBUF - 2), 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        load_w(min(kc + 1, L.KC - 1), rf, sf);
        __builtin_amdgcn_sched_barrier(0);
        dma(min(kc + NBUF - 1, L.KC - 1), (kc + NBUF - 1) % NBUF);
        __builtin_amdgcn_sched_barrier(0);
        f16x2 s2[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) s2[s] = e4m3x2_to_f16x2(sc[s] >> ((kc & 1) * 16));   // the low 16 bits
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(kc % NBUF, j, rc, s2);
      };
      if (L.KC & 1) {
        step(0, rA, sA, rB, sB);
        for (int kc = 1; kc < L.KC; kc += 2) {
          step(kc, rB, sB, rA, sA);
          step(kc + 1, rA, sA, rB, sB);
        }
      } else {
        for (int kc = 0; kc < L.KC; kc += 2) {
          step(kc, rA, sA, rB, sB);
          step(kc + 1, rB, sB, rA, sA);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // every load in flight lands before the workgroup exits

    // the epilogue factors of the lane's rows t * 16 + l16, t < TV, all loaded together (row
    // indices clamped to the tile's valid rows, values pinned: a load used only where the row
    // is valid is otherwise sunk into that branch and waited for there, one round trip per
    // slice, two for the gate_up's token -> row-scale chain)
    float rsc[TV];
    if constexpr (DOWNM) {
      if (a.hmin) {
        int hm[TV];
#pragma unroll
        for (int t = 0; t < TV; ++t) hm[t] = a.hmin[row0 + min(t * 16 + l16, nvalid - 1)];
#pragma unroll
        for (int t = 0; t < TV; ++t) asm volatile("" : "+v"(hm[t]));
#pragma unroll
        for (int t = 0; t < TV; ++t) rsc[t] = __builtin_ldexpf(wgs, -hm[t]);
      } else {
#pragma unroll
        for (int t = 0; t < TV; ++t) rsc[t] = a.xg[row0 + min(t * 16 + l16, nvalid - 1)];
#pragma unroll
        for (int t = 0; t < TV; ++t) asm volatile("" : "+v"(rsc[t]));
#pragma unroll
        for (int t = 0; t < TV; ++t) rsc[t] *= wgs;
      }
    } else {
      int tk[TV];
#pragma unroll
      for (int t = 0; t < TV; ++t) tk[t] = a.tok[row0 + min(t * 16 + l16, nvalid - 1)];
#pragma unroll
      for (int t = 0; t < TV; ++t) asm volatile("" : "+v"(tk[t]));
#pragma unroll
      for (int t = 0; t < TV; ++t) rsc[t] = a.xg[tk[t]];
#pragma unroll
      for (int t = 0; t < TV; ++t) asm volatile("" : "+v"(rsc[t]));
#pragma unroll
      for (int t = 0; t < TV; ++t) rsc[t] *= wgs;
    }
    if constexpr (DOWNM) {
      // y16 of the workgroup's M x COLS block goes through LDS (the ring is free once every
      // wave is past its last chunk) and leaves as whole row segments of COLS * 2 bytes, 16
      // bytes per lane, instead of 32-byte pieces of 16 rows per store instruction; the block
      // exponents follow as COLS / 16 bytes per row. Rows past the tile's valid ones are not
      // written.
      constexpr int COLS = WAVES * NSUB * 16, YP = COLS + 8, NBLK = COLS / 16;   // YP: +16 B per row
      static_assert(M * YP * 2 + M * NBLK <= NBUF * STAGE * 16, "the y block fits the LDS ring");
      uint16_t* ys = (uint16_t*)tile;
      int8_t* es = (int8_t*)(ys + M * YP);
      __syncthreads();   // every wave is done reading the ring
#pragma unroll
      for (int t = 0; t < TV; ++t) {
        const int rr = t * 16 + l16;
        if (rr >= nvalid) continue;
        // h16 from gate_up: the row's exponent P (2^-P); NVFP4 / FP8 h: its fp16 decode, the
        // row's scale
        const float scl = rsc[t];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          u32x2 p;
          const int e = y16_tile(acc[s][t], scl, p);
          *(u32x2*)(ys + rr * YP + (wave * NSUB + s) * 16 + 4 * lg) = p;
          if (lg == 0) es[rr * NBLK + wave * NSUB + s] = (int8_t)e;
        }
      }
      __syncthreads();
      const int col0 = item.nb * COLS;
      for (int i = threadIdx.x; i < nvalid * (COLS / 8); i += NT) {
        const int r = i / (COLS / 8), c = i - r * (COLS / 8);
        *(u32x4*)(a.yout + (size_t)(row0 + r) * a.N + col0 + c * 8) = *(const u32x4*)(ys + r * YP + c * 8);
      }
      for (int r = threadIdx.x; r < nvalid; r += NT) {
        int8_t* dst = a.yexp + (size_t)(row0 + r) * (a.N / 16) + col0 / 16;
        if constexpr (NBLK == 16)
          *(u32x4*)dst = *(const u32x4*)(es + r * NBLK);
        else
          *(u32x2*)dst = *(const u32x2*)(es + r * NBLK);
      }
      return;
    }
    // gate_up: h of the workgroup's M x HC block (HC = its h columns) likewise through LDS:
    // fp32 rows for the row quantisers (a.hf), or h16 in plain column order with one exponent
    // per 16-column block, whose minimum over the workgroup's blocks of a row is folded into
    // hmin[row] by one atomic per row
    constexpr int HC = WAVES * NSUB * 8, HNB = HC / 16;
    const int NO = a.N / 2, hcol0 = item.nb * HC;
    const float lim = g < a.clamp_groups ? a.swiglu_limit : INFINITY;
    __syncthreads();   // every wave is done reading the ring
    if (a.hf) {
      constexpr int FP = HC + 4;                         // floats per staged row (+16 B)
      static_assert(M * FP * 4 <= NBUF * STAGE * 16, "the fp32 h block fits the LDS ring");
      float* hs = (float*)tile;
      auto stage = [&](auto clampc) {
        constexpr bool CL = decltype(clampc)::value != 0;
#pragma unroll
        for (int t = 0; t < TV; ++t) {
          const int rr = t * 16 + l16;
          if (rr >= nvalid) continue;
          const float scl = rsc[t];
#pragma unroll
          for (int s = 0; s < NSUB; s += 2)
            *(f32x4*)(hs + rr * FP + ((wave * NSUB + s) >> 1) * 16 + 4 * lg) =
                h_pair<CL>(acc[s][t], acc[s + 1][t], scl, lim);
        }
      };
      if (lim == INFINITY) stage(IntC<0>());
      else stage(IntC<1>());
      __syncthreads();
      for (int i = threadIdx.x; i < nvalid * (HC / 4); i += NT) {
        const int r = i / (HC / 4), c = i - r * (HC / 4);
        *(f32x4*)(a.hf + (size_t)(row0 + r) * NO + hcol0 + c * 4) = *(const f32x4*)(hs + r * FP + c * 4);
      }
      return;
    }
    constexpr int HP = HC + 8;                           // halfs per staged row (+16 B)
    static_assert(M * HP * 2 + M * HNB <= NBUF * STAGE * 16, "the h16 block fits the LDS ring");
    uint16_t* hs = (uint16_t*)tile;
    int8_t* es = (int8_t*)(hs + M * HP);
    auto stage = [&](auto clampc) {
      constexpr bool CL = decltype(clampc)::value != 0;
#pragma unroll
      for (int t = 0; t < TV; ++t) {
        const int rr = t * 16 + l16;
        if (rr >= nvalid) continue;
        const float scl = rsc[t];
#pragma unroll
        for (int s = 0; s < NSUB; s += 2) {
          u32x2 p;
          const int e = h16_tile(h_pair<CL>(acc[s][t], acc[s + 1][t], scl, lim), p);
          const int hb = (wave * NSUB + s) >> 1;
          *(u32x2*)(hs + rr * HP + hb * 16 + 4 * lg) = p;
          if (lg == 0) es[rr * HNB + hb] = (int8_t)e;
        }
      }
    };
    if (lim == INFINITY) stage(IntC<0>());   // groups without a SwiGLU limit
    else stage(IntC<1>());
    __syncthreads();
    for (int i = threadIdx.x; i < nvalid * (HC / 8); i += NT) {
      const int r = i / (HC / 8), c = i - r * (HC / 8);
      *(u32x4*)(a.out + (size_t)(row0 + r) * NO + hcol0 + c * 8) = *(const u32x4*)(hs + r * HP + c * 8);
    }
    for (int r = threadIdx.x; r < nvalid; r += NT) {
      const int8_t* er = es + r * HNB;
      int m = H_EXP_INIT;
#pragma unroll
      for (int b = 0; b < HNB; ++b) m = min(m, (int)er[b]);
      int8_t* dst = a.hexp + (size_t)(row0 + r) * (NO / 16) + hcol0 / 16;
      if constexpr (HNB == 8)
        *(u32x2*)dst = *(const u32x2*)er;
      else
        *(uint32_t*)dst = *(const uint32_t*)er;
      if (a.hmin) atomicMin(&a.hmin[row0 + r], m);
    }
  };
  const int tv = (nvalid + 15) >> 4;
  if constexpr (TSUB == 8) {
    if (tv > 6) body(IntC<8>());
    else if (tv > 4) body(IntC<6>());
    else if (tv > 2) body(IntC<4>());
    else body(IntC<2>());
  } else if constexpr (TSUB == 6) {
    if (tv > 4) body(IntC<6>());
    else if (tv > 2) body(IntC<4>());
    else body(IntC<2>());
  } else {
    if (tv > 2) body(IntC<4>());
    else body(IntC<2>());
  }
}

template <int MODE, int NSUB, int TSUB, int NBUF, int WAVES, int OCC>
__global__ __launch_bounds__(64 * WAVES, OCC) void gemm_prefill_kernel(GemmArgs a) {
  __shared__ u32x4 tile[NBUF * TSUB * 16 * 16];
  prefill_body<MODE, NSUB, TSUB, NBUF, WAVES>(a, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, tile);
}

// ---------------------------------------------------------------- persistent prefill down
// The prefill down GEMM with P resident workgroups that each run a sequence of work items
// (tile slot, column block) and carry the load pipeline across them: the last chunks of an
// item issue the first weights and token chunks of the next, so its epilogue (y16 staging
// and the stores of the M x COLS block) runs while that data is in flight, and the stores
// drain under the next item's MFMAs instead of in one burst per round of workgroups.
// Items of XCD x (workgroups lin with lin % 8 = x, as the hardware deals them out) are the
// XCD's slots x per_xcd .. +per_xcd - 1 times the NB column blocks, taken in turn by the
// XCD's P / 8 workgroups, so the workgroups of an XCD share the tiles' rows and the experts'
// weights in its L2 as in the one-item-per-workgroup launch. The K chunk count is even (the
// two weight register sets then start every item in the same order).
// The epilogue stages y16 through the ring stage of the item's last chunk (the other two
// hold the next item's first chunks) in passes of 32 rows; block exponents and the rows'
// factors (hmin or xg, copied by a 4-byte LDS DMA at the item's start) have LDS arrays of
// their own. Stores go through buffer resources bounded at the item's valid rows, so every
// lane issues the same number of them (the hardware drops rows past the range) and the wait
// count of the next item's first chunk is a constant.
template <int NSUB, int TSUB, int NBUF, int WAVES>
__device__ __forceinline__ void prefill_down_run(const GemmArgs& a, int lin, int P, int NB, u32x4* tile,
                                                 int8_t* es, uint32_t* rowf) {
  static_assert(NBUF == 3 && TSUB == 6 && WAVES == 8 && (NSUB == 2 || NSUB == 1), "the 96-row 8-wave ring");
  constexpr int M = TSUB * 16, STAGE = M * 16, NT = 64 * WAVES, D = STAGE / NT;
  constexpr int COLS = WAVES * NSUB * 16, YP = COLS + 8, NBLK = COLS / 16;
  constexpr int PASS_T = 2, NPASS = TSUB / PASS_T, PASS_ROWS = PASS_T * 16;
  static_assert(PASS_ROWS * YP * 2 <= STAGE * 16, "a staging pass fits one ring stage");
  constexpr int SPP = PASS_ROWS * (COLS / 8) / NT;           // 16-byte y stores per thread and pass
  static_assert(SPP >= 1 && SPP * NT == PASS_ROWS * (COLS / 8), "whole store rounds");
  constexpr int S = NPASS * SPP + 1;                         // vector stores per thread per epilogue
  constexpr int W_ISSUE = D * (NBUF - 2);                    // loads a chunk may leave in flight
  constexpr int NO_LGKM = 15;                                // lgkmcnt field: no wait

  const int ntiles = a.tile_count[0];
  const int xcd = lin & 7, PX = P >> 3;
  const int per_xcd = (ntiles + 7) >> 3;
  const int slot_lo = xcd * per_xcd, slot_hi = min(ntiles, slot_lo + per_xcd);
  const ProjLayout L = proj_layout(a.N, a.K);
  const int KC = L.KC;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (WAVE - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const uint32_t lane_off = (uint32_t)lane * 16;

  // An item's slot, column block, group and first row are read one item before its row
  // count and weight scale, which are first needed in the previous item's last chunks and in
  // its epilogue: neither read waits on the other inside one item.
  struct Item {
    int ok, g, row0, nb, nvalid;
    float wgs;
  };
  // The plan's arrays and the weight scales are not written during the launch: read through
  // the constant address space they become scalar loads, which a vector memory wait (the
  // epilogue's stores, the next chunks in flight) never has to cover.
  typedef const int __attribute__((address_space(4))) cint;
  typedef const float __attribute__((address_space(4))) cfloat;
  auto item_head = [&](int m) {
    Item it;
    const int k = m / NB;
    it.ok = slot_lo + k < slot_hi;
    const int slot = it.ok ? slot_lo + k : 0;
    it.nb = m - k * NB;
    it.g = ((cint*)a.tile_group)[slot];
    it.row0 = ((cint*)a.tile_row0)[slot];
    it.nvalid = 1;
    it.wgs = 0.f;
    return it;
  };
  auto item_finish = [&](Item& it) {
    if (it.ok) {
      it.nvalid = min(M, ((cint*)a.offsets)[it.g + 1] - it.row0);
      it.wgs = ((cfloat*)a.wgs)[it.g];
    }
  };

  // loads of an item: weights of chunk kc into a register set; token rows of chunk kc into
  // ring stage st (rows past the item's valid ones repeat its last row); the rows' factors
  auto load_w = [&](const Item& it, int kc, u32x4 (&w)[NSUB], uint32_t (&sb)[NSUB]) {
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.wfp4 + (size_t)it.g * L.fp4_expert, (uint32_t)L.fp4_expert);
    const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(a.wsc + (size_t)it.g * L.sc_expert, (uint32_t)L.sc_expert);
    const int q0 = (it.nb * WAVES + wave) * NSUB;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      w[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, lane_off, (uint32_t)((q0 + s) * L.KC + kc) * 1024u, 0));
      sb[s] = __builtin_amdgcn_raw_buffer_load_b32(
          sr, lane_off, (uint32_t)((q0 + s) * L.KSG + (kc >> 3)) * 1024u + (uint32_t)(kc & 6) * 2u, 0);
    }
  };
  auto dma = [&](const Item& it, int kc, int st) {
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(a.x + (size_t)it.row0 * L.K, (uint32_t)it.nvalid * L.K * 2);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int r = 4 * (WAVES * i + wave) + lg;
      const uint32_t off = ((uint32_t)min(r, it.nvalid - 1) * (uint32_t)L.K + (l16 ^ lds_swz(r)) * 8) * 2;
      dma16(xr, off, (uint32_t)kc * (KCHUNK * 2), &tile[st * STAGE + (WAVES * i + wave) * 64]);
    }
  };
  // the rows' factors: wave w copies rows 64 w .. 64 w + 63 (zeros past the valid rows)
  auto dma_rowf = [&](const Item& it) {
    const void* src = a.hmin ? (const void*)(a.hmin + it.row0) : (const void*)(a.xg + it.row0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(src, (uint32_t)it.nvalid * 4u),
                                             (void __attribute__((address_space(3)))*)(rowf + wave * 64), 4,
                                             (int)((wave * 64 + lane) * 4), 0, 0, 0);
  };

  int m = lin >> 3;
  Item cur = item_head(m);
  if (!cur.ok) return;
  item_finish(cur);
  Item nxt = item_head(m + PX);
  u32x4 rA[NSUB], rB[NSUB];
  uint32_t sA[NSUB], sB[NSUB];
  load_w(cur, 0, rA, sA);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < NBUF - 1; ++c) dma(cur, min(c, KC - 1), c);
  dma_rowf(cur);
  __builtin_amdgcn_sched_barrier(0);
  int ring = 0;             // ring stage of the current item's chunk 0
  int first_wait = W_ISSUE + 1;   // chunk 0: the last token chunk, the factors (+ an epilogue's stores)

  auto run = [&](auto tvc) {
    constexpr int TV = decltype(tvc)::value;
    f32x4 acc[NSUB][TV];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int t = 0; t < TV; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](int st, int j, const u32x4 (&rc)[NSUB], const f16x2 (&s2)[NSUB]) {
      const u32x4* T0 = &tile[st * STAGE];
      const int c = (lg * 4 + j) ^ lds_swz(l16);
      u32x4 bop[TV];
#pragma unroll
      for (int t = 0; t < TV; ++t) bop[t] = T0[(t * 16 + l16) * 16 + c];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const f16x2 sj = j < 2 ? f16x2{s2[s].x, s2[s].x} : f16x2{s2[s].y, s2[s].y};
        const f16x8 w = dequant8_f16(pick_dword(rc[s], j), sj);
#pragma unroll
        for (int t = 0; t < TV; ++t) acc[s][t] = mfma16x16x32_f16(w, __builtin_bit_cast(f16x8, bop[t]), acc[s][t]);
      }
    };
    // chunk kc in ring stage rs: wait for its data, barrier, issue the weights (wi, wk) and
    // the token rows (di, dk) into stage ds, consume chunk kc. The body pairs load chunks of
    // this item only; the last pair issues the next item's first chunks (or this item's last
    // chunk again when there is none), so the per-chunk work of the body is that of a single
    // item. The LDS reads of chunk kc - 1 are complete (its MFMAs used them): only vmcnt is
    // waited.
    auto step = [&](int kc, int rs, int wait, const Item& wi, int wk, const Item& di, int dk, int ds,
                    const u32x4 (&rc)[NSUB], const uint32_t (&sc)[NSUB], u32x4 (&rf)[NSUB], uint32_t (&sf)[NSUB]) {
      if (wait == W_ISSUE + 1) __builtin_amdgcn_s_waitcnt(waitcnt_imm(W_ISSUE + 1, NO_LGKM));
      else if (wait == W_ISSUE + 1 + S) __builtin_amdgcn_s_waitcnt(waitcnt_imm(W_ISSUE + 1 + S, NO_LGKM));
      else __builtin_amdgcn_s_waitcnt(waitcnt_imm(W_ISSUE, NO_LGKM));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_w(wi, wk, rf, sf);
      __builtin_amdgcn_sched_barrier(0);
      dma(di, dk, ds);
      __builtin_amdgcn_sched_barrier(0);
      f16x2 s2[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) s2[s] = e4m3x2_to_f16x2(sc[s] >> ((kc & 1) * 16));
#pragma unroll
      for (int j = 0; j < 4; ++j) mma(rs, j, rc, s2);
    };
    // ring stages: chunk kc of the item sits in stage (st0 + kc) % 3; a step's DMA goes two
    // stages on, which is the stage read one step before
    const int st0 = ring;
    int rs = st0;
    auto adv = [](int x) { return x == NBUF - 1 ? 0 : x + 1; };
    int kc = 0;
    for (; kc < KC - 2; kc += 2) {
      const int r1 = adv(rs), r2 = adv(r1), r3 = adv(r2);
      step(kc, rs, kc == 0 ? first_wait : W_ISSUE, cur, kc + 1, cur, kc + 2, r2, rA, sA, rB, sB);
      step(kc + 1, r1, W_ISSUE, cur, kc + 2, cur, kc + 3, r3, rB, sB, rA, sA);
      rs = r2;
    }
    {
      // the last pair: the next item's weights of chunk 0 and its token chunks 0 and 1
      const bool n = nxt.ok;
      const Item& ti = n ? nxt : cur;
      const int r1 = adv(rs), r2 = adv(r1), r3 = adv(r2);
      step(kc, rs, kc == 0 ? first_wait : W_ISSUE, cur, kc + 1, ti, n ? 0 : KC - 1, r2, rA, sA, rB, sB);
      step(kc + 1, r1, W_ISSUE, ti, n ? 0 : KC - 1, ti, n ? 1 : KC - 1, r3, rB, sB, rA, sA);
    }

    // ---- epilogue of the item through the ring stage of its last chunk. Its per-lane
    // addresses derive from an opaque copy of the thread id, which keeps the compiler from
    // computing them once before the item loop and holding them through the K loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int el16 = tid & 15, elg = (tid >> 4) & 3;
    // y16 of every slice first, packed (half the registers of the fp32 accumulators, which
    // leaves room for the next item's weights in flight), block exponents straight to LDS
    u32x2 ypk[NSUB][TV];
#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const uint32_t f = rowf[t * 16 + el16];
      const float scl = a.hmin ? __builtin_ldexpf(cur.wgs, -(int)f) : cur.wgs * __uint_as_float(f);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int e = y16_tile(acc[s][t], scl, ypk[s][t]);
        if (elg == 0) es[(t * 16 + el16) * NBLK + wave * NSUB + s] = (int8_t)e;
      }
    }
    uint16_t* ys = (uint16_t*)&tile[((st0 + KC - 1) % NBUF) * STAGE];
    const __amdgpu_buffer_rsrc_t yr =
        buffer_rsrc(a.yout + (size_t)cur.row0 * a.N, (uint32_t)cur.nvalid * (uint32_t)a.N * 2u);
    const int col0 = cur.nb * COLS;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();                      // ... and every wave's: the stage is free
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
#pragma unroll
      for (int tt = 0; tt < PASS_T; ++tt) {
        const int t = p * PASS_T + tt;
        if (t < TV) {
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            *(u32x2*)(ys + (tt * 16 + el16) * YP + (wave * NSUB + s) * 16 + 4 * elg) = ypk[s][t];
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int k = 0; k < SPP; ++k) {
        const int i = tid + k * NT;
        const int r = i / (COLS / 8), c = i - r * (COLS / 8);
        const u32x4 v = *(const u32x4*)(ys + r * YP + c * 8);
        __builtin_amdgcn_raw_buffer_store_b128(v, yr, (uint32_t)((p * PASS_ROWS + r) * a.N + col0 + c * 8) * 2u,
                                               0, 0);
      }
      if (p + 1 < NPASS) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // the pass's LDS reads are done
        __builtin_amdgcn_s_barrier();
      }
    }
    {
      // block exponents: one row of NBLK bytes per thread (threads past the rows store out of range)
      const __amdgpu_buffer_rsrc_t er =
          buffer_rsrc(a.yexp + (size_t)cur.row0 * (a.N / 16), (uint32_t)cur.nvalid * (uint32_t)(a.N / 16));
      const int r = tid;
      const uint32_t off = r < M ? (uint32_t)(r * (a.N / 16) + col0 / 16) : 0x7FFFFFF0u;
      const int rs = min(r, M - 1);
      if constexpr (NBLK == 16)
        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(es + rs * NBLK), er, off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(*(const u32x2*)(es + rs * NBLK), er, off, 0, 0);
    }
  };

  while (true) {
    item_finish(nxt);
    const Item nn = item_head(m + 2 * PX);
    const int tv = (cur.nvalid + 15) >> 4;
    if (tv > 4) run(IntC<6>());
    else if (tv > 2) run(IntC<4>());
    else run(IntC<2>());
    if (!nxt.ok) break;
    dma_rowf(nxt);
    m += PX;
    ring = (ring + KC) % NBUF;
    cur = nxt;
    nxt = nn;
    first_wait = W_ISSUE + 1 + S;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // every load in flight lands before the workgroup exits
}

template <int NSUB, int TSUB, int NBUF, int WAVES, int OCC>
__global__ __launch_bounds__(64 * WAVES, OCC) void gemm_prefill_down_persist_kernel(GemmArgs a, int NB) {
  // one LDS object (ring, then block exponents, then row factors): with several, the
  // compiler's LDS-DMA wait tracking puts a vmcnt(0) before every ring read
  constexpr int RING = NBUF * TSUB * 16 * 16, ES = TSUB * 16 * WAVES * NSUB / 16, RF = 64 * WAVES / 4;
  __shared__ u32x4 lds[RING + ES + RF];
  prefill_down_run<NSUB, TSUB, NBUF, WAVES>(a, blockIdx.x, gridDim.x, NB, lds, (int8_t*)(lds + RING),
                                            (uint32_t*)(lds + RING + ES));
}

// Skewed prefill batches in one launch: workgroups 0 .. n_hot - 1 run the prefill GEMM over
// the first tile list (experts with many rows: compute bound), the rest the decode GEMM over
// the second (experts with a few rows: weight streaming), so the streaming work takes the
// compute units the hot tiles leave free and follows them as they finish, instead of waiting
// for the whole list. (Alternating the two kinds of work in groups of eight ids measured 25%
// slower than the hot tiles first.) Both parts use the workgroup's 8 waves (the decode part
// splits K eight ways) and one LDS buffer.
template <int MODE_HOT, int MODE_COLD, int TSUB, int NSUB_COLD>
__global__ __launch_bounds__(512, 4) void gemm_split_kernel(GemmArgs hot, GemmArgs cold, int n_hot, int NB,
                                                            int nbx) {
  constexpr int HOT_SLOTS = 3 * TSUB * 16 * 16;
  constexpr int COLD_SLOTS = 8 * NSUB_COLD * WAVE;
  __shared__ u32x4 smem[HOT_SLOTS > COLD_SLOTS ? HOT_SLOTS : COLD_SLOTS];
  const int lin = blockIdx.x;
  if (lin < n_hot) {
    prefill_body<MODE_HOT, 2, TSUB, 3, 8>(hot, lin, NB, smem);
  } else {
    const int c = lin - n_hot;
    decode_body<MODE_COLD, NSUB_COLD, 8>(cold, c % nbx, c / nbx, (f32x4*)smem);
  }
}

// -------------------------------------------------------- prefill GEMM, MX8 modes
// MXFP4 weights x MXFP8 activations on the block-scaled MFMA (16x16x128, no dequantisation).
// Tiles of M token rows of one expert (the plan's tile height: 96, or 64 when experts average
// fewer rows) x (WAVES x NSUB) 16-row weight tiles. Per 128-column chunk the token tile's E4M3
// codes (M rows x 128 bytes, 16-byte slots, piece c of row r at slot 8 r + (c ^ swz8(r))) and
// its E8M0 scales (4 bytes per row; every wave issues one dword DMA so that no branch splits
// the wait-count bookkeeping) arrive in LDS by DMA into a ring of three stages; each
// wave streams its weight tiles (16 bytes per lane per chunk, the scale tile's byte for the
// chunk) into three register sets, both two chunks ahead (an MX8 chunk is a quarter of the
// fp16 kernel's MFMA work per wave, too little to hide a load issued one chunk ahead). An
// MFMA's B operand is pieces lg and 4 + lg of a row (see mfma_mx); with swz8(r) = (r >> 1) & 7
// the 16 rows of a read land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

template <int MODE, int NSUB, int WAVES, int OCC, int M>
__global__ __launch_bounds__(64 * WAVES, OCC) void gemm_prefill_mx8_kernel(GemmArgs a) {
  static_assert(MODE == GEMM_GATEUP_MX8 || MODE == GEMM_DOWN_MX8, "MX8 modes");
  constexpr int TSUB = M / 16;
  constexpr int STAGE = M * 8;                        // 16-byte code slots per stage
  constexpr int SROWS = 64 * WAVES;                   // scale dwords per stage: a row per lane of every wave
  constexpr int NT = 64 * WAVES;
  constexpr int D = STAGE / NT;                       // code DMA instructions per lane per chunk
  static_assert(STAGE % NT == 0 && M <= SROWS && WAVES >= 2, "tile size");
  constexpr int NST = 3;                              // LDS stages (and weight register sets)
  // one LDS object per stage, so that the compiler sees that the DMA into one stage and the
  // reads of another never alias (with one array it waited for every DMA before each read)
  __shared__ u32x4 tile0[STAGE], tile1[STAGE], tile2[STAGE];
  __shared__ uint32_t stile0[SROWS], stile1[SROWS], stile2[SROWS];
  auto stage_tile = [&](auto stc) -> u32x4* {
    constexpr int S = decltype(stc)::value;
    return S == 0 ? tile0 : S == 1 ? tile1 : tile2;
  };
  auto stage_scales = [&](auto stc) -> uint32_t* {
    constexpr int S = decltype(stc)::value;
    return S == 0 ? stile0 : S == 1 ? stile1 : stile2;
  };

  const int ntiles = a.tile_count[0];
  const PrefillItem item = prefill_item(ntiles, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x);
  const int slot = item.slot;
  if (slot >= ntiles) return;
  const int g = __builtin_amdgcn_readfirstlane(a.tile_group[slot]);      // uniform: kept in SGPRs
  const int row0 = __builtin_amdgcn_readfirstlane(a.tile_row0[slot]);
  const ProjLayout L = proj_layout(a.N, a.K);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (WAVE - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const int q0 = (item.nb * WAVES + wave) * NSUB;
  const int nvalid = min(M, a.offsets[g + 1] - row0);
  // activation row of tile row r (clamped): gate_up gathers token rows (offsets from the
  // activation base: T K < 2^32 bytes), down its own rows relative to the tile's first row
  // (64-bit bases below, 32-bit offsets within the tile)
  auto src_row = [&](int r) {
    const int rl = min(r, nvalid - 1);
    return MODE == GEMM_DOWN_MX8 ? rl : a.tok[row0 + rl];
  };
  const uint8_t* qbase = a.xq + (MODE == GEMM_DOWN_MX8 ? (size_t)row0 * L.K : 0);
  const uint8_t* sbase = a.xs + (MODE == GEMM_DOWN_MX8 ? (size_t)row0 * (L.K / 32) : 0);
  // code DMA: instruction i of this wave fills slots (WAVES i + wave) * 64 + lane
  uint32_t src_off[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int sl = (WAVES * i + wave) * 64 + lane;
    const int r = sl >> 3;
    const int kp = (sl & 7) ^ swz8(r);
    src_off[i] = (uint32_t)src_row(r) * L.K + kp * 16;
  }
  // scale DMA: a row per lane of every wave (rows past the tile clamp to its last row)
  const uint32_t s_off = (uint32_t)src_row(wave * 64 + lane) * (L.K / 32);
  auto dma = [&](int kc, auto stc) {
    u32x4* T = stage_tile(stc);
    uint32_t* S = stage_scales(stc);
    const char* base = (const char*)qbase + (size_t)kc * KCHUNK;
#pragma unroll
    for (int i = 0; i < D; ++i) dma16(base + src_off[i], &T[(WAVES * i + wave) * 64]);
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(sbase + s_off + 4 * kc),
                                     (void __attribute__((address_space(3)))*)&S[wave * 64], 4, 0, 0);
  };

  const u32x4* wp[NSUB];
  const uint8_t* sp[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    wp[s] = fp4_tile(a, L, g, q0 + s, 0);
    sp[s] = (const uint8_t*)sc_tile(a, L, g, q0 + s, 0);
  }
  auto load_w = [&](int kc, u32x4 (&w)[NSUB], uint32_t (&sb)[NSUB]) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      w[s] = wp[s][(size_t)kc * WAVE];
      sb[s] = *(const uint32_t*)(sp[s] + (size_t)(kc >> 3) * (WAVE * 16) + (kc & 6) * 2);
    }
  };

  auto body = [&](auto tvc) {
    constexpr int TV = decltype(tvc)::value;
    f32x4 acc[NSUB][TV];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int t = 0; t < TV; ++t) acc[s][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // three register sets and LDS stages: chunk kc + 2 is loaded while chunk kc is consumed.
    // Chunk kc's DMA must have landed; the loads of chunk kc + 1 (weights: 2 NSUB ops; its DMA:
    // D code ops and one scale op) may still be in flight; past the last chunk nothing more is
    // issued and the wait is for everything. Issue order is pinned with scheduling barriers
    // (the wait count covers the LDS stages written by DMA, which the compiler does not track).
    u32x4 rw[NST][NSUB];
    uint32_t rs[NST][NSUB];
    load_w(0, rw[0], rs[0]);
    __builtin_amdgcn_sched_barrier(0);
    dma(0, IntC<0>());
    __builtin_amdgcn_sched_barrier(0);
    if (L.KC > 1) {
      load_w(1, rw[1], rs[1]);
      __builtin_amdgcn_sched_barrier(0);
      dma(1, IntC<1>());
    }
    __builtin_amdgcn_sched_barrier(0);
    auto step = [&](int kc, auto setc, auto kindc) {
      constexpr int C = decltype(setc)::value;          // kc % 3
      constexpr int KIND = decltype(kindc)::value;
      constexpr int NX = (C + 2) % NST;                 // set / stage of chunk kc + 2
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(KIND == STEP_LAST ? 0 : 2 * NSUB + D + 1, 0));
      __builtin_amdgcn_s_barrier();                     // chunk kc in LDS for every wave; stage NX free
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (KIND == STEP_FULL) {
        load_w(kc + 2, rw[NX], rs[NX]);
        __builtin_amdgcn_sched_barrier(0);
        dma(kc + 2, IntC<NX>());
        __builtin_amdgcn_sched_barrier(0);
      }
      const u32x4* T0 = stage_tile(IntC<C>());
      const uint8_t* S0 = (const uint8_t*)stage_scales(IntC<C>());
#pragma unroll
      for (int t = 0; t < TV; ++t) {
        const int r = t * 16 + l16;
        const u32x4 b0 = T0[r * 8 + (lg ^ swz8(r))];
        const u32x4 b1 = T0[r * 8 + ((4 + lg) ^ swz8(r))];
        const uint32_t sbv = S0[r * 4 + lg];
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          acc[s][t] = mfma_mx(rw[C][s], (rs[C][s] >> ((kc & 1) * 16)) & 0xFFu, b0, b1, sbv, acc[s][t]);
      }
    };
    run_chunks(L.KC, step);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // every load in flight lands before the workgroup exits

#pragma unroll
    for (int t = 0; t < TV; ++t) {
      const int rr = t * 16 + l16;
      if (rr >= nvalid) continue;
      const int orow = row0 + rr;
      if constexpr (MODE == GEMM_DOWN_MX8) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) epilogue_single(a, acc[s][t], 1.0f, orow, q0 + s);
      } else {
        const float lim = g < a.clamp_groups ? a.swiglu_limit : INFINITY;
#pragma unroll
        for (int s = 0; s < NSUB; s += 2) epilogue_pair<MODE>(a, acc[s][t], acc[s + 1][t], 1.0f, orow, (q0 + s) >> 1, lim);
      }
    }
  };
  const int tv = (nvalid + 15) >> 4;
  static_assert(TSUB == 6 || TSUB == 4, "row tiers assume 4 or 6 slices");
  if constexpr (TSUB == 6) {
    if (tv > 4) body(IntC<6>());
    else if (tv > 2) body(IntC<4>());
    else body(IntC<2>());
  } else {
    if (tv > 2) body(IntC<4>());
    else body(IntC<2>());
  }
}

// ---------------------------------------------------------------------- launch

template <typename K, typename... Args>
static void launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, const LaunchEvents& ev, const Args&... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Compute units of the current device (read once per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}


// The last launch-bound argument (OCC below) is the minimum number of waves per SIMD, which caps
// the registers of a wave at 512 / OCC.
constexpr int PRE_NSUB_GU = 2;    // prefill gate_up: 1 gate + 1 up tile per wave
constexpr int PRE_NSUB_DN = 2;    // prefill down: 2 tiles per wave
constexpr int PRE_TSUB = 6;       // prefill: 96 token rows per tile (measured 13% faster than 128 rows)
constexpr int PRE_NBUF_GU = 3;    // prefill GEMMs: LDS DMA ring depth (3 x 24 KiB)
constexpr int PRE_WAVES_GU = 8;   // fp16 gate_up and down: 8 waves x 2 tiles = 256 weight rows per token
constexpr int PRE_OCC_GU = 4;     // tile, two workgroups per CU (128 registers). Against 4 waves x 2 tiles
                                  // at 3 per CU: half the token-tile DMA per MFMA, gate_up 5-11% faster.
                                  // One workgroup per CU with weights and tiles two chunks ahead in three
                                  // sets (192 registers) measured 20% slower: occupancy hides more latency
constexpr int DEC_MIN_WGS = 2048; // decode: 8 workgroups per CU before 4 tiles per workgroup are used
constexpr int PERSIST_MAX_KC = 8; // prefill down with at most 8 K chunks (K <= 1024): the persistent
                                  // launch (Qwen3 K = 768: 133 -> 130 us; FP8 rows 130 -> 124 us). At
                                  // K = 2048 it measured 5% slower than one workgroup per item

// Decode split: 4 weight tiles per workgroup (twice the reuse of each token-operand load)
// when that still gives about 8 workgroups per CU, else 2; the K chunks go to the largest
// of 4 / 3 / 2 waves that divides them evenly (4 if none does).
template <int MODE>
static void launch_decode(int max_tiles, int est_tiles, const GemmArgs& a, hipStream_t s,
                          const LaunchEvents& ev) {
  const int nsub16 = a.N / 16, kc = a.K / KCHUNK;
  const bool many = nsub16 % 4 == 0 && (long)est_tiles * (nsub16 / 4) >= DEC_MIN_WGS;
  const bool wide = many || (MODE == GEMM_GATEUP_MX8 && a.hq8);   // MXFP8 h blocks: 4 tiles
  int nw = kc % 4 == 0 ? 4 : kc % 3 == 0 ? 3 : kc % 2 == 0 ? 2 : 4;
  nw = min(nw, kc);
  if constexpr (MODE == GEMM_GATEUP_MX8) {
    if (wide && (long)est_tiles * (nsub16 / 4) < DEC_MIN_WGS / 4 && kc % 8 == 0) {   // a small grid: 8 waves
      launch_k(gemm_decode_kernel<MODE, 4, 8>, dim3(nsub16 / 4, max_tiles), dim3(64 * 8), s, ev, a);
      return;
    }
  }
  if (wide) {
    launch_k(gemm_decode_kernel<MODE, 4>, dim3(nsub16 / 4, max_tiles), dim3(64 * nw), s, ev, a);
  } else {
    launch_k(gemm_decode_kernel<MODE, 2>, dim3(nsub16 / 2, max_tiles), dim3(64 * nw), s, ev, a);
  }
}

template <int MODE>
static hipError_t launch_mode(GemmRegime regime, int max_tiles, int est_tiles, const GemmArgs& a, hipStream_t s,
                              const LaunchEvents& ev) {
  if (regime == REGIME_DECODE_KSPLIT) {
    launch_decode<MODE>(max_tiles, est_tiles, a, s, ev);
  } else if constexpr (MODE == GEMM_GATEUP_F16 || MODE == GEMM_DOWN) {   // the prefill GEMMs: fp16 rows
    const int ny = (max_tiles + 7) / 8 * 8;
    constexpr int W = PRE_WAVES_GU, NS = MODE == GEMM_DOWN ? PRE_NSUB_DN : PRE_NSUB_GU;
    const bool t64 = a.tile_rows == 64;
    if (!t64 && a.tile_rows != PREFILL_TILE_ROWS) return hipErrorInvalidValue;
    const int NB = a.N / (16 * W * NS);
    const int kcs = a.K / KCHUNK;
    if (MODE == GEMM_DOWN && !t64 && a.N % (16 * W * NS) == 0 && kcs % 2 == 0 && kcs <= PERSIST_MAX_KC) {
      // resident workgroups, two per CU, each running a sequence of (tile, column block) items
      const int P = min(2 * device_cus() / 8 * 8, ny * NB);
      launch_k(gemm_prefill_down_persist_kernel<NS, PRE_TSUB, PRE_NBUF_GU, W, PRE_OCC_GU>, dim3(P), dim3(64 * W), s,
               ev, a, NB);
    } else if (a.N % (16 * W * NS) == 0)
      launch_k(t64 ? gemm_prefill_kernel<MODE, NS, 4, PRE_NBUF_GU, W, PRE_OCC_GU>
                   : gemm_prefill_kernel<MODE, NS, PRE_TSUB, PRE_NBUF_GU, W, PRE_OCC_GU>,
               dim3(a.N / (16 * W * NS), ny), dim3(64 * W), s, ev, a);
    else if (MODE == GEMM_DOWN)   // hidden a multiple of 128 only: one 16-column tile per wave covers it exactly
      launch_k(t64 ? gemm_prefill_kernel<MODE, 1, 4, PRE_NBUF_GU, W, PRE_OCC_GU>
                   : gemm_prefill_kernel<MODE, 1, PRE_TSUB, PRE_NBUF_GU, W, PRE_OCC_GU>,
               dim3(a.N / (16 * W), ny), dim3(64 * W), s, ev, a);
    else
      return hipErrorInvalidValue;   // gate_up: N = 2I, a multiple of 256
  } else {
    return hipErrorInvalidValue;     // the NVFP4 modes run in the decode regime only
  }
  return hipSuccess;
}

constexpr int PRE_WAVES_MX8 = 4;   // MX8 prefill: 4 waves x 2 weight tiles (a 2 x 2 wave layout with the
constexpr int PRE_NSUB_MX8 = 2;    // token rows split measured 9% slower), 2 workgroups per CU
constexpr int PRE_OCC_MX8 = 2;

template <int MODE>
static void launch_mx8(GemmRegime regime, int max_tiles, int est_tiles, const GemmArgs& a, hipStream_t s,
                       const LaunchEvents& ev) {
  if (regime == REGIME_DECODE_KSPLIT) {
    launch_decode<MODE>(max_tiles, est_tiles, a, s, ev);
    return;
  }
  constexpr int W = PRE_WAVES_MX8, NS = PRE_NSUB_MX8;   // N = 2I or H, multiples of 128
  const int ny = (max_tiles + 7) / 8 * 8;
  const dim3 grid(a.N / (16 * W * NS), ny);
  if (a.tile_rows == 64)
    launch_k(gemm_prefill_mx8_kernel<MODE, NS, W, PRE_OCC_MX8, 64>, grid, dim3(64 * W), s, ev, a);
  else
    launch_k(gemm_prefill_mx8_kernel<MODE, NS, W, PRE_OCC_MX8, PREFILL_TILE_ROWS>, grid, dim3(64 * W), s, ev, a);
}

hipError_t launch_gemm(GemmMode mode, GemmRegime regime, int max_tiles, int est_tiles, const GemmArgs& a,
                       hipStream_t s, const LaunchEvents& ev) {
  if (max_tiles <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  switch (mode) {
    case GEMM_GATEUP_F16: e = launch_mode<GEMM_GATEUP_F16>(regime, max_tiles, est_tiles, a, s, ev); break;
    case GEMM_GATEUP_FP4: e = launch_mode<GEMM_GATEUP_FP4>(regime, max_tiles, est_tiles, a, s, ev); break;
    case GEMM_DOWN: e = launch_mode<GEMM_DOWN>(regime, max_tiles, est_tiles, a, s, ev); break;
    case GEMM_DOWN_FP4: e = launch_mode<GEMM_DOWN_FP4>(regime, max_tiles, est_tiles, a, s, ev); break;
    case GEMM_GATEUP_MX8: launch_mx8<GEMM_GATEUP_MX8>(regime, max_tiles, est_tiles, a, s, ev); break;
    case GEMM_DOWN_MX8: launch_mx8<GEMM_DOWN_MX8>(regime, max_tiles, est_tiles, a, s, ev); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// ------------------------------------------------------------------- h rescale
// Between the prefill GEMMs: h16 rows of the first tile list's groups (plain column order, a
// power-of-two exponent per 16-column block) brought in place to the row's common exponent
// P = hmin[row] (the smallest block exponent, i.e. the scale of the row's largest block):
// h16 *= 2^(P - hexp[block]). The down GEMM then streams whole rows by LDS DMA and applies
// gs_e 2^-P in its epilogue. Grid (I / 128, tile bound): workgroup (c, slot) takes chunk c of
// the valid rows of tile `slot`; a thread rescales one 16-byte piece (8 columns of one block)
// at a time, so every element is read and written by the same thread.
__global__ __launch_bounds__(256) void h_rescale_kernel(uint16_t* __restrict__ h, const int8_t* __restrict__ hexp,
                                                        const int32_t* __restrict__ hmin,
                                                        const int32_t* __restrict__ tile_group,
                                                        const int32_t* __restrict__ tile_row0,
                                                        const int32_t* __restrict__ tile_count,
                                                        const int32_t* __restrict__ offsets, int tile_rows, int I) {
  const int slot = blockIdx.y;
  if (slot >= tile_count[0]) return;
  const int g = tile_group[slot], row0 = tile_row0[slot];
  const int nvalid = min(tile_rows, offsets[g + 1] - row0);
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < nvalid * 16; i += blockDim.x) {
    const size_t r = (size_t)row0 + (i >> 4);
    const int p = i & 15;
    uint16_t* ptr = h + r * I + c * KCHUNK + p * 8;
    const _Float16 f = h_factor(hmin[r] - (int)hexp[r * (I / 16) + c * 8 + (p >> 1)]);
    *(f16x8*)ptr = *(const f16x8*)ptr * f;
  }
}

hipError_t launch_h_rescale(uint16_t* h, const int8_t* hexp, const int32_t* hmin, const int32_t* tile_group,
                            const int32_t* tile_row0, const int32_t* tile_count, const int32_t* offsets,
                            int max_tiles, int tile_rows, int I, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(h_rescale_kernel, dim3(I / KCHUNK, max_tiles), dim3(256), 0, s, h, hexp, hmin, tile_group,
                     tile_row0, tile_count, offsets, tile_rows, I);
  return hipGetLastError();
}

// Skewed prefill batches: both tile lists in one launch (gemm_split_kernel). The hot part is
// the prefill GEMM at 8 waves x 2 tiles (N a multiple of 256); the cold part the decode GEMM at
// 4 tiles per workgroup (N a multiple of 64).
template <int MODE_HOT, int MODE_COLD>
static void launch_split_modes(dim3 grid, const GemmArgs& hot, const GemmArgs& cold, int n_hot, int NB, int nbx,
                               hipStream_t s, const LaunchEvents& ev) {
  auto kernel = gemm_split_kernel<MODE_HOT, MODE_COLD, 4, 4>;
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, dim3(512), 0, s, ev.start, ev.stop, 0, hot, cold, n_hot, NB, nbx);
  else
    hipLaunchKernelGGL(kernel, grid, dim3(512), 0, s, hot, cold, n_hot, NB, nbx);
}

hipError_t launch_gemm_split(GemmMode hot_mode, GemmMode cold_mode, int max_tiles, int cold_tiles,
                             const GemmArgs& hot, const GemmArgs& cold, hipStream_t s, const LaunchEvents& ev) {
  // 64-row hot tiles only (the plan's tile height for skewed batches)
  if (hot.N % (16 * PRE_WAVES_GU * 2) || cold.N % 64 || hot.tile_rows != 64)
    return hipErrorNotSupported;   // declined: nothing launched
  const int NB = hot.N / (16 * PRE_WAVES_GU * 2);
  const int n_hot = NB * ((max_tiles + 7) / 8 * 8);
  const int nbx = cold.N / 64;
  const long total = (long)n_hot + (long)nbx * cold_tiles;
  if (total <= 0 || total > (1L << 31) - 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total);
  if (hot_mode == GEMM_GATEUP_F16 && cold_mode == GEMM_GATEUP_F16)
    launch_split_modes<GEMM_GATEUP_F16, GEMM_GATEUP_F16>(grid, hot, cold, n_hot, NB, nbx, s, ev);
  else if (hot_mode == GEMM_DOWN && cold_mode == GEMM_DOWN)
    launch_split_modes<GEMM_DOWN, GEMM_DOWN>(grid, hot, cold, n_hot, NB, nbx, s, ev);
  else if (hot_mode == GEMM_DOWN && cold_mode == GEMM_DOWN_FP4)
    launch_split_modes<GEMM_DOWN, GEMM_DOWN_FP4>(grid, hot, cold, n_hot, NB, nbx, s, ev);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

// ---------------------------------------------------------------------- combine
// out[t] = bf16( sum_j w[t][j] * y[inv[t][j]]  (+ y_shared[t]) ), fp32, picks in
// order, shared expert last ([vllm.cpp] "Device-resident decode campaign",
// MoeCombineKernel: device FMA of the topk_weights over the expert outputs).
// Grid (T, H / 512): a 128-thread workgroup owns 512 columns of one token; the k row
// indices and weights are staged in LDS first so that all k row loads of a thread are
// independent and in flight together.
constexpr int COMBINE_COLS = 512;
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  __shared__ int s_inv[64];
  __shared__ float s_w[64];
  const int t = blockIdx.x;
  const int rows = a.T * a.k;
  if ((int)threadIdx.x < a.k) {
    s_inv[threadIdx.x] = a.inv[t * a.k + threadIdx.x];
    s_w[threadIdx.x] = a.w[t * a.k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * (COMBINE_COLS / 4) + threadIdx.x;   // 4-column group index
  if (c >= a.H / 4) return;
  // row r's columns 4c .. 4c+3: fp16 values and their block's exponent, exactly in fp32
  struct Raw {
    u32x2 q;
    int e;
  };
  auto fetch = [&](int r) {
    Raw v;
    v.q = *(const u32x2*)(a.y + (size_t)r * a.H + c * 4);
    v.e = a.yexp[(size_t)r * (a.H / 16) + (c >> 2)];
    return v;
  };
  auto decode = [](const Raw& v) {
    auto f = [&](uint32_t b) { return __builtin_ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)b), -v.e); };
    return f32x4{f(v.q.x & 0xFFFFu), f(v.q.x >> 16), f(v.q.y & 0xFFFFu), f(v.q.y >> 16)};
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // 8 rows per round, all loaded before any is summed: indices past k are clamped to the
  // last row and the loaded values pinned (otherwise each load is sunk into the branch of its
  // term and waited for there); the terms past k are skipped, so the sum runs in j order
  for (int j = 0; j < a.k; j += 8) {
    Raw v[8];
    float wq[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      v[q] = fetch(s_inv[min(j + q, a.k - 1)]);
      wq[q] = s_w[min(j + q, a.k - 1)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) asm volatile("" : "+v"(v[q].q.x), "+v"(v[q].q.y), "+v"(v[q].e), "+v"(wq[q]));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j + q < a.k) {
        const f32x4 d = decode(v[q]);
        const float wj = wq[q];
        acc.x = __builtin_fmaf(wj, d.x, acc.x);
        acc.y = __builtin_fmaf(wj, d.y, acc.y);
        acc.z = __builtin_fmaf(wj, d.z, acc.z);
        acc.w = __builtin_fmaf(wj, d.w, acc.w);
      }
  }
  for (int sh = 0; sh < a.S; ++sh) acc += decode(fetch(rows + sh * a.T + t));
  *(u32x2*)(a.out + (size_t)t * a.H + c * 4) =
      u32x2{f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16),
            f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16)};
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s, const LaunchEvents& ev) {
  if (a.T <= 0) return hipSuccess;
  const dim3 grid(a.T, (a.H + COMBINE_COLS - 1) / COMBINE_COLS);
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(combine_kernel, grid, dim3(128), 0, s, ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL(combine_kernel, grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvmoe

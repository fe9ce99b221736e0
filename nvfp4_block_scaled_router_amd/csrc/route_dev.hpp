// Device-side routing pieces shared by the routing kernels and the decode GEMM that plans
// its own tiles: orderable keys, DPP wave/row argmax and sums, per-token top-k (wave and
// 16-lane-row variants) and the LDS wave scan.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace nvmoe {

// Orderable 32-bit image of a finite float (larger float -> larger key); -0 maps to +0
// so that the two zeros tie and fall back to the expert id.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Logits l, l + STRIDE, ... of one token (lane l of a group of STRIDE lanes). The indices
// are clamped to the last expert rather than guarded, and each value is pinned by an empty
// asm statement: a load whose value is used only where e < E is otherwise sunk into a branch
// of its own and waited for there, one memory round trip per load. The values past E are
// never used.
template <int N, int STRIDE>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int l, float* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = row[min(l + STRIDE * i, E - 1)];
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Inverse of order_key (the value of a pick, without touching memory again).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// Max of the 64-bit keys (hi, lo) across the wave, with DPP butterflies inside each
// 16-lane row and lane reads across the 4 rows. The result is wave-uniform. Any
// reduction tree gives the same winner because the keys are a total order.
template <int CTRL>
__device__ __forceinline__ void dpp_max64(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, CTRL, 0xF, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, CTRL, 0xF, 0xF, false);
  const bool take = ohi > hi || (ohi == hi && olo > lo);
  hi = take ? ohi : hi;
  lo = take ? olo : lo;
}

// 64-bit key = (order_key(logit) << 32) | ~expert: the maximum is the largest logit with
// the lowest expert id. Finite logits give a non-zero high word, so 0 marks an empty or
// already taken slot.
__device__ __forceinline__ uint64_t pick_key(uint32_t okey, int e) {
  return ((uint64_t)okey << 32) | (uint32_t)~(uint32_t)e;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Max over the 16 lanes of a row; every lane of the row gets it.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_u64<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_u64<0x141>(v);   // row_half_mirror
  return dpp_max_u64<0x140>(v);   // row_mirror
}

__device__ __forceinline__ void wave_max64(uint32_t& hi, uint32_t& lo) {
  dpp_max64<0xB1>(hi, lo);    // quad_perm [1,0,3,2]
  dpp_max64<0x4E>(hi, lo);    // quad_perm [2,3,0,1]
  dpp_max64<0x141>(hi, lo);   // row_half_mirror
  dpp_max64<0x140>(hi, lo);   // row_mirror: every lane holds its row's max
  uint32_t bh = (uint32_t)__builtin_amdgcn_readlane((int)hi, 0), bl = (uint32_t)__builtin_amdgcn_readlane((int)lo, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_readlane((int)hi, r);
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_readlane((int)lo, r);
    if (h2 > bh || (h2 == bh && l2 > bl)) {
      bh = h2;
      bl = l2;
    }
  }
  hi = bh;
  lo = bl;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the wave in a fixed order (deterministic): butterflies inside 16-lane rows,
// then the four row sums added in row order. Wave-uniform result.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  float t = 0.0f;
#pragma unroll
  for (int r = 0; r < 64; r += 16) t += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), r));
  return t;
}

// One wave routes token t. EPL = experts per lane (E <= 64*EPL); lane l holds experts
// l, l+64, ... Key of expert e: (order_key(logit), ~e), so the maximum is the largest
// logit with the lowest id. Each lane keeps its best untaken candidate; after a pick only
// the owning lane rescans. Picks j < k end up in lane j. Outputs go to global memory and,
// if s_ids/s_w are given, to LDS.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lg, int E, int k, int score,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int32_t* __restrict__ ids_user, float* __restrict__ w_user,
                                            int t, int32_t* s_ids = nullptr, float* s_w = nullptr) {
  const int lane = threadIdx.x & (WAVE - 1);
  float v[EPL];
  load_logits<EPL, WAVE>(lg + (size_t)t * E, E, lane, v);
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) key[i] = lane + WAVE * i < E ? order_key(v[i]) : 0u;
  uint32_t taken = 0;
  auto local_best = [&](uint32_t& bh, uint32_t& bl) {
    bh = 0u;
    bl = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + WAVE * i;
      const uint32_t l = ~(uint32_t)e;
      // keys of real experts are > 0 in hi, so an empty slot (hi = 0, lo = 0) never wins
      if (e < E && !((taken >> i) & 1u) && (key[i] > bh || (key[i] == bh && l > bl))) {
        bh = key[i];
        bl = l;
      }
    }
  };
  uint32_t ch, cl;
  local_best(ch, cl);
  float my_v = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t wh = ch, wl = cl;
    wave_max64(wh, wl);
    const int e = (int)~wl;
    if (lane == (e & (WAVE - 1))) {
      taken |= 1u << (e / WAVE);
      local_best(ch, cl);
    }
    if (lane == j) {
      my_id = e;
      my_v = key_value(wh);
    }
  }
  // weights over the k picks, in fp32; lane j holds pick j
  const float lmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
  float s = 0.0f;
  if (lane < k) s = score == 0 ? __expf(my_v - lmax) : 1.0f / (1.0f + __expf(-my_v));
  const float sum = wave_sum(s);
  if (lane < k) {
    const float wj = s / sum;
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = wj;
    if (ids_user) ids_user[(size_t)t * k + lane] = my_id;
    if (w_user) w_user[(size_t)t * k + lane] = wj;
    if (s_ids) s_ids[t * k + lane] = my_id;
    if (s_w) s_w[t * k + lane] = wj;
  }
}

// ------------------------------------------------------------------------------
// Row-level routing: one 16-lane DPP row routes one token, so a wave routes four tokens
// at once and the pick reduction (4 DPP butterflies on the 64-bit key) never leaves the
// row: no cross-row lane reads, no scalar branches. Used when E <= 256.

// Sum over the 16 lanes of a row, identical in every lane of the row (a fixed butterfly;
// each addition is commutative, so all lanes compute the same bits).
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

// Descending sort of a lane's N keys in registers: Batcher's odd-even merge sort, a fixed
// network of compare-exchanges (19 for N = 8), fully unrolled.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t* a) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1)
#pragma unroll
    for (int kk = p; kk >= 1; kk >>= 1)
#pragma unroll
      for (int j = kk % p; j + kk < N; j += 2 * kk)
#pragma unroll
        for (int i = 0; i < kk; ++i)
          if (i + j + kk < N && (i + j) / (2 * p) == (i + j + kk) / (2 * p)) {
            const uint64_t x = a[i + j], y = a[i + j + kk];
            a[i + j] = x > y ? x : y;
            a[i + j + kk] = x > y ? y : x;
          }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  // old value 0, the identity of an unsigned max, so that the move fuses into v_max_u32_dpp
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return o > v ? o : v;
}
// Max over the 16 lanes of a row; every lane of the row gets it.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_u32<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_u32<0x141>(v);   // row_half_mirror
  return dpp_max_u32<0x140>(v);   // row_mirror
}

// Max over the wave, uniform: the row maxima, then the four rows' through lane reads.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max_u32(v);
  uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)v, r));
  return m;
}

// Lane r16 of the row holds experts r16, r16+16, ... (EPR = ceil(E/16) <= 16) as 64-bit
// pick keys, sorted descending in registers, so its best untaken key is always key[0].
// A pick is the row maximum of the lanes' first keys, found word by word: the largest
// high word (the logit), then among the lanes holding it the largest low word (the lowest
// expert id); the winning lane shifts its keys up by one. Everything is branch free except
// the final stores. Pick j (k <= 64) is kept by lane j % 16 in slot j / 16.
template <int EPR>
__device__ __forceinline__ void route_token_row(const float* __restrict__ lg, int E, int k, int score, int t,
                                                int32_t* __restrict__ ids, float* __restrict__ w,
                                                int32_t* __restrict__ ids_user, float* __restrict__ w_user,
                                                int32_t* s_ids) {
  const int r16 = threadIdx.x & 15;
  float v[EPR];
  load_logits<EPR, 16>(lg + (size_t)t * E, E, r16, v);
  uint64_t key[EPR];
#pragma unroll
  for (int i = 0; i < EPR; ++i) {
    const int e = r16 + 16 * i;
    key[i] = e < E ? pick_key(order_key(v[i]), e) : 0ull;
  }
  sort_desc<EPR>(key);
  uint64_t pk[4] = {0ull, 0ull, 0ull, 0ull};
  uint64_t key0 = 0ull;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jend = min(k, 16 * q + 16);
    for (int j = 16 * q; j < jend; ++j) {
      const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
      const uint32_t mh = row_max_u32(hi);
      const uint32_t ml = row_max_u32(hi == mh ? lo : 0u);
      const uint64_t win = ((uint64_t)mh << 32) | ml;   // row-uniform
      // the shift as a bit mask made opaque to the compiler: written as selects, it becomes an
      // indexed extract (a compare chain per key)
      uint32_t m = key[0] == win ? 0xFFFFFFFFu : 0u;
      asm volatile("" : "+v"(m));
      const uint64_t m64 = ((uint64_t)m << 32) | m;
#pragma unroll
      for (int i = 0; i + 1 < EPR; ++i) key[i] = (key[i + 1] & m64) | (key[i] & ~m64);
      key[EPR - 1] &= ~m64;
      if (q == 0 && j == 0) key0 = win;
      pk[q] = r16 == j - 16 * q ? win : pk[q];
    }
  }
  const float lmax = key_value((uint32_t)(key0 >> 32));
  float sv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    sv[q] = 0.0f;
    if (r16 + 16 * q < k) {
      const float v = key_value((uint32_t)(pk[q] >> 32));
      sv[q] = score == 0 ? __expf(v - lmax) : 1.0f / (1.0f + __expf(-v));
    }
  }
  const float sum = row_sum(((sv[0] + sv[1]) + sv[2]) + sv[3]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = r16 + 16 * q;
    if (j < k) {
      const float wj = sv[q] / sum;
      const int id = (int)~(uint32_t)pk[q];
      if (ids) ids[(size_t)t * k + j] = id;
      if (w) w[(size_t)t * k + j] = wj;
      if (ids_user) ids_user[(size_t)t * k + j] = id;
      if (w_user) w_user[(size_t)t * k + j] = wj;
      if (s_ids) s_ids[t * k + j] = id;
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (row shifts, then the two
// row broadcasts of the classic gfx9 scan).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Executed by one whole wave: exclusive scans of a[0..n) and b[0..n) in LDS (in place),
// totals written to a[n] and b[n]. Lane l owns a contiguous segment of ceil(n/64).
__device__ __forceinline__ void wave_dual_scan(int* a, int* b, int n) {
  const int lane = threadIdx.x & 63;
  const int seg = (n + 63) / 64, i0 = lane * seg, i1 = min(n, i0 + seg);
  int sa = 0, sb = 0;
  for (int i = i0; i < i1; ++i) {
    sa += a[i];
    sb += b[i];
  }
  const int ia = wave_inclusive_scan(sa), ib = wave_inclusive_scan(sb);
  int ra = ia - sa, rb = ib - sb;
  for (int i = i0; i < i1; ++i) {
    const int ca = a[i], cb = b[i];
    a[i] = ra;
    b[i] = rb;
    ra += ca;
    rb += cb;
  }
  if (lane == 63) {
    a[n] = ia;
    b[n] = ib;
  }
}

// Executed by one whole wave: exclusive scan of a[0..n) in LDS (in place), total in a[n].
__device__ __forceinline__ void wave_scan(int* a, int n) {
  const int lane = threadIdx.x & 63;
  const int seg = (n + 63) / 64, i0 = lane * seg, i1 = min(n, i0 + seg);
  int sa = 0;
  for (int i = i0; i < i1; ++i) sa += a[i];
  const int ia = wave_inclusive_scan(sa);
  int ra = ia - sa;
  for (int i = i0; i < i1; ++i) {
    const int ca = a[i];
    a[i] = ra;
    ra += ca;
  }
  if (lane == 63) a[n] = ia;
}

}  // namespace nvmoe

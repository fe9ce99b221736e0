// Routing: wave-level top-k with renormalised weights, per-expert histogram,
// prefix-scan offsets, stable expert-major permutation and the GEMM tile list.
//
// Selection order is the strict total order (logit desc, expert id asc): an argmax
// under a total order gives the same winner for any reduction tree, so the wave
// butterfly below is exact ([vllm.cpp] "DeepSeek-V4-Flash decode ds4-gap - Lever 3":
// one warp per token, per-lane argmax then a shuffle reduction, bit-identical to
// the one-thread loop). Counts come from integer LDS atomics (order free); the
// permutation from per-chunk token bitmaps, so it is unique and deterministic
// ([megamoe] CUDA_GRAPH_SYNC_INVENTORY: counts by scatter into a pre-allocated
// device buffer, offsets kept on device, no host read).
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
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + WAVE * i;
    key[i] = e < E ? order_key(lg[(size_t)t * E + e]) : 0u;
  }
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

// Lane r16 of the row holds experts r16, r16+16, ... (EPR = ceil(E/16) <= 16) as 64-bit
// pick keys; its candidate is the max of its keys, a picked expert's key is cleared to 0.
// Everything is branch free except the final stores. Pick j (k <= 64) is kept by lane
// j % 16 in slot j / 16.
template <int EPR>
__device__ __forceinline__ void route_token_row(const float* __restrict__ lg, int E, int k, int score, int t,
                                                int32_t* __restrict__ ids, float* __restrict__ w,
                                                int32_t* __restrict__ ids_user, float* __restrict__ w_user,
                                                int32_t* s_ids) {
  const int r16 = threadIdx.x & 15;
  uint64_t key[EPR];
#pragma unroll
  for (int i = 0; i < EPR; ++i) {
    const int e = r16 + 16 * i;
    key[i] = e < E ? pick_key(order_key(lg[(size_t)t * E + e]), e) : 0ull;
  }
  uint64_t pk[4] = {0ull, 0ull, 0ull, 0ull};
  uint64_t key0 = 0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t cand = key[0];
#pragma unroll
    for (int i = 1; i < EPR; ++i) cand = key[i] > cand ? key[i] : cand;
    const uint64_t win = row_max_u64(cand);           // row-uniform
    const int e = (int)~(uint32_t)win;
    if (j == 0) key0 = win;
#pragma unroll
    for (int i = 0; i < EPR; ++i) key[i] = (r16 + 16 * i == e) ? 0ull : key[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) pk[q] = (16 * q + r16 == j) ? win : pk[q];
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
      ids[(size_t)t * k + j] = id;
      w[(size_t)t * k + j] = wj;
      if (ids_user) ids_user[(size_t)t * k + j] = id;
      if (w_user) w_user[(size_t)t * k + j] = wj;
      if (s_ids) s_ids[t * k + j] = id;
    }
  }
}

// 256 threads = 16 rows = 16 tokens per workgroup.
template <int EPR>
__global__ __launch_bounds__(256) void route_row_kernel(RouteArgs a) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= a.T) return;   // whole rows leave together
  route_token_row<EPR>(a.logits, a.E, a.k, a.score, t, a.ids, a.w, a.ids_user, a.w_user, nullptr);
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

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  route_token<EPL>(a.logits, a.E, a.k, a.score, a.ids, a.w, a.ids_user, a.w_user, t);
}

// ------------------------------------------------------------------------------
// Generalised router, one wave per token (lane l holds experts l, l+64, ...):
//   s_e   FP64 score: softmax over all E (max logit, then the wave's fixed-order FP64
//         sum of exp), sigmoid, or sqrt(softplus(l)) computed as
//         sqrt(max(l, 0) + log1p(exp(-|l|)));
//   key_e binary32: fp32(s_e), plus the bias (a binary32 add) when one is packed;
//   group step: for each group its best and second-best key (two wave argmaxes),
//         the binary32 sum as the group score held by lane q, then topk_group wave
//         argmaxes over the lanes (lower group id on ties); experts of dropped groups
//         get the empty key 0;
//   picks: k wave argmaxes over (key, lower id) as in route_token;
//   w_j   = s_j / (FP64 wave sum of the picks' s) or s_j, times the routed scale.
// The pages name these variants: sqrt-softplus scores with a selection-only bias
// ([vllm.cpp] DeepSeek-V4 bring-up log, W6; [megamoe] archived CORRECTNESS_BACKLOG §5,
// Dense Router), the noaux_tc group step and routed scaling ([vllm.cpp] capability
// table: GLM-4.7-Flash and Laguna rows).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) v += __shfl_xor(v, m);   // same pairs in every lane
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

template <int EPL>
__device__ __forceinline__ void route_token_general(const RouteArgs& r, int t, int32_t* s_ids) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int E = r.E, k = r.k;
  const float* lg = r.logits + (size_t)t * E;
  float lv[EPL];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + WAVE * i;
    lv[i] = e < E ? lg[e] : 0.0f;
    if (e < E) lmax = fmaxf(lmax, lv[i]);
  }
  double denom = 1.0;
  if (r.score == 0) {
    lmax = wave_max_f32(lmax);
    double d = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + WAVE * i < E) d += exp((double)lv[i] - (double)lmax);
    denom = wave_sum_f64(d);
  }
  double sc[EPL];
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + WAVE * i;
    sc[i] = 0.0;
    key[i] = 0u;
    if (e < E) {
      const double l = (double)lv[i];
      double v;
      if (r.score == 0) v = exp(l - (double)lmax) / denom;
      else if (r.score == 1) v = 1.0 / (1.0 + exp(-l));
      else v = sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
      sc[i] = v;
      float kf = (float)v;
      if (r.bias) kf = kf + r.bias[e];
      key[i] = order_key(kf);
    }
  }
  if (r.n_group > 1) {
    const int gsz = E / r.n_group;
    float gscore = 0.0f;                                  // lane q: score of group q
    for (int q = 0; q < r.n_group; ++q) {
      uint64_t b1 = 0ull, b2 = 0ull;                      // this lane's two best keys in group q
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + WAVE * i;
        if (e < E && e / gsz == q) {
          const uint64_t pk = pick_key(key[i], e);
          if (pk > b1) {
            b2 = b1;
            b1 = pk;
          } else if (pk > b2) {
            b2 = pk;
          }
        }
      }
      uint32_t h1 = (uint32_t)(b1 >> 32), l1 = (uint32_t)b1;
      wave_max64(h1, l1);
      const uint64_t w1 = ((uint64_t)h1 << 32) | l1;
      const uint64_t c = b1 == w1 ? b2 : b1;              // the winner's lane offers its second
      uint32_t h2 = (uint32_t)(c >> 32), l2 = (uint32_t)c;
      wave_max64(h2, l2);
      const float g = h2 == 0u ? key_value(h1) : key_value(h1) + key_value(h2);
      if (lane == q) gscore = g;
    }
    uint64_t kept = 0ull;
    uint32_t gk = lane < r.n_group ? order_key(gscore) : 0u;
    for (int j = 0; j < r.topk_group; ++j) {
      uint32_t h = gk, l = gk ? ~(uint32_t)lane : 0u;
      wave_max64(h, l);
      const int q = (int)~l;
      kept |= 1ull << q;
      if (lane == q) gk = 0u;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + WAVE * i;
      if (e < E && !((kept >> (e / gsz)) & 1ull)) key[i] = 0u;
    }
  }
  // k picks: each lane keeps its best untaken candidate, only the owner rescans
  uint32_t taken = 0;
  auto local_best = [&](uint32_t& bh, uint32_t& bl) {
    bh = 0u;
    bl = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + WAVE * i;
      const uint32_t l = ~(uint32_t)e;
      if (key[i] != 0u && !((taken >> i) & 1u) && (key[i] > bh || (key[i] == bh && l > bl))) {
        bh = key[i];
        bl = l;
      }
    }
  };
  uint32_t ch, cl;
  local_best(ch, cl);
  double my_s = 0.0;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t wh = ch, wl = cl;
    wave_max64(wh, wl);
    const int e = (int)~wl;
    const int owner = e & (WAVE - 1), slot = e / WAVE;
    double se = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == slot) se = sc[i];
    se = __shfl(se, owner);
    if (lane == owner) {
      taken |= 1u << slot;
      local_best(ch, cl);
    }
    if (lane == j) {
      my_id = e;
      my_s = se;
    }
  }
  const double sum = wave_sum_f64(lane < k ? my_s : 0.0);
  if (lane < k) {
    const float wj = (float)((r.renorm ? my_s / sum : my_s) * (double)r.scaling);
    r.ids[(size_t)t * k + lane] = my_id;
    r.w[(size_t)t * k + lane] = wj;
    if (r.ids_user) r.ids_user[(size_t)t * k + lane] = my_id;
    if (r.w_user) r.w_user[(size_t)t * k + lane] = wj;
    if (s_ids) s_ids[t * k + lane] = my_id;
  }
}

template <int EPL>
__global__ __launch_bounds__(256) void route_general_kernel(RouteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;   // whole waves leave together
  route_token_general<EPL>(a, t, nullptr);
}

// Small batches (T <= 64, T*k <= 4096): routing, counts, offsets, permutation and tile
// list in one 1024-thread workgroup, everything in LDS. 64 DPP rows route up to 64 tokens
// at once (E <= 256; wider expert sets use one wave per token); one wave runs the two
// scans; global memory is read once (logits) and written at the end. A token's experts
// are distinct, so an expert's rank of token t is the number of earlier tokens in that
// expert's 64-bit token bitmap.
template <int EPL>
__global__ __launch_bounds__(1024) void plan_small_kernel(RouteArgs r, PlanArgs a) {
  extern __shared__ int lds[];
  const int G = a.G, E = a.E, T = a.T, k = a.k, rows = T * k, M = a.tile_rows;
  const int tid = threadIdx.x, nthr = blockDim.x;
  int* s_ids = lds;                          // [rows]
  int* cnt = s_ids + rows;                   // [G]
  int* off = cnt + G;                        // [G+1] row offsets
  int* tl = off + G + 1;                     // [G+1] tile starts
  uint32_t* bits = (uint32_t*)(tl + G + 1);  // [E][2] token bitmaps

  for (int g = tid; g < G; g += nthr) cnt[g] = g < E ? 0 : T;
  for (int i = tid; i < 2 * E; i += nthr) bits[i] = 0u;
  if (r.general) {           // the generalised router ran before: its picks are in r.ids
    for (int i = tid; i < rows; i += nthr) s_ids[i] = r.ids[i];
  } else if constexpr (EPL <= 4) {  // E <= 256: row-level routing, one token per 16-lane row
    const int t = tid >> 4;
    if (t < T) route_token_row<EPL * 4>(r.logits, E, k, r.score, t, r.ids, r.w, r.ids_user, r.w_user, s_ids);
  } else {
    for (int t = tid >> 6; t < T; t += nthr >> 6)
      route_token<EPL>(r.logits, E, k, r.score, r.ids, r.w, r.ids_user, r.w_user, t, s_ids, nullptr);
  }
  __syncthreads();
  for (int i = tid; i < rows; i += nthr) {
    const int e = s_ids[i], t = i / k;
    atomicAdd(&cnt[e], 1);
    atomicOr(&bits[2 * e + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  if (tid < 64) {
    for (int g = tid; g < G; g += 64) {
      off[g] = cnt[g];
      tl[g] = (cnt[g] + M - 1) / M;
    }
    wave_dual_scan(off, tl, G);   // same wave wrote the inputs: no barrier needed
  }
  __syncthreads();
  for (int i = tid; i < rows; i += nthr) {
    const int e = s_ids[i], t = i / k;
    const uint32_t lo = bits[2 * e], hi = bits[2 * e + 1];
    const int rank = t < 32 ? __popc(lo & ((1u << t) - 1u)) : __popc(lo) + __popc(hi & ((1u << (t - 32)) - 1u));
    const int pos = off[e] + rank;
    a.perm[pos] = i;
    a.inv[i] = pos;
    a.tok[pos] = t;
    a.hmin[pos] = H_EXP_INIT;
    if (a.perm_user) a.perm_user[pos] = i;
  }
  for (int q = tid; q < T * (G - E); q += nthr) {
    a.tok[rows + q] = q % T;
    a.hmin[rows + q] = H_EXP_INIT;
  }
  for (int g = tid; g <= G; g += nthr) {
    a.offsets[g] = off[g];
    if (g < G) a.counts[g] = cnt[g];
    if (g <= E && a.offsets_user) a.offsets_user[g] = off[g];
    if (g < E && a.counts_user) a.counts_user[g] = cnt[g];
  }
  for (int g = tid; g < G; g += nthr) {
    const int n = (cnt[g] + M - 1) / M;
    for (int q = 0; q < n; ++q) {
      a.tile_group[tl[g] + q] = g;
      a.tile_row0[tl[g] + q] = off[g] + q * M;
    }
  }
  if (tid == 0) a.tile_count[0] = tl[G];
}

// ------------------------------------------------------------------------------
// Large batches: three kernels after routing.
//  count:   one workgroup per block of PLAN_BLOCK tokens sets per-expert token bitmaps in
//           LDS, stores each (t, j)'s rank among the block's rows of its expert and the
//           block's per-expert counts;
//  scan:    one workgroup turns block counts into per-(block, expert) row bases, the
//           expert counts, offsets and the GEMM tile list;
//  scatter: base + local rank -> perm / inv / row->token map.
constexpr int PLAN_BLOCK = 256;

__global__ __launch_bounds__(PLAN_BLOCK) void plan_count_kernel(PlanArgs a, int32_t* local_rank,
                                                                int32_t* block_counts) {
  extern __shared__ uint32_t bmp[];          // [E][PLAN_BLOCK / 32]
  constexpr int WORDS = PLAN_BLOCK / 32;
  const int E = a.E, k = a.k, b = blockIdx.x, tid = threadIdx.x;
  const int t = b * PLAN_BLOCK + tid;
  for (int i = tid; i < E * WORDS; i += PLAN_BLOCK) bmp[i] = 0u;
  __syncthreads();
  if (t < a.T)
    for (int j = 0; j < k; ++j) atomicOr(&bmp[a.ids[(size_t)t * k + j] * WORDS + (tid >> 5)], 1u << (tid & 31));
  __syncthreads();
  if (t < a.T)
    for (int j = 0; j < k; ++j) {
      const uint32_t* be = bmp + a.ids[(size_t)t * k + j] * WORDS;
      int rank = __popc(be[tid >> 5] & ((1u << (tid & 31)) - 1u));
      for (int q = 0; q < (tid >> 5); ++q) rank += __popc(be[q]);
      local_rank[(size_t)t * k + j] = rank;
    }
  for (int e = tid; e < E; e += PLAN_BLOCK) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < WORDS; ++q) c += __popc(bmp[e * WORDS + q]);
    block_counts[(size_t)b * E + e] = c;
  }
}

__global__ __launch_bounds__(1024) void plan_scan_kernel(PlanArgs a, int32_t* block_counts, int nblocks) {
  extern __shared__ int sh[];
  const int G = a.G, E = a.E, T = a.T, M = a.tile_rows, tid = threadIdx.x;
  int* cnt = sh;               // [G]
  int* off = cnt + G;          // [G+1]
  int* tl = off + G + 1;       // [G+1]
  // per expert: running base over blocks (block_counts -> exclusive prefix in place)
  for (int e = tid; e < G; e += blockDim.x) {
    if (e < E) {
      int run = 0;
      for (int b = 0; b < nblocks; ++b) {
        const int c = block_counts[(size_t)b * E + e];
        block_counts[(size_t)b * E + e] = run;
        run += c;
      }
      cnt[e] = run;
    } else {
      cnt[e] = T;
    }
    off[e] = cnt[e];
    tl[e] = (cnt[e] + M - 1) / M;
  }
  __syncthreads();
  if (tid < 64) wave_dual_scan(off, tl, G);
  __syncthreads();
  for (int g = tid; g <= G; g += blockDim.x) {
    a.offsets[g] = off[g];
    if (g < G) a.counts[g] = cnt[g];
    if (g <= E && a.offsets_user) a.offsets_user[g] = off[g];
    if (g < E && a.counts_user) a.counts_user[g] = cnt[g];
  }
  for (int g = tid; g < G; g += blockDim.x) {
    const int n = (cnt[g] + M - 1) / M;
    for (int q = 0; q < n; ++q) {
      a.tile_group[tl[g] + q] = g;
      a.tile_row0[tl[g] + q] = off[g] + q * M;
    }
  }
  if (tid == 0) a.tile_count[0] = tl[G];
}

__global__ __launch_bounds__(256) void plan_scatter_kernel(PlanArgs a, const int32_t* local_rank,
                                                           const int32_t* block_base) {
  const int rows = a.T * a.k;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < rows) {
    const int t = i / a.k, e = a.ids[i];
    const int pos = a.offsets[e] + block_base[(size_t)(t / PLAN_BLOCK) * a.E + e] + local_rank[i];
    a.perm[pos] = i;
    a.inv[i] = pos;
    a.tok[pos] = t;
    a.hmin[pos] = H_EXP_INIT;
    if (a.perm_user) a.perm_user[pos] = i;
  } else if (i < rows + a.T * (a.G - a.E)) {
    a.tok[i] = (i - rows) % a.T;    // shared-expert rows read token (row - rows) % T
    a.hmin[i] = H_EXP_INIT;
  }
}

size_t plan_scratch_ints(int T, int k, int E) {
  const size_t nb = (size_t)(T + PLAN_BLOCK - 1) / PLAN_BLOCK;
  return (size_t)T * k + nb * E;       // local ranks + block counts
}

static size_t plan_small_lds_bytes(int rows, int E, int G) {
  return sizeof(int) * ((size_t)rows + G + 2 * ((size_t)G + 1) + 2 * (size_t)E);
}

bool plan_small_ok(int T, int k) { return T <= 64 && T * k <= 4096; }

template <int EPL>
static hipError_t launch_route_plan_t(const RouteArgs& r, const PlanArgs& p, int32_t* scratch, hipStream_t s) {
  if (r.general) hipLaunchKernelGGL(route_general_kernel<EPL>, dim3((r.T + 3) / 4), dim3(256), 0, s, r);
  if (plan_small_ok(p.T, p.k)) {
    hipLaunchKernelGGL(plan_small_kernel<EPL>, dim3(1), dim3(1024), plan_small_lds_bytes(p.T * p.k, p.E, p.G), s,
                       r, p);
    return hipGetLastError();
  }
  if (r.general) {
  } else if constexpr (EPL <= 4) {
    hipLaunchKernelGGL(route_row_kernel<EPL * 4>, dim3((r.T + 15) / 16), dim3(256), 0, s, r);
  } else {
    hipLaunchKernelGGL(route_kernel<EPL>, dim3((r.T + 3) / 4), dim3(256), 0, s, r);
  }
  const int nb = (p.T + PLAN_BLOCK - 1) / PLAN_BLOCK;
  int32_t* local_rank = scratch;
  int32_t* block_counts = scratch + (size_t)p.T * p.k;
  const size_t count_lds = sizeof(uint32_t) * (size_t)p.E * (PLAN_BLOCK / 32);
  hipLaunchKernelGGL(plan_count_kernel, dim3(nb), dim3(PLAN_BLOCK), count_lds, s, p, local_rank, block_counts);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), sizeof(int) * (3 * (size_t)p.G + 2), s, p, block_counts,
                     nb);
  const int n = p.T * p.k + p.T * (p.G - p.E);
  hipLaunchKernelGGL(plan_scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, local_rank, block_counts);
  return hipGetLastError();
}

hipError_t launch_route_plan(const RouteArgs& r, const PlanArgs& p, int32_t* scratch, hipStream_t s) {
  const int epl = (r.E + WAVE - 1) / WAVE;
  if (epl <= 1) return launch_route_plan_t<1>(r, p, scratch, s);
  if (epl <= 2) return launch_route_plan_t<2>(r, p, scratch, s);
  if (epl <= 4) return launch_route_plan_t<4>(r, p, scratch, s);
  if (epl <= 8) return launch_route_plan_t<8>(r, p, scratch, s);
  return launch_route_plan_t<16>(r, p, scratch, s);
}

}  // namespace nvmoe

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
#include "route_dev.hpp"
#include "rowq_dev.hpp"

namespace nvmoe {

__device__ __forceinline__ void side_rows(const RouteArgs& a, int j);

// 256 threads = 16 rows = 16 tokens per workgroup; with a side job, the workgroups past the
// routing ones convert the activation rows (side_rows).
template <int EPR>
__global__ __launch_bounds__(256) void route_row_kernel(RouteArgs a) {
  const int nb = (a.T + 15) / 16;
  if ((int)blockIdx.x >= nb) {
    side_rows(a, blockIdx.x - nb);
    return;
  }
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= a.T) return;   // whole rows leave together
  route_token_row<EPR>(a.logits, a.E, a.k, a.score, t, a.ids, a.w, a.ids_user, a.w_user, nullptr);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int nb = (a.T + 3) / 4;
  if ((int)blockIdx.x >= nb) {
    side_rows(a, blockIdx.x - nb);
    return;
  }
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
  // logits and biases at clamped indices, not guarded ones, so that all loads issue together
  // (values past E are never used)
  float lv[EPL], bv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    lv[i] = lg[min(lane + WAVE * i, E - 1)];
    bv[i] = 0.0f;
  }
  if (r.bias)
#pragma unroll
    for (int i = 0; i < EPL; ++i) bv[i] = r.bias[min(lane + WAVE * i, E - 1)];
  float lmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + WAVE * i < E) lmax = fmaxf(lmax, lv[i]);
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
      if (r.bias) kf = kf + bv[i];
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
  // k picks over the 64-bit keys (key, ~e), empty slots 0: each lane's keys sorted
  // descending in registers, so its best untaken one is always the first; a pick is the wave
  // maximum of the lanes' first keys, word by word (the largest key, then among its holders
  // the largest ~e, i.e. the lowest expert id); the winning lane shifts its keys up by one.
  // Pick j is recorded by lane j; its FP64 score is fetched from the expert's lane afterwards.
  uint64_t kk[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) kk[i] = key[i] != 0u ? pick_key(key[i], lane + WAVE * i) : 0ull;
  sort_desc<EPL>(kk);
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = (uint32_t)(kk[0] >> 32), lo = (uint32_t)kk[0];
    const uint32_t mh = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
    uint32_t m = kk[0] == (((uint64_t)mh << 32) | ml) ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(m));   // a bit mask, not a select (see route_token_row)
    const uint64_t m64 = ((uint64_t)m << 32) | m;
#pragma unroll
    for (int i = 0; i + 1 < EPL; ++i) kk[i] = (kk[i + 1] & m64) | (kk[i] & ~m64);
    kk[EPL - 1] &= ~m64;
    my_id = lane == j ? (int)~ml : my_id;
  }
  double my_s = 0.0;
  {
    const int owner = my_id & (WAVE - 1), slot = my_id / WAVE;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const double v = __shfl(sc[i], owner);
      my_s = i == slot ? v : my_s;
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

// The side job of a routing launch: workgroup j past the routing workgroups converts rows
// j * (waves per workgroup) + wave of side_x (MXFP8 or NVFP4 codes and scales, or fp16 rows
// and their factors), one wave per row.
__device__ __forceinline__ void side_rows(const RouteArgs& a, int j) {
  const int wpb = blockDim.x >> 6;
  const int t = j * wpb + (int)(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int K = a.side_K, lane = (int)(threadIdx.x & (WAVE - 1));
  const uint16_t* row = a.side_x + (size_t)t * K;
  if (a.side == SIDE_MXFP8)
    mxfp8_row_wave(row, K, a.side_q + (size_t)t * K, a.side_s + (size_t)t * (K / 32), lane);
  else if (a.side == SIDE_FP8)
    fp8_row_wave(row, K, a.side_q ? a.side_q + (size_t)t * K : nullptr, a.side_f + t, a.side_h + (size_t)t * K, lane);
  else if (a.side == SIDE_NVFP4)   // with side_h also the rows' fp16 decode (prefill batches)
    nvfp4_row_wave(row, K, a.side_q + (size_t)t * (K / 2), a.side_s + (size_t)t * (K / 16), a.side_f + t,
                   a.side_h ? a.side_h + (size_t)t * K : nullptr);
  else
    f16_row_wave(row, K, a.side_h + (size_t)t * K, a.side_f + t, lane);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_general_kernel(RouteArgs a) {
  const int nb = (a.T + 3) / 4;
  if ((int)blockIdx.x >= nb) {   // side-job workgroups (grid past the routing ones only with a side job)
    side_rows(a, blockIdx.x - nb);
    return;
  }
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;   // whole waves leave together
  route_token_general<EPL>(a, t, nullptr);
}

// Tile counts per group before the scans: list 1 takes groups with more than cold rows in
// ceil(c / M)-row tiles, list 2 groups with 1 .. cold rows in DECODE_TILE_ROWS-row tiles
// (cold = 0: every group in list 1).
__device__ __forceinline__ void tile_counts(int c, int M, int cold, int* tl, int* ct) {
  *tl = c > cold ? (c + M - 1) / M : 0;
  *ct = c > 0 && c <= cold ? (c + DECODE_TILE_ROWS - 1) / DECODE_TILE_ROWS : 0;
}

// The tile lists from the scanned offsets (off), list-1 tile starts (tl) and list-2 slots
// (ct): list 1 in slots 0 .. tl[G]-1, list 2 right after it; tile_count = {tl[G], ct[G]}.
__device__ __forceinline__ void write_tiles(const PlanArgs& a, const int* cnt, const int* off, const int* tl,
                                            const int* ct, int G, int tid, int nthr) {
  const int M = a.tile_rows;
  for (int g = tid; g < G; g += nthr) {
    if (cnt[g] > a.cold_rows) {
      const int n = (cnt[g] + M - 1) / M;
      for (int q = 0; q < n; ++q) {
        a.tile_group[tl[g] + q] = g;
        a.tile_row0[tl[g] + q] = off[g] + q * M;
      }
    } else {
      const int n = (cnt[g] + DECODE_TILE_ROWS - 1) / DECODE_TILE_ROWS;
      for (int q = 0; q < n; ++q) {
        a.tile_group[tl[G] + ct[g] + q] = g;
        a.tile_row0[tl[G] + ct[g] + q] = off[g] + q * DECODE_TILE_ROWS;
      }
    }
  }
  if (tid == 0) {
    a.tile_count[0] = tl[G];
    a.tile_count[1] = ct[G];
  }
}

// One wave: from the group counts cnt[0..G), the exclusive prefix sums of the counts (off),
// of the list-1 tile counts (tl) and of the list-2 tile counts (ct), each with its total at
// [G]. Lane l holds the run of ceil(G/64) <= OFFSETS_SEG consecutive groups from l ceil(G/64)
// in registers: the counts are read together (indices clamped, not guarded), the three scans
// run side by side, and every array is written once.
constexpr int OFFSETS_SEG = 8;
__device__ __forceinline__ void offsets_wave(const int* cnt, int* off, int* tl, int* ct, int G, int M, int cold) {
  const int lane = threadIdx.x & 63;
  const int seg = (G + 63) / 64, i0 = lane * seg;
  int c[OFFSETS_SEG], t1[OFFSETS_SEG], t2[OFFSETS_SEG];
#pragma unroll
  for (int u = 0; u < OFFSETS_SEG; ++u) c[u] = cnt[min(i0 + u, G - 1)];
  int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
  for (int u = 0; u < OFFSETS_SEG; ++u) {
    t1[u] = 0;
    t2[u] = 0;
    if (u < seg) {                              // the run length is the same in every lane
      if (i0 + u >= G) c[u] = 0;               // past the end: contributes nothing
      tile_counts(c[u], M, cold, &t1[u], &t2[u]);
      s0 += c[u];
      s1 += t1[u];
      s2 += t2[u];
    }
  }
  const int e0 = wave_inclusive_scan(s0), e1 = wave_inclusive_scan(s1), e2 = wave_inclusive_scan(s2);
  int r0 = e0 - s0, r1 = e1 - s1, r2 = e2 - s2;
#pragma unroll
  for (int u = 0; u < OFFSETS_SEG; ++u)
    if (u < seg && i0 + u < G) {
      off[i0 + u] = r0;
      tl[i0 + u] = r1;
      ct[i0 + u] = r2;
      r0 += c[u];
      r1 += t1[u];
      r2 += t2[u];
    }
  if (lane == 63) {
    off[G] = e0;
    tl[G] = e1;
    ct[G] = e2;
  }
}

// Small batches (T <= 64, T*k <= 4096): routing, counts, offsets, permutation and tile
// list in one 1024-thread workgroup, everything in LDS. 64 DPP rows route up to 64 tokens
// at once (E <= 256; wider expert sets use one wave per token); one wave runs the offset and
// tile-count scans; global memory is read once (logits) and written at the end. A token's experts
// are distinct, so an expert's rank of token t is the number of earlier tokens in that
// expert's 64-bit token bitmap.
template <int EPL>
__global__ __launch_bounds__(1024) void plan_small_kernel(RouteArgs r, PlanArgs a) {
  if (blockIdx.x > 0) {   // side-job workgroups (only with a side job)
    side_rows(r, blockIdx.x - 1);
    return;
  }
  extern __shared__ int lds[];
  const int G = a.G, E = a.E, T = a.T, k = a.k, rows = T * k, M = a.tile_rows;
  const int tid = threadIdx.x, nthr = blockDim.x;
  int* s_ids = lds;                          // [rows]
  int* cnt = s_ids + rows;                   // [G]
  int* off = cnt + G;                        // [G+1] row offsets
  int* tl = off + G + 1;                     // [G+1] list-1 tile starts
  int* ct = tl + G + 1;                      // [G+1] list-2 slots
  uint32_t* bits = (uint32_t*)(ct + G + 1);  // [E][2] token bitmaps

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
    if (G <= 64 * OFFSETS_SEG) {
      offsets_wave(cnt, off, tl, ct, G, M, a.cold_rows);
    } else {
      for (int g = tid; g < G; g += 64) {
        off[g] = cnt[g];
        tile_counts(cnt[g], M, a.cold_rows, &tl[g], &ct[g]);
      }
      wave_dual_scan(off, tl, G);   // same wave wrote the inputs: no barrier needed
      wave_scan(ct, G);
    }
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
  write_tiles(a, cnt, off, tl, ct, G, tid, nthr);
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
  // the picks' ids are read 8 at a time before their ranks are stored (a store between two
  // reads would make each read wait for the one before it)
  if (t < a.T)
    for (int j0 = 0; j0 < k; j0 += 8) {
      int id[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) id[u] = a.ids[(size_t)t * k + min(j0 + u, k - 1)];   // in bounds: no branch
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) {
          const uint32_t* be = bmp + id[u] * WORDS;
          int rank = __popc(be[tid >> 5] & ((1u << (tid & 31)) - 1u));
          for (int q = 0; q < (tid >> 5); ++q) rank += __popc(be[q]);
          local_rank[(size_t)t * k + j0 + u] = rank;
        }
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
  int* ct = tl + G + 1;        // [G+1]
  // per expert: running base over blocks (block_counts -> exclusive prefix in place). The
  // counts of 16 blocks are loaded together before their prefixes are stored: a store to the
  // array between two loads would make each load wait for the one before it.
  for (int e = tid; e < G; e += blockDim.x) {
    if (e < E) {
      int run = 0;
      for (int b0 = 0; b0 < nblocks; b0 += 16) {
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] = block_counts[(size_t)min(b0 + j, nblocks - 1) * E + e];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (b0 + j < nblocks) {
            block_counts[(size_t)(b0 + j) * E + e] = run;
            run += c[j];
          }
      }
      cnt[e] = run;
    } else {
      cnt[e] = T;
    }
    off[e] = cnt[e];
    tile_counts(cnt[e], M, a.cold_rows, &tl[e], &ct[e]);
  }
  __syncthreads();
  if (tid < 64) {
    wave_dual_scan(off, tl, G);
    wave_scan(ct, G);
  }
  __syncthreads();
  for (int g = tid; g <= G; g += blockDim.x) {
    a.offsets[g] = off[g];
    if (g < G) a.counts[g] = cnt[g];
    if (g <= E && a.offsets_user) a.offsets_user[g] = off[g];
    if (g < E && a.counts_user) a.counts_user[g] = cnt[g];
  }
  write_tiles(a, cnt, off, tl, ct, G, tid, blockDim.x);
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
  return sizeof(int) * ((size_t)rows + G + 3 * ((size_t)G + 1) + 2 * (size_t)E);
}

bool plan_small_ok(int T, int k) { return T <= 64 && T * k <= 4096; }

template <int EPL>
static hipError_t launch_route_plan_t(const RouteArgs& r, const PlanArgs& p, int32_t* scratch, hipStream_t s) {
  // the side job rides on the first launch: the general router's, the one-workgroup plan's
  // or the per-token router's
  bool side = r.side != SIDE_NONE;
  if (r.general) {
    hipLaunchKernelGGL(route_general_kernel<EPL>, dim3((r.T + 3) / 4 * (side ? 2 : 1)), dim3(256), 0, s, r);
    side = false;
  }
  if (plan_small_ok(p.T, p.k)) {
    hipLaunchKernelGGL(plan_small_kernel<EPL>, dim3(1 + (side ? (r.T + 15) / 16 : 0)), dim3(1024),
                       plan_small_lds_bytes(p.T * p.k, p.E, p.G), s, r, p);
    return hipGetLastError();
  }
  // the side job's workgroups (4 rows each) follow the routing ones in the same launch
  const int side_wgs = side ? (r.T + 3) / 4 : 0;
  if (r.general) {
  } else if constexpr (EPL <= 4) {
    hipLaunchKernelGGL(route_row_kernel<EPL * 4>, dim3((r.T + 15) / 16 + side_wgs), dim3(256), 0, s, r);
  } else {
    hipLaunchKernelGGL(route_kernel<EPL>, dim3((r.T + 3) / 4 + side_wgs), dim3(256), 0, s, r);
  }
  const int nb = (p.T + PLAN_BLOCK - 1) / PLAN_BLOCK;
  int32_t* local_rank = scratch;
  int32_t* block_counts = scratch + (size_t)p.T * p.k;
  const size_t count_lds = sizeof(uint32_t) * (size_t)p.E * (PLAN_BLOCK / 32);
  hipLaunchKernelGGL(plan_count_kernel, dim3(nb), dim3(PLAN_BLOCK), count_lds, s, p, local_rank, block_counts);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), sizeof(int) * (4 * (size_t)p.G + 3), s, p, block_counts,
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

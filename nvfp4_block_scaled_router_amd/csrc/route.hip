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

// Wave 0..: one wave routes one token. EPL = experts per lane (E <= 64*EPL).
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lg, int E, int k, int score,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int32_t* __restrict__ ids_user, float* __restrict__ w_user,
                                            int t) {
  const int lane = threadIdx.x & (WAVE - 1);
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + WAVE * i;
    v[i] = e < E ? lg[(size_t)t * E + e] : 0.0f;
  }
  uint32_t taken = 0;
  float my_v = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + WAVE * i;
      // ascending e within a lane: strict '>' keeps the lower id on ties
      if (e < E && !((taken >> i) & 1u) && (bi < 0 || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = WAVE / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, WAVE);
      const int oi = __shfl_xor(bi, off, WAVE);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == (bi & (WAVE - 1))) taken |= 1u << (bi / WAVE);
    if (lane == j) {
      my_v = bv;
      my_id = bi;
    }
  }
  // weights over the k picks, in fp32; lane j holds pick j
  const float lmax = __shfl(my_v, 0, WAVE);
  float s = 0.0f;
  if (lane < k) s = score == 0 ? __expf(my_v - lmax) : 1.0f / (1.0f + __expf(-my_v));
  float sum = s;
#pragma unroll
  for (int off = WAVE / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, WAVE);
  if (lane < k) {
    const float wj = s / sum;
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = wj;
    if (ids_user) ids_user[(size_t)t * k + lane] = my_id;
    if (w_user) w_user[(size_t)t * k + lane] = wj;
  }
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  route_token<EPL>(a.logits, a.E, a.k, a.score, a.ids, a.w, a.ids_user, a.w_user, t);
}

// Block-wide exclusive scan of n <= 2048 ints held in LDS (in place); returns the total.
__device__ int block_exclusive_scan(int* buf, int n, int* tmp /* [1024/64 + 1] */) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  int total = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + tid;
    int x = i < n ? buf[i] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) tmp[wv] = incl;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int q = 0; q < nw; ++q) {
        const int c = tmp[q];
        tmp[q] = run;
        run += c;
      }
      tmp[nw] = run;
    }
    __syncthreads();
    if (i < n) buf[i] = total + tmp[wv] + incl - x;
    total += tmp[nw];
    __syncthreads();
  }
  return total;
}

// One workgroup of 1024 threads. With ROUTE it first routes all T tokens itself
// (one wave per token); otherwise route_kernel ran before and ids are in global memory.
template <int EPL, bool ROUTE>
__global__ __launch_bounds__(1024) void plan_kernel(RouteArgs r, PlanArgs a) {
  extern __shared__ int lds[];
  const int G = a.G;                      // routed + shared groups
  int* cnt = lds;                         // [G]
  int* off = cnt + G + 1;                 // [G + 1]
  int* run = off + G + 1;                 // [E]   rows already placed per expert
  int* tiles = run + a.E;                 // [G + 1]
  int* tmp = tiles + G + 1;               // [17]
  uint32_t* bits = (uint32_t*)(tmp + 17); // [E][PLAN_CHUNK / 32]
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int T = a.T, k = a.k, E = a.E;
  const int rows = T * k;

  if (ROUTE) {
    for (int t = tid >> 6; t < T; t += nthr >> 6)
      route_token<EPL>(r.logits, E, k, r.score, r.ids, r.w, r.ids_user, r.w_user, t);
  }
  for (int g = tid; g < G; g += nthr) cnt[g] = g < E ? 0 : T;
  for (int e = tid; e < E; e += nthr) run[e] = 0;
  __syncthreads();
  for (int i = tid; i < rows; i += nthr) atomicAdd(&cnt[a.ids[i]], 1);
  __syncthreads();
  for (int g = tid; g < G; g += nthr) off[g] = cnt[g];
  __syncthreads();
  block_exclusive_scan(off, G, tmp);
  if (tid == 0) off[G] = rows + T * (G - E);
  __syncthreads();
  for (int g = tid; g <= G; g += nthr) {
    a.offsets[g] = off[g];
    if (g < G) a.counts[g] = cnt[g];
    if (g <= E && a.offsets_user) a.offsets_user[g] = off[g];
    if (g < E && a.counts_user) a.counts_user[g] = cnt[g];
  }

  // stable expert-major permutation, PLAN_CHUNK tokens at a time
  constexpr int WORDS = PLAN_CHUNK / 32;
  for (int c0 = 0; c0 < T; c0 += PLAN_CHUNK) {
    for (int i = tid; i < E * WORDS; i += nthr) bits[i] = 0u;
    __syncthreads();
    const int i = tid, t = c0 + tid;
    const bool live = i < PLAN_CHUNK && t < T;
    if (live)
      for (int j = 0; j < k; ++j) atomicOr(&bits[a.ids[t * k + j] * WORDS + (i >> 5)], 1u << (i & 31));
    __syncthreads();
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int e = a.ids[t * k + j];
        const uint32_t* be = bits + e * WORDS;
        int rank = __popc(be[i >> 5] & ((1u << (i & 31)) - 1u));
        for (int q = 0; q < (i >> 5); ++q) rank += __popc(be[q]);
        const int pos = off[e] + run[e] + rank;
        a.perm[pos] = t * k + j;
        a.inv[t * k + j] = pos;
        a.tok[pos] = t;
        if (a.perm_user) a.perm_user[pos] = t * k + j;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += nthr) {
      int c = 0;
      for (int q = 0; q < WORDS; ++q) c += __popc(bits[e * WORDS + q]);
      run[e] += c;
    }
    __syncthreads();
  }
  // shared-expert rows: row rows + s*T + t reads token t
  for (int q = tid; q < T * (G - E); q += nthr) a.tok[rows + q] = q % T;

  // GEMM tile list: ceil(count / M) tiles of M rows per group, in group order
  const int M = a.tile_rows;
  for (int g = tid; g < G; g += nthr) tiles[g] = (cnt[g] + M - 1) / M;
  __syncthreads();
  const int ntiles = block_exclusive_scan(tiles, G, tmp);
  for (int g = tid; g < G; g += nthr) {
    const int n = (cnt[g] + M - 1) / M;
    for (int m = 0; m < n; ++m) {
      a.tile_group[tiles[g] + m] = g;
      a.tile_row0[tiles[g] + m] = off[g] + m * M;
    }
  }
  if (tid == 0) a.tile_count[0] = ntiles;
}

size_t plan_lds_bytes(int E, int G) {
  return sizeof(int) * ((size_t)(G + 1) * 3 + E + 17) + sizeof(uint32_t) * (size_t)E * (PLAN_CHUNK / 32);
}

template <int EPL>
static hipError_t launch_route_plan_t(const RouteArgs& r, const PlanArgs& p, bool fused, hipStream_t s) {
  const size_t lds = plan_lds_bytes(p.E, p.G);
  if (lds > 65536) {  // large expert counts need more than the default dynamic LDS limit
    hipError_t e = hipFuncSetAttribute((const void*)plan_kernel<EPL, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)plan_kernel<EPL, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    if (e != hipSuccess) return e;
  }
  if (!fused) {
    hipLaunchKernelGGL(route_kernel<EPL>, dim3((r.T + 3) / 4), dim3(256), 0, s, r);
    hipLaunchKernelGGL((plan_kernel<EPL, false>), dim3(1), dim3(1024), plan_lds_bytes(p.E, p.G), s, r, p);
  } else {
    hipLaunchKernelGGL((plan_kernel<EPL, true>), dim3(1), dim3(1024), plan_lds_bytes(p.E, p.G), s, r, p);
  }
  return hipGetLastError();
}

hipError_t launch_route_plan(const RouteArgs& r, const PlanArgs& p, bool fused, hipStream_t s) {
  const int epl = (r.E + WAVE - 1) / WAVE;
  if (epl <= 1) return launch_route_plan_t<1>(r, p, fused, s);
  if (epl <= 2) return launch_route_plan_t<2>(r, p, fused, s);
  if (epl <= 4) return launch_route_plan_t<4>(r, p, fused, s);
  if (epl <= 8) return launch_route_plan_t<8>(r, p, fused, s);
  return launch_route_plan_t<16>(r, p, fused, s);
}

}  // namespace nvmoe

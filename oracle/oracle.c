/*
 * CPU oracle for the NVFP4 block-scaled fused-MoE layer.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library. It shares no
 * code, header, table or helper with the HIP path; both sides only share the
 * seeded input generator in synth/.
 *
 * Plain, slow and written to be checked by eye: FP64 everywhere except the
 * NVFP4 quantizer, whose result is a discrete encoding defined by binary32
 * operations and is therefore evaluated in binary32. Nearest-value encoders
 * are brute-force searches over every code, not bit tricks.
 *
 * Sources (the three web pages this method is described on):
 *   [b12x]     "b12x" README (github local-inference-lab/b12x)
 *   [vllm.cpp] "vllm.cpp docs/STATUS.md"
 *   [megamoe]  "nvfp4-megamoe-kernel" compare page (pre-b1...master)
 *
 * Parity pins: every function below is pinned by a test in tests/test_oracle_*.py
 * against something other than itself (hand tables, torch's float8 decoder,
 * brute force, closed forms, textbook special cases). None is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ decode */

/* E2M1 (float4_e2m1fn) nibble: bit 3 sign, bits 2..0 magnitude code.
 * [megamoe] README "NVFP4 throughout": weights are E2M1 packed two per byte
 * (float4_e2m1fn_x2); archived CORRECTNESS_BACKLOG §7: FP4 max = 6.
 * The eight magnitudes of the format are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1(uint32_t nib) {
  double m = E2M1_MAG[nib & 7u];
  return (nib & 8u) ? -m : m;
}

/* E4M3fn (float8_e4m3fn) byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448.
 * [megamoe] README "NVFP4 throughout" (FP8 E4M3 block scales, one per
 * 16-element microblock); archived CORRECTNESS_BACKLOG §7: E4M3 max = 448. */
double orc_e4m3fn(uint32_t byte) {
  uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    v = ldexp((double)m, -9);                 /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* bfloat16 bit pattern -> value (the upper half of a binary32). */
double orc_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* One NVFP4 weight element W[n][k] of an [N][K] projection, in the operand
 * layout the pages use: packed [N][K/2] (element 2i in the low nibble of byte
 * i, 2i+1 in the high nibble), block scales [N][K/16] (E4M3, block = 16
 * consecutive k), one FP32 global scale for the projection.
 * [vllm.cpp] capability table, GGUF loading row: the (weight_packed [N,K/2],
 * weight_scale [N,K/16]) operand pair and a per-expert weight_scale_2;
 * [megamoe] WALKING_BACK_SOME_QUANTS, "First: the CUDA illegal-memory-access":
 * dequant = E2M1 value * weight_scale repeated over 16 columns * weight_scale_2;
 * archived CORRECTNESS_BACKLOG §7: the weight global scale is weight_scale_2.
 * The product of an E2M1 value, an E4M3 value and a binary32 is exact in FP64. */
static uint32_t orc_nibble(const uint8_t* packed, int K, int n, int k) {
  uint8_t byte = packed[(size_t)n * (K / 2) + k / 2];
  return (k & 1) ? (byte >> 4) : (byte & 15u);
}

double orc_weight(const uint8_t* packed, const uint8_t* scales, float gs, int K, int n, int k) {
  return orc_e2m1(orc_nibble(packed, K, n, k)) * orc_e4m3fn(scales[(size_t)n * (K / 16) + k / 16]) * (double)gs;
}

/* MXFP4 weight element (the second weight format): E2M1 code times an E8M0 block
 * scale 2^(byte - 127) shared by 32 consecutive k, no global scale; byte 0xFF is
 * NaN. ([vllm.cpp] capability table, MXFP4 (compressed-tensors mxfp4-pack-quantized)
 * row: E8M0 dequant 2^(byte-127), group 32, no global scale; [b12x] "DeepSeek V4
 * Flash 0731 MoE reproduction": MXFP4 E8M0/K32 expert weights.) Exact in FP64. */
double orc_e8m0(uint32_t byte) {
  if (byte == 0xFFu) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

double orc_weight_mx(const uint8_t* packed, const uint8_t* scales, int K, int n, int k) {
  return orc_e2m1(orc_nibble(packed, K, n, k)) * orc_e8m0(scales[(size_t)n * (K / 32) + k / 32]);
}

/* --------------------------------------------------------------- quantizer */

/* Nearest non-negative finite E4M3fn value to v >= 0, ties to the even code
 * (the even mantissa), values >= 448 saturate to 448 (code 0x7E).
 * Brute force over the 127 codes 0x00..0x7E. */
static double E4M3_VALUE[0x7F];               /* decoded codes 0x00..0x7E */

__attribute__((constructor)) static void orc_init_tables(void) {
  for (uint32_t c = 0; c <= 0x7E; ++c) E4M3_VALUE[c] = orc_e4m3fn(c);
}

uint8_t orc_e4m3_encode(float v) {
  if (!(v > 0.0f)) return 0;                  /* 0, -0 (and NaN, not produced) */
  if (v >= 448.0f) return 0x7E;
  uint32_t best = 0;
  double bestd = (double)v;                   /* distance to code 0 (value 0) */
  for (uint32_t c = 1; c <= 0x7E; ++c) {
    double d = fabs(E4M3_VALUE[c] - (double)v);
    if (d < bestd || (d == bestd && (c & 1u) == 0 && (best & 1u) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)best;
}

/* Nearest E2M1 magnitude code (0..7) to r >= 0, ties to the even code,
 * r > 6 saturates to 6 (code 7). Brute force over the 8 magnitudes. */
uint8_t orc_e2m1_encode(float r) {
  if (!(r > 0.0f)) return 0;
  if (r >= 6.0f) return 7;
  uint32_t best = 0;
  double bestd = (double)r;
  for (uint32_t c = 1; c < 8; ++c) {
    double d = fabs(E2M1_MAG[c] - (double)r);
    if (d < bestd || (d == bestd && (c & 1u) == 0 && (best & 1u) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)best;
}

/* NVFP4 quantizer for rows[i][0..K), K a multiple of 16. Rows are grouped
 * `rows_per_gs` at a time; each group shares one FP32 global scale (1 row per
 * group for activations, all rows of a projection for a weight tensor).
 *
 * Global scale: [megamoe] archived CORRECTNESS_BACKLOG §7, "Runtime Activation
 * Global Scale": gs = max|x| / (6.0 * 448.0), so that no block scale overflows
 * E4M3. Block scales per 16 consecutive elements and E2M1 codes are the NVFP4
 * format of README "NVFP4 throughout"; the order of binary32 operations below
 * is the reading recorded with the design (the pages do not spell it out):
 *   A   = max |x| over the group                       (exact)
 *   gs  = A / 2688                                     (binary32 division)
 *   a_b = max |x| over block b                         (exact)
 *   s_b = gs == 0 ? 0 : E4M3_nearest(a_b / (6 * gs))   (binary32 mul, then div)
 *   d_b = value(s_b) * gs                              (binary32 mul)
 *   q_k = sign(x_k) | (d_b == 0 ? 0 : E2M1_nearest(|x_k| / d_b))
 * Outputs: packed [rows][K/2] (even k in the low nibble), scales [rows][K/16],
 * gs [rows / rows_per_gs]. */
void orc_quantize(const float* x, int64_t rows, int K, int64_t rows_per_gs,
                  uint8_t* packed, uint8_t* scales, float* gs_out) {
  int64_t groups = rows / rows_per_gs;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t g = 0; g < groups; ++g) {
    const float* xg = x + (size_t)g * rows_per_gs * K;
    float A = 0.0f;
    for (int64_t i = 0; i < rows_per_gs * K; ++i)
      if (fabsf(xg[i]) > A) A = fabsf(xg[i]);
    gs_out[g] = A / 2688.0f;
  }
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < rows; ++row) {
    float gs = gs_out[row / rows_per_gs];
    const float* xr = x + (size_t)row * K;
    for (int b = 0; b < K / 16; ++b) {
      float ab = 0.0f;
      for (int j = 0; j < 16; ++j)
        if (fabsf(xr[b * 16 + j]) > ab) ab = fabsf(xr[b * 16 + j]);
      uint8_t s = 0;
      if (gs != 0.0f) {
        float six_gs = 6.0f * gs;
        s = orc_e4m3_encode(ab / six_gs);
      }
      scales[(size_t)row * (K / 16) + b] = s;
      float d = (float)orc_e4m3fn(s) * gs;
      for (int j = 0; j < 16; ++j) {
        int k = b * 16 + j;
        float v = xr[k];
        uint32_t code = signbit(v) ? 8u : 0u;
        if (d != 0.0f) code |= orc_e2m1_encode(fabsf(v) / d);
        uint8_t* p = &packed[(size_t)row * (K / 2) + k / 2];
        if ((k & 1) == 0)
          *p = (uint8_t)((*p & 0xF0u) | code);
        else
          *p = (uint8_t)((*p & 0x0Fu) | (code << 4));
      }
    }
  }
}

/* ------------------------------------------------------ MXFP8 activations */

/* MXFP8 element: E4M3fn code times the block's E8M0 scale. */
double orc_mxfp8(uint32_t code, uint32_t scale) { return orc_e4m3fn(code) * orc_e8m0(scale); }

/* Decoded MXFP8 rows: x[r][k] = orc_mxfp8(codes[r][k], scales[r][k / 32]). */
void orc_mxfp8_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K, double* x) {
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k)
      x[(size_t)r * K + k] = orc_mxfp8(codes[(size_t)r * K + k], scales[(size_t)r * (K / 32) + k / 32]);
}

/* MXFP8 row quantiser: E4M3fn elements with one E8M0 scale per 32 consecutive k
 * (the MXFP8 activations of the W4A8 profile: [b12x] "DeepSeek V4 Flash 0731 MoE
 * reproduction"; E8M0 = 2^(byte-127) over groups of 32: [vllm.cpp] capability table,
 * MXFP4 row). Per block b of row r, in binary32:
 *   A_b    = max |x| over the block                          (exact)
 *   X_b    = floor(log2 A_b) - 8, clamped to [-127, 127]; A_b = 0 gives X_b = -127
 *            (8 = the exponent of E4M3's largest normal, 448 = 1.75 * 2^8)
 *   scale  = X_b + 127                                      (the E8M0 byte, value 2^X_b)
 *   code_k = sign(x_k) << 7 | E4M3_nearest(|x_k| * 2^-X_b)   (exact scaling; ratios above
 *            448 saturate to 448, ties to the even code)
 * The shared-exponent rule is the OCP microscaling one. Outputs codes [rows][K],
 * scales [rows][K/32]. */
void orc_mxfp8_quantize(const float* x, int64_t rows, int K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + (size_t)r * K;
    for (int b = 0; b < K / 32; ++b) {
      float A = 0.0f;
      for (int j = 0; j < 32; ++j)
        if (fabsf(xr[b * 32 + j]) > A) A = fabsf(xr[b * 32 + j]);
      int X = -127;
      if (A > 0.0f) {
        int E;
        frexpf(A, &E);                          /* A = f 2^E, f in [0.5, 1): floor(log2 A) = E - 1 */
        X = E - 1 - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      scales[(size_t)r * (K / 32) + b] = (uint8_t)(X + 127);
      for (int j = 0; j < 32; ++j) {
        const float v = xr[b * 32 + j];
        const uint32_t sign = signbit(v) ? 0x80u : 0u;
        codes[(size_t)r * K + b * 32 + j] = (uint8_t)(sign | orc_e4m3_encode(ldexpf(fabsf(v), -X)));
      }
    }
  }
}

/* ------------------------------------------- FP8 rows with a per-row scale */

/* FP8 row quantiser of the NVFP4-weight W4A8 path ([b12x] "What's in here": the unified
 * dynamic path's w4a8_nvfp4 variant, NVFP4 weights with FP8 activations; the pages name it
 * without its activation rule). Reading: E4M3fn codes with one FP32 scale per row taken
 * from the row's largest magnitude, which maps onto E4M3's largest value 448 -- the FP8
 * rule the same project applies to its KV rows ([megamoe] archived CORRECTNESS_BACKLOG,
 * section 7 "NVFP4 Quantization": FP8 KV quantisation with a per-row float32 scale from the
 * row amax), here applied to the activation rows. Per row r, in binary32:
 *   A      = max |x| over the row                           (exact)
 *   s      = A / 448                                        (binary32 division)
 *   code_k = sign(x_k) << 7 | (s == 0 ? 0 : E4M3_nearest(|x_k| / s))
 *            (binary32 division; ratios above 448 saturate to 448, ties to the even code)
 * Outputs codes [rows][K], scale [rows]. */
void orc_fp8_rows_quantize(const float* x, int64_t rows, int K, uint8_t* codes, float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + (size_t)r * K;
    float A = 0.0f;
    for (int k = 0; k < K; ++k)
      if (fabsf(xr[k]) > A) A = fabsf(xr[k]);
    const float s = A / 448.0f;
    scale[r] = s;
    for (int k = 0; k < K; ++k) {
      const uint32_t sign = signbit(xr[k]) ? 0x80u : 0u;
      codes[(size_t)r * K + k] = (uint8_t)(sign | (s == 0.0f ? 0u : orc_e4m3_encode(fabsf(xr[k]) / s)));
    }
  }
}

/* Decoded FP8 rows: x[r][k] = E4M3fn(codes[r][k]) * scale[r] (exact in FP64). */
void orc_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows, int K, double* x) {
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) x[(size_t)r * K + k] = orc_e4m3fn(codes[(size_t)r * K + k]) * (double)scale[r];
}

/* ----------------------------------------------------------------- routing */

/* Top-k routing of T tokens over E experts.
 * Selection: experts ordered by FP32 logit, larger first, equal values broken
 * by the lower expert index ([vllm.cpp] "DeepSeek-V4-Flash decode ds4-gap -
 * Lever 3": argmax under the strict total order (value, lower index)); every
 * token gets k distinct experts ([b12x] "DeepSeek V4 Flash 0731 MoE
 * reproduction": no duplicate expert inside one token). ids[t][j] is the j-th
 * pick. Comparison is numeric, so -0 and +0 tie.
 * Weights, renormalised over the k picks ([b12x] "What's in here": routing
 * scores kept in FP32 internally; [vllm.cpp] Lever 3 "exact renorm"):
 *   score 0 (softmax): w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max), i over picks
 *   score 1 (sigmoid): w_j = sig(l_j) / sum_i sig(l_i),  sig(z) = 1/(1+exp(-z))
 * ([vllm.cpp] capability table: sigmoid noaux_tc routers without the group step). */
void orc_route(const float* logits, int T, int E, int k, int score, int32_t* ids, double* w) {
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    double sum = 0.0, v[1024];
    for (int j = 0; j < k; ++j) {
      double lj = (double)l[ids[(size_t)t * k + j]];
      if (score == 0)
        v[j] = exp(lj - (double)l[ids[(size_t)t * k]]);
      else
        v[j] = 1.0 / (1.0 + exp(-lj));
      sum += v[j];
    }
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = v[j] / sum;
  }
  free(taken);
}

/* Generalised router: the score functions and selection rules the pages name
 * beside the plain top-k of orc_route.
 *   score s_e in FP64:
 *     0 softmax over all E experts: exp(l_e - l_max) / sum_i exp(l_i - l_max)
 *     1 sigmoid: 1 / (1 + exp(-l_e))
 *     2 sqrt-softplus: sqrt(log(1 + exp(l_e))), evaluated as
 *       sqrt(max(l,0) + log1p(exp(-|l|))) (the same number, no overflow)
 *       ([vllm.cpp] DeepSeek-V4 bring-up log, W6 sqrtsoftplus + hash-routed
 *       MoE: the V4 router score, distinct from V2/V3's sigmoid/softmax;
 *       [megamoe] archived CORRECTNESS_BACKLOG §5, Dense Router);
 *   selection key in binary32: key_e = fp32(s_e), plus bias_e (a binary32 add)
 *     when a bias is given. The bias steers selection only; the weights come from
 *     the unbiased scores ([vllm.cpp] DeepSeek-V4 bring-up log, W6: the correction
 *     bias enters selection only, the weights are gathered unbiased);
 *   group step (n_group > 1): the E experts form n_group equal groups of
 *     consecutive ids; a group's score is the binary32 sum of its two largest keys
 *     (its one key if the group has one expert); the topk_group groups with the
 *     largest scores are kept (lower group id on ties) and only their experts can
 *     be picked. The pages name this step of the DeepSeek-V3 noaux_tc router
 *     without spelling it out ([vllm.cpp] capability table: Laguna's router is
 *     noaux_tc minus the group step); this is DeepSeek-V3's definition;
 *   picks: the k largest keys among the pickable experts, lower id on ties
 *     (the total order of orc_route, on keys instead of logits);
 *   weights: w_j = s_j / sum_i s_i over the picks (renorm) or w_j = s_j, times
 *     `scaling` ([vllm.cpp] capability table: noaux_tc sigmoid router with
 *     routed scaling). */
static double orc_score(int score, double l, double lmax, double denom) {
  if (score == 0) return exp(l - lmax) / denom;
  if (score == 1) return 1.0 / (1.0 + exp(-l));
  return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
}

void orc_route_general(const float* logits, int T, int E, int k, int score, const float* bias,
                       int n_group, int topk_group, int renorm, double scaling, int32_t* ids,
                       double* w) {
  double* s = (double*)malloc(sizeof(double) * (size_t)E);
  float* key = (float*)malloc(sizeof(float) * (size_t)E);
  char* pickable = (char*)malloc((size_t)E);
  char* taken = (char*)malloc((size_t)E);
  float* gscore = (float*)malloc(sizeof(float) * (size_t)n_group);
  char* gkeep = (char*)malloc((size_t)n_group);
  const int gsz = E / n_group;
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    double lmax = l[0], denom = 0.0;
    for (int e = 1; e < E; ++e) lmax = fmax(lmax, (double)l[e]);
    if (score == 0)
      for (int e = 0; e < E; ++e) denom += exp((double)l[e] - lmax);
    for (int e = 0; e < E; ++e) {
      s[e] = orc_score(score, (double)l[e], lmax, denom);
      key[e] = (float)s[e];
      if (bias) key[e] = key[e] + bias[e];
    }
    /* group step: each group's two largest keys (lower id first on ties) */
    for (int q = 0; q < n_group; ++q) {
      int a = -1, b = -1;
      for (int e = q * gsz; e < (q + 1) * gsz; ++e) {
        if (a < 0 || key[e] > key[a]) {
          b = a;
          a = e;
        } else if (b < 0 || key[e] > key[b]) {
          b = e;
        }
      }
      gscore[q] = b < 0 ? key[a] : key[a] + key[b];
      gkeep[q] = 0;
    }
    for (int r = 0; r < topk_group; ++r) {
      int best = -1;
      for (int q = 0; q < n_group; ++q)
        if (!gkeep[q] && (best < 0 || gscore[q] > gscore[best])) best = q;
      gkeep[best] = 1;
    }
    for (int e = 0; e < E; ++e) {
      pickable[e] = gkeep[e / gsz];
      taken[e] = 0;
    }
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (pickable[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
      sum += s[best];
    }
    for (int j = 0; j < k; ++j) {
      const double sj = s[ids[(size_t)t * k + j]];
      w[(size_t)t * k + j] = (renorm ? sj / sum : sj) * scaling;
    }
  }
  free(s);
  free(key);
  free(pickable);
  free(taken);
  free(gscore);
  free(gkeep);
}

/* Per-expert counts, exclusive-scan offsets (offsets[E] = T*k), and the
 * expert-major permutation of the T*k (token, slot) pairs, tokens ascending
 * inside an expert; entries are t*k + j. inv[t*k+j] is the position of that
 * pair in perm. ([megamoe] CUDA_GRAPH_SYNC_INVENTORY: per-expert counts kept on
 * device in a fixed-shape buffer, expert offsets as device tensors; [vllm.cpp]
 * "Device-resident decode campaign": device topk_ids feed the grouped GEMM.) */
void orc_plan(const int32_t* ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
              int32_t* perm, int32_t* inv) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < (int64_t)T * k; ++i) counts[ids[i]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int e = 0; e < E; ++e)
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (ids[(size_t)t * k + j] == e) {
          perm[pos] = t * k + j;
          inv[(size_t)t * k + j] = (int32_t)pos;
          pos++;
        }
}

/* ------------------------------------------------------------- expert FFN */

typedef struct {
  const uint8_t* w1_packed;  /* [G][2I][H/2]; rows 0..I-1 gate, I..2I-1 up */
  const uint8_t* w1_scales;  /* [G][2I][H/16] (NVFP4) or [G][2I][H/32] (MXFP4) */
  const float* w1_gs;        /* [G] (NVFP4 only) */
  const uint8_t* w2_packed;  /* [G][H][I/2] */
  const uint8_t* w2_scales;  /* [G][H][I/16] or [G][H][I/32] */
  const float* w2_gs;        /* [G] */
  int32_t mx;                /* 0: NVFP4 (orc_weight), 1: MXFP4 (orc_weight_mx) */
} orc_proj_set;

/* Element (n, k) of expert g's projection in the set's format. */
static double proj_weight(const orc_proj_set* P, int second, int g, int N, int K, int n, int k) {
  const uint8_t* pk = (second ? P->w2_packed : P->w1_packed) + (size_t)g * N * (K / 2);
  const int bs = P->mx ? 32 : 16;
  const uint8_t* sc = (second ? P->w2_scales : P->w1_scales) + (size_t)g * N * (K / bs);
  if (P->mx) return orc_weight_mx(pk, sc, K, n, k);
  return orc_weight(pk, sc, (second ? P->w2_gs : P->w1_gs)[g], K, n, k);
}

/* One expert's SwiGLU MLP on one input row, FP64:
 *   g_i = sum_k W1[i][k] x_k,  u_i = sum_k W1[I+i][k] x_k,
 *   h_i = silu(g_i) * u_i = g_i / (1 + exp(-g_i)) * u_i,   y_n = sum_i W2[n][i] h_i.
 * ([megamoe] README "MoE kernel": fused SwiGLU grouped GEMM for gate/up, then
 * the down projection; [b12x] "What's in here": SiLU/SwiGLU activations.)
 * With clamp != 0 the clamped SwiGLU with limit L >= 0:
 *   h_i = silu(min(g_i, L)) * min(max(u_i, -L), L)
 * (gate clamped from above only, up from both sides: [vllm.cpp] DeepSeek-V4
 * bring-up log, W6; a limit of 0 zeroes the expert: the same log, ds4-file
 * loadability entry; limit 10: [b12x] "DeepSeek V4 Flash 0731 MoE reproduction",
 * [megamoe] archived CORRECTNESS_BACKLOG §6, Nvfp4MoE.)
 * With hq != 0 the down projection takes NVFP4 activations as the gate/up one
 * does in W4A4 ([megamoe] FINAL_STRETCH, Part B, B0: expert weights and
 * activations both E2M1 with E4M3 block scales; [megamoe] README, "NVFP4
 * throughout": FP4 activations once the epilogue quantises them): the row h is
 * rounded to binary32, quantised by orc_quantize as one row with its own global
 * scale (per row, as for x), and y uses its exact decode. hq == 2 quantises the
 * binary32 h with the MXFP8 quantiser instead (the W4A8 profile: both expert GEMMs
 * take MXFP8 activations, [b12x] "DeepSeek V4 Flash 0731 MoE reproduction"); hq == 3
 * with the per-row FP8 quantiser (orc_fp8_rows_quantize: the NVFP4-weight W4A8 path).
 * Weights are decoded element by element in the set's format (orc_weight or
 * orc_weight_mx). */
/* h = SwiGLU(W1 x) of one expert before any quantisation (the first half of the MLP). */
void orc_expert_h(const orc_proj_set* P, int g, int H, int I, const double* x, double* h, int clamp,
                  double limit) {
  for (int i = 0; i < I; ++i) {
    double gi = 0.0, ui = 0.0;
    for (int k = 0; k < H; ++k) {
      gi += proj_weight(P, 0, g, 2 * I, H, i, k) * x[k];
      ui += proj_weight(P, 0, g, 2 * I, H, I + i, k) * x[k];
    }
    if (clamp) {
      gi = fmin(gi, limit);
      ui = fmin(fmax(ui, -limit), limit);
    }
    h[i] = gi / (1.0 + exp(-gi)) * ui;
  }
}

void orc_expert_ffn_q(const orc_proj_set* P, int g, int H, int I, const double* x, double* y,
                      int clamp, double limit, int hq) {
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  orc_expert_h(P, g, H, I, x, h, clamp, limit);
  if (hq == 3) {   /* FP8 h with a per-row scale (the NVFP4-weight W4A8 path) */
    float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hc = (uint8_t*)malloc((size_t)I);
    float hs;
    for (int i = 0; i < I; ++i) h32[i] = (float)h[i];
    orc_fp8_rows_quantize(h32, 1, I, hc, &hs);
    orc_fp8_rows(hc, &hs, 1, I, h);
    free(h32);
    free(hc);
  } else if (hq == 2) {   /* MXFP8 h (W4A8 profile) */
    float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hc = (uint8_t*)malloc((size_t)I);
    uint8_t* hs = (uint8_t*)malloc((size_t)I / 32);
    for (int i = 0; i < I; ++i) h32[i] = (float)h[i];
    orc_mxfp8_quantize(h32, 1, I, hc, hs);
    for (int i = 0; i < I; ++i) h[i] = orc_mxfp8(hc[i], hs[i / 32]);
    free(h32);
    free(hc);
    free(hs);
  } else if (hq) {
    float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* hp = (uint8_t*)calloc((size_t)I / 2, 1);
    uint8_t* hs = (uint8_t*)malloc((size_t)I / 16);
    float hg;
    for (int i = 0; i < I; ++i) h32[i] = (float)h[i];
    orc_quantize(h32, 1, I, 1, hp, hs, &hg);
    for (int i = 0; i < I; ++i) h[i] = orc_weight(hp, hs, hg, I, 0, i);
    free(h32);
    free(hp);
    free(hs);
  }
  for (int n = 0; n < H; ++n) {
    double yn = 0.0;
    for (int i = 0; i < I; ++i) yn += proj_weight(P, 1, g, H, I, n, i) * h[i];
    y[n] = yn;
  }
  free(h);
}

void orc_expert_ffn_clamp(const orc_proj_set* P, int g, int H, int I, const double* x, double* y,
                          int clamp, double limit) {
  orc_expert_ffn_q(P, g, H, I, x, y, clamp, limit, 0);
}

void orc_expert_ffn(const orc_proj_set* P, int g, int H, int I, const double* x, double* y) {
  orc_expert_ffn_q(P, g, H, I, x, y, 0, 0.0, 0);
}

/* Layer output for a list of tokens, FP64, never rounded:
 *   out[t] = sum_j w[t][j] * FFN_{ids[t][j]}(x_t)   (+ FFN_shared(x_t), weight 1)
 * ([vllm.cpp] "Device-resident decode campaign", MoeCombineKernel: the
 * weighted sum of the expert outputs with topk_weights; [megamoe] archived
 * CORRECTNESS_BACKLOG §6: an always-on shared expert beside the routed ones.)
 * x: [n_tok][H] decoded inputs of the listed tokens; ids, w: [T][k] routing;
 * out: [n_tok][H]. clamp/limit select the clamped SwiGLU for the routed experts
 * (the pages state the limit for the routed experts and a plain SwiGLU for the
 * shared one: [megamoe] archived CORRECTNESS_BACKLOG §6, Nvfp4MoE and
 * Nvfp4SharedExpert); hq quantises h of every expert, routed and shared. */
void orc_moe_tokens_q(const orc_proj_set* routed, const orc_proj_set* shared, int num_shared,
                      int H, int I, int k, int n_tok, const int32_t* tokens, const double* x,
                      const int32_t* ids, const double* w, double* out, int clamp, double limit, int hq) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_tok; ++i) {
    int t = tokens[i];
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    double* o = out + (size_t)i * H;
    for (int n = 0; n < H; ++n) o[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      orc_expert_ffn_q(routed, ids[(size_t)t * k + j], H, I, x + (size_t)i * H, y, clamp, limit, hq);
      for (int n = 0; n < H; ++n) o[n] += w[(size_t)t * k + j] * y[n];
    }
    for (int s = 0; s < num_shared; ++s) {
      orc_expert_ffn_q(shared, s, H, I, x + (size_t)i * H, y, 0, 0.0, hq);
      for (int n = 0; n < H; ++n) o[n] += y[n];
    }
    free(y);
  }
}

void orc_moe_tokens_clamp(const orc_proj_set* routed, const orc_proj_set* shared, int num_shared,
                          int H, int I, int k, int n_tok, const int32_t* tokens, const double* x,
                          const int32_t* ids, const double* w, double* out, int clamp, double limit) {
  orc_moe_tokens_q(routed, shared, num_shared, H, I, k, n_tok, tokens, x, ids, w, out, clamp, limit, 0);
}

void orc_moe_tokens(const orc_proj_set* routed, const orc_proj_set* shared, int num_shared,
                    int H, int I, int k, int n_tok, const int32_t* tokens, const double* x,
                    const int32_t* ids, const double* w, double* out) {
  orc_moe_tokens_q(routed, shared, num_shared, H, I, k, n_tok, tokens, x, ids, w, out, 0, 0.0, 0);
}

/* Decoded NVFP4 activations: x[i][k] = E2M1(code) * E4M3(scale) * gs[i]. */
void orc_dequant_rows(const uint8_t* packed, const uint8_t* scales, const float* gs,
                      int64_t rows, int K, double* x) {
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) x[(size_t)r * K + k] = orc_weight(packed, scales, gs[r], K, (int)r, k);
}

/* Decoded bf16 activations. */
void orc_bf16_rows(const uint16_t* b, int64_t n, double* x) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_bf16(b[i]);
}

/* One expert projection decoded to FP64, row-major [N][K]: element (n, k) exactly as
 * proj_weight gives it (NVFP4: E2M1 x E4M3 x global scale; MXFP4: E2M1 x E8M0). The
 * per-expert evaluation of the layer (oracle/moe.py, forward_by_expert) decodes each
 * expert once with it instead of once per use; the values are the same. */
void orc_decode_proj(const orc_proj_set* P, int second, int g, int N, int K, double* W) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) W[(size_t)n * K + k] = proj_weight(P, second, g, N, K, n, k);
}

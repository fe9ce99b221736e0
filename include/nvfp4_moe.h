/*
 * nvfp4_moe.h — C ABI of libnvfp4moe.so, an NVFP4 block-scaled fused
 * mixture-of-experts layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (all steps run as HIP kernels on the caller's stream):
 *   1. route: top-k of the FP32 router logits under (value desc, expert id asc),
 *      weights renormalised over the k picks (softmax or sigmoid scores); or the
 *      generalised router (sqrt-softplus scores, a selection-only bias, the group
 *      step, routed scaling, weights without renormalisation);
 *   2. per-expert counts, exclusive-scan offsets, stable expert-major permutation;
 *   3. optional (W4A4) NVFP4 row quantisation of the activations;
 *   4. grouped gate/up GEMM over E2M1 weights with per-16 E4M3 block scales and an
 *      FP32 per-expert global scale, fused SwiGLU (silu(gate) * up, optionally
 *      clamped) epilogue;
 *   5. grouped down GEMM;
 *   6. weighted combine of the k expert outputs (+ an always-on shared expert).
 *
 * Sources (web pages the method is described on):
 *   [b12x]     "b12x" README (github local-inference-lab/b12x)
 *   [vllm.cpp] "vllm.cpp docs/STATUS.md"
 *   [megamoe]  "nvfp4-megamoe-kernel" compare page (pre-b1...master)
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device (or managed) memory allocated and owned
 *     by the caller; the library allocates no device memory and keeps no
 *     device pointer between calls. Host pointers are marked "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work and return; none synchronises or reads device memory
 *     on the host, so a call sequence with fixed pointers can be captured in a
 *     HIP graph. (Graph-safety rule of [megamoe] GETTING_CUDAGRAPH_READY: no
 *     host branch on a device value.)
 *   - Return codes ([megamoe] dsv4/kernels/attention/fmha_mixed_fp8_capi.cu:
 *     the launcher returns a negative code for a rejected shape, else the
 *     CUDA error; the Python wrapper raises on non-zero):
 *       0  enqueued
 *      <0  rejected on the host before anything was enqueued (MOE_ERR_*)
 *      >0  the hipError_t reported right after the enqueue
 *   - No call falls back to another path ([megamoe] fmha_mixed_fp8_op.py:
 *     hard error only).
 *   - Results are bit-identical across repeated calls: no floating-point
 *     atomics, fixed reduction orders.
 */
#ifndef NVFP4_MOE_H
#define NVFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped on any change of a struct layout or of an entry point's contract
 * ([vllm.cpp] capability table: a versioned C ABI). */
#define MOE_ABI_VERSION 2u

#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)     /* unsupported shape or descriptor field */
#define MOE_ERR_SIZE (-3)      /* packed or workspace buffer too small */
#define MOE_ERR_TOKENS (-4)    /* T < 0 or T > max_tokens */
#define MOE_ERR_ALIGN (-5)     /* a device pointer is not 16-byte aligned */
#define MOE_ERR_ABI (-6)       /* desc->abi_version is neither 1 nor MOE_ABI_VERSION */
#define MOE_ERR_ENUM (-7)      /* invalid enum value */
#define MOE_ERR_WEIGHT (-8)    /* invalid weight data (host validation) */
#define MOE_ERR_SCRATCH (-9)   /* moe_run_no_alloc: the plan's workspace exceeds MOE_STATIC_SCRATCH_BYTES */

/* Router score ([b12x] "What's in here": routing scores kept in FP32;
 * [vllm.cpp] capability table: sigmoid noaux_tc routers; [vllm.cpp] DeepSeek-V4
 * bring-up log, W6, and [megamoe] archived CORRECTNESS_BACKLOG §5, Dense Router:
 * the sqrt(softplus(x)) score). */
#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_SCORE_SQRT_SOFTPLUS 2   /* generalised router only */

/* Activation format ([b12x] "What's in here", moe: W4A16 = BF16 activations with
 * inline FP4 weight dequant; [megamoe] FINAL_STRETCH B0: expert weights and
 * activations both float4_e2m1fn_x2 = W4A4; [megamoe] README "NVFP4 throughout":
 * FP4 activations once the epilogue quantises them).
 *   MOE_ACT_BF16        both expert GEMMs take 16-bit activations (W4A16);
 *   MOE_ACT_NVFP4_ROWQ  x is row-quantised to NVFP4 (binary32 quantiser, one FP32
 *                       global scale per token row) before the gate/up GEMM;
 *   MOE_ACT_NVFP4_ALL   x as above, and h = silu(g)*u of every expert row (routed and
 *                       shared) is rounded to binary32 and row-quantised the same way,
 *                       with its own global scale, before the down GEMM. */
#define MOE_ACT_BF16 0
#define MOE_ACT_NVFP4_ROWQ 1
#define MOE_ACT_NVFP4_ALL 2
#define MOE_ACT_MXFP8 3   /* W4A8 ([b12x] "DeepSeek V4 Flash 0731 MoE reproduction": MXFP4
                             E8M0/K32 weights with MXFP8 activations); requires
                             MOE_WEIGHTS_MXFP4. x and h of every expert row are MXFP8-quantised:
                             per 32 consecutive k an E8M0 scale 2^X, X = floor(log2 max|v|) - 8
                             (clamped to [-127, 127]; -127 for a zero block), E4M3 codes of
                             |v| 2^-X rounded to nearest even and saturating at 448, sign kept.
                             Both GEMMs run gfx950's block-scaled MFMA on the raw codes. */
#define MOE_ACT_FP8_ROW 4 /* W4A8 on NVFP4 weights ([b12x] "What's in here", moe: the unified
                             dynamic path's w4a8_nvfp4 variant, NVFP4 weights with FP8
                             activations). x and h of every expert row are FP8 E4M3 with one FP32
                             scale per row, s = max|v| / 448 (binary32), codes sign | E4M3 of
                             |v| / s rounded to nearest even and saturating at 448 (0 if s == 0),
                             the per-row amax rule of [megamoe] archived CORRECTNESS_BACKLOG
                             section 7 (FP8 rows with a per-row float32 scale). Any weight format;
                             the GEMMs take the codes' exact fp16 decode and apply s in the
                             epilogue. */

/* Weight format of every projection ([vllm.cpp] capability table, MXFP4 row: E8M0
 * dequant 2^(byte-127), group 32, no global scale, distinct from NVFP4's group-16 fp8
 * scale path; [b12x] "DeepSeek V4 Flash 0731 MoE reproduction": MXFP4 E8M0/K32 expert
 * weights). */
#define MOE_WEIGHTS_NVFP4 0   /* E2M1 x E4M3 per 16 along K x FP32 per expert */
#define MOE_WEIGHTS_MXFP4 1   /* E2M1 x E8M0 (2^(byte-127)) per 32 along K */

/* Layer descriptor. Limits: hidden and inter multiples of 128 (hidden <= 16384,
 * inter <= 16384), 1 <= top_k <= min(64, num_experts), num_experts <= 1024,
 * 1 <= max_tokens <= 65536, num_shared in {0, 1}; renormalize in {0, 1};
 * n_group divides num_experts, n_group <= 64, 1 <= topk_group <= n_group and
 * topk_group * (num_experts / n_group) >= top_k; routed_scaling finite and > 0;
 * swiglu_limit finite and >= 0 when swiglu_clamp is set.
 * A descriptor with abi_version 1 ends after num_shared; its later fields take the
 * values of the plain layer (1, 1, 0, 0, 1.0, 0, MOE_WEIGHTS_NVFP4) and it must have
 * renormalize == 1.
 *
 * The plain router (score softmax or sigmoid, renormalize 1, no bias, n_group 1,
 * routed_scaling 1) selects on the logits. Any other setting runs the generalised
 * router, per token:
 *   s_e   = score in FP64: softmax over all E experts, sigmoid, or
 *           sqrt(softplus(l_e)) (MOE_SCORE_SQRT_SOFTPLUS);
 *   key_e = fp32(s_e) [+ bias_e, a binary32 add]: the bias (moe_pack_router_bias)
 *           steers selection only ([vllm.cpp] DeepSeek-V4 bring-up log, W6);
 *   group step (n_group > 1): groups of num_experts / n_group consecutive experts,
 *           a group's score the binary32 sum of its two largest keys, the topk_group
 *           best groups kept (lower group id on ties), picks only from those (the
 *           DeepSeek-V3 noaux_tc step the pages name: [vllm.cpp] capability table);
 *   picks = the k largest keys, lower id on ties;
 *   w_j   = s_j / sum of the picks' s (renormalize) or s_j, times routed_scaling
 *           ([vllm.cpp] capability table: noaux_tc sigmoid router with routed scaling).
 * swiglu_clamp: the routed experts use h = silu(min(g, L)) * clamp(u, -L, L),
 * L = swiglu_limit (gate clamped from above only; L = 0 zeroes them); the shared
 * expert keeps the plain SwiGLU ([vllm.cpp] DeepSeek-V4 bring-up log, W6 and the
 * ds4-file loadability entry; [megamoe] archived CORRECTNESS_BACKLOG §6, Nvfp4MoE
 * swiglu_limit 10 and Nvfp4SharedExpert). */
typedef struct {
  uint32_t abi_version;     /* MOE_ABI_VERSION (or 1, see above) */
  int32_t hidden;           /* H */
  int32_t inter;            /* I, per expert (the shared expert uses the same I) */
  int32_t num_experts;      /* E routed experts */
  int32_t top_k;            /* k experts per token */
  int32_t max_tokens;       /* T_max: capacity the workspace is sized for */
  int32_t score_fn;         /* MOE_SCORE_* */
  int32_t renormalize;      /* 1: weights renormalised over the k picks */
  int32_t act_format;       /* MOE_ACT_* */
  int32_t num_shared;       /* 0 or 1 always-on shared expert, weight 1.0 */
  /* since ABI 2 */
  int32_t use_bias;         /* 1: a per-expert selection bias is packed (moe_pack_router_bias) */
  int32_t n_group;          /* group step: expert groups (1 = none) */
  int32_t topk_group;       /* groups kept */
  int32_t swiglu_clamp;     /* 1: clamped SwiGLU for the routed experts */
  float routed_scaling;     /* factor on the routed weights */
  float swiglu_limit;       /* clamp limit L */
  int32_t weight_format;    /* MOE_WEIGHTS_* of every projection */
} moe_desc;

/* Opaque plan: host memory, immutable after moe_plan, safe to share between
 * threads. Concurrent moe_run calls need distinct workspaces. */
typedef struct moe_plan moe_plan_t;

/* One FP4 projection of G experts in the pages' operand layout ([vllm.cpp]
 * capability table, GGUF loading row: weight_packed [N,K/2] + weight_scale
 * [N,K/16] + per-expert weight_scale_2; [megamoe] archived CORRECTNESS_BACKLOG
 * §7: the weight global scale is weight_scale_2). Device pointers:
 *   packed       u8  [G][N][K/2]   E2M1 codes, element 2i in the low nibble of
 *                                  byte i, 2i+1 in the high nibble
 *   scales       u8  [G][N][K/16]  E4M3fn block scales, block = 16 consecutive k
 *   global_scale f32 [G]           per-expert global scale
 * W[g][n][k] = E2M1(code) * E4M3(scale[g][n][k/16]) * global_scale[g].
 * MXFP4 (weight_format MOE_WEIGHTS_MXFP4): scales u8 [G][N][K/32] E8M0 bytes,
 * global_scale unused (may be NULL), W[g][n][k] = E2M1(code) * 2^(scale[g][n][k/32]
 * - 127). Packing turns every MXFP4 expert exactly into the NVFP4 form the kernels
 * read: per-expert global scale 2^(m - 135), m = the expert's largest scale byte,
 * and E4M3 block scales 2^(byte - m + 8), exact while byte >= m - 17 (E4M3's
 * smallest power of two is 2^-9); moe_validate_weights_host rejects wider spans and
 * the NaN byte 0xFF, and packing gives such an expert a NaN global scale, so that
 * every output reading it is NaN (never a silently different value). With
 * MOE_ACT_MXFP8 the scale bytes are used as they are and any span is exact.
 * gate_up: N = 2I, K = H, rows 0..I-1 are the gate, rows I..2I-1 the up
 * projection; down: N = H, K = I. */
typedef struct {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* global_scale;
} moe_nvfp4_tensor;

/* Optional outputs of moe_run (every pointer may be NULL; device memory,
 * 4-byte aligned):
 *   topk_ids       i32 [T][k]  expert of pick j, picks in selection order
 *   topk_weights   f32 [T][k]  renormalised routing weight of pick j
 *   expert_counts  i32 [E]     rows routed to each expert
 *   expert_offsets i32 [E+1]   exclusive scan of counts, offsets[E] = T*k
 *   perm           i32 [T*k]   perm[offsets[e] + r] = t*k + j: expert-major,
 *                              tokens ascending inside an expert
 *   act_packed     u8  [T][H/2]   (NVFP4 x; MXFP8 and FP8 rows: [T][H] E4M3 codes) quantised
 *   act_scales     u8  [T][H/16]   activations, as moe_quantize_nvfp4_rows writes them (MXFP8:
 *   act_global     f32 [T]         [T][H/32] E8M0; FP8 rows: no block scales, act_global = the
 *                                  row scales, as moe_quantize_fp8_rows writes them) */
typedef struct {
  int32_t* topk_ids;
  float* topk_weights;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* perm;
  uint8_t* act_packed;
  uint8_t* act_scales;
  float* act_global;
} moe_routing_out;

/* Declare a layer. Host only, no HIP call, allocates only the host plan
 * ([b12x] "Using it": a plan declares the work, allocates no device storage
 * and compiles nothing; "What's in here": fixed-capacity scratch with live
 * row counts as runtime values). On success *plan is set and the two sizes
 * are the bytes the caller must provide for the packed weights and for the
 * workspace of any T <= max_tokens. */
int moe_plan(const moe_desc* desc, moe_plan_t** plan, size_t* packed_bytes,
             size_t* workspace_bytes);

/* Free a plan (NULL is ignored). */
void moe_plan_destroy(moe_plan_t* plan);

/* Re-lay the boundary-layout weights into the plan's packed buffer: a pure
 * byte permutation (gate/up 16-row interleave, 128-column K tiles in the
 * order the GEMM waves read them, block scales grouped per lane) plus a copy
 * of the global scales. ([vllm.cpp] capability table, GGUF row: NVFP4 weights
 * repacked at load as a pure byte permutation; [megamoe] CUDA_GRAPH_SYNC_INVENTORY
 * and WALKING_BACK_SOME_QUANTS: raw row-major scales re-laid once at finalize.)
 * gate_up and down describe the E routed experts; shared_gate_up/shared_down
 * the num_shared shared experts (NULL when num_shared == 0). The inputs must
 * stay valid until the enqueued work completes; `packed` must be 16-byte
 * aligned and at least packed_bytes long. The same inputs always produce the
 * same packed bytes. */
int moe_pack_weights(const moe_plan_t* plan, const moe_nvfp4_tensor* gate_up,
                     const moe_nvfp4_tensor* down, const moe_nvfp4_tensor* shared_gate_up,
                     const moe_nvfp4_tensor* shared_down, void* packed, size_t packed_bytes,
                     void* stream);

/* Copy the per-expert selection bias (device f32 [num_experts], finite values) into
 * the plan's packed buffer; required once per packed buffer when the descriptor has
 * use_bias = 1 (MOE_ERR_SHAPE otherwise). The bias is a layer parameter like the
 * weights: it only steers which experts are picked ([vllm.cpp] DeepSeek-V4 bring-up
 * log, W6; [megamoe] archived CORRECTNESS_BACKLOG §5, Dense Router e_bias). `packed`
 * as for moe_pack_weights; `bias` must stay valid until the copy completes. */
int moe_pack_router_bias(const moe_plan_t* plan, const float* bias, void* packed, size_t packed_bytes,
                         void* stream);

/* Run the layer on T live tokens (0 <= T <= max_tokens; T is a host int).
 *   packed        the buffer moe_pack_weights filled
 *   x             bf16 [T][H] activations (16-byte aligned)
 *   router_logits f32  [T][E] (16-byte aligned); finite values
 *   out           bf16 [T][H] = sum_j w[t][j] * FFN_{ids[t][j]}(x_t) (+ shared),
 *                 summed in FP32 in pick order, rounded to bf16 (RNE)
 *   routing       optional outputs (may be NULL)
 *   workspace     at least workspace_bytes, 16-byte aligned; contents on entry
 *                 are ignored, on return undefined
 * Intermediates: gate/up accumulate in FP32 and stay in registers through the
 * SwiGLU; h = silu(g*gs)*(u*gs) is stored as fp16 with one power-of-two exponent
 * per 16 columns (the block's largest |h| scaled into [2^14, 2^15)); before the fp16
 * MFMAs of the down GEMM every block is brought to the row's common exponent (that of
 * its largest block) by a power-of-two factor, which is exact except that values
 * pushed below fp16's normal range (more than 14 binades under the row's largest
 * block) lose low bits and those more than 24 binades under it become 0;
 * expert outputs are stored the same way (fp16 with a power-of-two exponent per 16
 * columns) and summed by the combine in fp32. With MOE_ACT_NVFP4_ALL, h is stored
 * as fp32, row-quantised (codes, E4M3 block scales, FP32 row global scale) and the
 * down GEMM decodes it exactly, applying the row's global scale in its epilogue.
 * ([megamoe] README "MoE kernel": fused SwiGLU grouped GEMM epilogue in
 * registers; [b12x] "What's in here": FP32 internal, BF16 boundary;
 * [vllm.cpp] "Device-resident decode campaign": device routing ids feed the
 * grouped GEMM, routing weights feed MoeCombineKernel.) T == 0 enqueues nothing. */
int moe_run(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
            const float* router_logits, uint16_t* out, const moe_routing_out* routing,
            void* workspace, size_t workspace_bytes, void* stream);

/* Stages of moe_run (for moe_run_timed); launch order ROUTE, GATE_UP, QUANT, DOWN, COMBINE. */
#define MOE_STAGE_QUANT 0      /* the preparation of h for the down GEMM: the h row quantisation
                                  (MOE_ACT_NVFP4_ALL, MOE_ACT_FP8_ROW, MOE_ACT_MXFP8 in the
                                  prefill regime) or the rescale of the h16 rows to their row
                                  exponent (16-bit h, prefill regime); empty otherwise (the
                                  activation preparation of x runs in the ROUTE stage) */
#define MOE_STAGE_ROUTE 1      /* top-k, counts, offsets, permutation, tile list, and the
                                  activation preparation (NVFP4 quantisation of x with, for
                                  prefill-regime batches, its exact fp16 decode; MXFP8
                                  quantisation; FP8 row quantisation with its exact fp16 decode;
                                  or the exact power-of-two rescale of bf16 rows into fp16) by
                                  extra workgroups of the first routing launch */
#define MOE_STAGE_GATE_UP 2    /* grouped gate/up GEMM + SwiGLU */
#define MOE_STAGE_DOWN 3       /* grouped down GEMM */
#define MOE_STAGE_COMBINE 4    /* weighted combine */
#define MOE_NUM_STAGES 5

/* moe_run with per-stage timing: stage_events holds 2*MOE_NUM_STAGES hipEvent_t
 * handles (as void*, any may be NULL), created by the caller with timing enabled.
 * For the single-kernel stages (GATE_UP, DOWN, COMBINE) events[2s] and events[2s+1]
 * are stamped by the kernel launch itself at the kernel's start and end, so their
 * elapsed time is the kernel's duration (a skewed batch's two tile lists run in one kernel;
 * where they run as two, the events stamp the first one's start and the second one's end);
 * for the others (QUANT: zero or one kernel, ROUTE: one to four kernels) they are recorded
 * on `stream` right before and after the stage. Results
 * are identical to moe_run. ([b12x] "Using it": per-kernel timing logs for tuning.) */
int moe_run_timed(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                  const float* router_logits, uint16_t* out, const moe_routing_out* routing,
                  void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events);

/* moe_run without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The workspace is a fixed array of MOE_STATIC_SCRATCH_BYTES inside the library, one
 * copy per GPU, held until the process ends; the call uses the copy of the current
 * device (hipGetDevice), so `stream` must belong to that device. Arguments, results and
 * error codes are moe_run's; MOE_ERR_SCRATCH if the plan's workspace_bytes exceeds
 * MOE_STATIC_SCRATCH_BYTES (64 MiB: any T_max of a decode-sized layer; the Qwen3-30B-A3B
 * shape up to about 1300 tokens). No call allocates or frees anything; the first call on
 * a device resolves the array's address there (hipGetSymbolAddress, no allocation). The
 * array keeps the previous call's contents, which the layer never reads: every value it
 * uses is written earlier in the same call. All calls on one GPU share the array, so calls
 * that may overlap in time on one GPU (different streams, or different threads) race and
 * must be serialised by the caller. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
int moe_run_no_alloc(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                     const float* router_logits, uint16_t* out, const moe_routing_out* routing,
                     void* stream);

/* NVFP4 row quantiser (the W4A4 activation step of moe_run, callable alone):
 * for each of `rows` bf16 rows of K elements (K a multiple of 16, <= 16384):
 *   gs   = max|x| / 2688, 2688 = 6 * 448 the largest E2M1 value times the largest
 *          E4M3 value ([megamoe] archived CORRECTNESS_BACKLOG §7, runtime activation
 *          global scale)
 *   s_b  = E4M3 nearest-even of a_b / (6 gs), saturating at 448; 0 if gs == 0
 *   d_b  = E4M3(s_b) * gs
 *   code = sign | E2M1 nearest-even of |x| / d_b, saturating at 6; 0 if d_b == 0
 * every step a binary32 operation rounded to nearest even (division correctly
 * rounded). Outputs packed u8 [rows][K/2], scales u8 [rows][K/16],
 * row_global f32 [rows]; all device pointers 16-byte aligned. */
int moe_quantize_nvfp4_rows(const uint16_t* x, int32_t rows, int32_t K, uint8_t* packed,
                            uint8_t* scales, float* row_global, void* stream);

/* FP8 row quantiser of MOE_ACT_FP8_ROW (NVFP4-weight W4A8; [b12x] "What's in here", moe,
 * w4a8_nvfp4; per-row amax scale as in [megamoe] archived CORRECTNESS_BACKLOG section 7):
 * per bf16 row of K columns,
 *   s    = max|x| / 448 (binary32)
 *   code = sign << 7 | E4M3 nearest-even of |x| / s (binary32 division), saturating at 448;
 *          0 if s == 0
 * Outputs codes u8 [rows][K] and row_scale f32 [rows] (device, caller-owned); x and codes
 * 16-byte aligned, row_scale 4-byte aligned; K a multiple of 16 up to 16384 (MOE_ERR_SHAPE
 * otherwise). Enqueued on `stream`; returns a HIP error code if the launch fails. */
int moe_quantize_fp8_rows(const uint16_t* x, int32_t rows, int32_t K, uint8_t* codes, float* row_scale,
                          void* stream);

/* The same quantiser with one global scale per group of `rows_per_group`
 * consecutive fp32 rows (a weight projection [N][K] is one group of N rows):
 * gs[g] = max|x| over the group / 2688, then blocks and codes as above.
 * Input w f32 [groups*rows_per_group][K]; outputs packed [..][K/2],
 * scales [..][K/16], group_global f32 [groups]. Used to prepare weights. */
int moe_quantize_nvfp4_weights(const float* w, int32_t groups, int32_t rows_per_group, int32_t K,
                               uint8_t* packed, uint8_t* scales, float* group_global,
                               void* stream);

/* Host-side weight check (host pointers, G experts of one projection):
 * rejects NaN block scales (E4M3fn S.1111.111), negative block scales and
 * non-finite or negative global scales with MOE_ERR_WEIGHT. which: 0 gate_up,
 * 1 down (routed, G = E), 2 shared gate_up, 3 shared down (G = num_shared).
 * ([megamoe] WALKING_BACK_SOME_QUANTS: validate scale sizes and contents at
 * the boundary instead of faulting inside a kernel.) */
int moe_validate_weights_host(const moe_desc* desc, const moe_nvfp4_tensor* host_copy, int32_t which);

/* Static description of a return code. */
const char* moe_strerror(int code);

/* MOE_ABI_VERSION of the loaded library. */
uint32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MOE_H */

// C ABI of libnvfp4moe.so: host validation, buffer layout and launch order.
// Declared in include/nvfp4_moe.h; see there for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/nvfp4_moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace nvmoe;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_HIDDEN = 16384;
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_TOPK = 64;
constexpr int MAX_TOKENS = 65536;
constexpr int MAX_GROUPS = 64;
// prefill: experts with at most this many rows run through the decode GEMM (second tile list)
constexpr int COLD_ROWS = 16;
constexpr int SPLIT_TILE_ROWS = 64;   // the first list's tile height in skewed and MX8 batches
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Upper bound on the GEMM tile list for T tokens and tile height M:
// sum over groups of ceil(c/M) <= rows/M + (non-empty groups).
int tile_bound(int T, int k, int E, int S, int M) {
  const long rows = (long)T * k;
  long b = rows / M + std::min<long>(E, rows);
  b += (long)S * ((T + M - 1) / M);
  return (int)b;
}

bool use_decode(int T, int k, int E) { return (long)T * k <= 16L * E; }

}  // namespace

struct moe_plan {
  moe_desc d;
  int G;
  ProjLayout w1, w2;
  size_t off_w1f, off_w1s, off_w1g, off_w2f, off_w2s, off_w2g, off_bias, packed_bytes;
  size_t ws_ids, ws_w, ws_counts, ws_offsets, ws_perm, ws_inv, ws_tok, ws_tgrp, ws_trow, ws_tcnt, ws_plan;
  size_t ws_xq, ws_xs, ws_xg, ws_x16, ws_h, ws_hexp, ws_hmin, ws_hf, ws_hq, ws_hs, ws_hg, ws_y, ws_yexp, ws_bytes;
  int max_tiles;
};

extern "C" {

uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer argument";
    case MOE_ERR_SHAPE: return "unsupported shape or descriptor field";
    case MOE_ERR_SIZE: return "packed or workspace buffer too small";
    case MOE_ERR_TOKENS: return "token count outside [0, max_tokens]";
    case MOE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_ERR_ABI: return "ABI version mismatch";
    case MOE_ERR_ENUM: return "invalid enum value";
    case MOE_ERR_WEIGHT: return "invalid weight data (NaN/negative scale or bad global scale)";
    case MOE_ERR_SCRATCH: return "the plan's workspace exceeds the static scratch of moe_run_no_alloc";
    default: break;
  }
  if (code > 0) return hipGetErrorString((hipError_t)code);
  return "unknown error";
}

// Bring a version-1 or current descriptor to the current layout (a version-1 one ends
// after num_shared; the later fields get the plain layer's values) and validate it.
static int load_desc(const moe_desc* in, moe_desc* out) {
  if (!in) return MOE_ERR_NULL;
  if (in->abi_version == 1u) {
    std::memset(out, 0, sizeof(*out));
    std::memcpy(out, in, offsetof(moe_desc, use_bias));
    out->n_group = 1;
    out->topk_group = 1;
    out->routed_scaling = 1.0f;
    if (in->renormalize != 1) return MOE_ERR_SHAPE;
  } else if (in->abi_version == MOE_ABI_VERSION) {
    *out = *in;
  } else {
    return MOE_ERR_ABI;
  }
  const moe_desc* d = out;
  if (d->score_fn != MOE_SCORE_SOFTMAX && d->score_fn != MOE_SCORE_SIGMOID && d->score_fn != MOE_SCORE_SQRT_SOFTPLUS)
    return MOE_ERR_ENUM;
  if (d->act_format != MOE_ACT_BF16 && d->act_format != MOE_ACT_NVFP4_ROWQ && d->act_format != MOE_ACT_NVFP4_ALL &&
      d->act_format != MOE_ACT_MXFP8 && d->act_format != MOE_ACT_FP8_ROW)
    return MOE_ERR_ENUM;
  if (d->hidden < 128 || d->hidden > MAX_HIDDEN || d->hidden % 128) return MOE_ERR_SHAPE;
  if (d->inter < 128 || d->inter > MAX_HIDDEN || d->inter % 128) return MOE_ERR_SHAPE;
  if (d->num_experts < 1 || d->num_experts > MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > MAX_TOPK || d->top_k > d->num_experts) return MOE_ERR_SHAPE;
  if (d->max_tokens < 1 || d->max_tokens > MAX_TOKENS) return MOE_ERR_SHAPE;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_SHAPE;
  if (d->num_shared < 0 || d->num_shared > 1) return MOE_ERR_SHAPE;
  if (d->use_bias != 0 && d->use_bias != 1) return MOE_ERR_ENUM;
  if (d->swiglu_clamp != 0 && d->swiglu_clamp != 1) return MOE_ERR_ENUM;
  if (d->n_group < 1 || d->n_group > MAX_GROUPS || d->num_experts % d->n_group) return MOE_ERR_SHAPE;
  if (d->topk_group < 1 || d->topk_group > d->n_group) return MOE_ERR_SHAPE;
  if ((long)d->topk_group * (d->num_experts / d->n_group) < d->top_k) return MOE_ERR_SHAPE;
  if (!std::isfinite(d->routed_scaling) || d->routed_scaling <= 0.0f) return MOE_ERR_SHAPE;
  if (d->swiglu_clamp && (!std::isfinite(d->swiglu_limit) || d->swiglu_limit < 0.0f)) return MOE_ERR_SHAPE;
  if (d->weight_format != MOE_WEIGHTS_NVFP4 && d->weight_format != MOE_WEIGHTS_MXFP4) return MOE_ERR_ENUM;
  // MXFP8 activations run the scaled MFMA on native MXFP4 weights only
  if (d->act_format == MOE_ACT_MXFP8 && d->weight_format != MOE_WEIGHTS_MXFP4) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The generalised router runs for anything but the plain top-k with renormalised
// softmax / sigmoid weights.
static bool general_router(const moe_desc& d) {
  return d.score_fn == MOE_SCORE_SQRT_SOFTPLUS || d.use_bias || d.n_group > 1 || d.renormalize == 0 ||
         d.routed_scaling != 1.0f;
}

int moe_plan(const moe_desc* desc, moe_plan_t** plan, size_t* packed_bytes, size_t* workspace_bytes) {
  if (!plan) return MOE_ERR_NULL;
  *plan = nullptr;
  moe_desc dd;
  const int rc = load_desc(desc, &dd);
  if (rc) return rc;
  struct moe_plan* p = new (std::nothrow) struct moe_plan;
  if (!p) return MOE_ERR_SIZE;
  std::memset(p, 0, sizeof(*p));
  p->d = dd;
  desc = &p->d;
  const int H = desc->hidden, I = desc->inter, E = desc->num_experts, k = desc->top_k;
  const int S = desc->num_shared, Tm = desc->max_tokens;
  p->G = E + S;
  p->w1 = proj_layout(2 * I, H);
  p->w2 = proj_layout(H, I);
  size_t o = 0;
  p->off_w1f = o; o = align_up(o + p->w1.fp4_expert * p->G);
  p->off_w1s = o; o = align_up(o + p->w1.sc_expert * p->G);
  p->off_w1g = o; o = align_up(o + sizeof(float) * p->G);
  p->off_w2f = o; o = align_up(o + p->w2.fp4_expert * p->G);
  p->off_w2s = o; o = align_up(o + p->w2.sc_expert * p->G);
  p->off_w2g = o; o = align_up(o + sizeof(float) * p->G);
  p->off_bias = o; o = align_up(o + (desc->use_bias ? sizeof(float) * E : 0));
  p->packed_bytes = o;

  const size_t routed = (size_t)Tm * k, rows = routed + (size_t)S * Tm;
  p->max_tiles = std::max(tile_bound(Tm, k, E, S, DECODE_TILE_ROWS), tile_bound(Tm, k, E, S, PREFILL_TILE_ROWS));
  o = 0;
  p->ws_ids = o; o = align_up(o + 4 * routed);
  p->ws_w = o; o = align_up(o + 4 * routed);
  p->ws_counts = o; o = align_up(o + 4 * (size_t)p->G);
  p->ws_offsets = o; o = align_up(o + 4 * ((size_t)p->G + 1));
  p->ws_perm = o; o = align_up(o + 4 * routed);
  p->ws_inv = o; o = align_up(o + 4 * routed);
  p->ws_tok = o; o = align_up(o + 4 * rows);
  // twice the bound: a second-list launch reads ahead of its count from anywhere in the list
  p->ws_tgrp = o; o = align_up(o + 8 * (size_t)p->max_tiles);
  p->ws_trow = o; o = align_up(o + 8 * (size_t)p->max_tiles);
  p->ws_tcnt = o; o = align_up(o + 16);
  p->ws_plan = o; o = align_up(o + 4 * plan_scratch_ints(Tm, k, E));
  const bool mx8 = desc->act_format == MOE_ACT_MXFP8, f8 = desc->act_format == MOE_ACT_FP8_ROW;
  const bool fp4x = desc->act_format != MOE_ACT_BF16 && !f8, fp4h = desc->act_format == MOE_ACT_NVFP4_ALL;
  // FP8 rows: x codes only go to the caller's act_packed; the GEMMs read the fp16 decode
  p->ws_xq = o; o = align_up(o + (fp4x ? (size_t)Tm * H / (mx8 ? 1 : 2) : 0));   // codes (MXFP8: a byte each)
  p->ws_xs = o; o = align_up(o + (fp4x ? (size_t)Tm * H / 16 : 0));
  p->ws_xg = o; o = align_up(o + 4 * (size_t)Tm);      // per-row activation factor (either format)
  p->ws_x16 = o; o = align_up(o + (mx8 ? 0 : 2 * (size_t)Tm * H));   // fp16 x rows (rescaled bf16 or NVFP4 decode)
  p->ws_h = o; o = align_up(o + (mx8 ? 0 : 2 * rows * I));              // h16 (NVFP4 / FP8 h: its fp16 decode)
  p->ws_hexp = o; o = align_up(o + (fp4h || mx8 || f8 ? 0 : rows * (I / 16)));  // per-16-column h exponents
  p->ws_hmin = o; o = align_up(o + 4 * rows);                       // per-row minimum h exponent
  p->ws_hf = o; o = align_up(o + (fp4h || mx8 || f8 ? 4 * rows * I : 0));   // NVFP4 / FP8 / prefill MXFP8 h: fp32
  p->ws_hq = o; o = align_up(o + (fp4h ? rows * I / 2 : mx8 ? rows * I : 0));   // h rows, their codes,
  p->ws_hs = o; o = align_up(o + (fp4h ? rows * (I / 16) : mx8 ? rows * (I / 32) : 0));   // block scales
  p->ws_hg = o; o = align_up(o + (fp4h || f8 ? 4 * rows : 0));     // and per-row scales
  p->ws_y = o; o = align_up(o + 2 * rows * H);         // y16
  p->ws_yexp = o; o = align_up(o + rows * (H / 16));  // per-16-column y exponents
  p->ws_bytes = o;
  if (packed_bytes) *packed_bytes = p->packed_bytes;
  if (workspace_bytes) *workspace_bytes = p->ws_bytes;
  *plan = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t* plan) { delete plan; }

static int check_tensor(const moe_nvfp4_tensor* t, bool mx) {
  if (!t || !t->packed || !t->scales || (!mx && !t->global_scale)) return MOE_ERR_NULL;
  if (!aligned16(t->packed) || !aligned16(t->scales) || (!mx && !aligned4(t->global_scale))) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int moe_pack_weights(const moe_plan_t* plan, const moe_nvfp4_tensor* gate_up, const moe_nvfp4_tensor* down,
                     const moe_nvfp4_tensor* shared_gate_up, const moe_nvfp4_tensor* shared_down, void* packed,
                     size_t packed_bytes, void* stream) {
  if (!plan || !packed) return MOE_ERR_NULL;
  const bool mx = plan->d.weight_format == MOE_WEIGHTS_MXFP4;
  int rc = check_tensor(gate_up, mx);
  if (!rc) rc = check_tensor(down, mx);
  if (!rc && plan->d.num_shared) {
    rc = check_tensor(shared_gate_up, mx);
    if (!rc) rc = check_tensor(shared_down, mx);
  }
  if (rc) return rc;
  if (!aligned16(packed)) return MOE_ERR_ALIGN;
  if (packed_bytes < plan->packed_bytes) return MOE_ERR_SIZE;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)packed;
  const int E = plan->d.num_experts;
  const moe_nvfp4_tensor* srcs[2][2] = {{gate_up, down}, {shared_gate_up, shared_down}};
  for (int shared = 0; shared <= (plan->d.num_shared ? 1 : 0); ++shared) {
    for (int proj = 0; proj < 2; ++proj) {
      const ProjLayout& L = proj ? plan->w2 : plan->w1;
      const moe_nvfp4_tensor* t = srcs[shared][proj];
      const size_t g0 = shared ? (size_t)E : 0;
      PackArgs a;
      a.packed = t->packed;
      a.scales = t->scales;
      a.gs = t->global_scale;
      a.G = shared ? plan->d.num_shared : E;
      a.N = L.N;
      a.K = L.K;
      a.gate_up = proj == 0;
      a.mx = !mx ? 0 : plan->d.act_format == MOE_ACT_MXFP8 ? 2 : 1;   // 2: native for the scaled MFMA
      a.fp4_out = base + (proj ? plan->off_w2f : plan->off_w1f) + g0 * L.fp4_expert;
      a.sc_out = base + (proj ? plan->off_w2s : plan->off_w1s) + g0 * L.sc_expert;
      a.gs_out = (float*)(base + (proj ? plan->off_w2g : plan->off_w1g)) + g0;
      const hipError_t e = launch_pack(a, s);
      if (e != hipSuccess) return (int)e;
    }
  }
  return MOE_OK;
}

int moe_pack_router_bias(const moe_plan_t* plan, const float* bias, void* packed, size_t packed_bytes,
                         void* stream) {
  if (!plan || !bias || !packed) return MOE_ERR_NULL;
  if (!plan->d.use_bias) return MOE_ERR_SHAPE;
  if (!aligned16(packed) || !aligned4(bias)) return MOE_ERR_ALIGN;
  if (packed_bytes < plan->packed_bytes) return MOE_ERR_SIZE;
  const hipError_t e = hipMemcpyAsync((uint8_t*)packed + plan->off_bias, bias, sizeof(float) * plan->d.num_experts,
                                      hipMemcpyDeviceToDevice, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : (int)e;
}

static int run_impl(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                    const float* router_logits, uint16_t* out, const moe_routing_out* routing, void* workspace,
                    size_t workspace_bytes, void* stream, void* const* ev);

int moe_run(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x, const float* router_logits,
            uint16_t* out, const moe_routing_out* routing, void* workspace, size_t workspace_bytes, void* stream) {
  return run_impl(plan, packed, T, x, router_logits, out, routing, workspace, workspace_bytes, stream, nullptr);
}

int moe_run_timed(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                  const float* router_logits, uint16_t* out, const moe_routing_out* routing, void* workspace,
                  size_t workspace_bytes, void* stream, void* const* stage_events) {
  return run_impl(plan, packed, T, x, router_logits, out, routing, workspace, workspace_bytes, stream,
                  stage_events);
}

// ---------------------------------------------------------------- no-allocation run
// moe_run_no_alloc runs the layer with the workspace in `scratch`, a fixed device array of
// the library (each GPU the library runs on holds its own copy until the process ends).
// Host code never uses the array's name as an address: it stands for a host-side shadow.
// The device address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept in scratch_ptr[device].
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];
}  // namespace

// The current device's address of `scratch` (resolved on the first call for the device).
static int static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= MAX_DEVICES) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || ((uintptr_t)p & (ALIGN - 1))) return (int)hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return MOE_OK;
}

int moe_run_no_alloc(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                     const float* router_logits, uint16_t* out, const moe_routing_out* routing, void* stream) {
  if (!plan) return MOE_ERR_NULL;
  if (plan->ws_bytes > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = static_scratch(&ws);
  if (rc) return rc;
  return run_impl(plan, packed, T, x, router_logits, out, routing, ws, plan->ws_bytes, stream, nullptr);
}

// Stages of several (or no) kernels are bracketed by event records on the stream; the
// single-kernel stages (the GEMMs, the combine) get kernel-stamped events instead.
static hipError_t mark(void* const* ev, int idx, hipStream_t s) {
  if (!ev || !ev[idx]) return hipSuccess;
  return hipEventRecord((hipEvent_t)ev[idx], s);
}

static LaunchEvents stage_events(void* const* ev, int stage) {
  LaunchEvents le;
  if (ev) {
    le.start = (hipEvent_t)ev[2 * stage];
    le.stop = (hipEvent_t)ev[2 * stage + 1];
  }
  return le;
}

static int run_impl(const moe_plan_t* plan, const void* packed, int32_t T, const uint16_t* x,
                    const float* router_logits, uint16_t* out, const moe_routing_out* routing, void* workspace,
                    size_t workspace_bytes, void* stream, void* const* ev) {
  if (!plan || !packed || !x || !router_logits || !out || !workspace) return MOE_ERR_NULL;
  const moe_desc& d = plan->d;
  if (T < 0 || T > d.max_tokens) return MOE_ERR_TOKENS;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(router_logits) || !aligned16(out) || !aligned16(workspace))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < plan->ws_bytes) return MOE_ERR_SIZE;
  moe_routing_out r;
  std::memset(&r, 0, sizeof(r));
  if (routing) {
    r = *routing;
    const void* p4[] = {r.topk_ids, r.topk_weights, r.expert_counts, r.expert_offsets, r.perm, r.act_global};
    for (const void* q : p4)
      if (q && !aligned4(q)) return MOE_ERR_ALIGN;
    if ((r.act_packed && !aligned16(r.act_packed)) || (r.act_scales && !aligned16(r.act_scales)))
      return MOE_ERR_ALIGN;
  }
  if (T == 0) return MOE_OK;

  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  const uint8_t* pk = (const uint8_t*)packed;
  const int H = d.hidden, I = d.inter, E = d.num_experts, k = d.top_k, S = d.num_shared;
  const bool mx8 = d.act_format == MOE_ACT_MXFP8;           // x and h MXFP8, scaled MFMA (W4A8)
  const bool f8 = d.act_format == MOE_ACT_FP8_ROW;          // x and h FP8 with a per-row scale (W4A8, NVFP4)
  const bool fp4 = d.act_format != MOE_ACT_BF16 && !mx8 && !f8;   // x row-quantised to NVFP4
  const bool fp4h = d.act_format == MOE_ACT_NVFP4_ALL;      // h too, before the down GEMM
  hipError_t e;

  uint8_t* xq = ((fp4 || mx8) && r.act_packed) ? r.act_packed : ws + plan->ws_xq;
  uint8_t* xs = ((fp4 || mx8) && r.act_scales) ? r.act_scales : ws + plan->ws_xs;
  float* xg = ((fp4 || f8) && r.act_global) ? r.act_global : (float*)(ws + plan->ws_xg);
  uint16_t* x16 = (uint16_t*)(ws + plan->ws_x16);
  const bool decode = use_decode(T, k, E);
  // Activation preparation: NVFP4 row quantisation, or the exact power-of-two rescale of bf16
  // rows into fp16 (its 1-op dequant route) for every batch: it rides on the routing launch,
  // and feeding small decode batches' bf16 rows to a bf16 MFMA instead (twice the dequant
  // work) measured slower (Qwen3 decode step at T = 1, 8, 32, 64: 0.2362 vs 0.2401 ms).
  // Prefill batches with NVFP4 x take its exact fp16 decode (written by the quantiser beside
  // the codes, the row's global scale in the epilogue) through the fp16 GEMM, whose token
  // tiles arrive by LDS DMA; decode batches read the codes.
  // FP8 x: its exact fp16 decode through the fp16 GEMM, the row's scale in the epilogue.
  const GemmMode gu_mode = mx8 ? GEMM_GATEUP_MX8
                          : f8 ? GEMM_GATEUP_F16
                          : fp4 ? (decode ? GEMM_GATEUP_FP4 : GEMM_GATEUP_F16)
                                : GEMM_GATEUP_F16;
  // the activation preparation runs in extra workgroups of the routing stage's first launch
  // (one wave per row); the QUANT stage times the preparation of h between the GEMMs

  // prefill batches averaging at most 64 rows per expert: experts with few rows (skewed
  // routing) go to the decode GEMM through a second tile list, in the same launch as the first
  const bool split = !decode && (long)T * k <= 64L * E;
  // MX8 prefill batches whose experts average under 80 rows, and the skewed batches, use
  // 64-row tiles (less of the last tile of each expert left empty, more workgroups)
  const int M = decode ? DECODE_TILE_ROWS
                       : ((mx8 && (long)T * k < 80L * E) || (split && !mx8)) ? SPLIT_TILE_ROWS : PREFILL_TILE_ROWS;
  const GemmRegime regime = decode ? REGIME_DECODE_KSPLIT : REGIME_PREFILL;
  RouteArgs ra;
  ra.logits = router_logits;
  ra.T = T;
  ra.E = E;
  ra.k = k;
  ra.score = d.score_fn;
  ra.ids = (int32_t*)(ws + plan->ws_ids);
  ra.w = (float*)(ws + plan->ws_w);
  ra.ids_user = r.topk_ids;
  ra.w_user = r.topk_weights;
  ra.general = general_router(d) ? 1 : 0;
  ra.bias = d.use_bias ? (const float*)(pk + plan->off_bias) : nullptr;
  ra.n_group = d.n_group;
  ra.topk_group = d.topk_group;
  ra.renorm = d.renormalize;
  ra.scaling = d.routed_scaling;
  ra.side = mx8                           ? SIDE_MXFP8
            : f8                            ? SIDE_FP8
            : fp4                           ? SIDE_NVFP4
                                            : SIDE_F16;
  ra.side_x = x;
  ra.side_K = H;
  ra.side_q = f8 ? r.act_packed : xq;      // FP8 codes only when the caller asks for them
  ra.side_s = xs;
  ra.side_f = xg;
  ra.side_h = (fp4 && decode) ? nullptr : x16;   // NVFP4 x of prefill batches: also its fp16 decode
  PlanArgs pa;
  pa.ids = ra.ids;
  pa.T = T;
  pa.E = E;
  pa.k = k;
  pa.G = plan->G;
  pa.tile_rows = M;
  pa.cold_rows = split ? COLD_ROWS : 0;
  pa.counts = (int32_t*)(ws + plan->ws_counts);
  pa.offsets = (int32_t*)(ws + plan->ws_offsets);
  pa.perm = (int32_t*)(ws + plan->ws_perm);
  pa.inv = (int32_t*)(ws + plan->ws_inv);
  pa.tok = (int32_t*)(ws + plan->ws_tok);
  pa.tile_group = (int32_t*)(ws + plan->ws_tgrp);
  pa.tile_row0 = (int32_t*)(ws + plan->ws_trow);
  pa.tile_count = (int32_t*)(ws + plan->ws_tcnt);
  pa.hmin = (int32_t*)(ws + plan->ws_hmin);
  pa.counts_user = r.expert_counts;
  pa.offsets_user = r.expert_offsets;
  pa.perm_user = r.perm;
  if ((e = mark(ev, 2 * MOE_STAGE_ROUTE, s)) != hipSuccess) return (int)e;
  e = launch_route_plan(ra, pa, (int32_t*)(ws + plan->ws_plan), s);
  if (e != hipSuccess) return (int)e;
  if ((e = mark(ev, 2 * MOE_STAGE_ROUTE + 1, s)) != hipSuccess) return (int)e;

  const int max_tiles = tile_bound(T, k, E, S, M);
  const int est_tiles = std::min(T * k, E) + S * ((T + M - 1) / M);   // exact when no expert overflows a tile
  GemmArgs g1;
  std::memset(&g1, 0, sizeof(g1));
  g1.wfp4 = pk + plan->off_w1f;
  g1.wsc = pk + plan->off_w1s;
  g1.wgs = (const float*)(pk + plan->off_w1g);
  g1.N = 2 * I;
  g1.K = H;
  g1.tok = pa.tok;
  g1.x = x16;
  g1.xq = xq;
  g1.xs = xs;
  g1.xg = xg;
  g1.tile_group = pa.tile_group;
  g1.tile_row0 = pa.tile_row0;
  g1.tile_count = pa.tile_count;
  g1.offsets = pa.offsets;
  g1.tile_rows = M;
  g1.out = (uint16_t*)(ws + plan->ws_h);
  g1.hexp = (int8_t*)(ws + plan->ws_hexp);
  g1.hmin = decode ? nullptr : pa.hmin;
  g1.h_natural = decode ? 0 : 1;                 // prefill: plain column order, rescaled before down
  // MXFP8 h: quantised in the decode GEMM's epilogue (a workgroup holds whole 32-column
  // blocks), or written as fp32 by the prefill GEMM and quantised by a row kernel
  g1.hf = fp4h || f8 || (mx8 && !decode) ? (float*)(ws + plan->ws_hf) : nullptr;
  if (mx8 && decode) {
    g1.hq8 = ws + plan->ws_hq;
    g1.hs8 = ws + plan->ws_hs;
  }
  g1.clamp_groups = d.swiglu_clamp ? E : 0;      // routed experts only
  g1.swiglu_limit = d.swiglu_limit;
  // second-list (cold) launches: the decode GEMM over list 2
  const int cold_tiles = split ? tile_bound(T, k, E, S, DECODE_TILE_ROWS) : 0;
  auto second = [&](GemmArgs g) {
    g.tile_first = pa.tile_count;
    g.tile_count = pa.tile_count + 1;
    g.h_natural = 0;                             // the decode GEMMs keep h16 permuted
    return g;
  };
  // the two lists of a skewed batch run in one launch where the split kernel takes the shapes
  // (the fp16 modes), else one after the other
  auto both_lists = [&](GemmMode hot_mode, GemmMode cold_mode, const GemmArgs& g, const LaunchEvents& le) {
    if (!mx8) {
      const hipError_t r = launch_gemm_split(hot_mode, cold_mode, max_tiles, cold_tiles, g, second(g), s, le);
      if (r != hipErrorNotSupported) return r;
    }
    hipError_t r = launch_gemm(hot_mode, regime, max_tiles, est_tiles, g, s, LaunchEvents{le.start, nullptr});
    if (r == hipSuccess)
      r = launch_gemm(cold_mode, REGIME_DECODE_KSPLIT, cold_tiles, cold_tiles, second(g), s,
                      LaunchEvents{nullptr, le.stop});
    return r;
  };
  {
    const LaunchEvents le = stage_events(ev, MOE_STAGE_GATE_UP);
    e = split ? both_lists(gu_mode, gu_mode, g1, le) : launch_gemm(gu_mode, regime, max_tiles, est_tiles, g1, s, le);
  }
  if (e != hipSuccess) return (int)e;

  GemmArgs g2 = g1;
  g2.wfp4 = pk + plan->off_w2f;
  g2.wsc = pk + plan->off_w2s;
  g2.wgs = (const float*)(pk + plan->off_w2g);
  g2.N = H;
  g2.K = I;
  g2.x = g1.out;
  g2.out = nullptr;
  g2.hf = nullptr;
  g2.hq8 = nullptr;
  g2.hs8 = nullptr;
  g2.yout = (uint16_t*)(ws + plan->ws_y);
  g2.yexp = (int8_t*)(ws + plan->ws_yexp);
  // NVFP4 h: decode batches read the codes; prefill batches take the quantiser's exact fp16
  // decode of every h row (the row's global scale in the epilogue) through the fp16 GEMM, and
  // their cold list (decode GEMM) reads the codes
  const GemmMode dn_mode = mx8 ? GEMM_DOWN_MX8 : (fp4h && decode) ? GEMM_DOWN_FP4 : GEMM_DOWN;
  const GemmMode dn_cold = fp4h ? GEMM_DOWN_FP4 : dn_mode;
  {
    // the QUANT stage brackets the preparation of h (none in the decode regime with 16-bit h)
    if ((e = mark(ev, 2 * MOE_STAGE_QUANT, s)) != hipSuccess) return (int)e;
    if (fp4h) {   // every h row (T*k routed, T per shared expert) quantised with its own global scale
      g2.xq = ws + plan->ws_hq;
      g2.xs = ws + plan->ws_hs;
      g2.xg = (const float*)(ws + plan->ws_hg);
      e = launch_quant_rows_f32(g1.hf, T * k + S * T, I, ws + plan->ws_hq, ws + plan->ws_hs,
                                (float*)(ws + plan->ws_hg), s, decode ? nullptr : (uint16_t*)(ws + plan->ws_h));
      if (!decode) {   // the fp16 decode, scaled per row by hg in the epilogue
        g2.x = (const uint16_t*)(ws + plan->ws_h);
        g2.hmin = nullptr;
      }
    } else if (f8) {   // every h row FP8-quantised with its own scale; the GEMMs take its fp16 decode
      e = launch_fp8_rows_f32(g1.hf, T * k + S * T, I, nullptr, (float*)(ws + plan->ws_hg),
                              (uint16_t*)(ws + plan->ws_h), s);
      g2.x = (const uint16_t*)(ws + plan->ws_h);
      g2.xg = (const float*)(ws + plan->ws_hg);
      g2.hexp = nullptr;
      g2.hmin = nullptr;
    } else if (mx8) {
      g2.xq = ws + plan->ws_hq;
      g2.xs = ws + plan->ws_hs;
      if (!decode) {   // every h row MXFP8-quantised (E8M0 per 32 columns)
        e = launch_mxfp8_rows_f32(g1.hf, T * k + S * T, I, ws + plan->ws_hq, ws + plan->ws_hs, s);
      }
    } else if (!decode) {   // h16 rows of the first tile list to their row's common exponent
      e = launch_h_rescale(g1.out, g1.hexp, pa.hmin, pa.tile_group, pa.tile_row0, pa.tile_count, pa.offsets,
                           max_tiles, M, I, s);
    }
    if (e != hipSuccess) return (int)e;
    if ((e = mark(ev, 2 * MOE_STAGE_QUANT + 1, s)) != hipSuccess) return (int)e;
    const LaunchEvents le = stage_events(ev, MOE_STAGE_DOWN);
    e = split ? both_lists(dn_mode, dn_cold, g2, le) : launch_gemm(dn_mode, regime, max_tiles, est_tiles, g2, s, le);
  }
  if (e != hipSuccess) return (int)e;

  CombineArgs c;
  c.y = (const uint16_t*)(ws + plan->ws_y);
  c.yexp = (const int8_t*)(ws + plan->ws_yexp);
  c.w = ra.w;
  c.inv = pa.inv;
  c.T = T;
  c.H = H;
  c.k = k;
  c.S = S;
  c.out = out;
  return (int)launch_combine(c, s, stage_events(ev, MOE_STAGE_COMBINE));
}

int moe_quantize_nvfp4_rows(const uint16_t* x, int32_t rows, int32_t K, uint8_t* packed, uint8_t* scales,
                            float* row_global, void* stream) {
  if (!x || !packed || !scales || !row_global) return MOE_ERR_NULL;
  if (rows < 0 || K < 16 || K > MAX_HIDDEN || K % 16) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(packed) || !aligned4(row_global)) return MOE_ERR_ALIGN;
  return (int)launch_quant_rows_bf16(x, rows, K, packed, scales, row_global, (hipStream_t)stream);
}

int moe_quantize_fp8_rows(const uint16_t* x, int32_t rows, int32_t K, uint8_t* codes, float* row_scale,
                          void* stream) {
  if (!x || !codes || !row_scale) return MOE_ERR_NULL;
  if (rows < 0 || K < 16 || K > MAX_HIDDEN || K % 16) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(row_scale)) return MOE_ERR_ALIGN;
  return (int)launch_fp8_rows_bf16(x, rows, K, codes, row_scale, nullptr, (hipStream_t)stream);
}

int moe_quantize_nvfp4_weights(const float* w, int32_t groups, int32_t rows_per_group, int32_t K, uint8_t* packed,
                               uint8_t* scales, float* group_global, void* stream) {
  if (!w || !packed || !scales || !group_global) return MOE_ERR_NULL;
  if (groups < 0 || rows_per_group < 1 || K < 16 || K > MAX_HIDDEN || K % 16) return MOE_ERR_SHAPE;
  if ((long)groups * rows_per_group > (1L << 30)) return MOE_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed) || !aligned4(group_global)) return MOE_ERR_ALIGN;
  return (int)launch_quant_groups_f32(w, groups, rows_per_group, K, packed, scales, group_global,
                                      (hipStream_t)stream);
}

int moe_validate_weights_host(const moe_desc* in, const moe_nvfp4_tensor* t, int32_t which) {
  moe_desc dd;
  const int rc = load_desc(in, &dd);
  if (rc) return rc;
  const moe_desc* desc = &dd;
  const bool mx = desc->weight_format == MOE_WEIGHTS_MXFP4;
  if (!t || !t->packed || !t->scales || (!mx && !t->global_scale)) return MOE_ERR_NULL;
  if (which < 0 || which > 3) return MOE_ERR_ENUM;
  const int G = which >= 2 ? desc->num_shared : desc->num_experts;
  const bool up = (which & 1) == 0;
  const size_t N = up ? 2 * (size_t)desc->inter : (size_t)desc->hidden;
  const size_t K = up ? (size_t)desc->hidden : (size_t)desc->inter;
  if (mx) {
    // E8M0: no NaN byte, and (when re-expressed as NVFP4 for 16-bit MFMAs, i.e. without
    // MXFP8 activations) every block within 17 binades of its expert's largest scale
    const size_t per = N * (K / 32);
    for (int g = 0; g < G; ++g) {
      const uint8_t* sc = t->scales + (size_t)g * per;
      int m = 0;
      for (size_t i = 0; i < per; ++i) {
        if (sc[i] == 0xFFu) return MOE_ERR_WEIGHT;
        m = std::max(m, (int)sc[i]);
      }
      if (desc->act_format != MOE_ACT_MXFP8)
        for (size_t i = 0; i < per; ++i)
          if ((int)sc[i] < m - MX_SCALE_SPAN) return MOE_ERR_WEIGHT;
    }
    return MOE_OK;
  }
  const size_t nsc = (size_t)G * N * (K / 16);
  for (size_t i = 0; i < nsc; ++i) {
    const uint8_t b = t->scales[i];
    if ((b & 0x7Fu) == 0x7Fu || (b & 0x80u)) return MOE_ERR_WEIGHT;
  }
  for (int g = 0; g < G; ++g) {
    const float v = t->global_scale[g];
    if (!std::isfinite(v) || v < 0.0f) return MOE_ERR_WEIGHT;
  }
  return MOE_OK;
}

}  // extern "C"

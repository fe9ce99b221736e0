// Internal launcher interface between api.cpp (host validation, planning) and the
// HIP kernels. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvmoe {

constexpr int DECODE_TILE_ROWS = 16;
constexpr int PREFILL_TILE_ROWS = 96;

struct RouteArgs {
  const float* logits;   // [T][E]
  int T, E, k, score;
  int32_t* ids;          // [T][k] workspace
  float* w;              // [T][k] workspace
  int32_t* ids_user;     // optional copies for the caller
  float* w_user;
  // generalised router (general != 0): FP64 scores, binary32 keys with an optional
  // selection-only bias, the group step, weights optionally renormalised and scaled
  int general;
  const float* bias;     // [E] or nullptr
  int n_group, topk_group, renorm;
  float scaling;
  // optional side job on the bf16 activation rows side_x [T][side_K], run by extra
  // workgroups of the first routing launch (one launch fewer for small batches):
  // SIDE_MXFP8: codes side_q [T][side_K] and E8M0 scales side_s [T][side_K/32];
  // SIDE_NVFP4: codes side_q [T][side_K/2], E4M3 scales side_s [T][side_K/16], global scales side_f [T]
  //   (and, with side_h set, the rows' exact fp16 decode without the global scale);
  // SIDE_F16: fp16 rows side_h [T][side_K] and their factors side_f [T];
  // SIDE_FP8: per-row FP8: scales side_f [T], fp16 decode side_h [T][side_K] and, when
  //   side_q is set, the E4M3 codes side_q [T][side_K]
  int side;
  const uint16_t* side_x;
  int side_K;
  uint8_t* side_q;
  uint8_t* side_s;
  float* side_f;
  uint16_t* side_h;
};
enum RouteSide { SIDE_NONE = 0, SIDE_MXFP8 = 1, SIDE_F16 = 2, SIDE_NVFP4 = 3, SIDE_FP8 = 4 };

struct PlanArgs {
  const int32_t* ids;    // [T][k]
  int T, E, k, G;        // G = E + shared groups
  int tile_rows;         // M of the GEMM tiles
  int cold_rows;         // > 0: groups with 1..cold_rows rows get one DECODE_TILE_ROWS tile in a
                         // second list (for the decode GEMM) after the first list's tiles
  int32_t* counts;       // [G]
  int32_t* offsets;      // [G+1]
  int32_t* perm;         // [T*k]
  int32_t* inv;          // [T*k]
  int32_t* tok;          // [T*k + S*T] token of each row
  int32_t* tile_group;   // [max tiles]
  int32_t* tile_row0;    // [max tiles]
  int32_t* tile_count;   // [2]: tiles of list 1, of list 2
  int32_t* hmin;         // [T*k + S*T] per-row minimum h exponent, set to H_EXP_INIT here
  int32_t* counts_user;  // optional [E]
  int32_t* offsets_user; // optional [E+1]
  int32_t* perm_user;    // optional [T*k]
};

// scratch: plan_scratch_ints(T, k, E) ints of workspace (large-T path only)
hipError_t launch_route_plan(const RouteArgs& r, const PlanArgs& p, int32_t* scratch, hipStream_t s);
size_t plan_scratch_ints(int T, int k, int E);
bool plan_small_ok(int T, int k);

// Activation / weight quantiser.
// With x16 != nullptr also the rows' exact fp16 decode without the global scale,
// E2M1 x E4M3 per element ([rows][K], plain column order).
hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int K, uint8_t* packed, uint8_t* scales,
                                  float* gs, hipStream_t s, uint16_t* x16 = nullptr);
// MXFP8 rows (codes [rows][K], E8M0 scales [rows][K/32]) from fp32 rows (h before the W4A8 down
// GEMM); the activation rows are converted by the routing launch (RouteArgs side jobs).
hipError_t launch_mxfp8_rows_f32(const float* x, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);
// FP8 rows with one scale per row (scale = max|x| / 448); codes [rows][K] and the fp16 decode
// x16 [rows][K] (without the scale) are each written when non-null
hipError_t launch_fp8_rows_bf16(const uint16_t* x, int rows, int K, uint8_t* codes, float* scale, uint16_t* x16,
                               hipStream_t s);
hipError_t launch_fp8_rows_f32(const float* x, int rows, int K, uint8_t* codes, float* scale, uint16_t* x16,
                               hipStream_t s);
// fp32 rows (h before the NVFP4 down GEMM), each with its own global scale.
hipError_t launch_quant_rows_f32(const float* x, int rows, int K, uint8_t* packed, uint8_t* scales, float* gs,
                                 hipStream_t s, uint16_t* x16 = nullptr);
hipError_t launch_quant_groups_f32(const float* x, int groups, int rows_per_group, int K, uint8_t* packed,
                                   uint8_t* scales, float* gs, hipStream_t s);

// Weight re-layout.
// MXFP4 packing: the E8M0 scale bytes of an expert lie within MX_SCALE_SPAN of its
// largest one m, so 2^(byte - m + 8) is an E4M3 value (2^-9 .. 2^8).
constexpr int MX_SCALE_SPAN = 17;

struct PackArgs {
  const uint8_t* packed;   // boundary layout [G][N][K/2]
  const uint8_t* scales;   // [G][N][K/16] E4M3 (NVFP4) or [G][N][K/32] E8M0 (MXFP4)
  const float* gs;         // [G] (NVFP4)
  int G, N, K;
  int gate_up;             // 1: interleave gate/up 16-row tiles
  int mx;                  // 1: MXFP4 input, re-expressed as E4M3 blocks + per-expert gs, or
                           // 2: MXFP4 kept native (raw E8M0 scale bytes for the scaled MFMA, gs 1)
  uint8_t* fp4_out;        // [G][N/16][KC][64][16]
  uint8_t* sc_out;         // [G][N/16][KSG][64][16]
  float* gs_out;           // [G]
};
hipError_t launch_pack(const PackArgs& a, hipStream_t s);

// Grouped GEMMs.
// gate_up modes: F16 = activations pre-scaled into fp16 (x16) and fp16 MFMA; BF16 = the
// caller's bf16 rows read directly, bf16 MFMA; FP4 = NVFP4 activation rows. down modes:
// DOWN = h16 rows; DOWN_FP4 = h row-quantised to NVFP4 (xq/xs/xg indexed by row).
// MX8 modes (MXFP4 weights with MXFP8 activations: xq = E4M3 codes [rows][K], xs = E8M0
// scales [rows][K/32]; gate_up gathers token rows, down reads its own rows) run the scaled
// MFMA on the raw codes, no dequantisation.
enum GemmMode {
  GEMM_GATEUP_F16 = 0, GEMM_GATEUP_FP4 = 1, GEMM_DOWN = 2, GEMM_DOWN_FP4 = 4, GEMM_GATEUP_MX8 = 5,
  GEMM_DOWN_MX8 = 6
};

struct GemmArgs {
  // weights (packed layout of one projection, G groups)
  const uint8_t* wfp4;
  const uint8_t* wsc;
  const float* wgs;        // [G]
  int N, K;                // projection rows, columns
  // token rows
  const int32_t* tok;      // row -> token (gather modes)
  const uint16_t* x;       // activations [T][K]: fp16 rescaled (GATEUP_F16); h16 [rows][K] (DOWN)
  const uint8_t* xq;       // [T][K/2]  (GATEUP_FP4; DOWN_FP4: [rows][K/2])
  const uint8_t* xs;       // [T][K/16] (DOWN_FP4: [rows][K/16])
  const float* xg;         // [T] per-row activation factor applied in the epilogue (DOWN_FP4: [rows])
  // tile list
  const int32_t* tile_group;
  const int32_t* tile_row0;
  const int32_t* tile_count;
  const int32_t* tile_first; // nullptr, or the index of the launch's first tile (list 2: &tile_count[0])
  const int32_t* offsets;  // [G+1] row ranges of the groups
  int tile_rows;           // the plan's tile height (prefill: PREFILL_TILE_ROWS, or 64 for skewed batches)
  // h = silu(g) u between the GEMMs, as h16 [rows][I] fp16 (columns permuted inside each
  // 128-column chunk, see h_pos) with, per row and 16-column block b, an exponent
  // hexp[row][b] such that h16 = fp16(h * 2^hexp) has the block's largest |h| in
  // [2^14, 2^15). gate_up writes both; down takes the row's smallest exponent P and
  // multiplies each block by 2^(P - hexp) so that a whole row shares the scale 2^P, undone
  // in its epilogue. With hmin set (large batches), gate_up also folds each block exponent
  // into hmin[row] (atomicMin) and down reads P there; without it (small batches, where a
  // few rows would take every block's atomic) down takes the minimum over the row's hexp.
  // The prefill GEMMs keep h16 in plain column order instead (h_natural = 1): a rescale pass
  // between the GEMMs (launch_h_rescale) brings every block of a row to the row's exponent
  // P = hmin[row] in place, and the prefill down GEMM streams those rows by LDS DMA.
  // DOWN with hexp and hmin both null: h16 rows in plain column order, each with one factor
  // xg[row] applied in the epilogue (the fp16 decode of h rows quantised with a per-row scale).
  uint16_t* out;           // gate_up: h16
  int8_t* hexp;            // [rows][I/16]
  int32_t* hmin;           // [rows] or nullptr
  int h_natural;           // gate_up: 1 = h16 in plain column order (prefill), 0 = permuted (decode)
  float* hf;               // gate_up: when set, h as fp32 [rows][I] in column order instead (the
                           // input of the row quantiser before DOWN_FP4); out/hexp/hmin unused
  uint8_t* hq8;            // GATEUP_MX8 decode kernel: when set, h MXFP8-quantised in the epilogue,
  uint8_t* hs8;            // codes [rows][I] and E8M0 scales [rows][I/32] (32-column blocks are
                           // local to a workgroup of 4 tiles); hf unused
  // down: y as fp16 [rows][N] with one exponent per row and 16-column block, the
  // block's largest |y| scaled into [2^14, 2^15): y = y16 * 2^-yexp
  uint16_t* yout;
  int8_t* yexp;            // [rows][N/16]
  // clamped SwiGLU for groups g < clamp_groups (0: none): silu(min(g, L)) * clamp(u, -L, L)
  int clamp_groups;
  float swiglu_limit;
};
// Kernel families: decode (<= 16 rows per tile, K split across the waves of a workgroup,
// direct token loads) and prefill (N split across the waves, 64- or 96-row token tiles in LDS).
enum GemmRegime { REGIME_DECODE_KSPLIT = 0, REGIME_PREFILL = 2 };
constexpr int H_EXP_INIT = 127;   // above any block exponent (start of a minimum)
constexpr int H_EXP_MAX = 120;    // block exponents are clamped to [-H_EXP_MAX, H_EXP_MAX]

// Optional timing of a single-kernel stage: when set, the kernel is launched with
// hipExtLaunchKernelGGL, which stamps the events at the kernel's own start and end (no
// enqueue or dispatch gap inside the measured interval).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// est_tiles: expected number of valid tile slots (sizes the decode split); max_tiles: grid bound.
hipError_t launch_gemm(GemmMode mode, GemmRegime regime, int max_tiles, int est_tiles, const GemmArgs& a,
                       hipStream_t s, const LaunchEvents& ev = LaunchEvents());

// Skewed prefill batches: the first tile list with the prefill GEMM (hot_mode: GATEUP_F16 or
// DOWN) and the second with the decode GEMM (cold_mode: GATEUP_F16, DOWN or DOWN_FP4) in one
// launch. hipErrorNotSupported (nothing launched) for shapes it does not take: hot N not a
// multiple of 256, tile rows other than 64; the caller then launches the lists apart.
hipError_t launch_gemm_split(GemmMode hot_mode, GemmMode cold_mode, int max_tiles, int cold_tiles,
                             const GemmArgs& hot, const GemmArgs& cold, hipStream_t s,
                             const LaunchEvents& ev = LaunchEvents());

struct CombineArgs {
  const uint16_t* y;       // fp16 [rows_total][H] expert outputs, scaled per 16-column block
  const int8_t* yexp;      // [rows_total][H/16]: y = y16 * 2^-yexp
  const float* w;          // [T][k]
  const int32_t* inv;      // [T*k]
  int T, H, k, S;
  uint16_t* out;           // bf16 [T][H]
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s, const LaunchEvents& ev = LaunchEvents());

// h16 rows of the first tile list's groups (plain column order, one exponent per 16 columns)
// brought in place to each row's common exponent P = hmin[row]: h16 *= 2^(P - hexp), exactly
// (a power of two; values that fall below fp16's normal range lose bits, as in the GEMM's own
// conversion of the decode path). I = columns per row.
hipError_t launch_h_rescale(uint16_t* h, const int8_t* hexp, const int32_t* hmin, const int32_t* tile_group,
                            const int32_t* tile_row0, const int32_t* tile_count, const int32_t* offsets,
                            int max_tiles, int tile_rows, int I, hipStream_t s);


}  // namespace nvmoe

// NVFP4 quantiser: per-group FP32 global scale, per-16 E4M3 block scales, E2M1 codes.
//
// Global scale gs = max|x| / (6 * 448) ([megamoe] archived CORRECTNESS_BACKLOG §7,
// "Runtime Activation Global Scale": computed at run time from the activation so
// that no E4M3 block scale overflows). The blocks follow the NVFP4 format of
// [megamoe] README "NVFP4 throughout" (16-element microblocks, E4M3 scales, E2M1
// values). Every step is one binary32 operation rounded to nearest even (no sums,
// so FP contraction cannot apply; division is correctly rounded), so the bytes
// are a pure function of the input bits:
//   s_b  = gs == 0 ? 0 : E4M3_rne_sat(a_b / (6 * gs))
//   d_b  = E4M3(s_b) * gs
//   code = signbit(x) << 3 | (d_b == 0 ? 0 : E2M1_rne_sat(|x| / d_b))
// One wave quantises one row (activations) or the rows of a group after a
// reduction kernel has produced the group's global scale (weights). The per-wave
// row quantisers sit in rowq_dev.hpp, shared with the routing kernels, which run
// them for the activation rows of decode batches.
#include "common.hpp"
#include "kernels.hpp"
#include "rowq_dev.hpp"

namespace nvmoe {

// One wave per row (nvfp4_row_wave): bf16 activation rows, or the fp32 h rows of the NVFP4
// down GEMM; with x16 also the rows' exact fp16 decode without the global scale (the
// operands of the prefill GEMMs).
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ x, int rows, int K,
                                                         uint8_t* __restrict__ packed,
                                                         uint8_t* __restrict__ scales, float* __restrict__ gs,
                                                         uint16_t* __restrict__ x16) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  nvfp4_row_wave(x + (size_t)r * K, K, packed + (size_t)r * (K / 2), scales + (size_t)r * (K / 16), gs + r,
                 x16 ? x16 + (size_t)r * K : nullptr);
}

// MXFP8 rows: one wave per row (mxfp8_row_wave), 4 rows per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void mxfp8_rows_kernel(const T* __restrict__ x, int rows, int K,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  mxfp8_row_wave(x + (size_t)r * K, K, codes + (size_t)r * K, scales + (size_t)r * (K / 32), threadIdx.x & (WAVE - 1));
}

// FP8 rows with a per-row scale: one wave per row (fp8_row_wave), 4 rows per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void fp8_rows_kernel(const T* __restrict__ x, int rows, int K,
                                                       uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                       uint16_t* __restrict__ x16) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  fp8_row_wave(x + (size_t)r * K, K, codes ? codes + (size_t)r * K : nullptr, scale + r,
               x16 ? x16 + (size_t)r * K : nullptr, threadIdx.x & (WAVE - 1));
}

// Group maxima: one 1024-thread workgroup per group, fixed reduction tree.
__global__ __launch_bounds__(1024) void group_gs_f32_kernel(const float* __restrict__ x, int rows_per_group, int K,
                                                            float* __restrict__ gs) {
  __shared__ float part[16];
  const float* base = x + (size_t)blockIdx.x * rows_per_group * K;
  const size_t n = (size_t)rows_per_group * K;
  float m = 0.0f;
  for (size_t i = (size_t)threadIdx.x * 4; i < n; i += (size_t)blockDim.x * 4) {
    const f32x4 a = *(const f32x4*)(base + i);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
  }
#pragma unroll
  for (int off = WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
  if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float A = 0.0f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) A = fmaxf(A, part[i]);
    gs[blockIdx.x] = A / 2688.0f;
  }
}

__global__ __launch_bounds__(256) void quant_rows_f32_kernel(const float* __restrict__ x, int rows, int K,
                                                             int rows_per_group, const float* __restrict__ gs,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ scales) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  wave_quant_row(x + (size_t)r * K, K, gs[r / rows_per_group], packed + (size_t)r * (K / 2),
                 scales + (size_t)r * (K / 16), (uint16_t*)nullptr);
}

hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int K, uint8_t* packed, uint8_t* scales,
                                  float* gs, hipStream_t s, uint16_t* x16) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel<uint16_t>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, packed,
                     scales, gs, x16);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f32(const float* x, int rows, int K, uint8_t* packed, uint8_t* scales, float* gs,
                                 hipStream_t s, uint16_t* x16) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, packed, scales,
                     gs, x16);
  return hipGetLastError();
}

hipError_t launch_mxfp8_rows_f32(const float* x, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_rows_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_rows_bf16(const uint16_t* x, int rows, int K, uint8_t* codes, float* scale, uint16_t* x16,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_rows_kernel<uint16_t>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, codes, scale, x16);
  return hipGetLastError();
}

hipError_t launch_fp8_rows_f32(const float* x, int rows, int K, uint8_t* codes, float* scale, uint16_t* x16,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_rows_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, codes, scale, x16);
  return hipGetLastError();
}

hipError_t launch_quant_groups_f32(const float* x, int groups, int rows_per_group, int K, uint8_t* packed,
                                   uint8_t* scales, float* gs, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(group_gs_f32_kernel, dim3(groups), dim3(1024), 0, s, x, rows_per_group, K, gs);
  const int rows = groups * rows_per_group;
  hipLaunchKernelGGL(quant_rows_f32_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, rows, K, rows_per_group,
                     gs, packed, scales);
  return hipGetLastError();
}

}  // namespace nvmoe

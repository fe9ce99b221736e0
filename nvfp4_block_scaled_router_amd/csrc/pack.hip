// Weight re-layout (moe_pack_weights): a pure byte permutation of the boundary
// operand pair (packed [N][K/2], scales [N][K/16]) into the tile order the GEMM
// waves read, plus a copy of the global scales. ([vllm.cpp] capability table, GGUF
// row: repacked at load as a pure byte permutation; [megamoe] CUDA_GRAPH_SYNC_INVENTORY:
// scales swizzled once at finalize into the layout the GEMM consumes.)
//
// fp4 tile (group g, 16-row tile q, chunk kc) = 64 lanes x 16 bytes, lane l holding
// row (l % 16) of the tile and bytes 16*(l/16) .. +15 of the chunk's 64 bytes, so one
// wave-wide 16-byte load reads 1 KiB of contiguous memory.
// scale tile (g, q, scale group sg) = 64 lanes x 16 bytes, lane l holding for the 8
// chunks kc = 8*sg + c the two block scales (8*kc + 2*(l/16), +1) of row (l % 16).
// For gate_up, tile q maps to boundary rows 16*(q/2) + r (q even: gate) or
// I + 16*(q/2) + r (q odd: up), so gate and up tiles of the same columns alternate.
#include "common.hpp"
#include "kernels.hpp"

namespace nvmoe {

__device__ __forceinline__ int boundary_row(int q, int r, int N, int gate_up) {
  if (!gate_up) return 16 * q + r;
  return (q & 1) ? (N / 2 + 16 * (q >> 1) + r) : (16 * (q >> 1) + r);
}

__global__ __launch_bounds__(256) void pack_fp4_kernel(PackArgs a) {
  const ProjLayout L = proj_layout(a.N, a.K);
  const size_t units = (size_t)a.G * (a.N / 16) * L.KC * WAVE;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(u % WAVE);
    size_t rest = u / WAVE;
    const int kc = (int)(rest % L.KC);
    rest /= L.KC;
    const int q = (int)(rest % (a.N / 16));
    const int g = (int)(rest / (a.N / 16));
    const int row = boundary_row(q, lane % 16, a.N, a.gate_up);
    const uint8_t* src = a.packed + ((size_t)g * a.N + row) * (a.K / 2) + (size_t)kc * 64 + (lane / 16) * 16;
    *(u32x4*)(a.fp4_out + u * 16) = *(const u32x4*)src;
  }
}

__global__ __launch_bounds__(256) void pack_scales_kernel(PackArgs a) {
  const ProjLayout L = proj_layout(a.N, a.K);
  const size_t units = (size_t)a.G * (a.N / 16) * L.KSG * WAVE;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(u % WAVE);
    size_t rest = u / WAVE;
    const int sg = (int)(rest % L.KSG);
    rest /= L.KSG;
    const int q = (int)(rest % (a.N / 16));
    const int g = (int)(rest / (a.N / 16));
    const int row = boundary_row(q, lane % 16, a.N, a.gate_up);
    const uint8_t* src = a.scales + ((size_t)g * a.N + row) * (a.K / 16);
    uint8_t b[16];
#pragma unroll
    for (int c = 0; c < SCALE_GROUP; ++c) {
      const int kc = sg * SCALE_GROUP + c;
      const bool in = kc < L.KC;
      b[2 * c] = in ? src[kc * 8 + 2 * (lane / 16)] : 0;
      b[2 * c + 1] = in ? src[kc * 8 + 2 * (lane / 16) + 1] : 0;
    }
    u32x4 v;
    v.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
    v.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
    v.z = b[8] | (b[9] << 8) | (b[10] << 16) | ((uint32_t)b[11] << 24);
    v.w = b[12] | (b[13] << 8) | (b[14] << 16) | ((uint32_t)b[15] << 24);
    *(u32x4*)(a.sc_out + u * 16) = v;
  }
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < a.G; g += blockDim.x) a.gs_out[g] = a.gs[g];
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  if (a.G <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_fp4_kernel, dim3(2048), dim3(256), 0, s, a);
  hipLaunchKernelGGL(pack_scales_kernel, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvmoe

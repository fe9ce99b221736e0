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
// MXFP4 input (E2M1 codes with E8M0 scales per 32 k, [vllm.cpp] capability table, MXFP4
// row) is re-expressed exactly in this form: per expert gs = 2^(m - 135), m its largest
// scale byte, and both E4M3 block scales of a 32-column block = 2^(byte - m + 8).
// With MXFP8 activations the MXFP4 weights stay native instead: the scale tile holds the
// raw E8M0 byte of each chunk's block (twice, in the two slots of the chunk) and gs = 1.
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

// E4M3 byte of 2^p: normal for p in [-6, 8] (exponent field p + 7), subnormal m 2^-9 for
// p in [-9, -7]; below that 0 (only for an expert whose global scale is NaN).
__device__ __forceinline__ uint8_t e4m3_pow2(int p) {
  if (p >= -6) return (uint8_t)((p + 7) << 3);
  if (p >= -9) return (uint8_t)(1 << (p + 9));
  return 0;
}

// MXFP4: per expert the largest E8M0 byte m -> gs_out[g] = 2^(m - 135) (one workgroup per
// expert, a max and a min over its N x K/32 scale bytes). An expert the NVFP4 form cannot hold
// exactly -- a byte more than MX_SCALE_SPAN below m, or the NaN byte 0xFF -- gets a NaN global
// scale instead, so that every output that reads it is NaN rather than silently different
// (the host validation rejects such weights before they get here).
__global__ __launch_bounds__(256) void pack_mx_gs_kernel(PackArgs a) {
  __shared__ int red_max[256], red_min[256];
  const int g = blockIdx.x;
  const size_t per = (size_t)a.N * (a.K / 32);
  const uint8_t* sc = a.scales + (size_t)g * per;
  int m = 0, mn = 255;
  for (size_t i = threadIdx.x; i < per; i += blockDim.x) {
    m = max(m, (int)sc[i]);
    mn = min(mn, (int)sc[i]);
  }
  red_max[threadIdx.x] = m;
  red_min[threadIdx.x] = mn;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red_max[threadIdx.x] = max(red_max[threadIdx.x], red_max[threadIdx.x + w]);
      red_min[threadIdx.x] = min(red_min[threadIdx.x], red_min[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const bool exact = red_max[0] != 0xFF && red_max[0] - red_min[0] <= MX_SCALE_SPAN;
    a.gs_out[g] = exact ? ldexpf(1.0f, red_max[0] - 135) : __builtin_nanf("");
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
    uint8_t b[16];
    if (a.mx == 2) {
      // MXFP4 for the scaled MFMA: the raw E8M0 byte of the lane's 32-column block of chunk kc
      const uint8_t* src = a.scales + ((size_t)g * a.N + row) * (a.K / 32);
#pragma unroll
      for (int c = 0; c < SCALE_GROUP; ++c) {
        const int kc = sg * SCALE_GROUP + c;
        const uint8_t e8 = kc < L.KC ? src[kc * 4 + lane / 16] : 0;
        b[2 * c] = e8;
        b[2 * c + 1] = e8;
      }
    } else if (a.mx) {
      // MXFP4: the lane's 32 columns of chunk kc are one E8M0 block, re-expressed as two
      // equal E4M3 block scales 2^(byte - m + 8) against the expert's gs = 2^(m - 135)
      const float gsv = a.gs_out[g];
      const int m = isfinite(gsv) ? ilogbf(gsv) + 135 : 255;   // NaN gs: the expert's outputs are NaN
      const uint8_t* src = a.scales + ((size_t)g * a.N + row) * (a.K / 32);
#pragma unroll
      for (int c = 0; c < SCALE_GROUP; ++c) {
        const int kc = sg * SCALE_GROUP + c;
        const uint8_t e4 = kc < L.KC ? e4m3_pow2((int)src[kc * 4 + lane / 16] - m + 8) : 0;
        b[2 * c] = e4;
        b[2 * c + 1] = e4;
      }
    } else {
      const uint8_t* src = a.scales + ((size_t)g * a.N + row) * (a.K / 16);
#pragma unroll
      for (int c = 0; c < SCALE_GROUP; ++c) {
        const int kc = sg * SCALE_GROUP + c;
        const bool in = kc < L.KC;
        b[2 * c] = in ? src[kc * 8 + 2 * (lane / 16)] : 0;
        b[2 * c + 1] = in ? src[kc * 8 + 2 * (lane / 16) + 1] : 0;
      }
    }
    u32x4 v;
    v.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
    v.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
    v.z = b[8] | (b[9] << 8) | (b[10] << 16) | ((uint32_t)b[11] << 24);
    v.w = b[12] | (b[13] << 8) | (b[14] << 16) | ((uint32_t)b[15] << 24);
    *(u32x4*)(a.sc_out + u * 16) = v;
  }
  if (blockIdx.x == 0 && a.mx != 1)   // NVFP4: the boundary's scales; native MXFP4: 1
    for (int g = threadIdx.x; g < a.G; g += blockDim.x) a.gs_out[g] = a.mx ? 1.0f : a.gs[g];
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  if (a.G <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_fp4_kernel, dim3(2048), dim3(256), 0, s, a);
  if (a.mx == 1) hipLaunchKernelGGL(pack_mx_gs_kernel, dim3(a.G), dim3(256), 0, s, a);
  hipLaunchKernelGGL(pack_scales_kernel, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvmoe

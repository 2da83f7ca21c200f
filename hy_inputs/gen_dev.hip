/*
 * Device build of the seeded input generator (see gen_core.h): fills large
 * tensors directly in HBM with values bit-identical to the host build.
 * Compiled with hipcc --offload-arch=gfx950 -O3 -ffp-contract=off.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "gen_core.h"

__global__ void __launch_bounds__(256) gen_gauss_kernel(uint64_t seed, uint32_t stream, uint64_t start,
                                                        uint64_t count, double std, uint16_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t o = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride)
    out[o] = gen_gauss_bf16_elem(seed, stream, start + o, std);
}

__global__ void __launch_bounds__(256) gen_uniform_kernel(uint64_t seed, uint32_t stream, uint64_t start,
                                                          uint64_t count, double lo, double width,
                                                          uint16_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t o = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride)
    out[o] = gen_uniform_bf16_elem(seed, stream, start + o, lo, width);
}

__global__ void __launch_bounds__(256) gen_u32_kernel(uint64_t seed, uint32_t stream, uint64_t start,
                                                      uint64_t count, uint32_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t o = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; o < count; o += stride)
    out[o] = gen_u32_elem(seed, stream, start + o);
}

static unsigned grid_for(uint64_t count) {
  uint64_t g = (count + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

extern "C" int hy_gen_gauss_bf16_dev(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
                                     double std, void* out, void* hip_stream) {
  if (count == 0) return 0;
  if (!out) return -1;
  hipLaunchKernelGGL(gen_gauss_kernel, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, start, count, std, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int hy_gen_uniform_bf16_dev(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
                                       double lo, double width, void* out, void* hip_stream) {
  if (count == 0) return 0;
  if (!out) return -1;
  hipLaunchKernelGGL(gen_uniform_kernel, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, start, count, lo, width, (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int hy_gen_u32_dev(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
                              void* out, void* hip_stream) {
  if (count == 0) return 0;
  if (!out) return -1;
  hipLaunchKernelGGL(gen_u32_kernel, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)hip_stream,
                     seed, stream, start, count, (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// moe_quant: MXFP8 quantization of activation rows for the routed experts of the FP8
// W8A8 format (the Hy4 preview release ships FP8 weights: app.myzaker.com Hy4 Preview
// news, section "MTP、FP8 与低价 API"; the activation format, OCP Microscaling MXFP8,
// is the reading this library takes). One thread per block of 32 values: it loads the
// block's 64 bytes of bf16, takes the block's largest magnitude, and writes 32 E4M3
// codes and one E8M0 scale byte.
#include "hy_moe.h"
#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads) mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t nblk,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (b >= nblk) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + 32 * b);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src[i];
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], e);
  uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
  dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
  dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
  scales[b] = (uint8_t)(e + 127);
}

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((nblk + kQuantThreads - 1) / kQuantThreads)),
                     dim3(kQuantThreads), 0, s, x, nblk, codes, scales);
  return hipGetLastError();
}

}  // namespace hymoe

extern "C" int hy_moe_mxfp8_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                                     void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return HY_MOE_ERR_INVALID_ARG;
  if (rows == 0) return HY_MOE_OK;
  if (!x || !codes || !scales) return HY_MOE_ERR_INVALID_ARG;
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15)) return HY_MOE_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) / cols) return HY_MOE_ERR_UNSUPPORTED;
  const hipError_t err = hymoe::launch_mx_quantize((const uint16_t*)x, rows, cols, (uint8_t*)codes,
                                                   (uint8_t*)scales, (hipStream_t)stream);
  return err == hipSuccess ? HY_MOE_OK : HY_MOE_ERR_HIP;
}

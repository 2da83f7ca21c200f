// Machine-peak probes: the bf16 and FP8 MFMA rates and the HBM read rate this GPU reaches,
// measured so that a layer's roofline fraction can be read against what the chip
// delivers as well as against its published peaks. Not part of the layer.
//
// MFMA: with random operand bits the chip draws more power per MFMA than with
// constant operands, and under its power cap the clock drops; the probe therefore
// takes its operands from a caller-filled buffer (random data gives the rate a real
// GEMM can reach). HBM: the best of three streaming passes of non-temporal 16-byte loads
// (each wave instruction reads 1 KB in order: the fastest read pattern measured, ~7.0
// TB/s against ~6.3 with plain loads) over a buffer much larger than the last-level cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hy_moe.h"
#include "common.h"

namespace hymoe {
// written only when a probe's result takes a value it practically never takes; with
// external linkage it cannot be dropped, so neither can the work feeding it
__device__ float g_probe_sink;
}  // namespace hymoe

namespace {

using namespace hymoe;

constexpr int kProbeThreads = 256;
constexpr int kProbeOps = 16;  // uint4 operands per lane (8 A, 8 B): 64 KB per workgroup
static_assert(kProbeThreads * kProbeOps * 16 == HY_MOE_PROBE_OPERAND_BYTES, "operand buffer size");

// 16 independent accumulators per wave (enough to keep the MFMA pipe full), 16
// MFMAs per iteration with operands rotated so consecutive MFMAs see different data.
__global__ void __launch_bounds__(kProbeThreads, 1) probe_mfma_kernel(const uint4* __restrict__ ops, int iters) {
  uint4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ops[threadIdx.x * kProbeOps + i];
    b[i] = ops[threadIdx.x * kProbeOps + 8 + i];
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma32x32x16(a[i], b[7 - i], acc[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma32x32x16(a[(i + 3) & 7], b[(i + 5) & 7], acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  if (s == 1.2345f) g_probe_sink = s;  // keeps the MFMAs live
}

// The FP8 probe: 32x32x64 E4M3 MFMAs with E8M0 block scales of 1.0 (the form the W8A8
// GEMM issues), 8 independent accumulators, operands of 8 registers rotated as above.
__global__ void __launch_bounds__(kProbeThreads, 1) probe_mfma_fp8_kernel(const uint4* __restrict__ ops, int iters) {
  i32x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 lo = ops[threadIdx.x * kProbeOps + 2 * i], hi = ops[threadIdx.x * kProbeOps + 2 * i + 1];
    const uint4 lo2 = ops[threadIdx.x * kProbeOps + 8 + 2 * i], hi2 = ops[threadIdx.x * kProbeOps + 9 + 2 * i];
    a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    b[i] = i32x8{(int)lo2.x, (int)lo2.y, (int)lo2.z, (int)lo2.w, (int)hi2.x, (int)hi2.y, (int)hi2.z, (int)hi2.w};
  }
  int one = 127;  // E8M0 1.0, in a register (the scale operands are VGPRs)
  asm volatile("" : "+v"(one));
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = mfma32x32x64_f8(a[i & 3], b[(7 - i) & 3], acc[i], one, one);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc[i] = mfma32x32x64_f8(a[(i + 3) & 3], b[(i + 5) & 3], acc[i], one, one);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  if (s == 1.2345f) g_probe_sink = s;  // keeps the MFMAs live
}

// Block-cyclic streaming: blocks of 8 x 256 vectors (32 KB), workgroup b reading
// blocks b, b + G, ..., 8 vectors per thread in flight; the vectors past the last
// whole block are read by workgroup 0.
constexpr int kReadUnroll = 8;
constexpr int kReadBlock = kReadUnroll * kProbeThreads;  // 16-byte vectors per block

__global__ void __launch_bounds__(kProbeThreads) probe_read_kernel(const uint4* __restrict__ p, size_t n) {
  uint32_t acc = 0;
  const size_t nblocks = n / kReadBlock;
  for (size_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
    const uint4* q = p + b * kReadBlock + threadIdx.x;
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = ldg16_stream(q + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (blockIdx.x == 0)
    for (size_t i = nblocks * kReadBlock + threadIdx.x; i < n; i += kProbeThreads) {
      const uint4 v = p[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  if (acc == 0x9E3779B9u) g_probe_sink = (float)acc;  // keeps the loads live
}

int cus_of_current_device() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// Times one launch made by `launch` on stream s; returns milliseconds or < 0.
template <class F>
float time_launch(hipStream_t s, F&& launch) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.f;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -1.f;
  }
  float ms = -1.f;
  if (hipEventRecord(e0, s) == hipSuccess) {
    launch();
    if (hipGetLastError() == hipSuccess && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      ms = -1.f;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

}  // namespace

extern "C" int hy_moe_probe_mfma_bf16(const void* operands, size_t operand_bytes, float* tflops, void* stream) {
  if (!operands || !tflops || ((uintptr_t)operands & 15) || operand_bytes < HY_MOE_PROBE_OPERAND_BYTES)
    return HY_MOE_ERR_INVALID_ARG;
  const int cus = cus_of_current_device();
  if (cus <= 0) return HY_MOE_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  const int grid = 4 * cus;
  // about 40 ms at 2.5 PFLOP/s: long enough for the clock to settle under load
  const int iters = (int)(4.0e13 / ((double)grid * 4 * 16 * 32768.0));
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)operands, 64);  // warm-up
  if (hipGetLastError() != hipSuccess) return HY_MOE_ERR_HIP;
  const float ms = time_launch(s, [&] {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)operands, iters);
  });
  if (ms <= 0.f) return HY_MOE_ERR_HIP;
  *tflops = (float)((double)grid * 4 * iters * 16 * 32768.0 / (ms * 1e-3) / 1e12);
  return HY_MOE_OK;
}

extern "C" int hy_moe_probe_mfma_fp8(const void* operands, size_t operand_bytes, float* tflops, void* stream) {
  if (!operands || !tflops || ((uintptr_t)operands & 15) || operand_bytes < HY_MOE_PROBE_OPERAND_BYTES)
    return HY_MOE_ERR_INVALID_ARG;
  const int cus = cus_of_current_device();
  if (cus <= 0) return HY_MOE_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  const int grid = 4 * cus;
  // about 40 ms at 5 PFLOP/s
  const int iters = (int)(2.0e14 / ((double)grid * 4 * 16 * 131072.0));
  hipLaunchKernelGGL(probe_mfma_fp8_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)operands, 64);
  if (hipGetLastError() != hipSuccess) return HY_MOE_ERR_HIP;
  const float ms = time_launch(s, [&] {
    hipLaunchKernelGGL(probe_mfma_fp8_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)operands, iters);
  });
  if (ms <= 0.f) return HY_MOE_ERR_HIP;
  *tflops = (float)((double)grid * 4 * iters * 16 * 131072.0 / (ms * 1e-3) / 1e12);
  return HY_MOE_OK;
}

extern "C" int hy_moe_probe_hbm_read(const void* buf, size_t bytes, float* gbps, void* stream) {
  if (!buf || !gbps || ((uintptr_t)buf & 15) || bytes < 16) return HY_MOE_ERR_INVALID_ARG;
  const int cus = cus_of_current_device();
  if (cus <= 0) return HY_MOE_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  const size_t n = bytes / 16;
  const int grid = 16 * cus;
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)buf, n);  // warm-up
  if (hipGetLastError() != hipSuccess) return HY_MOE_ERR_HIP;
  float ms = -1.f;
  for (int r = 0; r < 3; ++r) {  // the best of three passes
    const float t = time_launch(s, [&] {
      hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const uint4*)buf, n);
    });
    if (t <= 0.f) return HY_MOE_ERR_HIP;
    if (ms < 0.f || t < ms) ms = t;
  }
  *gbps = (float)((double)n * 16 / (ms * 1e-3) / 1e9);
  return HY_MOE_OK;
}

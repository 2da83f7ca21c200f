// moe_layout: the blocked layouts of HY_MOE_WEIGHTS_BF16_BLOCKED and
// HY_MOE_WEIGHTS_SHERRY_BLOCKED (the latter below). A row-major bf16 matrix
// [rows][cols] becomes one 2 KB block per 16-row group and 64-column slab, blocks in
// (row group, slab) order. Inside a block, the 16-byte piece q (columns [8 q, 8 q + 8) of
// the slab) of row r sits at piece 64 (q % 2) + 16 (q / 2) + r: the order in which the
// lanes of a streaming wave take them (lane 16 g + r holds row r, columns 16 g .. 16 g +
// 15 of the slab, as its pieces 16 g + r and 64 + 16 g + r), so each load instruction
// reads 1 KB in order. With row-major weights a wave's 16 rows lie a whole row apart (12
// KB at d = 6144) and HBM delivered ~5.75 TB/s for that pattern; whole 2 KB runs with
// rows in order inside gave ~6.15 TB/s; runs read in lane order with non-temporal loads
// ~7 TB/s. The grouped GEMM's load ops cover 8 rows x 8 pieces, still 8 whole lines. The
// conversion is a plain permutation of 16-byte pieces, run once when a model's weights
// are loaded.
#include "hy_moe.h"
#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kBlockThreads = 256;

// One thread per 16-byte piece (8 values) of the destination, written in order (whole
// lines); piece P of block (row group G, slab c) is piece q = 2 ((P / 16) % 4) + P / 64 of
// row 16 G + P % 16's slab c: a block's 128 threads read its 16 rows' 128-byte pieces whole.
__global__ void __launch_bounds__(kBlockThreads) block_bf16_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst, int64_t pieces,
                                                                    int64_t rows, int64_t cols) {
  const int64_t per_row = cols / 8, per_mat = rows * per_row, chunks = cols / 64;
  for (int64_t t = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; t < pieces;
       t += (int64_t)gridDim.x * kBlockThreads) {
    const int64_t m = t / per_mat, rem = t - m * per_mat;
    const int64_t b = rem / 128, pc = rem - b * 128;  // block (row group, slab) and its piece
    const int64_t g = b / chunks, c = b - g * chunks;
    const int64_t r = 16 * g + (pc & 15), q = 2 * ((pc >> 4) & 3) + (pc >> 6);
    dst[t] = src[m * per_mat + r * per_row + 8 * c + q];
  }
}

// Sherry codes: a row's K/512 slabs of 80 bytes (5 pieces each); slab c of row r lands at
// piece 80 ((r / 16) K/512 + c) + 5 (r % 16) of the matrix: 16 rows' slabs make one
// 1280-byte block, ten whole 128-byte lines (80-byte slabs at 80-byte strides straddle
// lines: the decode kernel fetched 1.57 times the code bytes it used).
__global__ void __launch_bounds__(kBlockThreads) block_sherry_kernel(const uint4* __restrict__ src,
                                                                      uint4* __restrict__ dst, int64_t pieces,
                                                                      int64_t rows, int64_t slabs) {
  const int64_t per_row = slabs * 5, per_mat = rows * per_row;
  for (int64_t t = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; t < pieces;
       t += (int64_t)gridDim.x * kBlockThreads) {
    const int64_t m = t / per_mat, rem = t - m * per_mat;
    const int64_t r = rem / per_row, q = rem - r * per_row;
    const int64_t c = q / 5, j = q - c * 5;
    dst[m * per_mat + ((r / 16) * slabs + c) * 80 + (r % 16) * 5 + j] = src[t];
  }
}

hipError_t launch_block_sherry(const uint32_t* src, uint32_t* dst, int64_t count, int64_t rows, int64_t cols,
                               hipStream_t s) {
  const int64_t slabs = cols / 512, pieces = count * rows * slabs * 5;
  if (pieces == 0) return hipSuccess;
  const int64_t want = (pieces + kBlockThreads - 1) / kBlockThreads;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(block_sherry_kernel, dim3(grid), dim3(kBlockThreads), 0, s, reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), pieces, rows, slabs);
  return hipGetLastError();
}

hipError_t launch_block_bf16(const uint16_t* src, uint16_t* dst, int64_t count, int64_t rows, int64_t cols,
                             hipStream_t s) {
  const int64_t pieces = count * rows * (cols / 8);
  if (pieces == 0) return hipSuccess;
  const int64_t want = (pieces + kBlockThreads - 1) / kBlockThreads;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(block_bf16_kernel, dim3(grid), dim3(kBlockThreads), 0, s, reinterpret_cast<const uint4*>(src),
                     reinterpret_cast<uint4*>(dst), pieces, rows, cols);
  return hipGetLastError();
}

}  // namespace hymoe

extern "C" int hy_moe_block_bf16(const void* src, void* dst, int64_t count, int64_t rows, int64_t cols,
                                 void* stream) {
  if (count < 0 || rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 64 != 0) return HY_MOE_ERR_INVALID_ARG;
  if (count == 0) return HY_MOE_OK;
  if (!src || !dst || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return HY_MOE_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) / cols || count > ((int64_t)1 << 40) / (rows * cols)) return HY_MOE_ERR_INVALID_ARG;
  const uintptr_t bytes = (uintptr_t)(count * rows * cols * 2);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return HY_MOE_ERR_INVALID_ARG;  // overlapping buffers
  const hipError_t err = hymoe::launch_block_bf16((const uint16_t*)src, (uint16_t*)dst, count, rows, cols,
                                                  (hipStream_t)stream);
  return err == hipSuccess ? HY_MOE_OK : HY_MOE_ERR_HIP;
}

extern "C" int hy_moe_block_sherry(const void* src, void* dst, int64_t count, int64_t rows, int64_t cols,
                                   void* stream) {
  if (count < 0 || rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 512 != 0) return HY_MOE_ERR_INVALID_ARG;
  if (count == 0) return HY_MOE_OK;
  if (!src || !dst || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return HY_MOE_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) / cols || count > ((int64_t)1 << 40) / (rows * cols)) return HY_MOE_ERR_INVALID_ARG;
  const uintptr_t bytes = (uintptr_t)(count * rows * (cols / 128 * 20));
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return HY_MOE_ERR_INVALID_ARG;  // overlapping buffers
  const hipError_t err = hymoe::launch_block_sherry((const uint32_t*)src, (uint32_t*)dst, count, rows, cols,
                                                    (hipStream_t)stream);
  return err == hipSuccess ? HY_MOE_OK : HY_MOE_ERR_HIP;
}

// moe_permute: per-expert histogram, prefix scan and deterministic token scatter
// into expert-contiguous rows, for batches of more than one 64-token block (a
// single block is dispatched inside the routing kernel).
//
// The experts selected for a token process it in parallel (m.xxqk.cn Hy4 preview
// explainer, section 2.2 "路由机制"); to run each expert as one dense contraction
// the (token, slot) pairs are grouped by expert: rows are expert-major, tokens
// ascending within an expert. Counts come from population counts of the per-block
// token masks written by the top-k kernel, so every position is fixed by the routing
// alone (no atomics whose order could vary).
#include "common.h"
#include "dispatch.h"
#include "kernels.h"

namespace hymoe {

// One block of 1024 threads. Expert e's token blocks are split into J = 1024 / E
// contiguous chunks, chunk j counted by thread j E + e; the chunk counts are combined
// in chunk order, so every position depends on the routing alone.
__global__ void __launch_bounds__(1024) permute_scan_kernel(const unsigned long long* __restrict__ mask, int nblk,
                                                            int T, int E, int k, int bm,
                                                            int32_t* __restrict__ blk_base,
                                                            int32_t* __restrict__ offs, int32_t* __restrict__ meta,
                                                            int32_t* __restrict__ touched, int4* __restrict__ tiles,
                                                            int32_t* __restrict__ counts_out,
                                                            int32_t* __restrict__ offsets_out) {
  __shared__ int wsum[17];
  __shared__ int part[1024];  // chunk counts, then chunk starts, [j][e]
  const int tid = threadIdx.x;
  const int J = max(1, (int)blockDim.x / E);
  const int cb = (nblk + J - 1) / J;  // blocks per chunk
  const int e = tid % E, j = tid / E;
  const bool mine = j < J;
  const int b0 = mine ? min(nblk, j * cb) : 0, b1 = mine ? min(nblk, b0 + cb) : 0;
  int c = 0;
#pragma unroll 8
  for (int b = b0; b < b1; ++b) c += __popcll(mask[(size_t)b * E + e]);
  if (mine) part[tid] = c;
  __syncthreads();
  // thread e < E: its total and the start of each chunk relative to the expert's first row
  int cnt = 0;
  if (tid < E) {
    for (int jj = 0; jj < J; ++jj) {
      const int v = part[jj * E + tid];
      part[jj * E + tid] = cnt;
      cnt += v;
    }
  }
  const int excl = build_work_lists(tid < E ? cnt : 0, T, E, k, bm, wsum, offs, meta, touched, tiles, counts_out,
                                    offsets_out);  // (synchronises the block)
  if (tid < E)
    for (int jj = 0; jj < J; ++jj) part[jj * E + tid] += excl;  // the expert's first row
  __syncthreads();
  if (mine) {
    int run = part[tid];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      blk_base[(size_t)b * E + e] = run;
      run += __popcll(mask[(size_t)b * E + e]);
    }
  }
}

// One block per 64-token block.
__global__ void __launch_bounds__(256) permute_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                              const unsigned long long* __restrict__ mask,
                                                              const int32_t* __restrict__ blk_base, int T, int E,
                                                              int k, int32_t* __restrict__ perm_src,
                                                              int32_t* __restrict__ pos) {
  const int blk = blockIdx.x;
  const int t_end = min((blk + 1) * kMaskBlock, T);
  for (int i = blk * kMaskBlock * k + threadIdx.x; i < t_end * k; i += blockDim.x) {
    const int t = i / k;
    const int e = topk_idx[i];
    const size_t be = (size_t)blk * E + e;
    const int p = dispatch_row(blk_base[be], mask[be], t - blk * kMaskBlock);
    perm_src[p] = i;
    pos[i] = p;
  }
}

hipError_t launch_permute(const Plan& p, int32_t* counts_out, int32_t* offsets_out, hipStream_t s, Marks& m) {
  if (p.nblk == 1) {
    // dispatched by the routing kernel; keep the stage events aligned
    hipError_t err = m.mark(s);
    return err == hipSuccess ? m.mark(s) : err;
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, p.mask, p.nblk, p.T, p.E, p.k, p.gemm_bm,
                     p.blk_base, p.offs, p.meta, p.touched, p.tiles, counts_out, offsets_out);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(p.nblk), dim3(256), 0, s, p.topk_idx, p.mask, p.blk_base, p.T,
                     p.E, p.k, p.perm_src, p.pos);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

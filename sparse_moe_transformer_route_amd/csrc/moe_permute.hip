// moe_permute: per-expert histogram, prefix scan and deterministic token scatter
// into expert-contiguous rows.
//
// The experts selected for a token process it in parallel (m.xxqk.cn Hy4 preview
// explainer, section 2.2 "路由机制"); to run each expert as one dense contraction
// the (token, slot) pairs are grouped by expert: rows are expert-major, tokens
// ascending within an expert, so row p of expert e is
//   offsets[e] + #{t' < t : e selected by t'}.
// Counts come from population counts of the per-block token masks written by the
// top-k kernel, so every position is fixed by the routing alone (no atomics whose
// order could vary).
#include "common.h"
#include "kernels.h"

namespace hymoe {

// Exclusive prefix sum over a block of up to 1024 threads; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int s = lane < nw ? wsum[lane] : 0;
    const int si = wave_inclusive_scan(s);
    if (lane < nw) wsum[lane] = si - s;
    if (lane == nw - 1) wsum[16] = si;
  }
  __syncthreads();
  const int res = inc - v + wsum[w];
  *total = wsum[16];
  __syncthreads();
  return res;
}

// One block of 1024 threads; thread e owns routed expert e.
__global__ void __launch_bounds__(1024) permute_scan_kernel(const unsigned long long* __restrict__ mask, int nblk,
                                                            int T, int E, int k, int bm,
                                                            int32_t* __restrict__ blk_base,
                                                            int32_t* __restrict__ offs, int32_t* __restrict__ meta,
                                                            int32_t* __restrict__ touched, int2* __restrict__ tiles,
                                                            int32_t* __restrict__ counts_out,
                                                            int32_t* __restrict__ offsets_out) {
  __shared__ int wsum[17];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E)
    for (int b = 0; b < nblk; ++b) cnt += __popcll(mask[(size_t)b * E + e]);
  int total = 0;
  const int excl = block_exclusive_scan(cnt, wsum, &total);
  if (e < E) {
    offs[e] = excl;
    if (counts_out) counts_out[e] = cnt;
    if (offsets_out) offsets_out[e] = excl;
    int run = excl;
    for (int b = 0; b < nblk; ++b) {
      blk_base[(size_t)b * E + e] = run;
      run += __popcll(mask[(size_t)b * E + e]);
    }
  }
  if (e == 0) {
    offs[E] = T * k;
    offs[E + 1] = T * k + T;
    if (offsets_out) offsets_out[E] = T * k;
  }

  // touched experts, ascending, then the shared expert
  const int flag = (e < E && cnt > 0) ? 1 : 0;
  int ntouched = 0;
  const int tpos = block_exclusive_scan(flag, wsum, &ntouched);
  if (flag) touched[tpos] = e;
  if (e == 0) touched[ntouched] = E;

  // grouped-GEMM M tiles: ceil(count/bm) per routed expert, then the shared expert's
  const int nt = (e < E) ? (cnt + bm - 1) / bm : 0;
  int routed_tiles = 0;
  const int toff = block_exclusive_scan(nt, wsum, &routed_tiles);
  for (int i = 0; i < nt; ++i) tiles[toff + i] = make_int2(e, i * bm);
  const int shared_tiles = (T + bm - 1) / bm;
  for (int i = e; i < shared_tiles; i += blockDim.x) tiles[routed_tiles + i] = make_int2(E, i * bm);
  if (e == 0) {
    meta[0] = ntouched + 1;
    meta[1] = routed_tiles + shared_tiles;
  }
}

// One block per kMaskBlock tokens: row of (t, j) = base of (block, expert) plus the
// number of earlier tokens of the block that selected the same expert.
__global__ void __launch_bounds__(256) permute_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                              const unsigned long long* __restrict__ mask,
                                                              const int32_t* __restrict__ blk_base, int T, int E,
                                                              int k, int32_t* __restrict__ perm_src,
                                                              int32_t* __restrict__ pos) {
  const int blk = blockIdx.x;
  const int t_end = min((blk + 1) * kMaskBlock, T);
  for (int i = blk * kMaskBlock * k + threadIdx.x; i < t_end * k; i += blockDim.x) {
    const int t = i / k;
    const int tl = t - blk * kMaskBlock;
    const int e = topk_idx[i];
    const unsigned long long m = mask[(size_t)blk * E + e];
    const int p = blk_base[(size_t)blk * E + e] + __popcll(m & ((1ull << tl) - 1ull));
    perm_src[p] = i;
    pos[i] = p;
  }
}

hipError_t launch_permute(const Plan& p, int32_t* counts_out, int32_t* offsets_out, hipStream_t s, Marks& m) {
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

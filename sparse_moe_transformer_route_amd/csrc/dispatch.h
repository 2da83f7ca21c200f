// Device-side building blocks of the dispatch step shared by the stand-alone
// permute kernels and the fused small-batch routing kernel.
//
// Rows are expert-major, tokens ascending within an expert: the row of (token t,
// expert e) is offsets[e] + #{t' < t : e selected by t'}. The shared expert is
// expert E with rows T*k .. T*k+T-1 in token order.
#pragma once

#include "common.h"
#include "kernels.h"

namespace hymoe {

// Exclusive prefix sum over a block of up to 1024 threads; *total gets the sum.
// wsum: 17 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
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

// Splits n rows into c = ceil(n/bm) tiles of (nearly) equal size in whole 32-row
// blocks: ceil(ceil(n/32)/c) blocks each, the last tile taking the rest (never empty).
// Equal tiles of one expert do the same work per k step, so running side by side they
// stay in step and share the expert's weight tiles through L2 (a short remainder tile
// would run ahead and fetch the weights again).
// Tile i = {e, first row, rows, index of the expert's first tile}.
__device__ __forceinline__ void write_tiles(int e, int n, int bm, int first, int4* __restrict__ tiles) {
  const int nt = (n + bm - 1) / bm;
  const int span = ((n + 31) / 32 + nt - 1) / nt * 32;
  for (int i = 0; i < nt; ++i) tiles[first + i] = make_int4(e, i * span, min(span, n - i * span), first);
}

// Thread e (< E) holds cnt = tokens routed to expert e; every thread of the block
// (blockDim >= E) must call. Writes offs[0..E+1], the touched-expert list (shared
// expert first, then routed experts with rows in ascending order), the grouped-GEMM
// M tiles (routed experts ascending, then the shared expert) and meta {touched
// count, tile count, routed tile count}; returns expert e's first row.
__device__ __forceinline__ int build_work_lists(int cnt, int T, int E, int k, int bm, int* wsum,
                                                int32_t* __restrict__ offs, int32_t* __restrict__ meta,
                                                int32_t* __restrict__ touched, int4* __restrict__ tiles,
                                                int32_t* __restrict__ counts_out,
                                                int32_t* __restrict__ offsets_out) {
  const int e = threadIdx.x;
  int total = 0;
  const int excl = block_exclusive_scan(cnt, wsum, &total);
  if (e < E) {
    offs[e] = excl;
    if (counts_out) counts_out[e] = cnt;
    if (offsets_out) offsets_out[e] = excl;
  }
  if (e == 0) {
    offs[E] = T * k;
    offs[E + 1] = T * k + T;
    if (offsets_out) offsets_out[E] = T * k;
  }
  // touched experts: the shared expert first (it has the most rows), then routed
  const int flag = (e < E && cnt > 0) ? 1 : 0;
  int ntouched = 0;
  const int tpos = block_exclusive_scan(flag, wsum, &ntouched);
  if (flag) touched[1 + tpos] = e;
  if (e == 0) touched[0] = E;
  // grouped-GEMM M tiles
  const int nt = (e < E) ? (cnt + bm - 1) / bm : 0;
  int routed_tiles = 0;
  const int toff = block_exclusive_scan(nt, wsum, &routed_tiles);
  if (nt > 0) write_tiles(e, cnt, bm, toff, tiles);
  if (e == 0) {
    write_tiles(E, T, bm, routed_tiles, tiles);
    meta[0] = ntouched + 1;
    meta[1] = routed_tiles + (T + bm - 1) / bm;
    meta[2] = routed_tiles;
  }
  // the grouped GEMM's work counters start at zero on every forward
  if (e >= kMetaSched && e < kMetaInts) meta[e] = 0;
  return excl;
}

// Row of (token t = blk*64 + tl, slot j) given the block's first row for expert e and
// the block's token mask for e.
__device__ __forceinline__ int dispatch_row(int base, unsigned long long m, int tl) {
  return base + __popcll(m & ((1ull << tl) - 1ull));
}

}  // namespace hymoe

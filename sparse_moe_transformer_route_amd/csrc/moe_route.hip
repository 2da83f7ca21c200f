// moe_route: router logits on bf16 MFMA, then per-token top-k selection with
// renormalised softmax weights and the per-block dispatch masks.
//
// The router scores each token against every routed expert and keeps the k best
// (m.xxqk.cn Hy4 preview explainer, section 2.2 "路由机制"; Hy4 preview: 256 routed
// experts, top-8, per the Tencent Hy4 preview model card). Scores are logits
// x.W_router[e] (+bias[e]) accumulated in fp32; ties go to the lower expert index;
// the merge weights are the softmax over the selected set.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace hymoe {

// ---------------------------------------------------------------------------
// Logits: one wave computes a 32-token x 64-expert tile over a slice of d.
// grid = (ceil(T/32), ceil(E/64), ks); part[z][t][e] holds slice z's partial sum.
// Operands are read straight from global memory: each lane streams 32 contiguous
// bytes of its row per 64-wide k step (the router is 0.5% of the layer's flops).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) route_logits_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          float* __restrict__ part, int T, int d, int E,
                                                          int kc) {
  const int lane = threadIdx.x;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 64, z = blockIdx.z;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t kbeg = (size_t)z * kc + 16 * g;

  const uint16_t* arow[2];
  const uint16_t* brow[4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    int t = min(t0 + 16 * tb + r16, T - 1);
    arow[tb] = x + (size_t)t * d + kbeg;
  }
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) {
    int e = min(e0 + 16 * eb + r16, E - 1);
    brow[eb] = wr + (size_t)e * d + kbeg;
  }

  f32x4 acc[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[tb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kk = 0; kk < kc; kk += 64) {
    uint4 a[2][2], b[4][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s = 0; s < 2; ++s) a[tb][s] = ldg16(arow[tb] + kk + 8 * s);
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int s = 0; s < 2; ++s) b[eb][s] = ldg16(brow[eb] + kk + 8 * s);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) acc[tb][eb] = mfma16x16x32(a[tb][s], b[eb][s], acc[tb][eb]);
  }

  float* dst = part + (size_t)z * T * E;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
      const int e = e0 + 16 * eb + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 16 * tb + 4 * g + q;
        if (t < T && e < E) dst[(size_t)t * E + e] = acc[tb][eb][q];
      }
    }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token, R = ceil(E/64) logits per lane; k rounds of a
// wave-wide argmax on (logit, -index), plus one round for the k/k+1 margin.
// The block of kMaskBlock tokens also builds mask[blk][e] (bit tl set when token
// blk*64+tl selected e), from which the permutation is derived.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void better(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
}

template <int R>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ part, int ks,
                                                         const float* __restrict__ bias, int T, int E, int k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w, float* __restrict__ margin,
                                                         unsigned long long* __restrict__ mask) {
  __shared__ unsigned long long smask[1024];
  for (int i = threadIdx.x; i < E; i += blockDim.x) smask[i] = 0ull;
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int blk = blockIdx.x;
  for (int tl = wv; tl < kMaskBlock; tl += 4) {
    const int t = blk * kMaskBlock + tl;
    if (t >= T) break;
    float v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = lane + 64 * r;
      if (e < E) {
        float s = 0.f;
        for (int z = 0; z < ks; ++z) s += part[((size_t)z * T + t) * E + e];
        if (bias) s += bias[e];
        v[r] = s;
      } else {
        v[r] = -FLT_MAX;
      }
    }
    unsigned taken = 0u;
    float myv = 0.f, top = 0.f, last = 0.f;
    int mye = 0;
    const int rounds = k < E ? k + 1 : k;
    for (int j = 0; j < rounds; ++j) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = lane + 64 * r;
        if (e < E && !((taken >> r) & 1u) && v[r] > bv) { bv = v[r]; be = e; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oe = __shfl_xor(be, o, 64);
        better(bv, be, ov, oe);
      }
      if (j < k) {
        if (lane == j) { myv = bv; mye = be; }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (j == 0) top = bv;
        last = bv;
      } else if (lane == 0 && margin) {
        margin[t] = last - bv;
      }
    }
    if (k == E && lane == 0 && margin) margin[t] = INFINITY;

    // merge weights: softmax over the selected set, shifted by its maximum
    const float ex = lane < k ? expf(myv - top) : 0.f;
    float zsum = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) zsum += __shfl_xor(zsum, o, 64);
    // ascending expert order: rank of this lane's expert among the selected
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const int oe = __shfl(mye, j, 64);
      rank += (oe < mye) ? 1 : 0;
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + rank] = mye;
      topk_w[(size_t)t * k + rank] = ex / zsum;
      atomicOr(&smask[mye], 1ull << tl);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += blockDim.x) mask[(size_t)blk * E + i] = smask[i];
}

static int pick_split(int T, int d, int E) {
  const int base = ((T + 31) / 32) * ((E + 63) / 64);
  const int target = 512;
  const int steps = d / 64;
  int best = 1;
  for (int s = 1; s <= steps; ++s)
    if (steps % s == 0 && base * s <= target) best = s;
  return best;
}

int route_split_for(int T, int d, int E) { return pick_split(T, d, E); }

hipError_t launch_route(const Plan& p, const uint16_t* x, const uint16_t* w_router, const float* bias,
                        float* margin_out, hipStream_t s, Marks& m) {
  dim3 g1((p.T + 31) / 32, (p.E + 63) / 64, p.ks);
  hipLaunchKernelGGL(route_logits_kernel, g1, dim3(64), 0, s, x, w_router, p.part, p.T, p.d, p.E, p.d / p.ks);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  dim3 g2(p.nblk);
  const int R = (p.E + 63) / 64;
  if (R <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, g2, dim3(256), 0, s, p.part, p.ks, bias, p.T, p.E, p.k, p.topk_idx,
                       p.topk_w, margin_out, p.mask);
  else if (R <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, g2, dim3(256), 0, s, p.part, p.ks, bias, p.T, p.E, p.k, p.topk_idx,
                       p.topk_w, margin_out, p.mask);
  else if (R <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, g2, dim3(256), 0, s, p.part, p.ks, bias, p.T, p.E, p.k, p.topk_idx,
                       p.topk_w, margin_out, p.mask);
  else if (R <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, g2, dim3(256), 0, s, p.part, p.ks, bias, p.T, p.E, p.k, p.topk_idx,
                       p.topk_w, margin_out, p.mask);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, g2, dim3(256), 0, s, p.part, p.ks, bias, p.T, p.E, p.k, p.topk_idx,
                       p.topk_w, margin_out, p.mask);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

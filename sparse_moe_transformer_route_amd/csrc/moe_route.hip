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
#include "dispatch.h"
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
// Logits for large T: a workgroup of 4 waves computes a 64-token x 256-expert tile
// over a slice of d (wave w: experts 64 w .. 64 w + 63). Each 64-wide k step of the
// 64 x-rows and 256 W_router rows (128 B per row, 40 KB) arrives in LDS through
// direct global->LDS loads in which 8 consecutive lanes cover one row (whole cache
// lines per lane quad: the address unit's fast case), then feeds 16x16x32 MFMAs
// from LDS. Two ring slots; 16-byte chunk c of row r sits at c ^ ((r / 2) mod 8): the
// LDS serves a 16-byte read 16 lanes at a time over 64 four-byte banks, and this key
// puts the 16 rows of such a group on distinct bank groups.
// Work w enumerates (slice, token tile, expert tile), expert tile fastest, and block
// b runs work (b mod 8) * per + b / 8: XCD x (b mod 8) takes the x-th contiguous
// eighth, so its workgroups share one or two slices of W_router in its L2.
// ---------------------------------------------------------------------------
constexpr int kLgTok = 64;                       // tokens per tile
constexpr int kLgExp = 256;                      // experts per tile
constexpr int kLgRows = kLgTok + kLgExp;         // staged rows per step
constexpr int kLgSlot = kLgRows * 128;           // 40 KB per ring slot
constexpr int kLgOps = kLgRows * 128 / 16 / 256; // 16-byte loads per thread per step (10)

template <int N>
__device__ __forceinline__ void lg_wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ void __launch_bounds__(256, 2) route_logits_lds_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr,
                                                                 float* __restrict__ part, int T, int d, int E,
                                                                 int kc, int ks) {
  __shared__ __attribute__((aligned(16))) uint8_t s0[kLgSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s1[kLgSlot];
  const int ntt = (T + kLgTok - 1) / kLgTok, nte = (E + kLgExp - 1) / kLgExp;
  const int nw = ntt * nte * ks;
  const int per = (nw + 7) >> 3;
  const int w = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (w >= nw) return;  // whole workgroup
  const int te = w % nte, rest = w / nte;
  const int tt = rest % ntt, z = rest / ntt;
  const int t0 = tt * kLgTok, e0 = te * kLgExp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // load op i of thread tid: staged row (256 i + tid) / 8, physical chunk tid % 8
  // holding logical chunk (tid % 8) ^ ((row / 2) % 8); rows 0..63 are tokens, 64.. experts,
  // both clamped to the last valid row (never stored)
  const uint16_t* src[kLgOps];
#pragma unroll
  for (int i = 0; i < kLgOps; ++i) {
    const int row = (256 * i + tid) >> 3, lc = (tid & 7) ^ ((row >> 1) & 7);
    const uint16_t* base = row < kLgTok ? x + (size_t)min(t0 + row, T - 1) * d
                                        : wr + (size_t)min(e0 + row - kLgTok, E - 1) * d;
    src[i] = base + (size_t)z * kc + 8 * lc;
  }
  // (the LDS address operand is the wave's base: lane l writes 16 bytes at base + 16 l)
  auto issue = [&](int st, uint8_t* slot) {
#pragma unroll
    for (int i = 0; i < kLgOps; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + 64 * st),
                                       (__attribute__((address_space(3))) void*)(slot + 4096 * i + 1024 * wv), 16, 0,
                                       0);
  };

  // fragment of 16 rows starting at row r0 for k group s (k 32 s .. 32 s + 31): lane
  // (r16, g) reads row r0 + r16, logical chunk 4 s + g
  const int r16 = lane & 15, g = lane >> 4;
  auto frag = [&](const uint8_t* slot, int r0, int s) {
    const int row = r0 + r16;
    return *reinterpret_cast<const uint4*>(slot + row * 128 + (((4 * s + g) ^ ((row >> 1) & 7)) << 4));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[tb][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* slot) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a[4], b[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) a[tb] = frag(slot, 16 * tb, s);
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) b[eb] = frag(slot, kLgTok + 64 * wv + 16 * eb, s);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) acc[tb][eb] = mfma16x16x32(a[tb], b[eb], acc[tb][eb]);
    }
  };
  // step st: its loads (issued one step earlier) landed everywhere, and every wave is
  // done with step st-1, whose slot then receives step st+1 while step st computes
  auto step = [&](int st, const uint8_t* cur, uint8_t* nxt, int nst) {
    lg_wait_vm<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + 1 < nst) issue(st + 1, nxt);
    compute(cur);
  };
  const int nst = kc / 64;
  issue(0, s0);
  for (int st = 0; st < nst; st += 2) {
    step(st, s0, s1, nst);
    if (st + 1 < nst) step(st + 1, s1, s0, nst);
  }

  float* dst = part + (size_t)z * T * E;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
      const int e = e0 + 64 * wv + 16 * eb + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 16 * tb + 4 * g + q;
        if (t < T && e < E) dst[(size_t)t * E + e] = acc[tb][eb][q];
      }
    }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token. Logits (the split-d partials summed in fixed order,
// plus the bias) are mapped to order-preserving 32-bit keys; the k-th largest key is
// found by an MSB-first radix select whose counts are wave ballots, then ties at the
// threshold go to the lowest expert indices. No lane shuffles in the search loop.
// The block of kMaskBlock tokens builds mask[blk][e] (bit tl set when token
// blk*64+tl selected e). With a single block (FUSED) the same workgroup also builds
// the dispatch lists and the permutation.
// ---------------------------------------------------------------------------
constexpr int kMaxSplit = 16;  // router split of d: at most this many partial sums per logit

__device__ __forceinline__ uint32_t mono_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int R, bool FUSED>
__global__ void __launch_bounds__(1024) route_select_kernel(const float* __restrict__ part, int ks,
                                                            const float* __restrict__ bias, int T, int E, int k,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w, float* __restrict__ margin,
                                                            unsigned long long* __restrict__ mask, Plan p,
                                                            int32_t* __restrict__ counts_out,
                                                            int32_t* __restrict__ offsets_out) {
  __shared__ unsigned long long smask[1024];
  __shared__ int sidx[FUSED ? kMaskBlock * 16 : 1];
  __shared__ int soff[FUSED ? 1024 : 1];
  __shared__ int wsum[17];
  for (int i = threadIdx.x; i < E; i += blockDim.x) smask[i] = 0ull;
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const unsigned long long below_lane = (1ull << lane) - 1ull;
  const int blk = blockIdx.x;
  const size_t TE = (size_t)T * E;
  for (int tl = wv; tl < kMaskBlock; tl += nwv) {
    const int t = blk * kMaskBlock + tl;
    if (t >= T) break;
    float val[R];
    uint32_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = lane + 64 * r;
      if (e < E) {
        // all partial loads issued before the (fixed-order) sum: unconditional, slices
        // past ks re-read the last one (cache hits) and are not added, so no load waits
        // behind a branch
        float pz[kMaxSplit];
#pragma unroll
        for (int z = 0; z < kMaxSplit; ++z) pz[z] = part[(size_t)min(z, ks - 1) * TE + (size_t)t * E + e];
        float sum = 0.f;
#pragma unroll
        for (int z = 0; z < kMaxSplit; ++z)
          if (z < ks) sum += pz[z];
        if (bias) sum += bias[e];
        val[r] = sum;
        key[r] = mono_key(sum);
      } else {
        val[r] = 0.f;
        key[r] = 0u;  // below every finite logit's key
      }
    }
    // k-th largest key
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int c = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) c += __popcll(__ballot(key[r] >= cand));
      if (c >= k) tau = cand;
    }
    int cgt = 0;
    unsigned long long eqm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cgt += __popcll(__ballot(key[r] > tau));
      eqm[r] = __ballot(key[r] == tau);
    }
    const int need = k - cgt;  // experts taken from those tied at the threshold
    bool sel[R];
    int eq_before = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int mine = __popcll(eqm[r] & below_lane);
      sel[r] = key[r] > tau || (((eqm[r] >> lane) & 1ull) && eq_before + mine < need);
      eq_before += __popcll(eqm[r]);
    }
    // margin = k-th minus (k+1)-th largest logit (wave-uniform branches)
    if (margin) {
      if (k == E) {
        if (lane == 0) margin[t] = INFINITY;
      } else if (eq_before > need) {
        if (lane == 0) margin[t] = 0.f;  // the (k+1)-th is tied with the k-th
      } else {
        uint32_t nb = 0u;
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (key[r] < tau && key[r] > nb) nb = key[r];
        nb = wave_max_u32(nb);
        if (lane == 0) margin[t] = key_value(tau) - key_value(nb);
      }
    }
    // softmax over the selected set, shifted by its largest logit
    uint32_t kmax = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) kmax = max(kmax, key[r]);
    const float top = key_value(wave_max_u32(kmax));
    float ex[R], part_sum = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ex[r] = sel[r] ? expf(val[r] - top) : 0.f;
      part_sum += ex[r];
    }
    const float zsum = wave_sum(part_sum);
    // ascending expert order: rank = selected experts with a smaller index
    int before = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned long long sm = __ballot(sel[r]);
      if (sel[r]) {
        const int e = lane + 64 * r;
        const int rank = before + __popcll(sm & below_lane);
        topk_idx[(size_t)t * k + rank] = e;
        topk_w[(size_t)t * k + rank] = ex[r] / zsum;
        atomicOr(&smask[e], 1ull << tl);
        if (FUSED) sidx[tl * 16 + rank] = e;
      }
      before += __popcll(sm);
    }
  }
  __syncthreads();
  if (!FUSED) {
    for (int i = threadIdx.x; i < E; i += blockDim.x) mask[(size_t)blk * E + i] = smask[i];
    return;
  }
  // single token block: counts, work lists and permutation here
  const int e = threadIdx.x;
  const int cnt = e < E ? __popcll(smask[e]) : 0;
  const int excl = build_work_lists(cnt, T, E, k, p.gemm_bm, wsum, p.offs, p.meta, p.touched, p.tiles, counts_out,
                                    offsets_out);
  if (e < E) soff[e] = excl;
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
    const int t = i / k, j = i - t * k;
    const int ee = sidx[t * 16 + j];
    const int row = dispatch_row(soff[ee], smask[ee], t);
    p.perm_src[row] = i;
    p.pos[i] = row;
  }
}

// The LDS-tiled logits kernel takes batches of at least this many tokens.
constexpr int kLgMinT = 1024;

// Split of d for the router: enough waves to stream W_router from HBM at small T
// (one-wave tiles), enough workgroups for two per CU at large T (LDS tiles); at most
// 16 partial sums per logit.
static int pick_split(int T, int d, int E) {
  const bool lds = T >= kLgMinT;
  const int base = lds ? ((T + kLgTok - 1) / kLgTok) * ((E + kLgExp - 1) / kLgExp)
                       : ((T + 31) / 32) * ((E + 63) / 64);
  const int target = lds ? 512 : 256;
  const int steps = d / 64;
  int best = 1;
  for (int s = 1; s <= steps && s <= kMaxSplit; ++s)
    if (steps % s == 0 && base * s <= target) best = s;
  return best;
}

int route_split_for(int T, int d, int E) { return pick_split(T, d, E); }

template <int R>
static void launch_select(const Plan& p, const float* bias, float* margin_out, int32_t* counts_out,
                          int32_t* offsets_out, hipStream_t s) {
  if (p.nblk == 1)
    hipLaunchKernelGGL((route_select_kernel<R, true>), dim3(1), dim3(1024), 0, s, p.part, p.ks, bias, p.T, p.E, p.k,
                       p.topk_idx, p.topk_w, margin_out, p.mask, p, counts_out, offsets_out);
  else
    hipLaunchKernelGGL((route_select_kernel<R, false>), dim3(p.nblk), dim3(1024), 0, s, p.part, p.ks, bias, p.T,
                       p.E, p.k, p.topk_idx, p.topk_w, margin_out, p.mask, p, counts_out, offsets_out);
}

hipError_t launch_route(const Plan& p, const uint16_t* x, const uint16_t* w_router, const float* bias,
                        float* margin_out, int32_t* counts_out, int32_t* offsets_out, hipStream_t s, Marks& m) {
  if (p.T >= kLgMinT) {
    const int nw = ((p.T + kLgTok - 1) / kLgTok) * ((p.E + kLgExp - 1) / kLgExp) * p.ks;
    hipLaunchKernelGGL(route_logits_lds_kernel, dim3(8 * ((nw + 7) / 8)), dim3(256), 0, s, x, w_router, p.part, p.T,
                       p.d, p.E, p.d / p.ks, p.ks);
  } else {
    dim3 g1((p.T + 31) / 32, (p.E + 63) / 64, p.ks);
    hipLaunchKernelGGL(route_logits_kernel, g1, dim3(64), 0, s, x, w_router, p.part, p.T, p.d, p.E, p.d / p.ks);
  }
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  const int R = (p.E + 63) / 64;
  if (R <= 1)
    launch_select<1>(p, bias, margin_out, counts_out, offsets_out, s);
  else if (R <= 2)
    launch_select<2>(p, bias, margin_out, counts_out, offsets_out, s);
  else if (R <= 4)
    launch_select<4>(p, bias, margin_out, counts_out, offsets_out, s);
  else if (R <= 8)
    launch_select<8>(p, bias, margin_out, counts_out, offsets_out, s);
  else
    launch_select<16>(p, bias, margin_out, counts_out, offsets_out, s);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

// Sparse-attention indexer: for each query, a score for every key of its sequence and
// the K best keys (Tencent Hy4 preview model card, configuration summary: every layer
// uses DeepSeek-style sparse attention whose indexer has 32 heads, head_dim 128 and
// top-k 2048, one 128-dim key per token shared by all heads; IndexCache lets 57 of the
// 78 layers reuse the selection of the layer before them, so only 21 layers run this).
// The score is read as sum over heads h of w[h] * max(0, q[h] . k): the pages give the
// indexer's shape, not its formula.
//
// indexer_scores_kernel: a workgroup takes 128 keys of one sequence. Their rows (256 B
// each) arrive in LDS by direct global->LDS loads, 16 lanes per row, 16-byte chunk c of
// key r stored at c ^ (r mod 16) so that the fragment reads (16 lanes = 16 keys, one
// chunk) hit 16 distinct bank groups. Each wave runs 32x32x16 bf16 MFMAs with the
// query's 32 heads as rows and 32 keys as columns: lane (key, half) then holds 16 heads
// of one key, weights and clips them in registers, and one shuffle adds the two halves.
// The kernel streams the keys once: HBM-bound.
//
// indexer_topk_kernel: one 1024-thread workgroup per query (for up to 64K keys each
// thread holds 64 of them, loaded once: 32 in registers, 32 in LDS). An MSB-first radix select over
// 8-bit digits of an order-preserving key of the fp32 scores finds the K-th score; the first digit (sign and exponent) takes few values, so its histogram counts
// are combined per wave (one LDS atomic per distinct digit), later digits are spread
// and go straight to per-wave histograms. Keys above the K-th, then the lowest-index
// keys equal to it, are written in ascending key order through block prefix sums.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "hy_moe.h"
#include "common.h"
#include "dispatch.h"

namespace hymoe {
namespace {

constexpr int kIxKeys = 128;      // keys per scoring workgroup (4 waves x 32)
constexpr int kIxHeads = 32;      // MFMA rows
constexpr int kIxSelThreads = 1024;
constexpr int kIxKeysPerThread = 64;  // selection keys held on chip per thread (S <= 64K)
constexpr int kIxChunk = 8192;        // keys per workgroup in the first stage of the two-stage selection

#define IX_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int D>
__global__ void __launch_bounds__(256) indexer_scores_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                             const uint16_t* __restrict__ keys, int S,
                                                             float* __restrict__ scores) {
  constexpr int CH = D / 8;                   // 16-byte chunks per key row
  constexpr int OPS = kIxKeys * CH / 256;     // direct-to-LDS ops per thread
  constexpr int NS = D / 16;                  // MFMA k steps
  static_assert(CH >= 16 && (CH & (CH - 1)) == 0, "D must be a power of two >= 128");
  __shared__ __attribute__((aligned(16))) uint8_t lk[kIxKeys * D * 2];
  const int b = blockIdx.y;
  const int s0 = blockIdx.x * kIxKeys;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const uint16_t* kb = keys + (size_t)b * S * D;
  // keys past S reload the last key (scores not stored); each key row is read once per
  // query and a wave's op covers 4 whole rows, so the loads take the non-temporal hint
  // (scoring 0.0953 -> 0.0914 ms at 32 x 64K keys)
#pragma unroll
  for (int i = 0; i < OPS; ++i) {
    const int pq = 256 * i + tid;
    const int row = pq / CH, lc = (pq % CH) ^ (row % 16);
    const int key = min(s0 + row, S - 1);
    __builtin_amdgcn_global_load_lds((const void*)(kb + (size_t)key * D + 8 * lc), IX_LDS(lk + 16 * (256 * i + 64 * wv)),
                                     16, 0, 2);
  }
  // the query's fragments (row = head) and the lane's 16 head weights, while the keys land
  uint4 fa[NS];
  const uint16_t* qb = q + ((size_t)b * kIxHeads + col) * D + 8 * hf;
#pragma unroll
  for (int s = 0; s < NS; ++s) fa[s] = *reinterpret_cast<const uint4*>(qb + 16 * s);
  float wl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wl[i] = w[(size_t)b * kIxHeads + 8 * (i / 4) + 4 * hf + (i % 4)];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int kr = 32 * wv + col;  // this lane's key row in the tile
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4 fb = *reinterpret_cast<const uint4*>(lk + kr * D * 2 + 16 * ((2 * s + hf) ^ (kr % 16)));
    acc = mfma32x32x16(fa[s], fb, acc);
  }
  // accumulator i: head 8 (i / 4) + 4 hf + i % 4 of key kr
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) v += wl[i] * fmaxf(acc[i], 0.f);
  v += __shfl_xor(v, 32, 64);
  if (hf == 0 && s0 + kr < S) scores[(size_t)b * S + s0 + kr] = v;
}

// order-preserving unsigned key of an fp32 value (larger value -> larger key)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the float an order key came from (order_key is a bijection on bit patterns)
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// KPT > 0: S <= kIxSelThreads * KPT, each thread holds the keys of indices
// [t KPT, t KPT + KPT) (loaded once, all loads in flight together);
// KPT == 0: any S, every pass reads the scores again (thread t: indices t, t + 1024, ...
// for the histograms, a contiguous range for the output).
// The K highest of the S scores sc[0..S) (ties to the lower position), written in
// ascending position order: out_idx[r] = remap ? remap[p] : offset + p, out_sc[r] = sc[p]
// when out_sc is given (REMAP: remap is given, and held in registers). Called by every
// thread of a kIxSelThreads block.
template <int KPT, bool REMAP = false>
__device__ __forceinline__ void topk_rows(const float* __restrict__ sc, int S, int K, const int32_t* __restrict__ remap,
                                          int offset, int32_t* __restrict__ out_idx, float* __restrict__ out_sc) {
  constexpr int NW = kIxSelThreads / 64;
  __shared__ uint32_t hist[NW][256];
  __shared__ uint32_t total[256];
  __shared__ int runc[256];  // per-wave running counts of the digit search
  __shared__ uint32_t sh_prefix, sh_need;
  __shared__ int wsum[17];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = min(K, S);
  // contiguous range of this thread (the output is written in index order)
  const int c = KPT > 0 ? KPT : (S + kIxSelThreads - 1) / kIxSelThreads;
  const int lo = min(S, tid * c), hi = min(S, lo + c);
  // keys j < KREG in registers, the rest in LDS (word [j - KREG][tid]: consecutive
  // threads on consecutive banks); all in registers spilled
  constexpr int KREG = KPT > 32 ? KPT / 2 : KPT > 0 ? KPT : 1;
  __shared__ uint32_t kl[KPT > 32 ? KPT - KPT / 2 : 1][kIxSelThreads];
  uint32_t kr[KREG];
  auto kget = [&](int j) -> uint32_t { return j < KREG ? kr[j] : kl[j - KREG][tid]; };
  if constexpr (KPT > 0) {
    if (KPT % 4 == 0 && ((uintptr_t)(sc + lo) & 15) == 0 && hi - lo == KPT) {
      // 16-byte loads: a quarter of the cache-line requests of 4-byte ones (a wave's
      // lanes are KPT * 4 bytes apart, each on its own line)
#pragma unroll
      for (int m = 0; m < KPT / 4; ++m) {
        const float4 v = *reinterpret_cast<const float4*>(sc + lo + 4 * m);
        const uint32_t k4[4] = {order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w)};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = 4 * m + t;
          if (j < KREG)
            kr[j] = k4[t];
          else
            kl[j - KREG][tid] = k4[t];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t key = lo + j < hi ? order_key(sc[lo + j]) : 0u;
        if (j < KREG)
          kr[j] = key;
        else
          kl[j - KREG][tid] = key;
      }
    }
  }
  // REMAP: the positions' output indices, loaded with the keys so that writing the
  // output waits on no load (a gather per taken key was a quarter of the merge stage)
  static_assert(!REMAP || (KPT > 0 && KPT <= 32), "remapped rows are held in registers");
  int32_t rv[REMAP ? KPT : 1];
  if constexpr (REMAP) {
    if (KPT % 4 == 0 && ((uintptr_t)(remap + lo) & 15) == 0 && hi - lo == KPT) {
#pragma unroll
      for (int m = 0; m < KPT / 4; ++m) {
        const int4 v = *reinterpret_cast<const int4*>(remap + lo + 4 * m);
        rv[4 * m] = v.x;
        rv[4 * m + 1] = v.y;
        rv[4 * m + 2] = v.z;
        rv[4 * m + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) rv[j] = lo + j < hi ? remap[lo + j] : 0;
    }
  }
  uint32_t prefix = 0, mask = 0, need = (uint32_t)n;  // need: keys still to take at or below the prefix
  // one key of the histogram pass: act = the key is a candidate
  auto count = [&](bool act, uint32_t dig, bool first) {
    if (first) {
      // few distinct leading digits: one atomic per distinct digit of the wave
      unsigned long long pend = __ballot(act);
      while (pend) {
        const int leader = __builtin_ctzll(pend);
        const uint32_t v = __shfl(dig, leader, 64);
        const unsigned long long same = __ballot(act && dig == v) & pend;
        if (lane == leader) atomicAdd(&hist[wv][v], (uint32_t)__popcll(same));
        pend &= ~same;
      }
    } else if (act) {
      atomicAdd(&hist[wv][dig], 1u);
    }
  };
#pragma unroll 1
  for (int d = 3; d >= 0; --d) {
    for (int i = tid; i < NW * 256; i += kIxSelThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    const int sh = 8 * d;
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t key = kget(j);
        count(lo + j < hi && (key & mask) == prefix, (key >> sh) & 255u, d == 3);
      }
    } else {
      for (int i0 = 0; i0 < S; i0 += kIxSelThreads) {
        const int i = i0 + tid;
        const uint32_t key = i < S ? order_key(sc[i]) : 0u;
        count(i < S && (key & mask) == prefix, (key >> sh) & 255u, d == 3);
      }
    }
    __syncthreads();
    // thread t < 256 takes digit 255 - t: its count, and by a scan over the 4 waves the
    // count of candidates with that digit or a larger one; the digit holding the
    // need-th largest candidate is the one where that running count reaches need
    if (tid < 256) {
      const int v = 255 - tid;
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < NW; ++k) cnt += (int)hist[k][v];
      const int incl = wave_inclusive_scan(cnt);
      if (lane == 63) wsum[wv] = incl;
      total[tid] = (uint32_t)cnt;
      runc[tid] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      int base = 0;
      for (int k = 0; k < wv; ++k) base += wsum[k];
      const int incl = base + runc[tid], cnt = (int)total[tid];
      if (incl >= (int)need && incl - cnt < (int)need) {
        sh_prefix = prefix | ((uint32_t)(255 - tid) << sh);
        sh_need = need - (uint32_t)(incl - cnt);
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
    mask |= 255u << sh;
  }
  // prefix = the K-th largest key; take every key above it and the `need` lowest-index
  // keys equal to it
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (KPT > 0)
      return kget(j);
    else
      return order_key(sc[lo + j]);
  };
  int n_gt = 0, n_eq = 0;
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (lo + j < hi) {
        const uint32_t key = kget(j);
        n_gt += key > prefix;
        n_eq += key == prefix;
      }
  } else {
    for (int j = 0; lo + j < hi; ++j) {
      const uint32_t key = key_at(j);
      n_gt += key > prefix;
      n_eq += key == prefix;
    }
  }
  int tot = 0;
  const int eq_before = block_exclusive_scan(n_eq, wsum, &tot);
  const int take_eq = max(0, min(n_eq, (int)need - eq_before));
  int pos = block_exclusive_scan(n_gt + take_eq, wsum, &tot);
  int eq_seen = 0;
  // the score written back is the key's own float (bit-exact), not a reload
  auto put = [&](int pos, int j, uint32_t key) {
    if constexpr (REMAP)
      out_idx[pos] = rv[j];
    else
      out_idx[pos] = remap ? remap[lo + j] : offset + lo + j;
    if (out_sc) out_sc[pos] = key_float(key);
  };
  auto emit = [&](int j, uint32_t key) {
    bool take = key > prefix;
    if (key == prefix) {
      take = eq_seen < take_eq;
      ++eq_seen;
    }
    if (take && pos < n) put(pos++, j, key);  // the bound only guards the buffer
  };
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (lo + j < hi) emit(j, kget(j));
  } else {
    for (int j = 0; lo + j < hi; ++j) emit(j, key_at(j));
  }
}

// One query per workgroup, all its scores at once.
template <int KPT>
__global__ void __launch_bounds__(kIxSelThreads) indexer_topk_kernel(const float* __restrict__ scores, int S, int K,
                                                                     int32_t* __restrict__ idx) {
  const int b = blockIdx.x;
  topk_rows<KPT>(scores + (size_t)b * S, S, K, nullptr, 0, idx + (size_t)b * min(K, S), nullptr);
}

// Two-stage selection, stage 1: workgroup (g, b) keeps the K best keys of [g C, g C + C)
// of query b (every key of the query's top K is among its chunk's top K), as (score,
// index) pairs in index order at slots [g K, ...) of the query's G K candidate slots
// (only the last chunk can hold fewer than K).
template <int KPT>
__global__ void __launch_bounds__(kIxSelThreads) indexer_topk_chunk_kernel(const float* __restrict__ scores, int S,
                                                                           int K, int C, float* __restrict__ cand_sc,
                                                                           int32_t* __restrict__ cand_idx) {
  const int g = blockIdx.x, b = blockIdx.y, G = gridDim.x;
  const int lo = g * C, len = min(C, S - lo);
  const size_t slot = ((size_t)b * G + g) * K;
  topk_rows<KPT>(scores + (size_t)b * S + lo, len, K, nullptr, lo, cand_idx + slot, cand_sc + slot);
}

// Stage 2: the K best of a query's L candidates (in index order, so ties still go to the
// lower key and the output stays ascending).
template <int KPT>
__global__ void __launch_bounds__(kIxSelThreads) indexer_topk_merge_kernel(const float* __restrict__ cand_sc,
                                                                           const int32_t* __restrict__ cand_idx, int L,
                                                                           int stride, int K, int32_t* __restrict__ idx) {
  const int b = blockIdx.x;
  topk_rows<KPT, true>(cand_sc + (size_t)b * stride, L, K, cand_idx + (size_t)b * stride, 0,
                       idx + (size_t)b * min(K, L), nullptr);
}

}  // namespace
}  // namespace hymoe

namespace {

size_t ix_align(size_t v) { return (v + 255) & ~(size_t)255; }

int ix_check(int64_t B, int64_t H, int64_t D, int64_t S, int64_t K) {
  if (B < 0 || H <= 0 || D <= 0 || S < 0 || K < 1) return HY_MOE_ERR_INVALID_ARG;
  if (H != 32 || D != 128 || B > 65535 || S >= ((int64_t)1 << 31) / 128 || B * S >= ((int64_t)1 << 31))
    return HY_MOE_ERR_UNSUPPORTED;
  return HY_MOE_OK;
}

}  // namespace

extern "C" size_t hy_indexer_workspace_size(int64_t B, int64_t S) {
  using namespace hymoe;
  if (B < 0 || S < 0) return 0;
  // the scores, then the two-stage selection's candidates (G chunks x at most C each)
  const size_t n = (size_t)(B * S > 0 ? B * S : 1), nc = (size_t)B * (size_t)(S + kIxChunk);
  return ix_align(sizeof(float) * n) + ix_align(sizeof(float) * nc) + ix_align(sizeof(int32_t) * nc);
}

extern "C" int hy_indexer_topk(const void* q, const float* w, const void* keys, int64_t B, int64_t H, int64_t D,
                               int64_t S, int64_t K, int32_t* idx, float* scores, void* workspace,
                               size_t workspace_bytes, void* const* stage_events, void* stream) {
  using namespace hymoe;
  const int rc = ix_check(B, H, D, S, K);
  if (rc != HY_MOE_OK) return rc;
  if (B == 0 || S == 0) return HY_MOE_OK;
  if (!q || !w || !keys || !idx || !workspace) return HY_MOE_ERR_INVALID_ARG;
  if (((uintptr_t)q & 15) || ((uintptr_t)keys & 15) || ((uintptr_t)w & 3) || ((uintptr_t)idx & 3) ||
      ((uintptr_t)scores & 3) || ((uintptr_t)workspace & 255))
    return HY_MOE_ERR_INVALID_ARG;
  if (workspace_bytes < hy_indexer_workspace_size(B, S)) return HY_MOE_ERR_WORKSPACE;
  uint8_t* ws = (uint8_t*)workspace;
  float* sc = scores ? scores : (float*)ws;
  const size_t nc = (size_t)B * (size_t)(S + kIxChunk);
  float* cand_sc = (float*)(ws + ix_align(sizeof(float) * (size_t)(B * S)));
  int32_t* cand_idx = (int32_t*)((uint8_t*)cand_sc + ix_align(sizeof(float) * nc));
  hipStream_t s = (hipStream_t)stream;
  // optional profiling events: before the scores, after them, after the selection
  auto mark = [&](int i) {
    return (stage_events && stage_events[i]) ? hipEventRecord((hipEvent_t)stage_events[i], s) : hipSuccess;
  };
  if (mark(0) != hipSuccess) return HY_MOE_ERR_HIP;
  hipLaunchKernelGGL(indexer_scores_kernel<128>, dim3((unsigned)((S + kIxKeys - 1) / kIxKeys), (unsigned)B), dim3(256),
                     0, s, (const uint16_t*)q, w, (const uint16_t*)keys, (int)S, sc);
  if (hipGetLastError() != hipSuccess || mark(1) != hipSuccess) return HY_MOE_ERR_HIP;
  const int k = (int)(K < S ? K : S);
  const int64_t G = (S + kIxChunk - 1) / kIxChunk;
  const int64_t L = (G - 1) * k + std::min<int64_t>(k, S - (G - 1) * kIxChunk);  // candidates per query
  const dim3 blk(kIxSelThreads);
  if (G >= 4 && k <= kIxChunk && L <= kIxSelThreads * 32) {
    // two stages: G chunks per query select in parallel, then one merge per query
    hipLaunchKernelGGL(indexer_topk_chunk_kernel<kIxChunk / kIxSelThreads>, dim3((unsigned)G, (unsigned)B), blk, 0, s,
                       (const float*)sc, (int)S, k, kIxChunk, cand_sc, cand_idx);
    if (hipGetLastError() != hipSuccess) return HY_MOE_ERR_HIP;
    const int stride = (int)(G * k);
    if (L <= kIxSelThreads * 16)
      hipLaunchKernelGGL(indexer_topk_merge_kernel<16>, dim3((unsigned)B), blk, 0, s, (const float*)cand_sc,
                         (const int32_t*)cand_idx, (int)L, stride, k, idx);
    else
      hipLaunchKernelGGL(indexer_topk_merge_kernel<32>, dim3((unsigned)B), blk, 0, s, (const float*)cand_sc,
                         (const int32_t*)cand_idx, (int)L, stride, k, idx);
  } else if (S <= kIxSelThreads * kIxKeysPerThread) {
    hipLaunchKernelGGL(indexer_topk_kernel<kIxKeysPerThread>, dim3((unsigned)B), blk, 0, s, (const float*)sc, (int)S,
                       k, idx);
  } else {
    hipLaunchKernelGGL(indexer_topk_kernel<0>, dim3((unsigned)B), blk, 0, s, (const float*)sc, (int)S, k, idx);
  }
  if (hipGetLastError() != hipSuccess || mark(2) != hipSuccess) return HY_MOE_ERR_HIP;
  return HY_MOE_OK;
}

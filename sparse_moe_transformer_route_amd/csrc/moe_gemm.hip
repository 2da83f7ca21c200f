// moe_grouped_gemm: expert FFNs for prefill-sized batches as grouped GEMMs on bf16
// MFMA (32x32x16, fp32 accumulate).
//
// Each expert is a SwiGLU FFN y = W_down (silu(W_gate x) * (W_up x)) applied to the
// tokens routed to it (m.xxqk.cn Hy4 preview explainer, sections 2.1 and 2.2); the
// always-on shared expert (Tencent Hy4 preview model card) is scheduled as expert E
// over all T tokens.
//
// Phase 1 (gate/up): an item is (M tile, 128 hidden units), computed as 256 MFMA
// columns (the 128 gate rows and the matching 128 up rows of the weights) so that one
// lane holds gate and up of the same (row, unit) and writes h = silu(gate) * up as
// bf16. A rows are gathered straight from x through the permutation.
// Phase 2 (down): an item is (M tile, 256 output columns) over k = I; y is bf16.
//
// M tiles: an expert's rows are cut into tiles of 256 rows plus a remainder. A
// workgroup is 4 waves, one per SIMD; wave w owns the tile's 32-row blocks w and w+4
// and all 256 columns (256 fp32 accumulators in AGPRs), so activation rows are
// loaded once per workgroup.
//
// Pipeline, per 32-wide k step: the 256 x 32 weight tile arrives in LDS by direct
// global->LDS loads into an 8-stage ring (16-byte chunks XOR-swizzled by row, so the
// MFMA fragment reads are conflict free), seven steps ahead: a slot is refilled right
// after the barrier that certifies it was read. Each wave's activation rows come into
// a 4-slot register ring, three steps ahead. Every step issues the same loads (steps
// outside the range reload a clamped one) so single vector-memory counts cover all
// waits; the barrier is a bare s_barrier so loads of later steps stay in flight.
// Persistent schedule: items are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i mod 8); within an expert they are ordered so that the
// 32 workgroups running together on an XCD cover a block of up to 4 M tiles x 8-32
// N tiles and share activations and weights through that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kThreads = 256;   // 4 waves, one per SIMD
constexpr int kRowsMax = 256;   // rows per M tile
constexpr int kBlk = 32;        // rows per MFMA block (32x32x16)
constexpr int kWaveBlocks = 2;  // row blocks per wave (4 waves x 2 x 32 = 256), dealt round-robin
constexpr int kNB = 8;          // 32-column blocks per wave and tile (256 columns)
constexpr int kBK = 32;         // k per step (two 32x32x16 MFMAs deep)
constexpr int kStages = 8;      // weight ring in LDS, kStages - 1 steps ahead
constexpr int kASlots = 4;      // activation ring in registers
constexpr int kAhead = kASlots - 1;              // activation prefetch distance (steps)
constexpr int kBRows = 256;                      // weight rows per tile
constexpr int kRowBytes = kBK * 2;               // 64 B per weight row per step
constexpr int kStageBytes = kBRows * kRowBytes;  // 16 KB
constexpr int kDma = kStageBytes / 16 / kThreads;  // direct-to-LDS ops per thread per step (4)
constexpr int kLoadsPerStep = kDma + 2 * kWaveBlocks;  // vector-memory ops a wave issues per step (8)
// When step ks starts, B(ks) must have landed. It was the first op of step
// ks-(kStages-1); after it come that step's A loads and the ops of the kStages-2
// following steps.
constexpr int kWaitB = 2 * kWaveBlocks + (kStages - 2) * kLoadsPerStep;

int grouped_gemm_bm() { return kRowsMax; }

struct GemmArgs {
  const uint16_t* x;
  const int32_t* perm_src;
  const int32_t* offs;
  const int32_t* meta;
  const int4* tiles;
  int Tk, k, d, I, E;
};

#define HY_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// lgkmcnt(0): this wave's LDS reads are complete.
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier without a memory fence (a fence would wait for every load in
// flight); the empty asm statements keep the compiler from moving memory operations
// across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte chunk c (of 4) of a 64-byte B-tile row sits at physical chunk c ^ f(row). f
// spreads the 16 rows read by one fragment load over distinct bank groups whether LDS
// serves 8 lanes (128 B) or 16 lanes (256 B) of a 16-byte read per cycle.
__device__ __forceinline__ int swz_key(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <bool GATEUP>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GemmArgs a, ExpertWeights w,
                                                                   uint16_t* __restrict__ h,
                                                                   uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st3[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st4[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st5[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st6[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st7[kStageBytes];
  uint8_t* const stage[kStages] = {st0, st1, st2, st3, st4, st5, st6, st7};

  const int K = GATEUP ? a.d : a.I;
  const int NT = GATEUP ? a.I / (kBRows / 2) : (a.d + kBRows - 1) / kBRows;
  const int total = a.meta[1] * NT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int per = (total + 7) >> 3;
  const int lo = xcd * per;
  const int hi = min(total, lo + per);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept scalar
  const int r32 = lane & 31, hf = lane >> 5;
  const int nks = K / kBK;
  // per-lane part of a fragment read for k-substep s: row r32 of a 32-row block, chunk
  // 2*hf + s (lane half hf holds k [16hf, 16hf+16) of a step), swizzled; the key
  // depends only on r32 because blocks start at multiples of 32
  const uint32_t frag_lo[2] = {(uint32_t)(r32 * kRowBytes + (((2 * hf) ^ swz_key(r32)) << 4)),
                               (uint32_t)(r32 * kRowBytes + (((2 * hf + 1) ^ swz_key(r32)) << 4))};

  for (int item = lo + slot; item < hi; item += nslot) {
    // items of one expert (its c M tiles x NT N tiles) are ordered in blocks of up to
    // 4 M tiles, N tile major within a block, so the workgroups running together on
    // an XCD share both the activation rows and the weight tiles through its L2
    const int4 any = a.tiles[item / NT];
    const int g0 = any.w;
    const int c = (a.offs[any.x + 1] - a.offs[any.x] + kRowsMax - 1) / kRowsMax;
    const int MG = min(c, 4);
    const int l = item - g0 * NT;
    const int blk = l / (MG * NT);
    const int mgh = min(MG, c - blk * MG);
    const int r = l - blk * MG * NT;
    const int nt = r / mgh;
    const int mt = g0 + blk * MG + (r - nt * mgh);
    const int4 tile = a.tiles[mt];
    // tile fields are workgroup-uniform: keep them scalar so the per-block guards below
    // are scalar branches
    const int e = __builtin_amdgcn_readfirstlane(tile.x);
    const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
    const int mrows = __builtin_amdgcn_readfirstlane(tile.z);
    const int ebase = __builtin_amdgcn_readfirstlane(a.offs[e]);
    const int nrb = (mrows + kBlk - 1) / kBlk;
    const bool routed = e < a.E;

    // A: block j of this wave is tile block wv + 4j; lane row r32, k run [16hf, 16hf+16)
    // of a step (32 contiguous bytes); 32-bit element offsets from x (gate/up) or h (down)
    const uint16_t* abase = GATEUP ? a.x : h;
    uint32_t aoff[kWaveBlocks];
#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j) {
      const int rr = min((wv + 4 * j) * kBlk + r32, mrows - 1);
      const int grow = ebase + m0 + rr;
      aoff[j] = GATEUP ? (uint32_t)(row_token(grow, a.perm_src, a.Tk, a.k) * a.d + 16 * hf)
                       : (uint32_t)(grow * a.I + 16 * hf);
    }
    // B: stage chunk q = 256 i + 64 wv + lane holds row q>>2, physical chunk q&3.
    // gate/up: rows 0..127 are gate units nt*128.., rows 128..255 the matching up units
    // (ops i < kDma/2 read gate rows, the rest up rows); down: rows are output columns
    // nt*256.. (clamped past d; those columns are not stored)
    const uint16_t* bbase[kDma];
    uint32_t boff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int q = kThreads * i + 64 * wv + lane;
      const int br = q >> 2, lc = (q & 3) ^ swz_key(br);
      if (GATEUP) {
        const uint16_t* mat = i < kDma / 2 ? (routed ? w.gate + (size_t)e * a.I * a.d : w.s_gate)
                                           : (routed ? w.up + (size_t)e * a.I * a.d : w.s_up);
        bbase[i] = mat + (size_t)nt * (kBRows / 2) * a.d;
        boff[i] = (uint32_t)((br & (kBRows / 2 - 1)) * a.d + 8 * lc);
      } else {
        bbase[i] = routed ? w.down + (size_t)e * a.d * a.I : w.s_down;
        boff[i] = (uint32_t)(min(nt * kBRows + br, a.d - 1) * a.I + 8 * lc);
      }
    }

    f32x16 acc[kWaveBlocks][kNB];
#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][nb][i] = 0.f;
    uint4 ar[kASlots][kWaveBlocks][2];

    // Every step t issues B(t + kStages - 1) then A(t + kAhead); steps outside [0, nks)
    // load a clamped (in-range) step, so each step issues the same ops in the same
    // order and a single vector-memory count covers every wait.
    auto issue_a = [&](int ks, int u) {
      const int kk = min(max(ks, 0), nks - 1) * kBK;
#pragma unroll
      for (int j = 0; j < kWaveBlocks; ++j) {
        ar[u][j][0] = ldg16(abase + aoff[j] + kk);
        ar[u][j][1] = ldg16(abase + aoff[j] + kk + 8);
      }
    };
    auto issue_b = [&](int ks, int u) {
      const int kk = min(ks, nks - 1) * kBK;
      uint8_t* dst = stage[u] + (64 * wv) * 16;
#pragma unroll
      for (int i = 0; i < kDma; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bbase[i] + boff[i] + kk), HY_LDS(dst + kThreads * 16 * i),
                                         16, 0, 0);
    };

    // prologue: steps -(kStages-1)..-1 fill the B ring (and issue A(0..kAhead-1) plus
    // clamped duplicates, so the op pattern matches the steady state)
#pragma unroll
    for (int t = -(kStages - 1); t < 0; ++t) {
      issue_b(t + kStages - 1, t + kStages - 1);
      issue_a(t + kAhead, (t + kAhead + 2 * kASlots) % kASlots);
    }

    const int nsteps = (nks + kStages - 1) / kStages * kStages;
    // the k loop, with this wave's number of active row blocks fixed at compile time
    // (no branches around the MFMAs: they would make the compiler wait for every load)
    auto k_loop = [&](auto nact_tag) {
      constexpr int NACT = decltype(nact_tag)::value;
      for (int k0 = 0; k0 < nsteps; k0 += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) {
          const int ks = k0 + u;
          wait_vm<kWaitB>();  // own B(ks) landed
          wait_lds();         // own fragment reads of the previous step done
          bare_barrier();     // everyone's B(ks) landed; the previous step's slot is free
          issue_b(ks + kStages - 1, (u + kStages - 1) % kStages);
          issue_a(ks + kAhead, (u + kAhead) % kASlots);
          if (NACT > 0 && ks < nks) {
            const uint8_t* L = stage[u];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
              for (int q4 = 0; q4 < kNB / 4; ++q4) {
                uint4 bf[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                  bf[nb] = *reinterpret_cast<const uint4*>(&L[(4 * q4 + nb) * 32 * kRowBytes + frag_lo[sub]]);
#pragma unroll
                for (int j = 0; j < NACT; ++j)
#pragma unroll
                  for (int nb = 0; nb < 4; ++nb)
                    acc[j][4 * q4 + nb] = mfma32x32x16(ar[u % kASlots][j][sub], bf[nb], acc[j][4 * q4 + nb]);
              }
            }
          }
        }
      }
    };
    const int nact = (wv + 4 < nrb) ? 2 : (wv < nrb ? 1 : 0);
    if (nact == 2)
      k_loop(std::integral_constant<int, 2>{});
    else if (nact == 1)
      k_loop(std::integral_constant<int, 1>{});
    else
      k_loop(std::integral_constant<int, 0>{});
    // all waves are done with the ring before the next item refills it
    __builtin_amdgcn_s_waitcnt(0);
    bare_barrier();

#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j) {
      const int rb = wv + 4 * j;
      if (rb >= nrb) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // 32x32 accumulator i of lane (r32, hf): row 8(i/4) + 4hf + i%4, column r32
        const int rr = rb * kBlk + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (rr >= mrows) continue;
        const size_t grow = (size_t)(ebase + m0 + rr);
        if (GATEUP) {
#pragma unroll
          for (int nb = 0; nb < kNB / 2; ++nb) {
            const float hv = silu(acc[j][nb][i]) * acc[j][nb + kNB / 2][i];
            h[grow * a.I + nt * (kBRows / 2) + nb * 32 + r32] = (uint16_t)f32_to_bf16_bits(hv);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const int col = nt * kBRows + nb * 32 + r32;
            if (col < a.d) y[grow * a.d + col] = (uint16_t)f32_to_bf16_bits(acc[j][nb][i]);
          }
        }
      }
    }
  }
}

static int g_grid[2][64];  // persistent grid per (phase, device), 0 = not yet computed

static int persistent_grid(int phase, const void* kernel) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int gsz = __atomic_load_n(&g_grid[phase][dev], __ATOMIC_ACQUIRE);
  if (gsz > 0) return gsz;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess || occ <= 0) occ = 1;
  gsz = ((cus * occ + 7) / 8) * 8;
  __atomic_store_n(&g_grid[phase][dev], gsz, __ATOMIC_RELEASE);
  return gsz;
}

hipError_t launch_grouped_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                  Marks& m) {
  GemmArgs a{x, p.perm_src, p.offs, p.meta, p.tiles, p.Tk, p.k, p.d, p.I, p.E};
  const int g1 = persistent_grid(0, reinterpret_cast<const void*>(&grouped_gemm_kernel<true>));
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(g1), dim3(kThreads), 0, s, a, w, p.h, (uint16_t*)p.y);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  const int g2 = persistent_grid(1, reinterpret_cast<const void*>(&grouped_gemm_kernel<false>));
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(g2), dim3(kThreads), 0, s, a, w, p.h, (uint16_t*)p.y);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

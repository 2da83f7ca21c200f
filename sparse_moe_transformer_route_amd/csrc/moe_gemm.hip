// moe_grouped_gemm: expert FFNs for prefill-sized batches as grouped GEMMs on bf16
// MFMA (16x16x32, fp32 accumulate).
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
// workgroup is 8 waves, two per SIMD: 4 along M (16-row blocks dealt round-robin) x 2
// along N (128 columns each), so the tile is 256 x 256 with 128 accumulators a wave.
//
// Pipeline, per 32-wide k step: the 256 x 32 weight tile arrives in LDS by direct
// global->LDS loads into an 8-stage ring (16-byte chunks XOR-swizzled by row, so the
// MFMA fragment reads are conflict free), seven steps ahead; each wave's A rows come
// into a 4-slot register ring, three steps ahead (the two N-waves of a row block read
// the same rows, mostly from L1). Every step issues the same loads (steps past the end
// reload the last one) so a single vector-memory count covers all waits. Waits are explicit vector-memory counts
// followed by a plain workgroup barrier, so loads of later steps stay in flight.
// Persistent schedule: items are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i mod 8); within an expert they are ordered so that the
// ~32 workgroups running together on an XCD cover a block of up to 4 M tiles x 8-32
// N tiles and share activations and weights through that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kThreads = 512;   // 8 waves: 4 along M x 2 along N, two per SIMD
constexpr int kRowsMax = 256;   // rows per M tile
constexpr int kBlk = 16;        // rows per MFMA block
constexpr int kWaveBlocks = 4;  // row blocks per wave (4 M-waves x 4 x 16 = 256)
constexpr int kWaveNB = 8;      // 16-column blocks per wave (2 N-waves x 8 x 16 = 256)
constexpr int kBK = 32;         // k per step (one 16x16x32 MFMA deep)
constexpr int kStages = 8;      // weight ring in LDS: 7 steps ahead
constexpr int kASlots = 4;      // activation ring in registers: 3 steps ahead
constexpr int kAhead = kASlots - 1;
constexpr int kBRows = 256;                      // weight rows per tile
constexpr int kRowBytes = kBK * 2;               // 64 B per weight row per step
constexpr int kStageBytes = kBRows * kRowBytes;  // 16 KB
constexpr int kDma = kStageBytes / 16 / kThreads;  // direct-to-LDS ops per thread per step (2)
constexpr int kLoadsPerStep = kDma + kWaveBlocks;  // vector-memory ops a wave issues per step (6)

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

// B-tile row of local column block nb of a wave (before adding nwrow).
template <bool GATEUP>
__device__ __forceinline__ constexpr int row_of_block(int nb) {
  return GATEUP ? (nb < 4 ? 16 * nb : 128 + 16 * (nb - 4)) : 16 * nb;
}

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
  const int mw = wv & 3, nw = wv >> 2;
  const int r16 = lane & 15, g = lane >> 4;
  const int nks = K / kBK;
  // this wave's 8 column blocks, as B-tile rows: nwrow + kRowOf[nb] (gate/up: 4 gate
  // blocks then the 4 up blocks of the same hidden units; down: 8 consecutive blocks)
  const int nwrow = GATEUP ? 64 * nw : 128 * nw;
  // per-lane part of a fragment read: row r16 of a 16-row block, chunk g, swizzled
  // (the swizzle key depends only on r16 because blocks start at multiples of 16)
  const uint32_t frag_lo = (uint32_t)(r16 * kRowBytes + ((g ^ swz_key(r16)) << 4));

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
    const int e = tile.x, m0 = tile.y, mrows = tile.z;
    const int ebase = a.offs[e];
    const int nrb = (mrows + kBlk - 1) / kBlk;
    const bool routed = e < a.E;

    // A: block j of this wave is tile block mw + 4j; lane row r16, k run [8g, 8g+8) of
    // a step; 32-bit element offsets from x (gate/up) or h (down)
    const uint16_t* abase = GATEUP ? a.x : h;
    uint32_t aoff[kWaveBlocks];
#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j) {
      const int rr = min((mw + 4 * j) * kBlk + r16, mrows - 1);
      const int grow = ebase + m0 + rr;
      aoff[j] = GATEUP ? (uint32_t)(row_token(grow, a.perm_src, a.Tk, a.k) * a.d + 8 * g)
                       : (uint32_t)(grow * a.I + 8 * g);
    }
    // B: stage chunk q = 512 i + 64 wv + lane holds row q>>2, physical chunk q&3.
    // gate/up: rows 0..127 are gate units nt*128.., rows 128..255 the matching up units
    // (op i < kDma/2 reads gate rows, the rest up rows); down: rows are output columns
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

    f32x4 acc[kWaveBlocks][kWaveNB];
#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j)
#pragma unroll
      for (int nb = 0; nb < kWaveNB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 ar[kASlots][kWaveBlocks];

    // Step t issues B(t + kStages - 1) then A(t + kAhead); steps past the end reload
    // the last real step so every step issues the same number of vector-memory ops and
    // one count covers all waits: when step ks starts, the ops newer than A(ks) are
    // those of the kAhead - 1 steps issued after it, and B(ks) is older than A(ks).
    auto issue_a = [&](int ks, int u) {
      const int kk = min(ks, nks - 1) * kBK;
#pragma unroll
      for (int j = 0; j < kWaveBlocks; ++j) ar[u][j] = ldg16(abase + aoff[j] + kk);
    };
    auto issue_b = [&](int ks, int u) {
      const int kk = min(ks, nks - 1) * kBK;
      uint8_t* dst = stage[u] + (64 * wv) * 16;
#pragma unroll
      for (int i = 0; i < kDma; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bbase[i] + boff[i] + kk), HY_LDS(dst + kThreads * 16 * i),
                                         16, 0, 0);
    };

#pragma unroll
    for (int t = -(kStages - 1); t < 0; ++t) {
      issue_b(t + kStages - 1, t + kStages - 1);
      if (t + kAhead >= 0) issue_a(t + kAhead, t + kAhead);
    }

    const int nsteps = (nks + kStages - 1) / kStages * kStages;
    for (int k0 = 0; k0 < nsteps; k0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int ks = k0 + u;
        wait_vm<(kAhead - 1) * kLoadsPerStep>();
        wait_lds();
        bare_barrier();
        issue_b(ks + kStages - 1, (u + kStages - 1) % kStages);
        issue_a(ks + kAhead, (u + kAhead) % kASlots);
        if (ks < nks) {
          const uint8_t* L = stage[u] + nwrow * kRowBytes;
#pragma unroll
          for (int q4 = 0; q4 < kWaveNB / 4; ++q4) {
            uint4 bf[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              bf[nb] = *reinterpret_cast<const uint4*>(&L[row_of_block<GATEUP>(4 * q4 + nb) * kRowBytes + frag_lo]);
#pragma unroll
            for (int j = 0; j < kWaveBlocks; ++j) {
              if (mw + 4 * j < nrb) {
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                  acc[j][4 * q4 + nb] = mfma16x16x32(ar[u % kASlots][j], bf[nb], acc[j][4 * q4 + nb]);
              }
            }
          }
        }
      }
    }
    // all waves are done reading the ring before the next item refills it
    __builtin_amdgcn_s_waitcnt(0);
    bare_barrier();

#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j) {
      const int rb = mw + 4 * j;
      if (rb >= nrb) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = rb * kBlk + 4 * g + q;
        if (rr >= mrows) continue;
        const size_t grow = (size_t)(ebase + m0 + rr);
        if (GATEUP) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const float hv = silu(acc[j][nb][q]) * acc[j][nb + 4][q];
            h[grow * a.I + nt * (kBRows / 2) + (4 * nw + nb) * 16 + r16] = (uint16_t)f32_to_bf16_bits(hv);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < kWaveNB; ++nb) {
            const int col = nt * kBRows + (8 * nw + nb) * 16 + r16;
            if (col < a.d) y[grow * a.d + col] = (uint16_t)f32_to_bf16_bits(acc[j][nb][q]);
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

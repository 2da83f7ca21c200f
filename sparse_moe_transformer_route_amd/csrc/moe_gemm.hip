// moe_grouped_gemm: expert FFNs for prefill-sized batches as grouped GEMMs on bf16
// MFMA (32x32x16, fp32 accumulate).
//
// Each expert is a SwiGLU FFN y = W_down (silu(W_gate x) * (W_up x)) applied to the
// tokens routed to it (m.xxqk.cn Hy4 preview explainer, sections 2.1 and 2.2); the
// always-on shared expert (Tencent Hy4 preview model card) is scheduled as expert E
// over all T tokens.
//
// Phase 1 (gate/up): tile = 256 dispatched rows x 64 hidden units, computed as 128
// MFMA columns (64 gate rows and the 64 matching up rows of the weights) so that the
// epilogue holds gate and up of the same (row, unit) in one lane and writes
// h = silu(gate) * up as bf16. A rows are gathered straight from x through the
// permutation (no gathered copy of x is materialised).
// Phase 2 (down): tile = 256 rows x 128 output columns over k = I; y is bf16.
//
// Per 64-wide k step a workgroup (4 waves, 64 rows each) stages the 128 x 64 weight
// tile in LDS (double-buffered, 16-byte chunks XOR-swizzled by row so the fragment
// reads are bank-conflict free); each wave reads its own A rows directly into
// registers. Persistent schedule: work items (M tile, N tile) are split into 8
// contiguous ranges, one per XCD (workgroup i runs on XCD i mod 8), so the N tiles of
// one M tile and the M tiles of one expert run together and share that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kBM = 256;
constexpr int kBK = 64;

int grouped_gemm_bm() { return kBM; }

struct GemmArgs {
  const uint16_t* x;
  const int32_t* perm_src;
  const int32_t* offs;
  const int32_t* meta;
  const int2* tiles;
  int Tk, k, d, I, E;
};

__device__ __forceinline__ uint32_t swz(int row, int chunk) { return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4)); }

template <bool GATEUP>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(GemmArgs a, ExpertWeights w, uint16_t* __restrict__ h,
                                                           uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][128 * 128];
  const int K = GATEUP ? a.d : a.I;
  const int NT = GATEUP ? a.I / 64 : a.d / 128;
  const int total = a.meta[1] * NT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int per = (total + 7) >> 3;
  const int lo = xcd * per;
  const int hi = min(total, lo + per);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nks = K / kBK;

  for (int item = lo + slot; item < hi; item += nslot) {
    const int mt = item / NT, nt = item - mt * NT;
    const int2 tile = a.tiles[mt];
    const int e = tile.x, mrow0 = tile.y;
    const int ebase = a.offs[e];
    const int mrows = min(kBM, a.offs[e + 1] - ebase - mrow0);
    const bool routed = e < a.E;
    const bool active = 64 * wv < mrows;

    // A operand rows of this wave: lane owns row 32*mb + (lane&31), k half (lane>>5)
    const uint16_t* arow[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = min(64 * wv + 32 * mb + (lane & 31), mrows - 1);
      const int grow = ebase + mrow0 + r;
      if (GATEUP)
        arow[mb] = a.x + (size_t)row_token(grow, a.perm_src, a.Tk, a.k) * a.d + 32 * (lane >> 5);
      else
        arow[mb] = h + (size_t)grow * a.I + 32 * (lane >> 5);
    }
    // B tile: 128 weight rows x 64 k; thread loads 4 chunks of 16 bytes
    const uint16_t* bsrc[4];
    uint32_t bdst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = threadIdx.x + 256 * i;
      const int br = q >> 3, c = q & 7;
      const uint16_t* base;
      if (GATEUP) {
        const uint16_t* wgt = br < 64 ? (routed ? w.gate + (size_t)e * a.I * a.d : w.s_gate)
                                      : (routed ? w.up + (size_t)e * a.I * a.d : w.s_up);
        base = wgt + (size_t)(nt * 64 + (br & 63)) * a.d;
      } else {
        base = (routed ? w.down + (size_t)e * a.d * a.I : w.s_down) + (size_t)(nt * 128 + br) * a.I;
      }
      bsrc[i] = base + 8 * c;
      bdst[i] = swz(br, c);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

    uint4 breg[4], acur[2][4], anxt[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) breg[i] = ldg16(bsrc[i]);
    if (active) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int s = 0; s < 4; ++s) acur[mb][s] = ldg16(arow[mb] + 8 * s);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&lds[0][bdst[i]]) = breg[i];
    __syncthreads();

    for (int ks = 0; ks < nks; ++ks) {
      const bool more = ks + 1 < nks;
      if (more) {
#pragma unroll
        for (int i = 0; i < 4; ++i) breg[i] = ldg16(bsrc[i] + (ks + 1) * kBK);
        if (active) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s = 0; s < 4; ++s) anxt[mb][s] = ldg16(arow[mb] + (ks + 1) * kBK + 8 * s);
        }
      }
      if (active) {
        const uint8_t* L = lds[ks & 1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 bf[4];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int br = nb * 32 + (lane & 31);
            bf[nb] = *reinterpret_cast<const uint4*>(&L[swz(br, 4 * (lane >> 5) + s)]);
          }
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma32x32x16(acur[mb][s], bf[nb], acc[mb][nb]);
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&lds[(ks + 1) & 1][bdst[i]]) = breg[i];
        if (active) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s = 0; s < 4; ++s) acur[mb][s] = anxt[mb][s];
        }
      }
      __syncthreads();
    }

    if (active) {
      const int col = lane & 31;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 64 * wv + 32 * mb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (r >= mrows) continue;
          const size_t grow = (size_t)(ebase + mrow0 + r);
          if (GATEUP) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              const float hv = silu(acc[mb][nb][i]) * acc[mb][nb + 2][i];
              h[grow * a.I + nt * 64 + nb * 32 + col] = (uint16_t)f32_to_bf16_bits(hv);
            }
          } else {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              y[grow * a.d + nt * 128 + nb * 32 + col] = (uint16_t)f32_to_bf16_bits(acc[mb][nb][i]);
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0) != hipSuccess || occ <= 0) occ = 1;
  gsz = ((cus * occ + 7) / 8) * 8;
  __atomic_store_n(&g_grid[phase][dev], gsz, __ATOMIC_RELEASE);
  return gsz;
}

hipError_t launch_grouped_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                  Marks& m) {
  GemmArgs a{x, p.perm_src, p.offs, p.meta, p.tiles, p.Tk, p.k, p.d, p.I, p.E};
  const int g1 = persistent_grid(0, reinterpret_cast<const void*>(&grouped_gemm_kernel<true>));
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(g1), dim3(256), 0, s, a, w, p.h, (uint16_t*)p.y);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  const int g2 = persistent_grid(1, reinterpret_cast<const void*>(&grouped_gemm_kernel<false>));
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(g2), dim3(256), 0, s, a, w, p.h, (uint16_t*)p.y);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

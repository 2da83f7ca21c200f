// moe_stream: expert FFNs for decode-sized batches, where every touched expert has
// only a few tokens and the layer is bound by reading each touched expert's weights
// once from HBM.
//
// Each expert is a SwiGLU FFN, y = W_down (silu(W_gate x) * (W_up x)); the tokens of
// an expert are run through it in parallel (m.xxqk.cn Hy4 preview explainer, sections
// 2.1 "FFN 层拆分" and 2.2 "路由机制"); the shared expert is treated as expert E whose
// rows are all T tokens (Hy4 preview: 1 shared expert on every token, Tencent Hy4
// preview model card).
//
// Work split: one workgroup = one touched expert x 64 output rows; a wave owns 16 rows
// and streams them along k in 64-element chunks: lane (r, g) reads row r, bytes
// [32g, 32g+32) of each chunk, with several chunks in flight. The 16 rows x 16 tokens
// product runs on 16x16x32 bf16 MFMA with fp32 accumulation (experts with more than
// 16 tokens take several passes). Sherry-ternary experts are decoded in registers from 5-bit codes
// through a 32-entry LDS table into bf16 +-1/0 and scaled per row after the sum; FP8
// (E4M3) experts stream 128-code chunks (one 128-byte line per row: lane (r, g) reads
// bytes [32g, 32g+32)) for two 16-row blocks per wave, 128 rows per workgroup, are
// converted to bf16 in registers (exact) and scaled per row likewise.
#include "common.h"
#include "kernels.h"

namespace hymoe {

struct StreamArgs {
  const uint16_t* x;     // bf16 [T][d]
  const int32_t* touched;
  const int32_t* meta;
  const int32_t* offs;
  const int32_t* perm_src;
  int Tk, k, d, I, E;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Activation loads are unconditional: lanes of unused token columns point at a valid
// row (the expert's first token) and their output columns, which depend only on their
// own activations, are never stored. A load guarded by the lane's own condition would
// become a branch, after which the compiler can no longer count the loads in flight.

// ------------------------------------------------------------- bf16 experts
// Weight streaming with a register ring: each lane keeps kDepth chunks of loads in
// flight (per chunk: 2 x 16 bytes of each weight row it covers, and the matching
// activations). Activations ride in the same ring as the weights because the
// vector-memory counter retires loads in issue order: a shallower activation
// prefetch would make every wait also wait for the newer weight loads.
// Row-major weights take plain loads: one load instruction covers 16 rows x 64 bytes,
// half of every line it touches, and with a non-temporal hint the line is not kept for
// the other half (measured markedly slower). In the blocked layout one load instruction
// of a wave reads 1 KB in order (whole lines), and there the hint lifts the streaming
// rate from ~6.3 to ~7.0 TB/s (weights are read exactly once per layer).
constexpr int kKV = 2;                  // 16-byte loads per lane per matrix per chunk
constexpr int kChunk = 4 * kKV * 8;     // elements of a row per chunk (4 lane groups)
// Ring depths with non-temporal blocked loads (same-process A/B, decode T=32, gate/up
// depth / down depth: 5/3 1.800 ms, 3/5 1.788, 5/5 1.793, 6/5 1.776: within ~1%);
// depth 3 keeps gate/up at 148 registers, three waves per SIMD.
constexpr int kDepthGateUp = 3;         // chunks in flight, gate/up (two matrices)
constexpr int kDepthDown = 5;           // chunks in flight, down (one matrix)
// In the ternary kernels only the shared expert streams bf16: a shallow ring keeps their
// register count, and so the number of waves hiding the code-table lookups, in check.
constexpr int kDepthSharedTern = 2;
// FP8 experts: each wave covers two 16-row blocks that share every activation load
// (with one block the activation loads are half of all loads per weight byte: down was
// 14% slower). A chunk is 128 codes of a row, one whole 128-byte line, as in the bf16
// kernels: with 64-code chunks each load instruction took half lines and gate/up moved
// 5.0 TB/s instead of 6.0. Ring depths: 2 chunks for gate/up (2 waves per SIMD), 1 for
// down (4 waves per SIMD).
constexpr int kFp8RowBlocks = 2;
constexpr int kFp8Chunk = 128;
constexpr int kDepthFp8GateUp = 2;
constexpr int kDepthFp8Down = 1;

// Weight formats of the streaming kernels.
// kWfBf16Blk: bf16 in the blocked layout (2 KB per 16 rows x 64 columns, in lane order,
// moe_layout.hip): a wave's 16 rows of one 64-column chunk are one contiguous 2 KB run,
// the next chunk 2 KB further on; lane l's two loads of a chunk are its pieces l and 64 + l.
constexpr int kWfBf16 = 0, kWfTern = 1, kWfFp8 = 2, kWfBf16Blk = 3;
constexpr int kBlkChunk = 16 * kChunk;  // elements from one chunk of a row to the next, blocked layout

// Drives a register ring of D + 1 slots over n items in order: load(i, slot) issues
// the loads of item i into a slot, use(slot) consumes it, D items ahead of the loads.
// When n is a multiple of D + 1 the loop body has no branch (loads past the end fetch
// item n - 1 again, from cache), so the compiler can count the loads in flight and
// waits for exactly the item it consumes; a guarded prefetch would make it drain the
// whole ring once per period. Other n take uniform guards.
template <int D, class Load, class Use>
__device__ __forceinline__ void ring_stream(int n, Load&& load, Use&& use) {
  if (n % (D + 1) == 0) {
#pragma unroll
    for (int s = 0; s < D; ++s) load(min(s, n - 1), s);
    for (int c0 = 0; c0 < n; c0 += D + 1) {
#pragma unroll
      for (int u = 0; u <= D; ++u) {
        // sched_barrier(0): the scheduler would otherwise sink the loads below the
        // MFMAs (shorter live ranges) and shrink the ring
        load(min(c0 + u + D, n - 1), (u + D) % (D + 1));
        __builtin_amdgcn_sched_barrier(0);
        use(u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < D; ++s)
      if (s < n) load(s, s);
    for (int c0 = 0; c0 < n; c0 += D + 1) {
#pragma unroll
      for (int u = 0; u <= D; ++u) {
        if (c0 + u < n) {
          if (c0 + u + D < n) load(c0 + u + D, (u + D) % (D + 1));
          use(u);
        }
      }
    }
  }
}

// Weights of a lane: WS elements from one chunk to the next (kChunk row-major, kBlkChunk
// blocked), VS from its first 16-byte load of a chunk to its second (8 row-major, 512
// blocked); BLK: non-temporal loads (see above).
template <bool BLK>
__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  return BLK ? ldg16_stream(p) : ldg16(p);
}

template <int D, bool BLK = false>
__device__ __forceinline__ void gateup_bf16_block(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                  const uint16_t* __restrict__ xr, int d, f32x4& accg,
                                                  f32x4& accu) {
  constexpr int WS = BLK ? kBlkChunk : kChunk, VS = BLK ? 512 : 8;
  uint4 rg[D + 1][kKV], ru[D + 1][kKV], rx[D + 1][kKV];
  ring_stream<D>(
      d / kChunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          rg[slot][v] = ldw<BLK>(wg + ch * WS + VS * v);
          ru[slot][v] = ldw<BLK>(wu + ch * WS + VS * v);
          rx[slot][v] = ldg16(xr + ch * kChunk + 8 * v);
        }
      },
      [&](int u) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          accg = mfma16x16x32(rg[u][v], rx[u][v], accg);
          accu = mfma16x16x32(ru[u][v], rx[u][v], accu);
        }
      });
}

// The same for two 16-token passes at once (the shared expert, whose rows are all T
// tokens): each weight chunk is loaded once for both activation sets. Depth 2 keeps the
// ring at the routed path's register count.
template <int D, bool BLK>
__device__ __forceinline__ void gateup_bf16_block_x2(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                     const uint16_t* __restrict__ xr0, const uint16_t* __restrict__ xr1,
                                                     int d, f32x4 (&accg)[2], f32x4 (&accu)[2]) {
  constexpr int WS = BLK ? kBlkChunk : kChunk, VS = BLK ? 512 : 8;
  uint4 rg[D + 1][kKV], ru[D + 1][kKV], rx[D + 1][2][kKV];
  ring_stream<D>(
      d / kChunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          rg[slot][v] = ldw<BLK>(wg + ch * WS + VS * v);
          ru[slot][v] = ldw<BLK>(wu + ch * WS + VS * v);
          rx[slot][0][v] = ldg16(xr0 + ch * kChunk + 8 * v);
          rx[slot][1][v] = ldg16(xr1 + ch * kChunk + 8 * v);
        }
      },
      [&](int u) {
#pragma unroll
        for (int v = 0; v < kKV; ++v)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            accg[p] = mfma16x16x32(rg[u][v], rx[u][p][v], accg[p]);
            accu[p] = mfma16x16x32(ru[u][v], rx[u][p][v], accu[p]);
          }
      });
}

template <int D, bool BLK>
__device__ __forceinline__ void down_bf16_block_x2(const uint16_t* __restrict__ wd, const uint16_t* __restrict__ hr0,
                                                   const uint16_t* __restrict__ hr1, int I, f32x4 (&acc)[2]) {
  constexpr int WS = BLK ? kBlkChunk : kChunk, VS = BLK ? 512 : 8;
  uint4 rw[D + 1][kKV], rx[D + 1][2][kKV];
  ring_stream<D>(
      I / kChunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          rw[slot][v] = ldw<BLK>(wd + ch * WS + VS * v);
          rx[slot][0][v] = ldg16(hr0 + ch * kChunk + 8 * v);
          rx[slot][1][v] = ldg16(hr1 + ch * kChunk + 8 * v);
        }
      },
      [&](int u) {
#pragma unroll
        for (int v = 0; v < kKV; ++v)
#pragma unroll
          for (int p = 0; p < 2; ++p) acc[p] = mfma16x16x32(rw[u][v], rx[u][p][v], acc[p]);
      });
}

// ------------------------------------------------------------- FP8 experts
// Per chunk, lane group g loads the 32 codes of k [32 g, 32 g + 32) of each of its rows
// (two 16-byte loads) and the 32 matching activations (four); MFMA m of the chunk takes
// k [32 g + 8 m, +8) in every lane group, codes widened to bf16 right before it.
template <int D, int NR>
__device__ __forceinline__ void gateup_fp8_block(const uint8_t* const (&wg)[NR], const uint8_t* const (&wu)[NR],
                                                 const uint16_t* __restrict__ xr, int d, f32x4 (&accg)[NR],
                                                 f32x4 (&accu)[NR]) {
  uint4 rg[D + 1][NR][2], ru[D + 1][NR][2], rx[D + 1][4];
  ring_stream<D>(
      d / kFp8Chunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            rg[slot][r][v] = ldg16(wg[r] + ch * kFp8Chunk + 16 * v);
            ru[slot][r][v] = ldg16(wu[r] + ch * kFp8Chunk + 16 * v);
          }
#pragma unroll
        for (int m = 0; m < 4; ++m) rx[slot][m] = ldg16(xr + ch * kFp8Chunk + 8 * m);
      },
      [&](int u) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            accg[r] = mfma16x16x32(e4m3x8_bf16(rg[u][r][v].x, rg[u][r][v].y), rx[u][2 * v], accg[r]);
            accu[r] = mfma16x16x32(e4m3x8_bf16(ru[u][r][v].x, ru[u][r][v].y), rx[u][2 * v], accu[r]);
            accg[r] = mfma16x16x32(e4m3x8_bf16(rg[u][r][v].z, rg[u][r][v].w), rx[u][2 * v + 1], accg[r]);
            accu[r] = mfma16x16x32(e4m3x8_bf16(ru[u][r][v].z, ru[u][r][v].w), rx[u][2 * v + 1], accu[r]);
          }
      });
}

template <int D, int NR>
__device__ __forceinline__ void down_fp8_block(const uint8_t* const (&wd)[NR], const uint16_t* __restrict__ hr, int I,
                                               f32x4 (&acc)[NR]) {
  uint4 rw[D + 1][NR][2], rx[D + 1][4];
  ring_stream<D>(
      I / kFp8Chunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int v = 0; v < 2; ++v) rw[slot][r][v] = ldg16(wd[r] + ch * kFp8Chunk + 16 * v);
#pragma unroll
        for (int m = 0; m < 4; ++m) rx[slot][m] = ldg16(hr + ch * kFp8Chunk + 8 * m);
      },
      [&](int u) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            acc[r] = mfma16x16x32(e4m3x8_bf16(rw[u][r][v].x, rw[u][r][v].y), rx[u][2 * v], acc[r]);
            acc[r] = mfma16x16x32(e4m3x8_bf16(rw[u][r][v].z, rw[u][r][v].w), rx[u][2 * v + 1], acc[r]);
          }
      });
}

template <int D, bool BLK = false>
__device__ __forceinline__ void down_bf16_block(const uint16_t* __restrict__ wd, const uint16_t* __restrict__ hr,
                                                int I, f32x4& acc) {
  constexpr int WS = BLK ? kBlkChunk : kChunk, VS = BLK ? 512 : 8;
  uint4 rw[D + 1][kKV], rx[D + 1][kKV];
  ring_stream<D>(
      I / kChunk,
      [&](int ch, int slot) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          rw[slot][v] = ldw<BLK>(wd + ch * WS + VS * v);
          rx[slot][v] = ldg16(hr + ch * kChunk + 8 * v);
        }
      },
      [&](int u) {
#pragma unroll
        for (int v = 0; v < kKV; ++v) acc = mfma16x16x32(rw[u][v], rx[u][v], acc);
      });
}

// ---------------------------------------------------------- ternary experts
// 32-entry table: code -> four bf16 values (two packed dwords).
__device__ __forceinline__ void build_code_table(uint2* lut) {
  const int c = threadIdx.x;
  if (c < 32) {
    const int z = c & 3;
    uint32_t v[4];
    int nz = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q == z) {
        v[q] = 0u;
      } else {
        v[q] = ((c >> (2 + nz)) & 1) ? 0xBF80u : 0x3F80u;
        ++nz;
      }
    }
    lut[c] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
  }
}

// Ternary streaming with the same register ring as the bf16 path, over packed blocks of
// 128 weights (5 words, 1.25 bits per weight). The MFMA's k assignment gives lane
// group g the 32 weights [32g, 32g + 32) of a block, i.e. groups 8g .. 8g+7, whose 40
// code bits start at bit 40g: words (5g)/4 and (5g)/4 + 1, shifted right by 8g. Code
// bits [10m, 10m + 10) of that window are the two groups of k-step m (m < 4), decoded
// through the LDS table into the 8 bf16 weights of the MFMA's A operand; the matching
// activations are x[128 b + 32 g + 8 m, +8).
constexpr int kTernDepth = 3;  // blocks in flight (48 and 16 blocks per row divide by 4)
constexpr int kTernRowBlocks = 2;  // 16-row blocks per wave: a workgroup covers 128 rows

__device__ __forceinline__ uint4 tern_operand(uint64_t v, int m, const uint2* lut) {
  const uint2 lo = lut[(uint32_t)(v >> (10 * m)) & 31u];
  const uint2 hi = lut[(uint32_t)(v >> (10 * m + 5)) & 31u];
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

__device__ __forceinline__ uint64_t tern_window(const uint32_t* c, int g) {
  return ((uint64_t)c[0] | ((uint64_t)c[1] << 32)) >> (8 * g);
}

// NM weight matrices (gate and up, or down) x NR blocks of 16 rows against up to 16
// token columns; the row blocks share each activation operand. q[mi][r]: this lane's
// row in row block r of matrix mi, already offset by the lane's first code word; xr:
// this lane's token row offset by 32 g.
template <int NM, int NR, int D>
__device__ __forceinline__ void tern_rows_block(const uint32_t* const (*q)[NR], const uint16_t* __restrict__ xr,
                                                int nb, int g, const uint2* lut, f32x4 (*acc)[NR]) {
  uint32_t rc[D + 1][NM][NR][2];
  uint4 rx[D + 1][4];
  ring_stream<D>(
      nb,
      [&](int blk, int slot) {
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            rc[slot][mi][r][0] = q[mi][r][5 * blk];
            rc[slot][mi][r][1] = q[mi][r][5 * blk + 1];
          }
#pragma unroll
        for (int m = 0; m < 4; ++m) rx[slot][m] = ldg16(xr + 128 * blk + 8 * m);
      },
      [&](int u) {
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const uint64_t v = tern_window(rc[u][mi][r], g);
#pragma unroll
            for (int m = 0; m < 4; ++m)
              acc[mi][r] = mfma16x16x32(tern_operand(v, m, lut), rx[u][m], acc[mi][r]);
          }
      });
}

// ------------------------------------------------------------------ kernels
// Grid rows (blockIdx.y): in the ternary and FP8 kernels (128 rows per workgroup) the
// first ones each take one 16-token pass and one 64-row half of the shared expert (bf16
// there, and larger than a ternary or FP8 expert), so its passes run side by side from
// the start instead of one after another; in the bf16 kernels the shared expert has one
// row. Then one touched routed expert each (touched[0] is the shared expert).
__device__ __forceinline__ int shared_slots(const StreamArgs& a, bool tern) {
  return tern ? ((a.Tk / a.k + 15) / 16) * 2 : 1;
}

// bf16 kernels: three workgroups (waves per SIMD) per CU, the shared expert's two-pass
// path included
template <int WF>
__global__ void __launch_bounds__(256, (WF == kWfBf16 || WF == kWfBf16Blk) ? 3 : 1)
    stream_gateup_kernel(StreamArgs a, ExpertWeights w, uint16_t* __restrict__ h) {
  constexpr bool TERN = WF == kWfTern, FP8 = WF == kWfFp8, WIDE = TERN || FP8, BLK = WF == kWfBf16Blk;
  __shared__ uint2 lut[32];
  if (TERN) {
    build_code_table(lut);
    __syncthreads();
  }
  // plain scalars (a struct here ended up in scratch memory)
  const int sh = shared_slots(a, WIDE), slot = blockIdx.y;
  const bool shared_part = slot < sh;
  const int ridx = slot - sh + 1;
  if (!shared_part && ridx >= a.meta[0]) return;
  const int e = shared_part ? a.E : a.touched[ridx];
  // ternary and FP8 kernels: a shared-expert row takes one 16-token pass and one 64-row half
  const int cb_first = (WIDE && shared_part) ? 16 * (slot >> 1) : 0;
  const int sub_first = (WIDE && shared_part) ? (slot & 1) : 0;
  const int sub_last = WIDE ? (shared_part ? sub_first + 1 : 2) : 1;
  const int row0 = a.offs[e];
  const int n = (WIDE && shared_part) ? min(a.offs[e + 1] - row0, cb_first + 16) : a.offs[e + 1] - row0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int d = a.d, I = a.I;
  const bool routed = e < a.E;

  if (FP8 && routed) {
    // E4M3 routed expert: rows i0 + 16 r + r16 (r < NR), 16 token columns per pass, each
    // row's sums times its fp32 scale; D row 4g + j of block r is unit i0 + 16r + 4g + j
    constexpr int NR = kFp8RowBlocks;
    const int i0 = blockIdx.x * 128 + wv * 16 * NR;
    const uint8_t* wg[NR];
    const uint8_t* wu[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wg[r] = w.f8gate + ((size_t)e * I + i0 + 16 * r + r16) * d + 32 * g;
      wu[r] = w.f8up + ((size_t)e * I + i0 + 16 * r + r16) * d + 32 * g;
    }
    for (int cb = 0; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      const uint16_t* xr = a.x + (size_t)row_token(col, a.perm_src, a.Tk, a.k) * d + 32 * g;
      f32x4 accg[NR], accu[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) accg[r] = accu[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      gateup_fp8_block<kDepthFp8GateUp, NR>(wg, wu, xr, d, accg, accu);
      if (valid) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // the scales are read here, not kept across the ring (registers: occupancy)
            const size_t unit = (size_t)e * I + i0 + 16 * r + 4 * g + j;
            hv[j] = silu(accg[r][j] * w.f8sgate[unit]) * (accu[r][j] * w.f8sup[unit]);
          }
          *reinterpret_cast<uint2*>(h + (size_t)col * I + i0 + 16 * r + 4 * g) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
      }
    }
    return;
  }

  if (!TERN || !routed) {
    // bf16 weights: 64 rows per pass (a ternary-kernel workgroup covers 128 rows),
    // 16 token columns per pass
#pragma unroll 1
    for (int sub = sub_first; sub < sub_last; ++sub) {
    const int i0 = blockIdx.x * (WIDE ? 128 : 64) + sub * 64 + wv * 16;
    // row i0 + r16, columns [16 g, 16 g + 16) of each 64-column chunk: row-major, or in
    // block row i0 / 16 of the blocked layout pieces 16 g + r16 and 64 + 16 g + r16 (the
    // lane's pieces, in lane order: a load instruction reads 1 KB in order)
    const size_t roff = BLK ? (size_t)(i0 / 16) * (d / 64) * 1024 + 8 * lane : (size_t)(i0 + r16) * d + kKV * 8 * g;
    const uint16_t* wg = (routed ? w.gate + (size_t)e * I * d : w.s_gate) + roff;
    const uint16_t* wu = (routed ? w.up + (size_t)e * I * d : w.s_up) + roff;
    int cb = cb_first;
    if (!WIDE && !routed) {
      // the shared expert: two 16-token passes per weight stream
      for (; cb + 16 < n; cb += 32) {
        int col[2];
        bool valid[2];
        const uint16_t* xr[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          valid[p] = cb + 16 * p + r16 < n;
          col[p] = valid[p] ? row0 + cb + 16 * p + r16 : row0;
          xr[p] = a.x + (size_t)row_token(col[p], a.perm_src, a.Tk, a.k) * d + kKV * 8 * g;
        }
        f32x4 accg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, accu[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        gateup_bf16_block_x2<2, BLK>(wg, wu, xr[0], xr[1], d, accg, accu);
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (valid[p]) {
            uint2 v = make_uint2(pack_bf16x2(silu(accg[p][0]) * accu[p][0], silu(accg[p][1]) * accu[p][1]),
                                 pack_bf16x2(silu(accg[p][2]) * accu[p][2], silu(accg[p][3]) * accu[p][3]));
            *reinterpret_cast<uint2*>(h + (size_t)col[p] * I + i0 + 4 * g) = v;
          }
      }
    }
    for (; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      const uint16_t* xr = a.x + (size_t)row_token(col, a.perm_src, a.Tk, a.k) * d + kKV * 8 * g;
      f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
      gateup_bf16_block<WIDE ? kDepthSharedTern : kDepthGateUp, BLK>(wg, wu, xr, d, accg, accu);
      if (valid) {
        uint2 v = make_uint2(pack_bf16x2(silu(accg[0]) * accu[0], silu(accg[1]) * accu[1]),
                             pack_bf16x2(silu(accg[2]) * accu[2], silu(accg[3]) * accu[3]));
        *reinterpret_cast<uint2*>(h + (size_t)col * I + i0 + 4 * g) = v;
      }
    }
    }
    return;
  }

  // Sherry-ternary routed expert: rows i0 + 16 r + r16 (r < kTernRowBlocks), 16 token
  // columns per pass, scaled per row at the end
  constexpr int NR = kTernRowBlocks;
  const int i0 = blockIdx.x * 128 + wv * 16 * NR;
  const int nb = d / 128, wpr = nb * 5;
  const int w0 = (5 * g) >> 2;
  const uint32_t* q[2][NR];
  float sg[NR][4], su[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    q[0][r] = w.qgate + ((size_t)e * I + i0 + 16 * r + r16) * wpr + w0;
    q[1][r] = w.qup + ((size_t)e * I + i0 + 16 * r + r16) * wpr + w0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // D row 4g + j of row block r is hidden unit i0 + 16r + 4g + j
      sg[r][j] = bf16_bits_to_f32(w.sgate[(size_t)e * I + i0 + 16 * r + 4 * g + j]);
      su[r][j] = bf16_bits_to_f32(w.sup[(size_t)e * I + i0 + 16 * r + 4 * g + j]);
    }
  }
  for (int cb = 0; cb < n; cb += 16) {
    const bool valid = cb + r16 < n;
    const int col = valid ? row0 + cb + r16 : row0;
    const uint16_t* xr = a.x + (size_t)row_token(col, a.perm_src, a.Tk, a.k) * d + 32 * g;
    f32x4 acc[2][NR];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[mi][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    tern_rows_block<2, NR, kTernDepth>(q, xr, nb, g, lut, acc);
    if (valid) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[j] = silu(acc[0][r][j] * sg[r][j]) * (acc[1][r][j] * su[r][j]);
        *reinterpret_cast<uint2*>(h + (size_t)col * I + i0 + 16 * r + 4 * g) =
            make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      }
    }
  }
}

template <int WF>
__global__ void __launch_bounds__(256) stream_down_kernel(StreamArgs a, ExpertWeights w,
                                                          const uint16_t* __restrict__ h, float* __restrict__ y) {
  constexpr bool TERN = WF == kWfTern, FP8 = WF == kWfFp8, WIDE = TERN || FP8, BLK = WF == kWfBf16Blk;
  __shared__ uint2 lut[32];
  if (TERN) {
    build_code_table(lut);
    __syncthreads();
  }
  // plain scalars (a struct here ended up in scratch memory)
  const int sh = shared_slots(a, WIDE), slot = blockIdx.y;
  const bool shared_part = slot < sh;
  const int ridx = slot - sh + 1;
  if (!shared_part && ridx >= a.meta[0]) return;
  const int e = shared_part ? a.E : a.touched[ridx];
  // ternary and FP8 kernels: a shared-expert row takes one 16-token pass and one 64-row half
  const int cb_first = (WIDE && shared_part) ? 16 * (slot >> 1) : 0;
  const int sub_first = (WIDE && shared_part) ? (slot & 1) : 0;
  const int sub_last = WIDE ? (shared_part ? sub_first + 1 : 2) : 1;
  const int row0 = a.offs[e];
  const int n = (WIDE && shared_part) ? min(a.offs[e + 1] - row0, cb_first + 16) : a.offs[e + 1] - row0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int d = a.d, I = a.I;
  const bool routed = e < a.E;

  if (FP8 && routed) {
    // E4M3 routed expert: output rows m0 + 16 r + r16 (r < NR), sums times the rows'
    // fp32 scales
    constexpr int NR = kFp8RowBlocks;
    const int m0 = blockIdx.x * 128 + wv * 16 * NR;
    const uint8_t* wd[NR];
    float sd[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wd[r] = w.f8down + ((size_t)e * d + m0 + 16 * r + r16) * I + 32 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) sd[r][j] = w.f8sdown[(size_t)e * d + m0 + 16 * r + 4 * g + j];
    }
    for (int cb = 0; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      f32x4 acc[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      down_fp8_block<kDepthFp8Down, NR>(wd, h + (size_t)col * I + 32 * g, I, acc);
      if (valid) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
          *reinterpret_cast<float4*>(y + (size_t)col * d + m0 + 16 * r + 4 * g) =
              make_float4(acc[r][0] * sd[r][0], acc[r][1] * sd[r][1], acc[r][2] * sd[r][2], acc[r][3] * sd[r][3]);
      }
    }
    return;
  }

  if (!TERN || !routed) {
#pragma unroll 1
    for (int sub = sub_first; sub < sub_last; ++sub) {
    const int m0 = blockIdx.x * (WIDE ? 128 : 64) + sub * 64 + wv * 16;
    // (lane pieces of the blocked layout as in the gate/up kernel)
    const size_t roff = BLK ? (size_t)(m0 / 16) * (I / 64) * 1024 + 8 * lane : (size_t)(m0 + r16) * I + kKV * 8 * g;
    const uint16_t* wd = (routed ? w.down + (size_t)e * d * I : w.s_down) + roff;
    int cb = cb_first;
    if (!WIDE && !routed) {
      // the shared expert: two 16-token passes per weight stream
      for (; cb + 16 < n; cb += 32) {
        int col[2];
        bool valid[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          valid[p] = cb + 16 * p + r16 < n;
          col[p] = valid[p] ? row0 + cb + 16 * p + r16 : row0;
        }
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        down_bf16_block_x2<2, BLK>(wd, h + (size_t)col[0] * I + kKV * 8 * g, h + (size_t)col[1] * I + kKV * 8 * g, I,
                                   acc);
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (valid[p])
            *reinterpret_cast<float4*>(y + (size_t)col[p] * d + m0 + 4 * g) =
                make_float4(acc[p][0], acc[p][1], acc[p][2], acc[p][3]);
      }
    }
    for (; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      down_bf16_block<WIDE ? kDepthSharedTern : kDepthDown, BLK>(wd, h + (size_t)col * I + kKV * 8 * g, I, acc);
      if (valid)
        *reinterpret_cast<float4*>(y + (size_t)col * d + m0 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    }
    return;
  }

  // Sherry-ternary routed expert: output rows m0 + 16 r + r16 (r < kTernRowBlocks), 16
  // token columns per pass, scaled per row at the end
  constexpr int NR = kTernRowBlocks;
  const int m0 = blockIdx.x * 128 + wv * 16 * NR;
  const int nb = I / 128, wpr = nb * 5;
  const uint32_t* q[1][NR];
  float sd[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    q[0][r] = w.qdown + ((size_t)e * d + m0 + 16 * r + r16) * wpr + ((5 * g) >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) sd[r][j] = bf16_bits_to_f32(w.sdown[(size_t)e * d + m0 + 16 * r + 4 * g + j]);
  }
  for (int cb = 0; cb < n; cb += 16) {
    const bool valid = cb + r16 < n;
    const int col = valid ? row0 + cb + r16 : row0;
    f32x4 acc[1][NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[0][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    tern_rows_block<1, NR, kTernDepth>(q, h + (size_t)col * I + 32 * g, nb, g, lut, acc);
    if (valid) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        *reinterpret_cast<float4*>(y + (size_t)col * d + m0 + 16 * r + 4 * g) =
            make_float4(acc[0][r][0] * sd[r][0], acc[0][r][1] * sd[r][1], acc[0][r][2] * sd[r][2],
                        acc[0][r][3] * sd[r][3]);
    }
  }
}

// The shared expert (bf16, rows = all T tokens in order) beside the LDS-staged ternary
// kernels: one wave, 16 rows (gate/up: hidden units i0w..; down: output rows m0w..),
// token columns [cb, min(n, cb + 16)).
__device__ __forceinline__ void shared_gateup_pass(const StreamArgs& a, const ExpertWeights& w,
                                                   uint16_t* __restrict__ h, int i0w, int row0, int cb, int n) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int d = a.d;
  const uint16_t* wg = w.s_gate + (size_t)(i0w + r16) * d + kKV * 8 * g;
  const uint16_t* wu = w.s_up + (size_t)(i0w + r16) * d + kKV * 8 * g;
  const bool valid = cb + r16 < n;
  const int col = valid ? row0 + cb + r16 : row0;
  const uint16_t* xr = a.x + (size_t)row_token(col, a.perm_src, a.Tk, a.k) * d + kKV * 8 * g;
  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  gateup_bf16_block<kDepthSharedTern>(wg, wu, xr, d, accg, accu);
  if (valid)
    *reinterpret_cast<uint2*>(h + (size_t)col * a.I + i0w + 4 * g) =
        make_uint2(pack_bf16x2(silu(accg[0]) * accu[0], silu(accg[1]) * accu[1]),
                   pack_bf16x2(silu(accg[2]) * accu[2], silu(accg[3]) * accu[3]));
}

__device__ __forceinline__ void shared_down_pass(const StreamArgs& a, const ExpertWeights& w,
                                                 const uint16_t* __restrict__ h, float* __restrict__ y, int m0w,
                                                 int row0, int cb, int n) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int I = a.I;
  const uint16_t* wd = w.s_down + (size_t)(m0w + r16) * I + kKV * 8 * g;
  const bool valid = cb + r16 < n;
  const int col = valid ? row0 + cb + r16 : row0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  down_bf16_block<kDepthSharedTern>(wd, h + (size_t)col * I + kKV * 8 * g, I, acc);
  if (valid)
    *reinterpret_cast<float4*>(y + (size_t)col * a.d + m0w + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// ------------------------------------------- ternary experts, staged in LDS
// Routed Sherry experts when d and I are multiples of 512. Loading the operands
// straight into registers in the MFMA layout (above) puts 16 rows on consecutive
// lanes, so each lane quad touches four cache lines and the address unit, not HBM,
// bounds the kernel. Here a workgroup covers 256 code rows (gate/up: 128 hidden units
// of both matrices; down: 256 output rows) of one touched expert and walks k in
// chunks of 4 blocks (512 weights): the chunk's code bytes (80 B per row) and the
// pass's 4 activation rows (1 KB each) arrive in LDS by direct global->LDS loads
// with consecutive lanes on consecutive 16-byte pieces, in a 2-slot ring filled one
// chunk ahead; the four waves share the activations. The kernel is bound by latency
// (code-table lookups feeding each MFMA), so occupancy matters more than ring depth:
// 4 tokens per pass keep a slot at 24 KB and 3 workgroups fit per CU (decode experts
// have ~1.6 tokens; a 3-slot ring at 2 workgroups per CU measured 15-20% slower). The
// MFMA's other 12 token columns repeat token 3 and are not stored. Activation piece c
// of token slot t is stored at c ^ t, so a fragment read's token rows fall on
// distinct banks.
constexpr int kTlBlocks = 4;                             // 128-weight blocks per chunk
constexpr int kTlRows = 256;                             // code rows per workgroup
constexpr int kTlRowBytes = kTlBlocks * 20;              // code bytes per row per chunk
constexpr int kTlCodeBytes = kTlRows * kTlRowBytes;      // 20 KB
constexpr int kTlTok = 4;                                // tokens per pass
constexpr int kTlTokBytes = kTlBlocks * 128 * 2;         // activation bytes per token per chunk
constexpr int kTlXBytes = kTlTok * kTlTokBytes;          // 4 KB
constexpr int kTlSlot = kTlCodeBytes + kTlXBytes;        // 24 KB per ring slot
constexpr int kTlCodeOps = kTlCodeBytes / (256 * 16);    // 16-byte loads per thread per chunk: 5
constexpr int kTlWgPerCu = 3;                            // workgroups per CU (2 slots: 48 KB each)
// cache-policy operand of a load: non-temporal (blocked codes: each load op reads 1 KB in
// order, whole lines, and every code byte is read once per layer)
constexpr int kLoadNt = 2;
// one 1 KB activation piece per wave and token slot
static_assert(kTlCodeOps * 256 * 16 == kTlCodeBytes && kTlXBytes == 4 * 1024 && kTlTok == 4, "whole load ops");

bool tern_lds_eligible(const Plan& p, const ExpertWeights& w) {
  auto a16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  // (buffer resources address one expert's code matrix, I d 20 / 128 bytes, with 32-bit offsets)
  return w.ternary && p.d % 512 == 0 && p.I % 512 == 0 && a16(w.qgate) && a16(w.qup) && a16(w.qdown) &&
         (int64_t)p.I * (p.d / 128 * 20) < ((int64_t)1 << 31);
}

// NM = 2: gate and up (act = x through the permutation, out = h bf16, K = d);
// NM = 1: down (act = h rows, out = y fp32, K = I). Grid (rows / (256 / NM),
// shared slots + touched routed experts). The first grid rows run the bf16 shared
// expert, one 16-token pass and one 64-row quarter (down) or half (gate/up) of the
// workgroup's rows each, so that they start first and overlap the routed experts.
template <int NM>
__host__ __device__ constexpr int tern_shared_subs() { return kTlRows / NM / 64; }

// TB: code matrices in the blocked layout ([rows/16][K/512][16][80 B]): a 16-row group's
// chunk is one 1280-byte run and the next chunk of a row is 1280 bytes on.
template <int NM, bool TB>
__global__ void __launch_bounds__(256, kTlWgPerCu) tern_lds_kernel(StreamArgs a, ExpertWeights w,
                                                        const uint16_t* __restrict__ act, void* __restrict__ out) {
  __shared__ uint2 lut[32];
  __shared__ __attribute__((aligned(16))) uint8_t s0[kTlSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s1[kTlSlot];
  constexpr int SUBS = tern_shared_subs<NM>();
  const int T = a.Tk / a.k;
  const int sh = w.tshared ? (T + kTlTok - 1) / kTlTok : ((T + 15) / 16) * SUBS;
  if (!w.tshared && (int)blockIdx.y < sh) {
    const int pass = blockIdx.y / SUBS, sub = blockIdx.y - pass * SUBS;
    const int r0 = blockIdx.x * (kTlRows / NM) + sub * 64 + (threadIdx.x >> 6) * 16;
    if (NM == 2)
      shared_gateup_pass(a, w, reinterpret_cast<uint16_t*>(out), r0, a.offs[a.E], 16 * pass, T);
    else
      shared_down_pass(a, w, act, reinterpret_cast<float*>(out), r0, a.offs[a.E], 16 * pass, T);
    return;
  }
  // a Sherry-packed shared expert (expert E, all T tokens) takes the first grid rows, one
  // pass of kTlTok tokens each; then one touched routed expert per row (touched[0] is the
  // shared expert)
  const bool shared_row = (int)blockIdx.y < sh;
  const int ridx = blockIdx.y - sh + 1;
  if (!shared_row && ridx >= a.meta[0]) return;  // whole workgroup
  build_code_table(lut);
  __syncthreads();  // the table's LDS writes are visible to every wave before the first decode
  const int e = shared_row ? a.E : a.touched[ridx];
  const int row0 = a.offs[e];
  const int cb_first = shared_row ? kTlTok * (int)blockIdx.y : 0;
  const int n = shared_row ? min(a.offs[e + 1] - row0, cb_first + kTlTok) : a.offs[e + 1] - row0;
  const int K = NM == 2 ? a.d : a.I;
  const int R = NM == 2 ? a.I : a.d;  // rows of each matrix
  const int wpr = K / 128 * 5;        // code words per row
  const int rbase = blockIdx.x * (kTlRows / NM);
  const int nch = K / (128 * kTlBlocks);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;

  // Direct-to-LDS loads go through buffer resources (wave-uniform base and size, 32-bit
  // per-lane offsets): the compiler then counts LDS reads in order and waits only for
  // the ones an MFMA needs (with global_load_lds ops in flight it waits for every LDS
  // read). Code op i of wave wv fills LDS piece q = 5 wv + i (1 KB): pieces j = 64 q +
  // lane, workgroup code row j / 5, 16-byte piece j % 5 of the row's 80 chunk bytes
  // (LDS [row][80 B]). With NM = 2, waves 0-1 load gate rows and waves 2-3 up rows.
  const uint32_t* cm = (NM == 2 ? (wv >= 2 ? w.qup : w.qgate) : w.qdown) + (size_t)e * R * wpr;  // the expert's matrix
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(cm), (short)0, R * wpr * 4, kBufferRsrcWord3);
  int coff[kTlCodeOps];
#pragma unroll
  for (int i = 0; i < kTlCodeOps; ++i) {
    const int j = 64 * (5 * wv + i) + lane, row = j / 5, piece = j - 5 * row;
    const int mr = rbase + (NM == 2 ? (row & 127) : row);  // matrix row
    coff[i] = TB ? (mr / 16) * (K / 512) * 1280 + 80 * (mr % 16) + 16 * piece : mr * wpr * 4 + 16 * piece;
  }
  // this wave's row blocks: NM = 2: (gate, up) x 2 blocks of 16 units at rbase + 32 wv;
  // NM = 1: 4 blocks of 16 output rows at rbase + 64 wv
  auto crow = [&](int qb) { return NM == 2 ? (qb >> 1) * 128 + 32 * wv + 16 * (qb & 1) + r16 : 64 * wv + 16 * qb + r16; };
  const int w0 = (5 * g) >> 2;  // lane group g's first code word of a block
  float sc[4][4];               // row scales of the rows this lane's results belong to
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int orow = crow(qb) - r16 + 4 * g + j;  // D row 4g + j of the block
      const int mat = NM == 2 ? orow >> 7 : 0, rr = NM == 2 ? (orow & 127) : orow;
      const uint16_t* sp = NM == 2 ? (mat ? w.sup : w.sgate) : w.sdown;
      sc[qb][j] = bf16_bits_to_f32(sp[(size_t)e * R + rbase + rr]);
    }

  for (int cb = cb_first; cb < n; cb += kTlTok) {  // token passes (uniform)
    // activations: wave wv loads token slot wv of the pass (unused slots repeat a valid
    // row), lane l piece l of each chunk's 1 KB, stored at piece l ^ wv
    const int col = cb + wv < n ? row0 + cb + wv : row0 + cb_first;
    // (routed rows are below Tk: their token is perm_src / k; the shared expert's rows
    // follow in token order)
    const uint16_t* arow = NM == 2 ? act + (size_t)(col < a.Tk ? (uint32_t)a.perm_src[col] / (uint32_t)a.k
                                                               : (uint32_t)(col - a.Tk)) * a.d
                                   : act + (size_t)col * a.I;
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(arow), (short)0, K * 2, kBufferRsrcWord3);
    const int xoff = 16 * (lane ^ wv);
    auto issue = [&](int c, uint8_t* slot) {
      // (the LDS operand is the wave's base: lane l writes 16 bytes at base + 16 l)
#pragma unroll
      for (int i = 0; i < kTlCodeOps; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (__attribute__((address_space(3))) void*)(slot + 1024 * (5 * wv + i)),
                                                 16, coff[i], (TB ? 16 * kTlRowBytes : kTlRowBytes) * c, 0,
                                                 TB ? kLoadNt : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void*)(slot + kTlCodeBytes + 1024 * wv),
                                               16, xoff, kTlTokBytes * c, 0, 0);
    };
    f32x4 acc[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) acc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A chunk is 16 MFMA groups i = 4 b + qb (block b, row block qb), each 4 MFMAs. The
    // LDS reads run ahead in program order, fenced by scheduling barriers: group i+2's
    // code words, group i+1's table lookups and (in the second group of a block) the next
    // block's activations are issued before group i's MFMAs, so each MFMA waits for
    // lookups issued a whole group earlier rather than right before it.
    auto compute = [&](const uint8_t* slot) {
      constexpr int NG = 4 * kTlBlocks;
      const int tk = min(r16, kTlTok - 1);  // this lane's token column (repeats past the pass)
      const uint8_t* xs = slot + kTlCodeBytes + tk * kTlTokBytes;
      auto xload = [&](int b, uint4* xf) {
#pragma unroll
        for (int m = 0; m < 4; ++m) xf[m] = *reinterpret_cast<const uint4*>(xs + 16 * ((16 * b + 4 * g + m) ^ tk));
      };
      auto words = [&](int i, uint32_t* cw) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(slot + crow(i & 3) * kTlRowBytes + 20 * (i >> 2)) + w0;
        cw[0] = p[0];
        cw[1] = p[1];
      };
      auto decode = [&](const uint32_t* cw, uint4* op) {
        const uint64_t v = tern_window(cw, g);
#pragma unroll
        for (int m = 0; m < 4; ++m) op[m] = tern_operand(v, m, lut);
      };
      uint32_t cw[3][2];
      uint4 op[2][4], xf[2][4];
      xload(0, xf[0]);
      words(0, cw[0]);
      words(1, cw[1]);
      decode(cw[0], op[0]);
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < NG) words(i + 2, cw[(i + 2) % 3]);
        if (i + 1 < NG) decode(cw[(i + 1) % 3], op[(i + 1) & 1]);
        if ((i & 3) == 1 && (i >> 2) + 1 < kTlBlocks) xload((i >> 2) + 1, xf[((i >> 2) + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[i & 3] = mfma16x16x32(op[i & 1][m], xf[(i >> 2) & 1][m], acc[i & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // chunk c: its loads (issued a chunk earlier) landed everywhere and every wave is
    // done with chunk c-1, whose slot then receives chunk c+1 while chunk c computes
    auto step = [&](int c, const uint8_t* cur, uint8_t* nxt) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (gfx9 encoding, other counters untouched)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (c + 1 < nch) issue(c + 1, nxt);
      compute(cur);
    };
    issue(0, s0);
    for (int c = 0; c < nch; c += 2) {
      step(c, s0, s1);
      if (c + 1 < nch) step(c + 1, s1, s0);
    }
    if (r16 < kTlTok && cb + r16 < n) {
      const int col = row0 + cb + r16;
      if (NM == 2) {
        uint16_t* h = reinterpret_cast<uint16_t*>(out);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) hv[j] = silu(acc[r][j] * sc[r][j]) * (acc[2 + r][j] * sc[2 + r][j]);
          *reinterpret_cast<uint2*>(h + (size_t)col * a.I + rbase + 32 * wv + 16 * r + 4 * g) =
              make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
      } else {
        float* y = reinterpret_cast<float*>(out);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          *reinterpret_cast<float4*>(y + (size_t)col * a.d + rbase + 64 * wv + 16 * qb + 4 * g) =
              make_float4(acc[qb][0] * sc[qb][0], acc[qb][1] * sc[qb][1], acc[qb][2] * sc[qb][2],
                          acc[qb][3] * sc[qb][3]);
      }
    }
    __syncthreads();  // every wave is done with both slots before the next pass loads them
  }
}

hipError_t launch_stream_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                 Marks& m) {
  StreamArgs a{x, p.touched, p.meta, p.offs, p.perm_src, p.Tk, p.k, p.d, p.I, p.E};
  const int routed = p.Tk < p.E ? p.Tk : p.E;  // at most this many touched routed experts
  const int sh = (w.ternary || w.fp8) ? ((p.T + 15) / 16) * 2 : 1;
  const int passes = (p.T + 15) / 16;
  if (tern_lds_eligible(p, w)) {
    // LDS-staged ternary kernels, the shared expert's rows first in each grid (bf16: one
    // row per 16-token pass and row quarter; Sherry: one per kTlTok-token pass)
    const auto gu = w.tblocked ? tern_lds_kernel<2, true> : tern_lds_kernel<2, false>;
    const auto dn = w.tblocked ? tern_lds_kernel<1, true> : tern_lds_kernel<1, false>;
    const int tsh = (p.T + kTlTok - 1) / kTlTok;
    hipLaunchKernelGGL(gu, dim3(p.I / (kTlRows / 2), (w.tshared ? tsh : passes * tern_shared_subs<2>()) + routed),
                       dim3(256), 0, s, a, w, x, (void*)p.h);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess) err = m.mark(s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dn, dim3(p.d / kTlRows, (w.tshared ? tsh : passes * tern_shared_subs<1>()) + routed),
                       dim3(256), 0, s, a, w, (const uint16_t*)p.h, (void*)p.y);
    err = hipGetLastError();
    return err == hipSuccess ? m.mark(s) : err;
  }
  const int slots = routed + sh;
  // ternary and FP8 kernels: 128 rows per workgroup (d and I are multiples of 128)
  const int rows_wg = (w.ternary || w.fp8) ? 128 : 64;
  dim3 g1(p.I / rows_wg, slots), g2(p.d / rows_wg, slots);
  const auto gu = w.ternary ? stream_gateup_kernel<kWfTern>
                  : w.fp8   ? stream_gateup_kernel<kWfFp8>
                  : w.blocked ? stream_gateup_kernel<kWfBf16Blk>
                              : stream_gateup_kernel<kWfBf16>;
  const auto dn = w.ternary ? stream_down_kernel<kWfTern>
                  : w.fp8   ? stream_down_kernel<kWfFp8>
                  : w.blocked ? stream_down_kernel<kWfBf16Blk>
                              : stream_down_kernel<kWfBf16>;
  hipLaunchKernelGGL(gu, g1, dim3(256), 0, s, a, w, p.h);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dn, g2, dim3(256), 0, s, a, w, p.h, (float*)p.y);
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

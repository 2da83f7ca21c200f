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
// through a 32-entry LDS table into bf16 +-1/0 and scaled per row after the sum.
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

// ------------------------------------------------------------- bf16 experts
// Weight streaming with a register ring: each lane keeps kDepth chunks of loads in
// flight (per chunk: 2 x 16 bytes of each weight row it covers, and the matching
// activations). Activations ride in the same ring as the weights because the
// vector-memory counter retires loads in issue order: a shallower activation
// prefetch would make every wait also wait for the newer weight loads.
// Plain loads: non-temporal hints measured markedly slower on gfx950.
constexpr int kKV = 2;                  // 16-byte loads per lane per matrix per chunk
constexpr int kChunk = 4 * kKV * 8;     // elements of a row per chunk (4 lane groups)
constexpr int kDepthGateUp = 5;         // chunks in flight, gate/up (two matrices)
constexpr int kDepthDown = 7;           // chunks in flight, down (one matrix)

template <int D>
__device__ __forceinline__ void gateup_bf16_block(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                  const uint16_t* __restrict__ xr, bool xv, int d, f32x4& accg,
                                                  f32x4& accu) {
  const int nch = d / kChunk;
  uint4 rg[D + 1][kKV], ru[D + 1][kKV], rx[D + 1][kKV];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    if (s < nch) {
#pragma unroll
      for (int v = 0; v < kKV; ++v) {
        rg[s][v] = ldg16(wg + s * kChunk + 8 * v);
        ru[s][v] = ldg16(wu + s * kChunk + 8 * v);
        rx[s][v] = xv ? ldg16(xr + s * kChunk + 8 * v) : zero4();
      }
    }
  }
  for (int c0 = 0; c0 < nch; c0 += D + 1) {
#pragma unroll
    for (int u = 0; u <= D; ++u) {
      const int ch = c0 + u;
      if (ch < nch) {
        const int nx = ch + D;
        const int ns = (u + D) % (D + 1);
        if (nx < nch) {
#pragma unroll
          for (int v = 0; v < kKV; ++v) {
            rg[ns][v] = ldg16(wg + nx * kChunk + 8 * v);
            ru[ns][v] = ldg16(wu + nx * kChunk + 8 * v);
            rx[ns][v] = xv ? ldg16(xr + nx * kChunk + 8 * v) : zero4();
          }
        }
#pragma unroll
        for (int v = 0; v < kKV; ++v) {
          accg = mfma16x16x32(rg[u][v], rx[u][v], accg);
          accu = mfma16x16x32(ru[u][v], rx[u][v], accu);
        }
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void down_bf16_block(const uint16_t* __restrict__ wd, const uint16_t* __restrict__ hr,
                                                bool hv, int I, f32x4& acc) {
  const int nch = I / kChunk;
  uint4 rw[D + 1][kKV], rx[D + 1][kKV];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    if (s < nch) {
#pragma unroll
      for (int v = 0; v < kKV; ++v) {
        rw[s][v] = ldg16(wd + s * kChunk + 8 * v);
        rx[s][v] = hv ? ldg16(hr + s * kChunk + 8 * v) : zero4();
      }
    }
  }
  for (int c0 = 0; c0 < nch; c0 += D + 1) {
#pragma unroll
    for (int u = 0; u <= D; ++u) {
      const int ch = c0 + u;
      if (ch < nch) {
        const int nx = ch + D;
        const int ns = (u + D) % (D + 1);
        if (nx < nch) {
#pragma unroll
          for (int v = 0; v < kKV; ++v) {
            rw[ns][v] = ldg16(wd + nx * kChunk + 8 * v);
            rx[ns][v] = hv ? ldg16(hr + nx * kChunk + 8 * v) : zero4();
          }
        }
#pragma unroll
        for (int v = 0; v < kKV; ++v) acc = mfma16x16x32(rw[u][v], rx[u][v], acc);
      }
    }
  }
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

// 5-bit code of group q (0..31) of a 160-bit block held in w[0..4].
__device__ __forceinline__ uint32_t group_code(const uint32_t* w, int q) {
  const int bit = 5 * q;
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if (sh > 27) v |= w[wi + 1] << (32 - sh);
  return v & 31u;
}

// Accumulates one packed block (128 weights of this lane's row) against NCB token
// blocks; xr[c] points at the matching 128 activations of the lane's token.
template <int NCB>
__device__ __forceinline__ void ternary_block_mfma(const uint32_t* w, const uint2* lut, const uint16_t* const* xr,
                                                   const bool* xv, f32x4* acc) {
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const uint2 lo = lut[group_code(w, 2 * s)];
    const uint2 hi = lut[group_code(w, 2 * s + 1)];
    const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const uint4 b = xv[c] ? ldg16(xr[c] + 8 * s) : zero4();
      acc[c] = mfma16x16x32(a, b, acc[c]);
    }
  }
}

__device__ __forceinline__ void load_block5(const uint32_t* p, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < 5; ++i) w[i] = __builtin_nontemporal_load(p + i);
}

// ------------------------------------------------------------------ kernels
struct TokenCols {
  int col[2];
  bool valid[2];
};

__device__ __forceinline__ TokenCols token_cols(const StreamArgs& a, int row0, int n, int cb, int r16) {
  TokenCols tc;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int j = cb + 16 * c + r16;
    tc.valid[c] = j < n;
    tc.col[c] = tc.valid[c] ? row0 + j : row0;
  }
  return tc;
}

template <bool TERN>
__global__ void __launch_bounds__(256) stream_gateup_kernel(StreamArgs a, ExpertWeights w, uint16_t* __restrict__ h) {
  __shared__ uint2 lut[32];
  if (TERN) {
    build_code_table(lut);
    __syncthreads();
  }
  const int slot = blockIdx.y;
  if (slot >= a.meta[0]) return;
  const int e = a.touched[slot];
  const int row0 = a.offs[e], n = a.offs[e + 1] - row0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int i0 = blockIdx.x * 64 + wv * 16;
  const int d = a.d, I = a.I;
  const bool routed = e < a.E;

  if (!TERN || !routed) {
    // bf16 weights: 16 token columns per pass
    const uint16_t* wg = (routed ? w.gate + (size_t)e * I * d : w.s_gate) + (size_t)(i0 + r16) * d + kKV * 8 * g;
    const uint16_t* wu = (routed ? w.up + (size_t)e * I * d : w.s_up) + (size_t)(i0 + r16) * d + kKV * 8 * g;
    for (int cb = 0; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      const uint16_t* xr = a.x + (size_t)row_token(col, a.perm_src, a.Tk, a.k) * d + kKV * 8 * g;
      f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
      gateup_bf16_block<kDepthGateUp>(wg, wu, xr, valid, d, accg, accu);
      if (valid) {
        uint2 v = make_uint2(pack_bf16x2(silu(accg[0]) * accu[0], silu(accg[1]) * accu[1]),
                             pack_bf16x2(silu(accg[2]) * accu[2], silu(accg[3]) * accu[3]));
        *reinterpret_cast<uint2*>(h + (size_t)col * I + i0 + 4 * g) = v;
      }
    }
    return;
  }

  for (int cb = 0; cb < n; cb += 32) {
    const TokenCols tc = token_cols(a, row0, n, cb, r16);
    const bool two = n - cb > 16;
    f32x4 accg[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 accu[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const uint16_t* xrow[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) xrow[c] = a.x + (size_t)row_token(tc.col[c], a.perm_src, a.Tk, a.k) * d;
    {
      const int nb = d / 128, wpr = nb * 5;
      const uint32_t* qg = w.qgate + ((size_t)e * I + i0 + r16) * wpr;
      const uint32_t* qu = w.qup + ((size_t)e * I + i0 + r16) * wpr;
      for (int b0 = 0; b0 < nb; b0 += 4) {
        const int b = b0 + g;
        const bool bv = b < nb;
        uint32_t bg[5], bu[5];
        if (bv) {
          load_block5(qg + 5 * b, bg);
          load_block5(qu + 5 * b, bu);
        } else {
#pragma unroll
          for (int i = 0; i < 5; ++i) bg[i] = bu[i] = 0u;
        }
        const uint16_t* xr[2] = {xrow[0] + 128 * b, xrow[1] + 128 * b};
        const bool xv[2] = {tc.valid[0] && bv, tc.valid[1] && bv};
        if (two) {
          ternary_block_mfma<2>(bg, lut, xr, xv, accg);
          ternary_block_mfma<2>(bu, lut, xr, xv, accu);
        } else {
          ternary_block_mfma<1>(bg, lut, xr, xv, accg);
          ternary_block_mfma<1>(bu, lut, xr, xv, accu);
        }
      }
      // per-row scales: D row 4g+q is hidden unit i0 + 4g + q
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sg = bf16_bits_to_f32(w.sgate[(size_t)e * I + i0 + 4 * g + q]);
        const float su = bf16_bits_to_f32(w.sup[(size_t)e * I + i0 + 4 * g + q]);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          accg[c][q] *= sg;
          accu[c][q] *= su;
        }
      }
    }
    // h[row][i0 + 4g + q] = silu(gate) * up, as bf16
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c == 1 && !two) break;
      if (!tc.valid[c]) continue;
      const float h0 = silu(accg[c][0]) * accu[c][0];
      const float h1 = silu(accg[c][1]) * accu[c][1];
      const float h2 = silu(accg[c][2]) * accu[c][2];
      const float h3 = silu(accg[c][3]) * accu[c][3];
      uint2 v = make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
      *reinterpret_cast<uint2*>(h + (size_t)tc.col[c] * I + i0 + 4 * g) = v;
    }
  }
}

template <bool TERN>
__global__ void __launch_bounds__(256) stream_down_kernel(StreamArgs a, ExpertWeights w,
                                                          const uint16_t* __restrict__ h, float* __restrict__ y) {
  __shared__ uint2 lut[32];
  if (TERN) {
    build_code_table(lut);
    __syncthreads();
  }
  const int slot = blockIdx.y;
  if (slot >= a.meta[0]) return;
  const int e = a.touched[slot];
  const int row0 = a.offs[e], n = a.offs[e + 1] - row0;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * 64 + wv * 16;
  const int d = a.d, I = a.I;
  const bool routed = e < a.E;

  if (!TERN || !routed) {
    const uint16_t* wd = (routed ? w.down + (size_t)e * d * I : w.s_down) + (size_t)(m0 + r16) * I + kKV * 8 * g;
    for (int cb = 0; cb < n; cb += 16) {
      const bool valid = cb + r16 < n;
      const int col = valid ? row0 + cb + r16 : row0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      down_bf16_block<kDepthDown>(wd, h + (size_t)col * I + kKV * 8 * g, valid, I, acc);
      if (valid)
        *reinterpret_cast<float4*>(y + (size_t)col * d + m0 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    return;
  }

  for (int cb = 0; cb < n; cb += 32) {
    const TokenCols tc = token_cols(a, row0, n, cb, r16);
    const bool two = n - cb > 16;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      const int nb = I / 128, wpr = nb * 5;
      const uint32_t* qd = w.qdown + ((size_t)e * d + m0 + r16) * wpr;
      for (int b0 = 0; b0 < nb; b0 += 4) {
        const int b = b0 + g;
        const bool bv = b < nb;
        uint32_t bw[5];
        if (bv) {
          load_block5(qd + 5 * b, bw);
        } else {
#pragma unroll
          for (int i = 0; i < 5; ++i) bw[i] = 0u;
        }
        const uint16_t* hr[2] = {h + (size_t)tc.col[0] * I + 128 * b, h + (size_t)tc.col[1] * I + 128 * b};
        const bool hv[2] = {tc.valid[0] && bv, tc.valid[1] && bv};
        if (two)
          ternary_block_mfma<2>(bw, lut, hr, hv, acc);
        else
          ternary_block_mfma<1>(bw, lut, hr, hv, acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sd = bf16_bits_to_f32(w.sdown[(size_t)e * d + m0 + 4 * g + q]);
        acc[0][q] *= sd;
        acc[1][q] *= sd;
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c == 1 && !two) break;
      if (!tc.valid[c]) continue;
      *reinterpret_cast<float4*>(y + (size_t)tc.col[c] * d + m0 + 4 * g) =
          make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    }
  }
}

hipError_t launch_stream_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                 Marks& m) {
  StreamArgs a{x, p.touched, p.meta, p.offs, p.perm_src, p.Tk, p.k, p.d, p.I, p.E};
  const int slots = (p.Tk < p.E ? p.Tk : p.E) + 1;
  dim3 g1(p.I / 64, slots), g2(p.d / 64, slots);
  if (w.ternary) {
    hipLaunchKernelGGL(stream_gateup_kernel<true>, g1, dim3(256), 0, s, a, w, p.h);
  } else {
    hipLaunchKernelGGL(stream_gateup_kernel<false>, g1, dim3(256), 0, s, a, w, p.h);
  }
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = m.mark(s);
  if (err != hipSuccess) return err;
  if (w.ternary) {
    hipLaunchKernelGGL(stream_down_kernel<true>, g2, dim3(256), 0, s, a, w, p.h, (float*)p.y);
  } else {
    hipLaunchKernelGGL(stream_down_kernel<false>, g2, dim3(256), 0, s, a, w, p.h, (float*)p.y);
  }
  err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

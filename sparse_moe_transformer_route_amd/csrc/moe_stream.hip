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
// and streams them along k, 32 contiguous bytes per lane per weight matrix per 64-wide
// step... in 128-wide chunks: lane (r, g) reads row r, bytes [64g, 64g+64) of the chunk.
// The 16 rows x up-to-32 tokens product runs on 16x16x32 bf16 MFMA with fp32
// accumulation. Sherry-ternary experts are decoded in registers from 5-bit codes
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
template <int NCB>
__device__ __forceinline__ void gateup_bf16_block(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                  const uint16_t* const* xr, const bool* xv, int d, f32x4* accg,
                                                  f32x4* accu) {
  uint4 cg[4], cu[4], cx[NCB][4];
  uint4 ng[4], nu[4], nx[NCB][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    cg[s] = ldg16_stream(wg + 8 * s);
    cu[s] = ldg16_stream(wu + 8 * s);
#pragma unroll
    for (int c = 0; c < NCB; ++c) cx[c][s] = xv[c] ? ldg16(xr[c] + 8 * s) : zero4();
  }
  for (int kk = 128; kk <= d; kk += 128) {
    const bool more = kk < d;
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ng[s] = ldg16_stream(wg + kk + 8 * s);
        nu[s] = ldg16_stream(wu + kk + 8 * s);
#pragma unroll
        for (int c = 0; c < NCB; ++c) nx[c][s] = xv[c] ? ldg16(xr[c] + kk + 8 * s) : zero4();
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        accg[c] = mfma16x16x32(cg[s], cx[c][s], accg[c]);
        accu[c] = mfma16x16x32(cu[s], cx[c][s], accu[c]);
      }
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        cg[s] = ng[s];
        cu[s] = nu[s];
#pragma unroll
        for (int c = 0; c < NCB; ++c) cx[c][s] = nx[c][s];
      }
    }
  }
}

template <int NCB>
__device__ __forceinline__ void down_bf16_block(const uint16_t* __restrict__ wd, const uint16_t* const* hr,
                                                const bool* hv, int I, f32x4* acc) {
  uint4 cw[4], cx[NCB][4], nw[4], nx[NCB][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    cw[s] = ldg16_stream(wd + 8 * s);
#pragma unroll
    for (int c = 0; c < NCB; ++c) cx[c][s] = hv[c] ? ldg16(hr[c] + 8 * s) : zero4();
  }
  for (int kk = 128; kk <= I; kk += 128) {
    const bool more = kk < I;
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        nw[s] = ldg16_stream(wd + kk + 8 * s);
#pragma unroll
        for (int c = 0; c < NCB; ++c) nx[c][s] = hv[c] ? ldg16(hr[c] + kk + 8 * s) : zero4();
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[c] = mfma16x16x32(cw[s], cx[c][s], acc[c]);
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        cw[s] = nw[s];
#pragma unroll
        for (int c = 0; c < NCB; ++c) cx[c][s] = nx[c][s];
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

  for (int cb = 0; cb < n; cb += 32) {
    const TokenCols tc = token_cols(a, row0, n, cb, r16);
    const bool two = n - cb > 16;
    f32x4 accg[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 accu[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const uint16_t* xrow[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) xrow[c] = a.x + (size_t)row_token(tc.col[c], a.perm_src, a.Tk, a.k) * d;

    if (!TERN || !routed) {
      const uint16_t* wg = (routed ? w.gate + (size_t)e * I * d : w.s_gate) + (size_t)(i0 + r16) * d + 32 * g;
      const uint16_t* wu = (routed ? w.up + (size_t)e * I * d : w.s_up) + (size_t)(i0 + r16) * d + 32 * g;
      const uint16_t* xr[2] = {xrow[0] + 32 * g, xrow[1] + 32 * g};
      if (two)
        gateup_bf16_block<2>(wg, wu, xr, tc.valid, d, accg, accu);
      else
        gateup_bf16_block<1>(wg, wu, xr, tc.valid, d, accg, accu);
    } else {
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

  for (int cb = 0; cb < n; cb += 32) {
    const TokenCols tc = token_cols(a, row0, n, cb, r16);
    const bool two = n - cb > 16;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (!TERN || !routed) {
      const uint16_t* wd = (routed ? w.down + (size_t)e * d * I : w.s_down) + (size_t)(m0 + r16) * I + 32 * g;
      const uint16_t* hr[2] = {h + (size_t)tc.col[0] * I + 32 * g, h + (size_t)tc.col[1] * I + 32 * g};
      if (two)
        down_bf16_block<2>(wd, hr, tc.valid, I, acc);
      else
        down_bf16_block<1>(wd, hr, tc.valid, I, acc);
    } else {
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

// moe_combine: the merge of expert outputs into the layer output (m.xxqk.cn Hy4
// preview explainer, section 2.2 "路由机制": the selected experts' results are merged
// as the layer's output), plus the always-on shared expert (Tencent Hy4 preview model
// card):
//   out[t] = bf16( sum_j w[t][j] * y[pos(t, j)] + y_shared[t] )
// summed in fp32 over the slots in ascending expert order and rounded once to nearest
// even. Each output element is owned by one thread, so the sum order is fixed.
#include "common.h"
#include "kernels.h"

namespace hymoe {

__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// bf16 expert outputs (grouped path): every y row is read once, and a wave reads 1 KB of
// it in order, so the loads take the non-temporal hint (T=8192: ~25 us off the combine's
// ~0.21 ms; results unchanged)
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 a = ldg16_stream(p);
  const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(u[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
  }
}

// One workgroup = one token x 8 NT output columns, 8 consecutive columns per thread.
// fp32 y (streaming path, a decode batch of a few tokens): 128 threads, so the few
// tokens still spread over many CUs. bf16 y (grouped path, thousands of tokens): 768
// threads, a whole 6144-column row per workgroup, so each y row is read in one 12 KB
// run (T=8192: 0.165 -> 0.157 ms against 128 threads; 768 threads on the fp32 path:
// 6.1 -> 7.0 us at T=32).
template <typename YT>
constexpr int combine_threads() {
  return sizeof(YT) == 4 ? 128 : 768;
}

template <typename YT>
__global__ void __launch_bounds__(combine_threads<YT>()) combine_kernel(const YT* __restrict__ y,
                                                                         const int32_t* __restrict__ pos,
                                                                         const float* __restrict__ topk_w, int k,
                                                                         int d, int Tk, uint16_t* __restrict__ out) {
  constexpr int NT = combine_threads<YT>();
  const int t = blockIdx.x;
  const int c = blockIdx.y * (8 * NT) + threadIdx.x * 8;
  if (c >= d) return;
  const int32_t* pp = pos + (size_t)t * k;
  const float* ww = topk_w + (size_t)t * k;
  float s[8];  // the shared expert's row, loaded first (added last)
  load8(y + (size_t)(Tk + t) * d + c, s);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // slots in groups of 4 with all 4 rows in flight before they are added, then the
  // remaining slots one by one; ascending slot order throughout
  int j = 0;
  for (; j + 4 <= k; j += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(y + (size_t)pp[j + u] * d + c, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wj = ww[j + u];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[u][i], acc[i]);
    }
  }
  for (; j < k; ++j) {
    const float wj = ww[j];
    float v[8];
    load8(y + (size_t)pp[j] * d + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[i], acc[i]);
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0] + s[0], acc[1] + s[1]);
  o.y = pack_bf16x2(acc[2] + s[2], acc[3] + s[3]);
  o.z = pack_bf16x2(acc[4] + s[4], acc[5] + s[5]);
  o.w = pack_bf16x2(acc[6] + s[6], acc[7] + s[7]);
  *reinterpret_cast<uint4*>(out + (size_t)t * d + c) = o;
}

hipError_t launch_combine(const Plan& p, bool y_is_f32, uint16_t* out, hipStream_t s, Marks& m) {
  if (y_is_f32) {
    constexpr int nt = combine_threads<float>();
    hipLaunchKernelGGL(combine_kernel<float>, dim3(p.T, (p.d + 8 * nt - 1) / (8 * nt)), dim3(nt), 0, s,
                       (const float*)p.y, p.pos, p.topk_w, p.k, p.d, p.Tk, out);
  } else {
    constexpr int nt = combine_threads<uint16_t>();
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(p.T, (p.d + 8 * nt - 1) / (8 * nt)), dim3(nt), 0, s,
                       (const uint16_t*)p.y, p.pos, p.topk_w, p.k, p.d, p.Tk, out);
  }
  hipError_t err = hipGetLastError();
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

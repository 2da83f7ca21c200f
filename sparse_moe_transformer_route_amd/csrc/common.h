// Device helpers shared by the MoE layer's HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Rows per expert-block in the dispatch masks (one bit per token of a block).
constexpr int kMaskBlock = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D[16x16] += A[16x32] B[32x16]; lane l holds row (l&15) of A, column (l&15) of B and
// column (l&15), rows 4*(l>>4)+[0,4) of D. Each lane's 8 k-values of A and B sit at the
// same k positions, so any fixed assignment of k to (lane>>4, element) is a valid
// reduction order: the kernels use it to load longer contiguous runs per lane.
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D[32x32] += A[32x16] B[16x32]; lane l holds row (l&31) of A, column (l&31) of B and
// column (l&31) of D, rows 8*(i/4) + 4*(l>>5) + (i%4) for accumulator i.
__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Fourth word of a raw buffer resource (no index stride, no swizzle): data format
// 32-bit (field value 4 at bit 15), the value CDNA buffer loads expect for untyped
// byte-addressed access.
constexpr int kBufferRsrcWord3 = 0x00020000;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// D[32x32] += A[32x64] B[64x32] on E4M3 codes with E8M0 block scales sa (A) and sb (B)
// (byte 0 of each; 127 = 1). Lane (r, h) holds row / column r: bytes 0-15 are k
// [16h, 16h + 16) and bytes 16-31 are k [32 + 16h, 32 + 16h + 16) of the 64, and the scale
// of 32-k block b of row / column r comes from lane (r, b). D as the bf16 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma32x32x64_f8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming load of data read exactly once (expert weights): non-temporal hint.
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Wave-wide inclusive prefix sum (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Row r of the dispatched row space -> token index. Rows [0, T*k) are the routed
// (token, slot) pairs in expert-contiguous order; rows [T*k, T*k+T) belong to the
// shared expert in token order.
__device__ __forceinline__ int row_token(int r, const int* __restrict__ perm_src, int Tk, int k) {
  return r < Tk ? perm_src[r] / k : r - Tk;
}

// Eight FP8 E4M3 codes (code i in byte i of lo, hi) to eight bf16 values with the gfx950
// conversion instruction; every E4M3 value, subnormals included, is a bf16 value, so the
// conversion is exact (NaN codes give NaN).
template <bool HI>  // codes 0-1 or 2-3 of the word
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, HI));
}
__device__ __forceinline__ uint4 e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  return make_uint4(e4m3x2_bf16<false>(lo), e4m3x2_bf16<true>(lo), e4m3x2_bf16<false>(hi), e4m3x2_bf16<true>(hi));
}

// ---- MXFP8 (OCP Microscaling v1.0): blocks of 32 values share a scale 2^e (E8M0 byte
// e + 127), e = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero block);
// elements are E4M3 (nearest, ties to even) of v * 2^-e saturated to +-448.

// The block exponent e of a block whose largest magnitude is amax (finite).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 9;  // frexp exponent - 1 = floor(log2 amax)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values scaled by 2^-e to four E4M3 codes in one word (value i in byte i).
__device__ __forceinline__ uint32_t mx_pack4(float v0, float v1, float v2, float v3, int e) {
  auto q = [e](float v) { return __builtin_amdgcn_fmed3f(__builtin_ldexpf(v, -e), -448.f, 448.f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q(v0), q(v1), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q(v2), q(v3), lo, true);
}

}  // namespace hymoe

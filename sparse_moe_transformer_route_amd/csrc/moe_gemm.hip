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
// M tiles: an expert's rows are cut into near-equal tiles of at most 256 rows (whole
// 32-row blocks). A workgroup is 4 waves, one per SIMD, in a 2 x 2 layout: wave
// (wm, wn) owns the 32-row blocks 2j + wm (j < 4, dealt alternately so a short tile
// keeps both M-waves busy) and the 128 columns [128 wn, 128 wn + 128) of the 256 x 256
// tile: 256 fp32 accumulators in AGPRs.
//
// Pipeline, per 64-wide k step: the step's 256 activation rows and 256 weight rows
// (128 B each: one cache line per row, so the vector L1's limited number of
// outstanding misses carries twice the bytes of 64-byte pieces) arrive in LDS by
// direct global->LDS loads into two rings of 32 KB slots: 2 activation slots and 3
// weight slots (all 160 KB: the weights come from HBM and get more lead than the
// activations, mostly L2 hits). 16-byte chunks are XOR-swizzled by row so the MFMA
// fragment reads are conflict free. Activation rows are gathered from x through the
// permutation (gate/up) or read from h (down). Only LDS-bound loads are in flight in
// the k loop, so the vector-memory wait is an explicit count. A step runs 4 MFMA
// groups (k = 16 each), each group's fragments read while the previous group's MFMAs
// run; at the end of the step one bare barrier certifies that the next step has
// landed and that this step's slots are free. Their next loads (the activations of
// the step after next, the weights of the step after that) go out in 4-op pieces
// between the following step's MFMA groups, so the address unit works through them
// while MFMAs run.
// Persistent schedule: items are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i mod 8) and claimed in order through per-XCD counters, so
// workgroups that finish early take more work; within an expert, items are ordered so
// that the workgroups running together on an XCD cover a block of up to 4 M tiles x
// 8-32 N tiles and share activations and weights through that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hymoe {

constexpr int kThreads = 256;   // 4 waves, one per SIMD
constexpr int kRowsMax = 256;   // rows per M tile
constexpr int kBlk = 32;        // rows per MFMA block (32x32x16)
constexpr int kWaveBlocks = 4;  // row blocks per wave (2 M-waves x 4 x 32 = 256)
constexpr int kNB = 4;          // 32-column blocks per wave (2 N-waves x 4 x 32 = 256)
constexpr int kBK = 64;         // k per step (four 32x32x16 MFMAs deep); K % (2 kBK) == 0
constexpr int kSub = kBK / 16;  // MFMA groups per step
constexpr int kRowBytes = kBK * 2;               // 128 B per row per step
constexpr int kHalf = kRowsMax * kRowBytes;      // 32 KB: one operand's ring slot
constexpr int kDma = kHalf / 16 / kThreads;      // direct-to-LDS ops per operand per thread per step (8)
// Sherry ternary weights: a row's 64 weights of a k step are 16 five-bit codes (10
// bytes at byte 10 ks of the row); each row gets a 16-byte line of a 4 KB code slot
// holding the 3 words from byte 4 floor(10 ks / 4) (the codes start at bit 16 (ks % 2)
// of them), loaded with 4 one-word direct-to-LDS ops per thread per step.
constexpr int kCodePitch = 16;
constexpr int kCodeSlot = kRowsMax * kCodePitch;  // 4 KB
constexpr int kCodeOps = kCodeSlot / 4 / kThreads;  // 4
constexpr int kScaleBytes = 512;                    // an item's 256 row scales (bf16)
// FP8 (E4M3) weights: a row's 64 codes of a k step (4 pieces of 16 bytes) go to the
// row's 64-byte line of a 16 KB slot, piece p at p ^ f8_key(row). The k order within a
// step is permuted for FP8 (activations alike) so that each lane's codes for MFMA groups
// 2q and 2q + 1 are one piece: one 16-byte LDS read per two groups, conflict free,
// converted to bf16 (exact) right before each group's MFMAs.
constexpr int kF8Pitch = 64;
constexpr int kF8Slot = kRowsMax * kF8Pitch;         // 16 KB
constexpr int kF8Ops = kF8Slot / 16 / kThreads;      // 4 direct-to-LDS ops per thread per step
constexpr int kF8ScaleBytes = kRowsMax * 4;          // an item's 256 row scales (fp32)
static_assert(kF8Ops == kCodeOps, "the code and FP8 load offsets share storage");

// Weight formats of the routed experts' tiles. kGemmW8A8: FP8 weights and MXFP8
// activations on the FP8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4): a k step is
// 128 codes (128 bytes per row, as the bf16 step's 64 values), two MFMA groups of 64;
// the activations' E8M0 block scales reach the MFMAs from registers.
// kGemmBf16Blk: bf16 weights in the blocked layout (2 KB per 16 rows x 64 columns, pieces
// in lane order, blk_piece): a step's weight slot holds the tile's 16 blocks of that step
// as they are in memory (block g of the slot: tile rows 16 g .. 16 g + 15), so each load
// op copies 1 KB in order (half a block), and a fragment read (32 rows of one 16-byte
// column piece) takes two runs of 256 contiguous bytes: no conflicts without a swizzle.
// kGemmTernBlk: Sherry codes in the blocked layout ([rows/16][K/512][16][80 B]): the
// ternary kernel with row r's window of step ks at 1280 ((r / 16) K/512 + ks / 8) +
// 80 (r % 16) + 4 floor(10 (ks % 8) / 4) instead of K/128 20 r + 4 floor(10 ks / 4).
constexpr int kGemmBf16 = 0, kGemmTern = 1, kGemmFp8 = 2, kGemmW8A8 = 3, kGemmBf16Blk = 4, kGemmTernBlk = 5;
constexpr int kBK8 = 128;        // W8A8: k per step
constexpr int kSub8 = kBK8 / 64;  // W8A8: MFMA groups per step

// Blocked bf16 layout: the 16-byte piece of row r (< 16) holding its columns
// [8 q, 8 q + 8) of a 64-column slab is piece 64 (q % 2) + 16 (q / 2) + r of the slab's
// 2 KB block.
__device__ __forceinline__ uint32_t blk_piece(int r, int q) {
  return 64u * (uint32_t)(q & 1) + 16u * (uint32_t)(q >> 1) + (uint32_t)r;
}

// Two 16-byte LDS reads into one 8-register operand.
__device__ __forceinline__ i32x8 lds_pair(const uint8_t* p0, const uint8_t* p1) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p0);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}


int grouped_gemm_bm() { return kRowsMax; }

struct GemmArgs {
  const uint16_t* x;
  // W8A8: this launch's activation codes and block scales (gate/up: the token rows,
  // [T][d] and [T][d / 32]; down: the routed hidden rows, [T k][I] and [T k][I / 32]) and,
  // for gate/up, where the hidden rows' codes and scales go
  const uint8_t* aq;
  const uint8_t* as;
  uint8_t* hq;
  uint8_t* hs;
  const int32_t* perm_src;
  const int32_t* offs;
  int32_t* meta;  // [1] M tiles, [2] routed M tiles; [kMetaSched..] per-XCD work counters, zeroed by the
                  // routing kernels
  const int4* tiles;
  int Tk, k, d, I, E;
  int sel;  // M tiles to run: 0 every one, 1 the routed experts', 2 the shared expert's
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

// 16-byte chunk c (of 8) of a 128-byte row sits at physical chunk c ^ ((row / 2) % 8).
// The LDS has 64 banks of 4 bytes and serves a 16-byte read 16 lanes at a time; the 16
// rows of one such group fall pairwise (even, odd row) on the two 128-byte halves of
// the banks, and the key gives each pair a different chunk: no conflicts. (A key of
// row % 8 puts rows r and r + 8 on the same banks: every fragment read took twice
// as long.)
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }

// FP8 piece swizzle: the 16 lanes of a 16-byte LDS read (rows r..r+15, one logical piece)
// fall on 16 distinct bank quads; without it, on 4 (8-byte reads of the unpermuted order
// measured ~3 conflict cycles per LDS instruction).
__device__ __forceinline__ int f8_key(int row) { return (row >> 2) & 3; }

// Two floats to packed bf16 (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each;
// the result is rounded to bf16 right after). Large negative z gives -0, large
// positive z gives z.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * z));
}

// Calls f(integral_constant<int, T>) for T in the sequence, in order.
template <int... T, class F>
__device__ __forceinline__ void for_seq(std::integer_sequence<int, T...>, F&& f);

// The 5-bit code at bit P of a 3-word window (P + 5 <= 96).
template <int P>
__device__ __forceinline__ uint32_t code5(const uint32_t (&w)[3]) {
  constexpr int W = P / 32, O = P % 32;
  static_assert(P >= 0 && P + 5 <= 96, "code position");
  if constexpr (O <= 27)
    return (w[W] >> O) & 31u;
  else
    return __builtin_amdgcn_alignbit(w[W + 1], w[W], O) & 31u;
}

// bf16 pair to floats.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Scheduling pattern for one MFMA group's region: MFMA, global load, MFMA, global
// load, ..., then MFMA, LDS read, ..., then the rest, so the loads and reads issue
// while the MFMA pipe is busy instead of ahead of the group's first MFMA (loads first:
// measured ~1% faster than reads first; spreading them evenly was slower).
template <int NMFMA, int NREAD, int NVMEM>
__device__ __forceinline__ void interleave_group() {
  constexpr int N = NMFMA > NREAD + NVMEM ? NMFMA : NREAD + NVMEM;
  for_seq(std::make_integer_sequence<int, N>{}, [&](auto i_tag) {
    constexpr int I = decltype(i_tag)::value;
    if constexpr (I < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (I < NVMEM)
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // vector memory
    else if constexpr (I - NVMEM < NREAD)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  });
}

// Calls f(integral_constant<int, T>) for T in the sequence, in order.
template <int... T, class F>
__device__ __forceinline__ void for_seq(std::integer_sequence<int, T...>, F&& f) {
  (f(std::integral_constant<int, T>{}), ...);
}

// TAILR = (K / kBK) mod 6 (0, 2 or 4: K is a multiple of 128): the k loop runs whole
// periods of the 2 x 3 slot pattern and ends with a tail of that many steps.
// WF = kGemmTern: routed experts' weights are Sherry ternary codes with bf16 row scales
// (the shared expert's tiles run in the bf16 kernel); each lane decodes the codes of
// its B fragments through a 32-entry LDS table into bf16 +1/0/-1, and the scales are
// applied in the epilogue. WF = kGemmFp8: E4M3 codes with fp32 row scales, converted
// to bf16 per fragment, scales likewise in the epilogue.
template <bool GATEUP, int TAILR, int WF>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GemmArgs a, ExpertWeights w,
                                                                   uint16_t* __restrict__ h,
                                                                   uint16_t* __restrict__ y) {
  constexpr bool TERN = WF == kGemmTern || WF == kGemmTernBlk, FP8 = WF == kGemmFp8, A8 = WF == kGemmW8A8,
                 BLK = WF == kGemmBf16Blk, TB = WF == kGemmTernBlk;
  constexpr int BS = 3;  // weight (or code) ring slots
  constexpr int kBOps = TERN ? kCodeOps : FP8 ? kF8Ops : kDma;  // weight-side load ops per thread per step
  constexpr int BKE = A8 ? kBK8 : kBK;     // k per step (128 bytes per row either way)
  // Separate LDS arrays rather than one carved buffer: the compiler tells direct-to-LDS
  // loads and LDS reads of different arrays apart; within one array it would wait for
  // every such load in flight before each LDS read.
  uint8_t *sa0, *sa1, *sb0 = nullptr, *sb1 = nullptr;  // activation slots; sb0, sb1: epilogue pieces 2, 3
  uint8_t* sr[3];                  // weight (bf16, FP8) or code (ternary) ring slots
  uint2* lut = nullptr;            // ternary: the code table
  uint8_t* ssc = nullptr;          // ternary, FP8: the item's row scales
  if constexpr (FP8) {
    // the down epilogue stages its 4 pieces in two rounds through the activation slots
    __shared__ __attribute__((aligned(16))) uint8_t fa0[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t fa1[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t fr0[kF8Slot];
    __shared__ __attribute__((aligned(16))) uint8_t fr1[kF8Slot];
    __shared__ __attribute__((aligned(16))) uint8_t fr2[kF8Slot];
    __shared__ __attribute__((aligned(16))) uint8_t fsc[kF8ScaleBytes];
    sa0 = fa0, sa1 = fa1;
    sr[0] = fr0, sr[1] = fr1, sr[2] = fr2;
    ssc = fsc;
  } else if constexpr (TERN) {
    __shared__ __attribute__((aligned(16))) uint8_t ta0[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t ta1[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t te0[GATEUP ? 16 : kHalf];  // the down epilogue only
    __shared__ __attribute__((aligned(16))) uint8_t te1[GATEUP ? 16 : kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t tc0[kCodeSlot];
    __shared__ __attribute__((aligned(16))) uint8_t tc1[kCodeSlot];
    __shared__ __attribute__((aligned(16))) uint8_t tc2[kCodeSlot];
    __shared__ __attribute__((aligned(16))) uint8_t tsc[kScaleBytes];
    __shared__ uint2 tlut[32];
    sa0 = ta0, sa1 = ta1, sb0 = te0, sb1 = te1;
    sr[0] = tc0, sr[1] = tc1, sr[2] = tc2;
    lut = tlut, ssc = tsc;
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t ba0[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t ba1[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t bb0[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t bb1[kHalf];
    __shared__ __attribute__((aligned(16))) uint8_t bb2[kHalf];
    sa0 = ba0, sa1 = ba1, sb0 = bb0, sb1 = bb1;
    sr[0] = bb0, sr[1] = bb1, sr[2] = bb2;
  }
  uint8_t* const sa[2] = {sa0, sa1};
  uint8_t* const* const sb = sr;
  if constexpr (TERN) {
    // code -> four bf16 values: bits 0-1 the position of the zero, bits 2-4 the signs
    // of the other three in order (1 = negative)
    const int c = threadIdx.x;
    if (c < 32) {
      uint32_t v[4];
      int nz = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q == (c & 3)) {
          v[q] = 0u;
        } else {
          v[q] = ((c >> (2 + nz)) & 1) ? 0xBF80u : 0x3F80u;
          ++nz;
        }
      }
      lut[c] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
    }
  }
  // the claimed item is handed to the workgroup through the first activation slot,
  // idle between items
  int* const next_item = reinterpret_cast<int*>(sa0);

  const int K = GATEUP ? a.d : a.I;
  const int NT = GATEUP ? a.I / (kRowsMax / 2) : (a.d + kRowsMax - 1) / kRowsMax;
  const int t_lo = a.sel == 2 ? a.meta[2] : 0;  // this launch's M tiles [t_lo, t_hi)
  const int t_hi = a.sel == 1 ? a.meta[2] : a.meta[1];
  const int total = (t_hi - t_lo) * NT;
  const int xcd = blockIdx.x & 7;
  const int per = (total + 7) >> 3;
  int32_t* const counters = a.meta + kMetaSched + (GATEUP ? 0 : 8) + (a.sel == 2 ? 16 : 0);
  // Items are split into 8 contiguous ranges, one per XCD; a workgroup takes the next
  // item of its own XCD's range (so the items in flight on an XCD are neighbours), and
  // once that range is used up, the next unclaimed item of another XCD's range.
  // steal: the next unclaimed item of the other XCDs' ranges, or -1
  auto steal = [&]() -> int {
    for (int t = 1; t < 8; ++t) {
      const int x = (xcd + t) & 7;
      const int lo = x * per, hi = min(total, lo + per);
      if (lo >= hi) continue;
      const int v = atomicAdd(&counters[x], 1);
      if (lo + v < hi) return lo + v;
    }
    return -1;
  };
  // v: the value an atomic increment of this XCD's own counter returned
  auto own_or_steal = [&](int v) -> int {
    const int lo = xcd * per, hi = min(total, lo + per);
    return lo + v < hi ? lo + v : steal();
  };
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept scalar
  const int wm = wv & 1, wn = wv >> 1;
  const int nks = K / BKE;
  const uint32_t fa_off = wm * kBlk * kRowBytes;              // block 2j + wm
  const uint32_t fb_off = wn * (kRowsMax / 2) * kRowBytes;    // columns 128 wn..

  // Thread 0 claims each item during the previous item's last k step (the atomic's
  // latency hides behind that step's MFMAs; its result is read after the k loop) and
  // hands it over through LDS between items.
  int claimed = 0, own_ticket = 0;
  if (threadIdx.x == 0) claimed = own_or_steal(atomicAdd(&counters[xcd], 1));
  for (;;) {
    if (threadIdx.x == 0) *next_item = claimed;
    __syncthreads();
    const int claim = __builtin_amdgcn_readfirstlane(*next_item);  // uniform: kept scalar
    __syncthreads();  // everyone has read it before the slot is loaded
    if (claim < 0) break;
    const int item = claim + t_lo * NT;
    // The thread index is made opaque once per item so that per-lane address math is
    // redone per item (a few ALU ops) rather than hoisted out of the item loop, where it
    // would be spilled across the k loop and reloaded with full vector-memory waits.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int r32 = lane & 31, hf = lane >> 5;
    // per-lane part of a fragment read for k group s: row r32 of a 32-row block, chunk
    // 2s + hf (lane half hf holds k [8(2s+hf), 8(2s+hf)+8) of the step), swizzled; the key
    // depends only on r32 because blocks start at multiples of 32
    // (FP8: group s and half hf take chunk 4 (s / 2) + 2 hf + s % 2 instead of 2 s + hf,
    // the same bijection of the step's 8 chunks for activations and weights)
    uint32_t frag_lo[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      const int c = FP8 ? 4 * (s >> 1) + 2 * hf + (s & 1) : 2 * s + hf;
      frag_lo[s] = (uint32_t)(r32 * kRowBytes + ((c ^ swz_key(r32)) << 4));
    }
    // blocked weights: piece c of block row r32 within the 32-row block (blocks of 16 rows,
    // 2 KB apart)
    uint32_t fragb_lo[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s)
      fragb_lo[s] = BLK ? 2048u * (uint32_t)(r32 >> 4) + 16u * blk_piece(r32 & 15, 2 * s + hf) : frag_lo[s];
    // FP8: the codes of groups 2q, 2q + 1 (chunks 4q + 2hf, 4q + 2hf + 1: bytes
    // [32 q + 16 hf, +16) of the row's step) are piece 2q + hf, stored at piece
    // (2q + hf) ^ f8_key(r32) of the row's line (blocks start at multiples of 32 rows)
    uint32_t f8o[kSub / 2];
#pragma unroll
    for (int q = 0; q < kSub / 2; ++q) f8o[q] = (uint32_t)(r32 * kF8Pitch + 16 * ((2 * q + hf) ^ f8_key(r32)));
    // W8A8: group s (k [64 s, 64 s + 64) of the step) takes the lane's two 16-byte pieces,
    // chunks 4 s + hf and 4 s + 2 + hf of the row's 128 bytes (the FP8 MFMA's byte order)
    uint32_t a8o[kSub8][2];
#pragma unroll
    for (int q = 0; q < kSub8; ++q)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        a8o[q][p] = (uint32_t)(r32 * kRowBytes + (((4 * q + 2 * p + hf) ^ swz_key(r32)) << 4));
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
    // tile fields are workgroup-uniform: keep them scalar
    const int e = __builtin_amdgcn_readfirstlane(tile.x);
    const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
    const int mrows = __builtin_amdgcn_readfirstlane(tile.z);
    const int ebase = __builtin_amdgcn_readfirstlane(a.offs[e]);
    const int nrb = (mrows + kBlk - 1) / kBlk;
    const bool routed = e < a.E;

    // Loads: op i of a thread covers stage rows 32 i + 8 wv + lane/8, physical chunk
    // lane % 8, i.e. chunk (lane % 8) ^ key(row) of the row's 128-byte k window.
    // Activations: tile rows past the tile's end reload its last row (never used).
    // Weights: gate/up rows 64 q .. 64 q + 63 (q = i / 2) are gate (q even) or up (q odd)
    // units nt*128 + 64 (q / 2) + [0, 64), so wave (., wn) holds gate and up of the
    // same 64 units; down rows are output columns nt*256 + row, clamped past d (not
    // stored).
    // Addresses are a workgroup-uniform base (scalar registers) plus a 32-bit byte offset
    // per lane (the grouped path requires x, h and every expert matrix under 4 GiB).
    const char* const abase = A8 ? reinterpret_cast<const char*>(a.aq)
                                 : reinterpret_cast<const char*>(GATEUP ? a.x : h);
    uint32_t aoff[kDma], boff[kDma];
    const char* bbase[kDma];
    // gate/up: the token of each loaded row (rows past Tk are the shared expert's, in
    // token order); the permutation entries are all loaded before any is used
    uint32_t src[kDma];
    if (GATEUP) {
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        const int grow = ebase + m0 + min((kThreads * i + 64 * wv + lane) >> 3, mrows - 1);
        src[i] = (uint32_t)a.perm_src[min(grow, a.Tk - 1)];
      }
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        const int grow = ebase + m0 + min((kThreads * i + 64 * wv + lane) >> 3, mrows - 1);
        src[i] = grow < a.Tk ? src[i] / (uint32_t)a.k : (uint32_t)(grow - a.Tk);
      }
    }
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int q = kThreads * i + 64 * wv + lane;
      const int row = q >> 3, lc = (q & 7) ^ swz_key(row);
      const int grow = ebase + m0 + min(row, mrows - 1);
      if constexpr (A8) {  // byte addressing of E4M3 codes (routed tiles only)
        if (GATEUP) {
          aoff[i] = src[i] * (uint32_t)a.d + 16 * lc;
          const int qq = i >> 1;
          const uint8_t* mat = ((qq & 1) == 0 ? w.f8gate : w.f8up) + (size_t)e * a.I * a.d;
          bbase[i] = reinterpret_cast<const char*>(mat + (size_t)(nt * (kRowsMax / 2) + 64 * (qq >> 1)) * a.d);
          boff[i] = (uint32_t)(row & 63) * (uint32_t)a.d + 16 * lc;
        } else {
          aoff[i] = (uint32_t)grow * (uint32_t)a.I + 16 * lc;
          bbase[i] = reinterpret_cast<const char*>(w.f8down + ((size_t)e * a.d + (size_t)nt * kRowsMax) * a.I);
          boff[i] = (uint32_t)(min(nt * kRowsMax + row, a.d - 1) - nt * kRowsMax) * (uint32_t)a.I + 16 * lc;
        }
      } else if (GATEUP) {
        aoff[i] = (src[i] * (uint32_t)a.d + 8 * lc) * 2u;
        const int qq = i >> 1;  // 64-row quarter of the tile
        const uint16_t* mat = (qq & 1) == 0 ? (routed ? w.gate + (size_t)e * a.I * a.d : w.s_gate)
                                            : (routed ? w.up + (size_t)e * a.I * a.d : w.s_up);
        const int r0 = nt * (kRowsMax / 2) + 64 * (qq >> 1), rr = row & 63;  // the quarter's first unit, row in it
        if constexpr (BLK) {
          // slot piece q of the step: block q / 128 of the tile (block 2 (i % 2) + wv / 2 of
          // quarter qq = i / 2), piece q % 128 of it
          bbase[i] = reinterpret_cast<const char*>(mat + (size_t)(r0 / 16) * (a.d / 64) * 1024);
          boff[i] = ((uint32_t)(2 * (i & 1) + (wv >> 1)) * (uint32_t)(a.d / 64) * 1024u +
                     8u * (uint32_t)(q & 127)) * 2u;
        } else {
          bbase[i] = reinterpret_cast<const char*>(mat + (size_t)r0 * a.d);
          boff[i] = ((uint32_t)rr * (uint32_t)a.d + 8 * lc) * 2u;
        }
      } else {
        aoff[i] = ((uint32_t)grow * (uint32_t)a.I + 8 * lc) * 2u;
        const uint16_t* mat = routed ? w.down + (size_t)e * a.d * a.I : w.s_down;
        const int rr = min(nt * kRowsMax + row, a.d - 1) - nt * kRowsMax;  // output column in the tile, clamped
        if constexpr (BLK) {
          // slot piece q: block q / 128 of the tile (output columns nt*256 + 16 (q / 128) ..,
          // a block past d clamped to the last one: not stored), piece q % 128 of it
          const int gb = min(nt * (kRowsMax / 16) + (q >> 7), a.d / 16 - 1) - nt * (kRowsMax / 16);
          bbase[i] = reinterpret_cast<const char*>(mat + (size_t)(nt * kRowsMax / 16) * (a.I / 64) * 1024);
          boff[i] = ((uint32_t)gb * (uint32_t)(a.I / 64) * 1024u + 8u * (uint32_t)(q & 127)) * 2u;
        } else {
          bbase[i] = reinterpret_cast<const char*>(mat + (size_t)nt * kRowsMax * a.I);
          boff[i] = ((uint32_t)rr * (uint32_t)a.I + 8 * lc) * 2u;
        }
      }
    }
    // Ternary codes: op i of a thread loads word min(lane % 4, 2) of the step's window of
    // tile row 64 i + 16 wv + lane / 4 (gate/up: the rows of quarter i, as above; down:
    // output columns clamped past d) into byte 16 row + 4 (lane % 4) of the code slot.
    const char* cbase[kCodeOps];  // workgroup-uniform
    uint32_t coff[kCodeOps];
    if constexpr (TERN) {
      const uint32_t rw = (uint32_t)(K / 128 * 20);  // code bytes per weight row
      const int rr = 16 * wv + (lane >> 2);
      const uint32_t wo = 4u * (uint32_t)min(lane & 3, 2);
      const uint32_t bstride = (uint32_t)(K / 512) * 1280u;  // blocked: bytes per 16-row group
#pragma unroll
      for (int i = 0; i < kCodeOps; ++i) {
        // the quarter's (or tile's) first row b0 and this lane's row relative to it
        const int b0 = GATEUP ? nt * (kRowsMax / 2) + 64 * (i >> 1) : nt * kRowsMax;
        const int rel = GATEUP ? rr : min(nt * kRowsMax + 64 * i + rr, a.d - 1) - nt * kRowsMax;
        const uint32_t* mat = GATEUP ? ((i & 1) == 0 ? w.qgate : w.qup) : w.qdown;
        const char* m = reinterpret_cast<const char*>(mat) + (size_t)e * (GATEUP ? a.I : a.d) * rw;
        if constexpr (TB) {
          cbase[i] = m + (size_t)(b0 / 16) * bstride;
          coff[i] = (uint32_t)(rel / 16) * bstride + (uint32_t)(rel % 16) * 80u + wo;
        } else {
          cbase[i] = m + (size_t)b0 * rw;
          coff[i] = (uint32_t)rel * rw + wo;
        }
      }
      // the item's row scales into LDS (wave 0; these loads are older than every k-loop
      // load, so the counted waits below cover them): gate/up units nt*128 + [0, 128) of
      // the gate then the up matrix, or down columns nt*256 + [0, 256) clamped past d
      if (wv == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint16_t* src =
              GATEUP ? (i == 0 ? w.sgate : w.sup) + (size_t)e * a.I + nt * (kRowsMax / 2) + 2 * lane
                     : w.sdown + (size_t)e * a.d + min(nt * kRowsMax + 2 * (64 * i + lane), a.d - 2);
          __builtin_amdgcn_global_load_lds((const void*)src, HY_LDS(ssc + 256 * i), 4, 0, 0);
        }
      }
    }
    // FP8 codes: op i of a thread loads physical piece lane % 4 (logical piece
    // (lane % 4) ^ f8_key(row)) of the step's 64 bytes of tile row 64 i + 16 wv + lane / 4
    // (rows as for the ternary codes) into byte 16 (4 row + lane % 4) of the slot
    if constexpr (FP8) {
      const uint32_t rb = (uint32_t)K;  // code bytes per weight row
      const int rr = 16 * wv + (lane >> 2);
      const uint32_t po = 16u * (uint32_t)((lane & 3) ^ f8_key(rr));  // f8_key(64 i + rr) == f8_key(rr)
#pragma unroll
      for (int i = 0; i < kF8Ops; ++i) {
        if (GATEUP) {
          const uint8_t* mat = (i & 1) == 0 ? w.f8gate : w.f8up;
          cbase[i] = reinterpret_cast<const char*>(mat) + ((size_t)e * a.I + nt * (kRowsMax / 2) + 64 * (i >> 1)) * rb;
          coff[i] = (uint32_t)rr * rb + po;
        } else {
          cbase[i] = reinterpret_cast<const char*>(w.f8down) + ((size_t)e * a.d + nt * kRowsMax) * rb;
          coff[i] = (uint32_t)(min(nt * kRowsMax + 64 * i + rr, a.d - 1) - nt * kRowsMax) * rb + po;
        }
      }
      // the item's fp32 row scales into LDS (wave 0, older than every k-loop load):
      // gate/up units nt*128 + [0, 128) of the gate then the up matrix, or down columns
      // nt*256 + [0, 256) clamped past d
      if (wv == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* src = GATEUP ? (i < 2 ? w.f8sgate : w.f8sup) + (size_t)e * a.I + nt * (kRowsMax / 2) +
                                          64 * (i & 1) + lane
                                    : w.f8sdown + (size_t)e * a.d + min(nt * kRowsMax + 64 * i + lane, a.d - 1);
          __builtin_amdgcn_global_load_lds((const void*)src, HY_LDS(ssc + 256 * i), 4, 0, 0);
        }
      }
    }
    // W8A8: the activation block scales of the lane's 4 row blocks (rows (2 j + wm) 32 +
    // r32, clamped to the tile), one word per row per step (blocks 4 ks .. 4 ks + 3),
    // loaded into registers one step ahead and double-buffered by step parity
    uint32_t soff[kWaveBlocks];
    uint32_t sreg[2][kWaveBlocks];
    if constexpr (A8) {
      const uint32_t bpr = (uint32_t)(K / 32);  // scale bytes per row
#pragma unroll
      for (int j = 0; j < kWaveBlocks; ++j) {
        const int grow = ebase + m0 + min((2 * j + wm) * kBlk + r32, mrows - 1);
        const uint32_t srow = GATEUP ? (uint32_t)a.perm_src[grow] / (uint32_t)a.k : (uint32_t)grow;
        soff[j] = srow * bpr;
      }
    }
    auto issue_s = [&](int ks, auto par_tag) __attribute__((always_inline)) {
      if constexpr (A8) {
#pragma unroll
        for (int j = 0; j < kWaveBlocks; ++j)
          sreg[decltype(par_tag)::value][j] = *reinterpret_cast<const uint32_t*>(a.as + soff[j] + 4 * ks);
      }
    };
    auto issue_f8 = [&](int ks, uint8_t* st) {
      uint8_t* dc = st + 1024 * wv;
#pragma unroll
      for (int i = 0; i < kF8Ops; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(cbase[i] + coff[i] + kF8Pitch * ks), HY_LDS(dc + 4096 * i), 16,
                                         0, 0);
    };
    // the step's code words: byte 4 floor(10 ks / 4) of each row (blocked: of its 512-weight
    // slab ks / 8, 1280 bytes per slab); the codes start at bit 16 (ks % 2) either way
    auto issue_c = [&](int ks, uint8_t* st) {
      const uint32_t so = TB ? (uint32_t)(ks >> 3) * 1280u + ((uint32_t)(10 * (ks & 7)) & ~3u) : (uint32_t)(10 * ks) & ~3u;
      uint8_t* dc = st + 256 * wv;
#pragma unroll
      for (int i = 0; i < kCodeOps; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(cbase[i] + coff[i] + so), HY_LDS(dc + 1024 * i), 4, 0, 0);
    };
    // ops [I0, I1) of a step's activation / weight load group
    // (a step is 128 bytes of every row: 64 bf16 values or 128 E4M3 codes)
    auto issue_a = [&](int ks, uint8_t* st, auto i0_tag, auto i1_tag) {
      const int kb = ks * kRowBytes;
      uint8_t* da = st + (64 * wv) * 16;
#pragma unroll
      for (int i = decltype(i0_tag)::value; i < decltype(i1_tag)::value; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(abase + aoff[i] + kb), HY_LDS(da + kThreads * 16 * i), 16, 0,
                                         0);
    };
    auto issue_b = [&](int ks, uint8_t* st, auto i0_tag, auto i1_tag) {
      const int kb = ks * (BLK ? 16 * kRowBytes : kRowBytes);  // blocked: the next 2 KB block
      uint8_t* db = st + (64 * wv) * 16;
#pragma unroll
      for (int i = decltype(i0_tag)::value; i < decltype(i1_tag)::value; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bbase[i] + boff[i] + kb), HY_LDS(db + kThreads * 16 * i), 16,
                                         0, 0);
    };
    using C0 = std::integral_constant<int, 0>;
    using CH = std::integral_constant<int, kDma / 2>;
    using CF = std::integral_constant<int, kDma>;

    f32x16 acc[kWaveBlocks][kNB];
#pragma unroll
    for (int j = 0; j < kWaveBlocks; ++j)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][nb][i] = 0.f;

    // prologue: steps 0 and 1 of the weights, step 0 and the first half of step 1 of
    // the activations in flight (K >= 128 gives at least 2 steps), step 0 landed
    // everywhere; the rest of step 1 and the weights of step 2 follow in step 0
    // W8A8: the scales of steps 0 and 1 go out first, fenced off: the counted wait below
    // takes them as the oldest loads (were the compiler to place an ordinary load after
    // the weights' direct-to-LDS loads, the count would leave some of those unwaited)
    issue_s(0, std::integral_constant<int, 0>{});
    issue_s(1, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    issue_a(0, sa0, C0{}, CF{});
    if constexpr (TERN) {
      issue_c(0, sb[0]);
      issue_c(1, sb[1]);
    } else if constexpr (FP8) {
      issue_f8(0, sb[0]);
      issue_f8(1, sb[1]);
    } else {
      issue_b(0, sb[0], C0{}, CF{});
      issue_b(1, sb[1], C0{}, CF{});
    }
    // (W8A8: all of step 1's activations; its steps load the activations two steps ahead)
    if constexpr (A8)
      issue_a(1, sa1, C0{}, CF{});
    else
      issue_a(1, sa1, C0{}, CH{});
    wait_vm<kBOps + (A8 ? kDma : kDma / 2)>();
    bare_barrier();

    // the k loop, with this wave's number of active row blocks fixed at compile time
    // (no branches around the MFMAs)
    auto k_loop = [&](auto nact_tag) {
      constexpr int NACT = decltype(nact_tag)::value;
      uint4 fa[2][kWaveBlocks], fb[2][kNB];
      uint4 fc[2][kNB];  // FP8: the raw codes of a pair of groups, converted right before each group's MFMAs
      // W8A8: 32 codes per lane per operand (two pieces), one buffer: each register is
      // refilled with the next group's fragment right after the MFMA that last reads it
      i32x8 fa8[kWaveBlocks], fb8[kNB];
      // The previous group's reads are waited for (long done: a whole MFMA group ran
      // since) before this group's are issued, so at most 8 are in flight and the
      // MFMAs that follow need no wait.
      auto read_frags = [&](const uint8_t* La, const uint8_t* Lb, int s) {
        wait_lds();
#pragma unroll
        for (int j = 0; j < NACT; ++j)
          fa[s & 1][j] = *reinterpret_cast<const uint4*>(La + fa_off + j * 2 * kBlk * kRowBytes + frag_lo[s]);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          if constexpr (FP8) {
            if ((s & 1) == 0)  // the pair's codes, read with its first group
              fc[(s >> 1) & 1][nb] = *reinterpret_cast<const uint4*>(Lb + (128 * wn + 32 * nb) * kF8Pitch + f8o[s >> 1]);
          } else
            fb[s & 1][nb] = *reinterpret_cast<const uint4*>(Lb + fb_off + nb * kBlk * kRowBytes + fragb_lo[s]);
        }
      };
      // Ternary: the step's code windows of the lane's 4 weight rows (128 wn + 32 nb +
      // r32), read once per step; group S of the step (k [8 (2S + hf), +8)) takes the two
      // codes at bit 16 PAR + 20 S + 10 hf of its row's window, PAR = step parity (the
      // windows are shifted right by 10 hf when group 0 is read).
      uint32_t cw[kNB][3];
      auto read_codes = [&](const uint8_t* Lc) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const uint4 t = *reinterpret_cast<const uint4*>(Lc + kCodePitch * (128 * wn + 32 * nb + r32));
          cw[nb][0] = t.x;
          cw[nb][1] = t.y;
          cw[nb][2] = t.z;
        }
      };
      auto read_frags_t = [&](const uint8_t* La, auto s_tag, auto par_tag) {
        constexpr int S = decltype(s_tag)::value;
        constexpr int PAR = decltype(par_tag)::value;
        wait_lds();
        if constexpr (S == 0) {
          const uint32_t sh = 10u * (uint32_t)hf;
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            cw[nb][0] = __builtin_amdgcn_alignbit(cw[nb][1], cw[nb][0], sh);
            cw[nb][1] = __builtin_amdgcn_alignbit(cw[nb][2], cw[nb][1], sh);
            cw[nb][2] >>= sh;
          }
        }
#pragma unroll
        for (int j = 0; j < NACT; ++j)
          fa[S & 1][j] = *reinterpret_cast<const uint4*>(La + fa_off + j * 2 * kBlk * kRowBytes + frag_lo[S]);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const uint2 lo = lut[code5<16 * PAR + 20 * S>(cw[nb])];
          const uint2 hi = lut[code5<16 * PAR + 20 * S + 5>(cw[nb])];
          fb[S & 1][nb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      };
      // operands in (weights, activations) order: the accumulators hold the transposed
      // tile, so lane (r32, hf) has output row r32 and 4 consecutive columns per
      // accumulator quad (see the epilogue); row blocks [J0, J1)
      auto mfmas_rows = [&](int s, auto j0_tag, auto j1_tag) {
#pragma unroll
        for (int j = decltype(j0_tag)::value; j < decltype(j1_tag)::value; ++j)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) acc[j][nb] = mfma32x32x16(fb[s & 1][nb], fa[s & 1][j], acc[j][nb]);
      };
      // W8A8 group S of a step of parity PAR: MFMAs column block major (nb, then row
      // block j); the lane's activation scale for row block j is byte 2 S + hf of that
      // step's scale word. With REFILL, fb8[nb] takes the fragment of group SN from
      // (La, Lb) right after its last MFMA (row block NACT - 1), and fa8[j] right after
      // column block kNB - 1's MFMA of row block j. vm(t) issues the group's vector-memory
      // op t (t < NV): op m goes out right after MFMA m, in program order as well as in
      // the scheduling pattern (issued ahead of the group, the scheduler sent all of them
      // in one burst before the first MFMA), and ops past the group's MFMAs follow them.
      auto rd_a8 = [&](const uint8_t* La, int s, int j) __attribute__((always_inline)) {
        const uint8_t* base = La + fa_off + j * 2 * kBlk * kRowBytes;
        fa8[j] = lds_pair(base + a8o[s][0], base + a8o[s][1]);
      };
      auto rd_b8 = [&](const uint8_t* Lb, int s, int nb) __attribute__((always_inline)) {
        const uint8_t* base = Lb + fb_off + nb * kBlk * kRowBytes;
        fb8[nb] = lds_pair(base + a8o[s][0], base + a8o[s][1]);
      };
      auto group8 = [&](auto s_tag, auto par_tag, auto refill_tag, auto sn_tag, auto nv_tag, const uint8_t* La,
                        const uint8_t* Lb, auto&& vm) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value, PAR = decltype(par_tag)::value;
        constexpr bool REFILL = decltype(refill_tag)::value;
        constexpr int SN = decltype(sn_tag)::value, NV = decltype(nv_tag)::value;
        constexpr int NM = kNB * NACT;  // the group's MFMAs
        if constexpr (NACT > 0) {
          int one = 127;  // E8M0 1.0 for the weights (their fp32 row scales apply in the epilogue)
          asm volatile("" : "+v"(one));
          int sc[kWaveBlocks];
#pragma unroll
          for (int j = 0; j < NACT; ++j) sc[j] = (int)((sreg[PAR][j] >> (16 * S + 8 * hf)) & 0xFFu);
          for_seq(std::make_integer_sequence<int, kNB>{}, [&](auto nb_tag) {
            constexpr int NB = decltype(nb_tag)::value;
            for_seq(std::make_integer_sequence<int, NACT>{}, [&](auto j_tag) {
              constexpr int J = decltype(j_tag)::value;
              acc[J][NB] = mfma32x32x64_f8(fb8[NB], fa8[J], acc[J][NB], one, sc[J]);
              if constexpr (NB * NACT + J < NV) vm(std::integral_constant<int, NB * NACT + J>{});
              if constexpr (REFILL && J == NACT - 1) rd_b8(Lb, SN, NB);
              if constexpr (REFILL && NB == kNB - 1) rd_a8(La, SN, J);
            });
          });
          // MFMA m = NB NACT + J, then a vector-memory op (the first NV MFMAs), then the
          // reads that follow it
          for_seq(std::make_integer_sequence<int, kNB * NACT>{}, [&](auto m_tag) {
            constexpr int M = decltype(m_tag)::value, NB = M / NACT, J = M % NACT;
            constexpr int NR = REFILL ? 2 * ((J == NACT - 1) ? 1 : 0) + 2 * ((NB == kNB - 1) ? 1 : 0) : 0;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (M < NV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
          });
        }
        if constexpr (NV > NM) {
          for_seq(std::make_integer_sequence<int, NV - NM>{}, [&](auto t_tag) {
            vm(std::integral_constant<int, NM + decltype(t_tag)::value>{});
          });
          __builtin_amdgcn_sched_group_barrier(0x010, NV - NM, 0);
        }
      };
      auto mfmas = [&](int s) {
        if constexpr (FP8) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const uint4 c = fc[(s >> 1) & 1][nb];
            fb[s & 1][nb] = (s & 1) == 0 ? e4m3x8_bf16(c.x, c.y) : e4m3x8_bf16(c.z, c.w);
          }
        }
        mfmas_rows(s, std::integral_constant<int, 0>{}, std::integral_constant<int, NACT>{});
      };
      // One step ks on activation slot UA = ks % 2 and weight slot UB = ks % BS. The
      // slots step ks-1 used were freed by the barrier that ended it; their next loads
      // (the second half of the activations of step ks+1, the weights of step ks+2) go
      // out in 4-op pieces between this step's MFMA groups, so the address unit works
      // through them while the MFMAs run instead of stalling the waves in one burst.
      // PA: step ks+1 exists (its activations are loaded); PB: step ks+2 exists (its
      // weights, and the first half of its activations at the end of this step, are
      // loaded); NEXT: there is a next step. sched_barrier(0) keeps each group
      // in place: the fragment reads stay ahead of the MFMAs that run while they are in
      // flight.
      auto step = [&](auto ua_tag, auto ub_tag, auto next_tag, auto pa_tag, auto pb_tag, int ks) {
        constexpr int UA = decltype(ua_tag)::value;
        constexpr int UB = decltype(ub_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool PA = decltype(pa_tag)::value;
        constexpr bool PB = decltype(pb_tag)::value;
        for_seq(std::integer_sequence<int, 1, 2, 3>{}, [&](auto s_tag) {
          constexpr int S = decltype(s_tag)::value;
          if constexpr (TERN)
            read_frags_t(sa[UA], std::integral_constant<int, S>{}, ua_tag);  // ks % 2 == UA
          else
            read_frags(sa[UA], sb[UB], S);
          if constexpr (S == 1 && PA) issue_a(ks + 1, sa[UA ^ 1], CH{}, CF{});
          if constexpr (TERN) {
            if constexpr (S == 2 && PB) issue_c(ks + 2, sb[(UB + 2) % BS]);
          } else if constexpr (FP8) {
            if constexpr (S == 2 && PB) issue_f8(ks + 2, sb[(UB + 2) % BS]);
          } else {
            if constexpr (S == 2 && PB) issue_b(ks + 2, sb[(UB + 2) % BS], C0{}, CH{});
            if constexpr (S == 3 && PB) issue_b(ks + 2, sb[(UB + 2) % BS], CH{}, CF{});
          }
          mfmas(S - 1);
          constexpr int NV = (TERN || FP8) ? ((S == 1 && PA) ? kDma / 2 : (S == 2 && PB) ? kBOps : 0)
                                           : ((S == 1 && PA) || (S >= 2 && PB)) ? kDma / 2 : 0;
          constexpr int NREAD = NACT + (TERN ? 2 * kNB : (FP8 && (S & 1)) ? 0 : kNB);
          interleave_group<NACT * kNB, NREAD, NV>();
          __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (NEXT) {
          // own loads of step ks+1 landed: all but this step's weight loads (the newest)
          wait_vm<PB ? kBOps : 0>();
          wait_lds();      // own reads of this step done
          bare_barrier();  // everyone's step ks+1 landed; this step's slots are free
          if constexpr (PB) issue_a(ks + 2, sa[UA], C0{}, CH{});
          if constexpr (TERN) {
            // the next step's code windows first; half of this step's last MFMA group
            // runs while they are read, then group 0 of the next step is decoded
            constexpr int H = (NACT + 1) / 2;
            read_codes(sb[(UB + 1) % BS]);
            mfmas_rows(kSub - 1, std::integral_constant<int, 0>{}, std::integral_constant<int, H>{});
            __builtin_amdgcn_sched_group_barrier(0x100, kNB, 0);  // the code reads
            interleave_group<H * kNB, 0, PB ? kDma / 2 : 0>();
            __builtin_amdgcn_sched_barrier(0);
            read_frags_t(sa[UA ^ 1], std::integral_constant<int, 0>{}, std::integral_constant<int, UA ^ 1>{});
            mfmas_rows(kSub - 1, std::integral_constant<int, H>{}, std::integral_constant<int, NACT>{});
            interleave_group<(NACT - H) * kNB, NACT + 2 * kNB, 0>();
          } else {
            read_frags(sa[UA ^ 1], sb[(UB + 1) % BS], 0);
            mfmas(kSub - 1);
            interleave_group<NACT * kNB, NACT + kNB, PB ? kDma / 2 : 0>();
          }
        } else {
          // the last step: claim the next item (read after the k loop)
          if (threadIdx.x == 0) own_ticket = atomicAdd(&counters[xcd], 1);
          __builtin_amdgcn_sched_barrier(0);
          mfmas(kSub - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // W8A8 step ks: group 0 on fragments already in registers (refilling group 1's from
      // this step's slots) with step ks+2's weights issued over it; then the barrier that
      // frees this step's activation slot and lands step ks+1's; group 1 refilling the next
      // step's group 0, with all of step ks+2's activations issued over it into the slot
      // just freed; then the scales of step ks+2 into the parity's registers, which group 1
      // was the last to read. Each load thus has two (activations) or three (weights) MFMA
      // groups to land before the barrier that waits for it (with half of step ks+1's
      // activations issued over group 0 instead, they had one group: gate/up 1.5% slower).
      auto step8 = [&](auto ua_tag, auto ub_tag, auto next_tag, auto pa_tag, auto pb_tag, int ks)
                       __attribute__((always_inline)) {
        constexpr int UA = decltype(ua_tag)::value;
        constexpr int UB = decltype(ub_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr bool PB = decltype(pb_tag)::value;  // (step ks+1's loads went out in step ks-1)
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        // group 0's ops: step ks+2's weights
        auto vm0 = [&](auto t_tag) __attribute__((always_inline)) {
          constexpr int T = decltype(t_tag)::value;
          issue_b(ks + 2, sb[(UB + 2) % BS], std::integral_constant<int, T>{}, std::integral_constant<int, T + 1>{});
        };
        group8(I0{}, ua_tag, std::true_type{}, I1{}, std::integral_constant<int, PB ? kDma : 0>{}, sa[UA], sb[UB],
               vm0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NEXT) {
          wait_vm<PB ? kBOps : 0>();  // all but step ks+2's weights (the newest)
          wait_lds();
          bare_barrier();
          // group 1's ops: step ks+2's activations
          auto vm1 = [&](auto t_tag) __attribute__((always_inline)) {
            constexpr int T = decltype(t_tag)::value;
            issue_a(ks + 2, sa[UA], std::integral_constant<int, T>{}, std::integral_constant<int, T + 1>{});
          };
          group8(I1{}, ua_tag, std::true_type{}, I0{}, std::integral_constant<int, PB ? kDma : 0>{}, sa[UA ^ 1],
                 sb[(UB + 1) % BS], vm1);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (PB) issue_s(ks + 2, ua_tag);
        } else {
          group8(I1{}, ua_tag, std::false_type{}, I0{}, I0{}, nullptr, nullptr, [](auto) {});
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // whole periods of P = 6 steps (slots repeat with period 6), then the last R steps
      // (R = TAILR, or 6 when TAILR is 0), all with compile-time slots
      constexpr int P = 6;
      constexpr int R = TAILR == 0 ? P : TAILR;
      if constexpr (A8) {
#pragma unroll
        for (int j = 0; j < NACT; ++j) rd_a8(sa[0], 0, j);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) rd_b8(sb[0], 0, nb);
        int k0 = 0;
        for (; k0 + R < nks; k0 += P)
          for_seq(std::make_integer_sequence<int, P>{}, [&](auto t) {
            constexpr int T = decltype(t)::value;
            step8(std::integral_constant<int, T % 2>{}, std::integral_constant<int, T % 3>{}, std::true_type{},
                  std::true_type{}, std::true_type{}, k0 + T);
          });
        // the next item's claim goes out before the last steps rather than inside the last
        // one: a branch after the tail's MFMAs let the compiler sink them all below it,
        // away from their fragment reads (every fragment of the tail live at once)
        if (threadIdx.x == 0) own_ticket = atomicAdd(&counters[xcd], 1);
        for_seq(std::make_integer_sequence<int, R>{}, [&](auto t) {
          constexpr int T = decltype(t)::value;
          step8(std::integral_constant<int, T % 2>{}, std::integral_constant<int, T % 3>{},
                std::integral_constant<bool, (T + 1 < R)>{}, std::integral_constant<bool, (T + 1 < R)>{},
                std::integral_constant<bool, (T + 2 < R)>{}, k0 + T);
        });
      } else {
        if constexpr (TERN) {
          read_codes(sb[0]);
          read_frags_t(sa[0], std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        } else {
          read_frags(sa[0], sb[0], 0);
        }
        int k0 = 0;
        for (; k0 + R < nks; k0 += P)
          for_seq(std::make_integer_sequence<int, P>{}, [&](auto t) {
            constexpr int T = decltype(t)::value;
            step(std::integral_constant<int, T % 2>{}, std::integral_constant<int, T % 3>{}, std::true_type{},
                 std::true_type{}, std::true_type{}, k0 + T);
          });
        for_seq(std::make_integer_sequence<int, R>{}, [&](auto t) {
          constexpr int T = decltype(t)::value;
          step(std::integral_constant<int, T % 2>{}, std::integral_constant<int, T % 3>{},
               std::integral_constant<bool, (T + 1 < R)>{}, std::integral_constant<bool, (T + 1 < R)>{},
               std::integral_constant<bool, (T + 2 < R)>{}, k0 + T);
        });
      }
    };
    const int nact = min(kWaveBlocks, max(0, (nrb - wm + 1) >> 1));
    if (nact == 4)
      k_loop(std::integral_constant<int, 4>{});
    else if (nact == 3)
      k_loop(std::integral_constant<int, 3>{});
    else if (nact == 2)
      k_loop(std::integral_constant<int, 2>{});
    else if (nact == 1)
      k_loop(std::integral_constant<int, 1>{});
    else
      k_loop(std::integral_constant<int, 0>{});
    // all waves are done with the ring: it now stages the output tile
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x == 0) claimed = own_or_steal(own_ticket);
    bare_barrier();

    // Epilogue through LDS: the tile is written as 256-row x 64-column bf16 pieces of
    // 32 KB (sa0, sa1, sb0, sb1; 128 B per row; 16-byte chunk c of row r sits at
    // c ^ swz_key(r)), then leaves with 16-byte stores of whole row segments. Accumulator
    // i of lane (r32, hf) is output row r32 of its 32-row block, column 8 (i / 4) + 4 hf +
    // i % 4 of its 32-column block, so each quad of accumulators is 8 contiguous bytes:
    // one 8-byte LDS write. gate/up: piece wn holds h units nt*128 + 64 wn + [0, 64);
    // down: piece 2 wn + nb/2 holds y columns nt*256 + 64 (2 wn + nb/2) + [0, 64). The FP8
    // down kernel has no sb0/sb1 (its weight ring and the activation slots fill the LDS):
    // it stages pieces 0-1 (waves wn = 0), writes them out, then pieces 2-3, both in
    // sa0/sa1.
    if constexpr (A8 && GATEUP) {
      // W8A8 gate/up: h = silu(g) * u in fp32 (weight row scales from memory), quantized
      // to MXFP8 per 32 hidden units of a row: the two lanes (r32, 0) and (r32, 1) hold a
      // block's 32 values, so one exchange gives its largest magnitude. The codes are
      // staged in sa0 (row r's 128 codes of the item, 16-byte chunk c at c ^ swz_key(r))
      // and leave as 16-byte row segments; lane (r32, 0) writes the block's scale byte.
      const size_t sbase = (size_t)e * a.I + nt * (kRowsMax / 2);
      const int hbpr = a.I / 32;
#pragma unroll
      for (int j = 0; j < kWaveBlocks; ++j) {
        const int rb = 2 * j + wm;
        if (rb >= nrb) continue;  // wave-uniform
        const int row = rb * kBlk + r32;
#pragma unroll
        for (int nb = 0; nb < kNB / 2; ++nb) {
          float v[16];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int c0 = 64 * wn + 32 * nb + 8 * qd + 4 * hf;
            float sg[4], su[4];  // (scales are only 4-byte aligned: one load each)
#pragma unroll
            for (int t = 0; t < 4; ++t) sg[t] = w.f8sgate[sbase + c0 + t], su[t] = w.f8sup[sbase + c0 + t];
#pragma unroll
            for (int t = 0; t < 4; ++t)
              v[4 * qd + t] = silu_fast(acc[j][nb][4 * qd + t] * sg[t]) * (acc[j][nb + kNB / 2][4 * qd + t] * su[t]);
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          const int ex = mx_exponent(amax);
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int chunk = 4 * wn + 2 * nb + (qd >> 1);
            *reinterpret_cast<uint32_t*>(sa0 + row * kRowBytes + ((chunk ^ swz_key(row)) << 4) + 8 * (qd & 1) +
                                         4 * hf) = mx_pack4(v[4 * qd], v[4 * qd + 1], v[4 * qd + 2], v[4 * qd + 3], ex);
          }
          if (hf == 0 && row < mrows)
            a.hs[(size_t)(ebase + m0 + row) * hbpr + nt * 4 + 2 * wn + nb] = (uint8_t)(ex + 127);
        }
      }
      wait_lds();
      bare_barrier();
      {
        const int orow = tid >> 3, ch = tid & 7;
        const uint32_t pl = (uint32_t)(orow * kRowBytes + ((ch ^ swz_key(orow)) << 4));
        uint8_t* const ob = a.hq + (size_t)(ebase + m0 + orow) * a.I + nt * (kRowsMax / 2) + 16 * ch;
        uint4 v[kRowsMax / 32];
#pragma unroll
        for (int it = 0; it < kRowsMax / 32; ++it) v[it] = *reinterpret_cast<const uint4*>(sa0 + pl + it * 32 * kRowBytes);
#pragma unroll
        for (int it = 0; it < kRowsMax / 32; ++it)
          if (it * 32 + orow < mrows) *reinterpret_cast<uint4*>(ob + (size_t)it * 32 * a.I) = v[it];
      }
      wait_lds();
      bare_barrier();
      continue;
    }
    constexpr int NPIECE = GATEUP ? 2 : 4;
    constexpr int ROUNDS = (FP8 && !GATEUP) ? 2 : 1;
    constexpr int PPR = NPIECE / ROUNDS;  // pieces staged per round
    auto piece_buf = [&](int lp) -> uint8_t* { return lp == 0 ? sa0 : lp == 1 ? sa1 : lp == 2 ? sb0 : sb1; };
    // A piece's 8 row groups are read from LDS first, then stored, so no store waits on
    // another.
    const int ldc = GATEUP ? a.I : a.d;
    const int orow = tid >> 3, ch = tid & 7;
    const uint32_t pl_off = (uint32_t)(orow * 128 + ((ch ^ swz_key(orow)) << 4));
    uint16_t* const obase = (GATEUP ? h : y) + (size_t)(ebase + m0 + orow) * ldc + ch * 8;
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
#pragma unroll
      for (int j = 0; j < kWaveBlocks; ++j) {
        const int rb = 2 * j + wm;
        if (rb >= nrb) continue;  // wave-uniform
        const int row = rb * kBlk + r32;
#pragma unroll
        for (int nb = 0; nb < (GATEUP ? kNB / 2 : kNB); ++nb) {
          const int piece = GATEUP ? wn : 2 * wn + (nb >> 1);
          if constexpr (ROUNDS > 1) {
            if (piece / PPR != rd) continue;  // wave-uniform
          }
          uint8_t* const pb = piece_buf(piece - rd * PPR);
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            // ternary, FP8: the row scales of the quad's 4 columns (gate/up: unit 64 wn +
            // 32 nb + 8 qd + 4 hf + t of the item's gate scales, then of its up scales at
            // +128; down: column 128 wn + 32 nb + 8 qd + 4 hf + t)
            float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
            const int c0 = (GATEUP ? 64 : 128) * wn + 32 * nb + 8 * qd + 4 * hf;
            if constexpr (TERN) {
              const uint2 g2 = *reinterpret_cast<const uint2*>(ssc + 2 * c0);
              sg[0] = bf_lo(g2.x), sg[1] = bf_hi(g2.x), sg[2] = bf_lo(g2.y), sg[3] = bf_hi(g2.y);
              if constexpr (GATEUP) {
                const uint2 u2 = *reinterpret_cast<const uint2*>(ssc + 2 * (c0 + kRowsMax / 2));
                su[0] = bf_lo(u2.x), su[1] = bf_hi(u2.x), su[2] = bf_lo(u2.y), su[3] = bf_hi(u2.y);
              }
            } else if constexpr (A8) {  // down: the output columns' row scales, from memory
#pragma unroll
              for (int t = 0; t < 4; ++t) sg[t] = w.f8sdown[(size_t)e * a.d + nt * kRowsMax + c0 + t];
            } else if constexpr (FP8) {
              const float4 g4 = *reinterpret_cast<const float4*>(ssc + 4 * c0);
              sg[0] = g4.x, sg[1] = g4.y, sg[2] = g4.z, sg[3] = g4.w;
              if constexpr (GATEUP) {
                const float4 u4 = *reinterpret_cast<const float4*>(ssc + 4 * (c0 + kRowsMax / 2));
                su[0] = u4.x, su[1] = u4.y, su[2] = u4.z, su[3] = u4.w;
              }
            }
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i = 4 * qd + t;
              if constexpr (TERN || FP8 || A8)
                v[t] = GATEUP ? silu_fast(acc[j][nb][i] * sg[t]) * (acc[j][nb + kNB / 2][i] * su[t])
                              : acc[j][nb][i] * sg[t];
              else
                v[t] = GATEUP ? silu_fast(acc[j][nb][i]) * acc[j][nb + kNB / 2][i] : acc[j][nb][i];
            }
            const int chunk = GATEUP ? 4 * nb + qd : 4 * (nb & 1) + qd;  // 16-byte chunk of the piece row
            const uint32_t off = row * 128 + ((chunk ^ swz_key(row)) << 4) + 8 * hf;
            *reinterpret_cast<uint2*>(pb + off) = make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
          }
        }
      }
      wait_lds();
      bare_barrier();
#pragma unroll
      for (int pc = rd * PPR; pc < (rd + 1) * PPR; ++pc) {
        const int col0 = GATEUP ? nt * (kRowsMax / 2) + 64 * pc : nt * kRowsMax + 64 * pc;
        if (!GATEUP && col0 >= a.d) continue;  // d is a multiple of 128: whole pieces fall outside
        const uint8_t* pbase = piece_buf(pc - rd * PPR);
        uint4 v[kRowsMax / 32];
#pragma unroll
        for (int it = 0; it < kRowsMax / 32; ++it)  // row it*32 + orow: same swizzle as orow
          v[it] = *reinterpret_cast<const uint4*>(pbase + pl_off + it * 32 * 128);
#pragma unroll
        for (int it = 0; it < kRowsMax / 32; ++it)
          if (it * 32 + orow < mrows) *reinterpret_cast<uint4*>(obase + (size_t)it * 32 * ldc + col0) = v[it];
      }
      if constexpr (ROUNDS > 1) {
        if (rd + 1 < ROUNDS) {  // the next round's pieces overwrite the buffers just read
          wait_lds();
          bare_barrier();
        }
      }
    }
    // every thread has read its pieces before the next item's loads overwrite them
    wait_lds();
    bare_barrier();
  }
}

static int g_grid[12][64];  // persistent grid per (kernel kind, device), 0 = not yet computed

static int persistent_grid(int kind, const void* kernel) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int gsz = __atomic_load_n(&g_grid[kind][dev], __ATOMIC_ACQUIRE);
  if (gsz > 0) return gsz;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess || occ <= 0) occ = 1;
  gsz = ((cus * occ + 7) / 8) * 8;
  __atomic_store_n(&g_grid[kind][dev], gsz, __ATOMIC_RELEASE);
  return gsz;
}

using GemmKern = void (*)(GemmArgs, ExpertWeights, uint16_t*, uint16_t*);

// kernel for (phase, weight format, K): indexed by (steps of K) mod 6 / 2
template <bool GATEUP, int WF>
static GemmKern pick_gemm(int K) {
  static const GemmKern k[3] = {grouped_gemm_kernel<GATEUP, 0, WF>, grouped_gemm_kernel<GATEUP, 2, WF>,
                                grouped_gemm_kernel<GATEUP, 4, WF>};
  return k[(K / (WF == kGemmW8A8 ? kBK8 : kBK)) % 6 / 2];
}

static hipError_t launch_gemm(GemmKern kern, int kind, GemmArgs a, int sel, const ExpertWeights& w, const Plan& p,
                              hipStream_t s) {
  a.sel = sel;
  const int g = persistent_grid(kind, reinterpret_cast<const void*>(kern));
  hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), 0, s, a, w, p.h, (uint16_t*)p.y);
  return hipGetLastError();
}

hipError_t launch_grouped_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                  Marks& m) {
  GemmArgs a{x, nullptr, nullptr, nullptr, nullptr, p.perm_src, p.offs, p.meta, p.tiles, p.Tk, p.k, p.d, p.I, p.E, 0};
  hipError_t err;
  if (w.a8) {
    // W8A8: the token rows to MXFP8, then the FP8-MFMA kernels over the routed tiles and
    // the bf16 kernels over the shared expert's, per phase (the quantization is timed
    // with gate/up)
    err = launch_mx_quantize(x, p.T, p.d, p.xq, p.xs, s);
    a.aq = p.xq, a.as = p.xs, a.hq = p.hq, a.hs = p.hs;
    if (err == hipSuccess) err = launch_gemm(pick_gemm<true, kGemmW8A8>(p.d), 6, a, 1, w, p, s);
    if (err == hipSuccess) err = launch_gemm(pick_gemm<true, kGemmBf16>(p.d), 0, a, 2, w, p, s);
    if (err == hipSuccess) err = m.mark(s);
    a.aq = p.hq, a.as = p.hs, a.hq = nullptr, a.hs = nullptr;
    if (err == hipSuccess) err = launch_gemm(pick_gemm<false, kGemmW8A8>(p.I), 7, a, 1, w, p, s);
    if (err == hipSuccess) err = launch_gemm(pick_gemm<false, kGemmBf16>(p.I), 1, a, 2, w, p, s);
    return err == hipSuccess ? m.mark(s) : err;
  }
  if (!w.ternary && !w.fp8) {
    const GemmKern gu = w.blocked ? pick_gemm<true, kGemmBf16Blk>(p.d) : pick_gemm<true, kGemmBf16>(p.d);
    const GemmKern dn = w.blocked ? pick_gemm<false, kGemmBf16Blk>(p.I) : pick_gemm<false, kGemmBf16>(p.I);
    err = launch_gemm(gu, w.blocked ? 8 : 0, a, 0, w, p, s);
    if (err == hipSuccess) err = m.mark(s);
    if (err == hipSuccess) err = launch_gemm(dn, w.blocked ? 9 : 1, a, 0, w, p, s);
    return err == hipSuccess ? m.mark(s) : err;
  }
  // ternary or FP8 routed experts, then the bf16 shared expert, per phase
  const GemmKern gu = w.tblocked  ? pick_gemm<true, kGemmTernBlk>(p.d)
                     : w.ternary ? pick_gemm<true, kGemmTern>(p.d)
                                 : pick_gemm<true, kGemmFp8>(p.d);
  const GemmKern dn = w.tblocked  ? pick_gemm<false, kGemmTernBlk>(p.I)
                     : w.ternary ? pick_gemm<false, kGemmTern>(p.I)
                                 : pick_gemm<false, kGemmFp8>(p.I);
  const int kind = w.tblocked ? 10 : w.ternary ? 2 : 4;
  if (w.tshared) {
    // a Sherry-packed shared expert is expert E of the code arrays: one launch over every tile
    err = launch_gemm(gu, kind, a, 0, w, p, s);
    if (err == hipSuccess) err = m.mark(s);
    if (err == hipSuccess) err = launch_gemm(dn, kind + 1, a, 0, w, p, s);
    return err == hipSuccess ? m.mark(s) : err;
  }
  err = launch_gemm(gu, kind, a, 1, w, p, s);
  if (err == hipSuccess) err = launch_gemm(pick_gemm<true, kGemmBf16>(p.d), 0, a, 2, w, p, s);
  if (err == hipSuccess) err = m.mark(s);
  if (err == hipSuccess) err = launch_gemm(dn, kind + 1, a, 1, w, p, s);
  if (err == hipSuccess) err = launch_gemm(pick_gemm<false, kGemmBf16>(p.I), 1, a, 2, w, p, s);
  return err == hipSuccess ? m.mark(s) : err;
}

}  // namespace hymoe

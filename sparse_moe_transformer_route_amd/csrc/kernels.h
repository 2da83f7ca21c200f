// Launchers of the MoE layer's kernels; each enqueues on `stream` and returns the
// launch status. Argument shapes are validated by the C ABI before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymoe {

// Optional profiling events recorded after each kernel (caller-created hipEvent_t).
struct Marks {
  void* const* ev;
  int next;
  hipError_t mark(hipStream_t s) {
    hipError_t e = (ev && ev[next]) ? hipEventRecord((hipEvent_t)ev[next], s) : hipSuccess;
    ++next;
    return e;
  }
};

// Per-call device state carved from the workspace.
constexpr int kMetaInts = 64;
constexpr int kMetaSched = 16;  // first grouped-GEMM work counter in meta

struct Plan {
  int T, d, E, k, I;
  int Tk;          // routed rows, T*k
  int rows;        // routed + shared rows, T*k + T
  int nblk;        // token blocks of kMaskBlock
  int ks;          // router split-K factor
  int gemm_bm;     // grouped-GEMM M tile
  int max_tiles;   // upper bound of grouped-GEMM M tiles
  // workspace buffers
  float* part;               // [ks][T][E] router partial logits
  int32_t* topk_idx;         // [T][k]
  float* topk_w;             // [T][k]
  unsigned long long* mask;  // [nblk][E] token bitmask per (block, expert)
  int32_t* blk_base;         // [nblk][E] first row of (block, expert)
  int32_t* offs;             // [E+2] row offsets, expert E = shared
  int32_t* meta;             // [kMetaInts]: [0] touched experts incl. shared, [1] grouped-GEMM M tiles,
                             // [2] routed experts' M tiles (the shared expert's follow), [16..23] gate/up and
                             // [24..31] down work counters, one per XCD; [32..47] the same for a launch over
                             // the shared expert's tiles alone
  int32_t* touched;          // [E+1] touched experts: shared (E) first, then routed ascending
  int4* tiles;               // [max_tiles] {expert, first row within expert, rows, expert's first tile}
  int32_t* perm_src;         // [T*k]
  int32_t* pos;              // [T*k] inverse of perm_src
  uint16_t* h;               // bf16 [rows][I]
  void* y;                   // [rows][d]: fp32 (stream path) or bf16 (grouped path)
  // FP8 W8A8 only (MXFP8 activations of the routed experts)
  uint8_t* xq;               // [T][d] E4M3 codes of the token rows
  uint8_t* xs;               // [T][d / 32] E8M0 block scales
  uint8_t* hq;               // [T*k][I] codes of the routed hidden rows
  uint8_t* hs;               // [T*k][I / 32] their block scales
};

hipError_t launch_route(const Plan& p, const uint16_t* x, const uint16_t* w_router, const float* bias,
                        float* margin_out, int32_t* counts_out, int32_t* offsets_out, hipStream_t s, Marks& m);
hipError_t launch_permute(const Plan& p, int32_t* counts_out, int32_t* offsets_out, hipStream_t s, Marks& m);

struct ExpertWeights {
  // bf16 routed experts
  const uint16_t* gate;
  const uint16_t* up;
  const uint16_t* down;
  // Sherry ternary routed experts
  const uint32_t* qgate;
  const uint32_t* qup;
  const uint32_t* qdown;
  const uint16_t* sgate;
  const uint16_t* sup;
  const uint16_t* sdown;
  // FP8 (E4M3) routed experts: codes [E][rows][cols], fp32 scales [E][rows]
  const uint8_t* f8gate;
  const uint8_t* f8up;
  const uint8_t* f8down;
  const float* f8sgate;
  const float* f8sup;
  const float* f8sdown;
  // bf16 shared expert
  const uint16_t* s_gate;
  const uint16_t* s_up;
  const uint16_t* s_down;
  bool ternary;
  bool fp8;
  bool a8;       // with fp8: MXFP8 activations (W8A8)
  bool blocked;   // bf16 in the blocked layout (2 KB per 16 rows x 64 columns, per matrix, shared expert too)
  bool tblocked;  // with ternary: code matrices in the blocked layout ([rows/16][cols/512][16][80 B])
  bool tshared;   // with ternary: the shared expert is Sherry-packed, expert E of the code and scale arrays
};

hipError_t launch_stream_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                 Marks& m);
hipError_t launch_grouped_experts(const Plan& p, const uint16_t* x, const ExpertWeights& w, hipStream_t s,
                                  Marks& m);
hipError_t launch_combine(const Plan& p, bool y_is_f32, uint16_t* out, hipStream_t s, Marks& m);

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_block_bf16(const uint16_t* src, uint16_t* dst, int64_t count, int64_t rows, int64_t cols,
                             hipStream_t s);
hipError_t launch_block_sherry(const uint32_t* src, uint32_t* dst, int64_t count, int64_t rows, int64_t cols,
                               hipStream_t s);

int grouped_gemm_bm();
int route_split_for(int T, int d, int E);

}  // namespace hymoe

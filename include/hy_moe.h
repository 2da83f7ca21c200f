/*
 * hy_moe.h — C ABI of an MI355X-native (gfx950) forward pass of one sparse
 * Mixture-of-Experts FFN layer.
 *
 * What the layer computes (m.xxqk.cn Hy4 preview explainer, sections 2.1
 * "FFN 层拆分" and 2.2 "路由机制"; Tencent Hy4 preview model card; the
 * app.myzaker.com Hy4 Preview news, section "770B 不是简单堆参数"):
 *   the FFN is split into E routed experts plus one shared expert; a router
 *   scores each token against every routed expert, the top-k are activated,
 *   every token also passes through the shared expert, and the expert outputs
 *   are merged into the layer output. Hy4 preview: E = 256, k = 8, d = 6144.
 * Readings taken where the pages are silent (each is a fixed part of this ABI):
 *   logits   l[t][e] = sum_i x[t][i] W_router[e][i] (+ router_bias[e]), fp32 accumulate
 *   select   the k largest logits, ties to the lower expert index
 *   weights  w[t][e] = softmax over the selected set: exp(l_e - l_max) / sum
 *   expert   y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z)
 *   output   out[t] = bf16( y_shared(x_t) + sum_{e in S_t} w[t][e] y_e(x_t) ),
 *            the sum taken in fp32 over the set in ascending expert order and
 *            rounded once (nearest even).
 *
 * Conventions for every entry point:
 *  - Tensors are row-major and contiguous. "bf16" means IEEE bfloat16 bit
 *    patterns. Weight matrices are stored [out][in] (the input dimension is
 *    contiguous): W_gate/W_up [E][I][d], W_down [E][d][I], shared [I][d]/[d][I].
 *  - Pointers documented as DEVICE must point to memory of the device current on
 *    the calling thread; the caller owns every buffer and the library never
 *    frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work
 *    is enqueued on it and the call returns without waiting; device-side faults
 *    surface at the caller's next synchronisation.
 *  - Every argument check runs before anything is enqueued. On error nothing is
 *    enqueued and the outputs are untouched.
 *  - Results are deterministic: the same inputs on the same device give
 *    bitwise-identical outputs (no floating-point atomics anywhere).
 *  - Supported envelope: 1 <= k <= min(E, 16), E <= 1024, d % 128 == 0,
 *    I % 128 == 0, T * k < 2^31. T == 0 is a no-op returning HY_MOE_OK.
 *    HY_MOE_PATH_GROUPED further needs T * d * 2 and T * (k + 1) * I * 2 (the bytes
 *    of x and of the hidden activations) below 2^32; HY_MOE_PATH_AUTO takes the
 *    streaming path where they are not.
 */
#ifndef HY_MOE_H
#define HY_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HY_MOE_OK = 0,
  HY_MOE_ERR_INVALID_ARG = -1, /* null required pointer, negative size, k < 1, k > E */
  HY_MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported envelope */
  HY_MOE_ERR_WORKSPACE = -3,   /* workspace given but smaller than hy_moe_workspace_size() */
  HY_MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} hy_moe_status;

/* Storage format of the routed experts' weights (the shared expert is bf16). */
typedef enum {
  HY_MOE_WEIGHTS_BF16 = 0,
  /* Sherry sparse-ternary weights (ai.chattools.top article on compressing Hy4
   * preview to 214GB, section "极限压缩背后的技术支柱：Sherry 与 MIX-STQ1_0"):
   * groups of 4 consecutive weights along a row hold values in {-1,0,+1} with
   * exactly one zero (4 positions x 2^3 signs = 32 codes = 5 bits, 1.25 bits
   * per weight); weight = row scale (bf16) * ternary value.
   * Packed layout: a row of C weights is C/128 blocks of 5 uint32 words. The
   * 5 words of a block, little-endian, form a 160-bit integer B; group g of the
   * block (weights 4g..4g+3) has code (B >> 5g) & 31. Code bits 0-1 give the
   * position of the zero in the group; bits 2, 3, 4 give the signs of the
   * first, second and third non-zero weight in ascending position (1 means -1).
   * Every bit pattern is a valid block. */
  HY_MOE_WEIGHTS_SHERRY_TERNARY = 1,
  /* FP8 weights (the Hy4 preview release ships BF16 and FP8 weights, FP8 halving
   * the weight storage: app.myzaker.com Hy4 Preview news, section "MTP、FP8 与
   * 低价 API"). The pages give no encoding or scale layout; taken here: each
   * routed expert weight is one OCP 8-bit float in the E4M3 encoding (sign bit 7,
   * exponent bits 6-3 with bias 7, mantissa bits 2-0; exponent 0 is subnormal,
   * S.1111.111 is NaN, no infinities), each output row has one fp32 scale, and
   * weight = scale * value. Activations and the shared expert stay bf16; a NaN
   * code gives NaN outputs. The kernels convert the codes to bf16 exactly (every
   * E4M3 value is a bf16 value) and scale the fp32 sums. */
  HY_MOE_WEIGHTS_FP8_E4M3 = 2,
  /* FP8 weights with FP8 activations (W8A8; same pages, which name no activation
   * format). Weights, scales and their layout exactly as HY_MOE_WEIGHTS_FP8_E4M3.
   * The routed experts' activations (the token rows entering gate/up and the hidden
   * rows entering down) are quantized to MXFP8 as OCP Microscaling Formats v1.0
   * defines it (see hy_moe_mxfp8_quantize) and the products run on the FP8 matrix
   * cores, block scales applied in hardware, fp32 accumulation; the hidden rows are
   * quantized from fp32. The router and the shared expert stay bf16. Runs on the
   * grouped path only (AUTO picks it; HY_MOE_PATH_STREAM -> HY_MOE_ERR_UNSUPPORTED) and
   * needs d % 256 == 0 and I % 256 == 0. */
  HY_MOE_WEIGHTS_FP8_W8A8 = 3,
  /* bf16 weights as HY_MOE_WEIGHTS_BF16 (the same layer, m.xxqk.cn Hy4 preview explainer
   * section 2.1; the same pointers W_gate/W_up/W_down and Ws_gate/Ws_up/Ws_down, the same
   * sizes), every expert matrix, routed and shared, stored in this library's blocked
   * layout: a matrix of R rows by K columns (R = I and K = d for gate and up, R = d and
   * K = I for down) becomes one 1024-value (2 KB) block per 16-row group and 64-column
   * slab, blocks in (row group, slab) order; the 8 values of row r in columns
   * [64 c + 8 q, 64 c + 8 q + 8) (q < 8) start at element
   * 1024 * ((r / 16) * (K / 64) + c) + 8 * (64 * (q % 2) + 16 * (q / 2) + r % 16).
   * Each 16-row group's 64-column slab is then one contiguous 2 KB run, in the order the
   * streaming path's load instructions take it (1 KB in order each), which HBM delivers
   * faster than 16 rows a whole row apart. Results are bitwise identical to
   * HY_MOE_WEIGHTS_BF16 on the same weights. hy_moe_block_bf16 converts row-major
   * matrices. */
  HY_MOE_WEIGHTS_BF16_BLOCKED = 4,
  /* Sherry ternary codes as HY_MOE_WEIGHTS_SHERRY_TERNARY (the same pointers, scales and
   * sizes; ai.chattools.top article, section on Sherry and MIX-STQ1_0), each code matrix
   * stored in this library's blocked layout: a matrix of R rows whose K weights per row
   * pack into K/128 * 20 bytes becomes [R/16][K/512][16][80 bytes]: the 80 code bytes of
   * row r for weights [512 c, 512 c + 512) start at byte 1280 * ((r / 16) * (K / 512) + c)
   * + 80 * (r % 16). Each 16-row group's slab is then 1280 bytes, exactly ten 128-byte
   * lines, instead of 16 pieces of 80 bytes that straddle lines. Needs d % 512 == 0,
   * I % 512 == 0 and I * d * 20 / 128 < 2^31 (one expert's code matrix), and 16-byte
   * aligned code arrays (HY_MOE_ERR_UNSUPPORTED / HY_MOE_ERR_INVALID_ARG otherwise). Results are bitwise identical to
   * HY_MOE_WEIGHTS_SHERRY_TERNARY on the same codes. hy_moe_block_sherry converts. */
  HY_MOE_WEIGHTS_SHERRY_BLOCKED = 5
} hy_moe_wfmt;

/* Which kernels run the experts. AUTO picks by the average rows per expert. */
typedef enum {
  HY_MOE_PATH_AUTO = 0,
  HY_MOE_PATH_STREAM = 1,  /* weight-streaming kernels: each touched expert's weights read once per
                              pass of up to 16 of its tokens (4 in the LDS-staged Sherry kernels,
                              used when d and I are multiples of 512); meant for decode-sized
                              batches */
  HY_MOE_PATH_GROUPED = 2  /* LDS-tiled grouped GEMM on bf16 MFMA; prefill-sized batches. Sherry
                              and FP8 codes are decoded to bf16 operands on the fly (the row scales
                              are applied to the sums); with them the bf16 shared expert runs in
                              its own launches of the bf16 kernel */
} hy_moe_path;

/*
 * hy_moe_forward — the whole layer, bf16 weights, no router bias.
 *   x         DEVICE bf16 [T][d]       token activations
 *   W_router  DEVICE bf16 [E][d]
 *   W_gate    DEVICE bf16 [E][I][d]    routed experts
 *   W_up      DEVICE bf16 [E][I][d]
 *   W_down    DEVICE bf16 [E][d][I]
 *   Ws_gate   DEVICE bf16 [I][d]       shared expert
 *   Ws_up     DEVICE bf16 [I][d]
 *   Ws_down   DEVICE bf16 [d][I]
 *   out       DEVICE bf16 [T][d]       written in full
 * Scratch memory is allocated stream-ordered on `stream` (hipMallocAsync) and
 * released stream-ordered before returning; use hy_moe_forward_ex with a
 * caller workspace to avoid any allocation.
 */
int hy_moe_forward(const void* x, const void* W_router, const void* W_gate, const void* W_up,
                   const void* W_down, const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                   int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, void* out, void* stream);

/* Full argument set of hy_moe_forward_ex. Zero-initialise, then fill. */
typedef struct hy_moe_args {
  /* inputs (DEVICE) */
  const void* x;             /* bf16 [T][d] */
  const void* W_router;      /* bf16 [E][d] */
  const float* router_bias;  /* fp32 [E] or NULL; added to the logits before both the
                                selection and the softmax */
  hy_moe_wfmt expert_format;
  const void* W_gate;        /* BF16: bf16 [E][I][d] */
  const void* W_up;          /* BF16: bf16 [E][I][d] */
  const void* W_down;        /* BF16: bf16 [E][d][I] */
  const void* Wq_gate;       /* SHERRY_TERNARY: uint32 [E][I][d/128*5]; FP8_E4M3: uint8 [E][I][d] */
  const void* Wq_up;         /* SHERRY_TERNARY: uint32 [E][I][d/128*5]; FP8_E4M3: uint8 [E][I][d] */
  const void* Wq_down;       /* SHERRY_TERNARY: uint32 [E][d][I/128*5]; FP8_E4M3: uint8 [E][d][I]
                                (FP8 codes 16-byte aligned, everything else 4-byte) */
  const void* S_gate;        /* row scales. SHERRY_TERNARY: bf16 [E][I]; FP8_E4M3: fp32 [E][I] */
  const void* S_up;          /* SHERRY_TERNARY: bf16 [E][I]; FP8_E4M3: fp32 [E][I] */
  const void* S_down;        /* SHERRY_TERNARY: bf16 [E][d]; FP8_E4M3: fp32 [E][d] */
  const void* Ws_gate;       /* bf16 [I][d] */
  const void* Ws_up;         /* bf16 [I][d] */
  const void* Ws_down;       /* bf16 [d][I] */
  int64_t T, d, E, k, I;
  /* output (DEVICE) */
  void* out;                 /* bf16 [T][d] */
  /* scratch (DEVICE): NULL => allocated stream-ordered on the stream */
  void* workspace;
  size_t workspace_bytes;
  /* optional routing outputs (DEVICE, NULL to skip) */
  int32_t* topk_idx;         /* [T][k] selected experts, ascending expert id */
  float* topk_w;             /* [T][k] merge weights, same order */
  int32_t* counts;           /* [E]    tokens per routed expert */
  int32_t* offsets;          /* [E+1]  exclusive prefix sum of counts */
  int32_t* perm_src;         /* [T*k]  t*k+j of the pair at expert-contiguous row p
                                (experts ascending, tokens ascending within one) */
  float* margin;             /* [T]    k-th minus (k+1)-th largest logit (fp32); +inf if k == E */
  hy_moe_path path;
  /* optional profiling hook: NULL, or HY_MOE_NUM_STAGE_EVENTS hipEvent_t handles (created
     by the caller) recorded on the stream before the first kernel and after each kernel,
     in the order listed below; event i+1 minus event i is the duration of kernel i. A NULL
     entry is skipped (that point is not recorded). */
  void** stage_events;
  /* optional hidden-row output, HY_MOE_WEIGHTS_FP8_W8A8 only (DEVICE, NULL to skip; both or
     neither): the routed experts' hidden rows exactly as the down projection reads them,
     in dispatched-row order (row p belongs to the pair perm_src[p]). hidden_codes: uint8
     [T*k][I] E4M3 codes, 16-byte aligned; hidden_scales: uint8 [T*k][I/32] E8M0 block
     scales. When given they replace the workspace's copy (no extra traffic). */
  void* hidden_codes;
  void* hidden_scales;
  /* The shared expert's weight format (ai.chattools.top article, section on Sherry and
     MIX-STQ1_0: Sherry packing is chosen per layer, so a layer's shared expert may be
     packed like its routed experts). HY_MOE_WEIGHTS_BF16 (0, what a zero-initialized
     struct holds): bf16 Ws_gate/Ws_up/Ws_down. Or the expert format itself, when that is
     HY_MOE_WEIGHTS_SHERRY_TERNARY or HY_MOE_WEIGHTS_SHERRY_BLOCKED: the shared expert is
     expert E of Wq_gate/Wq_up/Wq_down and S_gate/S_up/S_down, which then hold E+1
     experts; Ws_* are not read (may be NULL). This needs d % 512 == 0, I % 512 == 0,
     I * d * 20 / 128 < 2^31 and 16-byte aligned code arrays (HY_MOE_ERR_UNSUPPORTED /
     HY_MOE_ERR_INVALID_ARG otherwise); any other value is HY_MOE_ERR_INVALID_ARG. */
  hy_moe_wfmt shared_format;
} hy_moe_args;

/* Kernels of one call, in launch order (indices into the stage events). */
enum {
  HY_MOE_K_ROUTE_LOGITS = 0, /* router logits (MFMA) */
  HY_MOE_K_ROUTE_TOPK = 1,   /* top-k selection, weights, dispatch masks (and, for T <= 64, the
                                dispatch lists and permutation: kernels 2 and 3 are then empty) */
  HY_MOE_K_PERMUTE_SCAN = 2, /* per-expert counts, offsets, work lists */
  HY_MOE_K_PERMUTE_SCATTER = 3,
  HY_MOE_K_EXPERT_GATEUP = 4, /* gate/up + SwiGLU of every touched expert and the shared expert */
  HY_MOE_K_EXPERT_DOWN = 5,   /* down projection */
  HY_MOE_K_COMBINE = 6,       /* weighted merge + shared-expert add */
  HY_MOE_NUM_KERNELS = 7,
  HY_MOE_NUM_STAGE_EVENTS = 8
};

/* hy_moe_forward_ex — the layer with every option. Returns a hy_moe_status. */
int hy_moe_forward_ex(const hy_moe_args* args, void* stream);

/*
 * hy_moe_forward_noalloc — hy_moe_forward_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same layer and the same kernels; the scratch memory is a buffer of
 * HY_MOE_NOALLOC_SCRATCH_BYTES that the library keeps per device (a device global,
 * present from the library's load on that device until the process ends). The call
 * allocates nothing and frees nothing.
 *   args  as for hy_moe_forward_ex, with workspace NULL and workspace_bytes 0
 *         (HY_MOE_ERR_INVALID_ARG otherwise).
 * Shapes whose hy_moe_workspace_size() exceeds HY_MOE_NOALLOC_SCRATCH_BYTES are
 * rejected with HY_MOE_ERR_WORKSPACE before anything is enqueued; at the Hy4 preview
 * layer shape (d = 6144, E = 256, k = 8, I = 2048) that admits T <= 251 (T <= 383 with
 * HY_MOE_WEIGHTS_FP8_W8A8, whose grouped path keeps its expert outputs in bf16). All calls on
 * one device share that device's buffer and it keeps the last call's contents: calls
 * that overlap in time on one device (other streams, other threads) race and their
 * results are undefined, so serialize them. Nothing in the buffer needs to start at
 * zero: each call writes everything it reads before reading it.
 */
#define HY_MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int hy_moe_forward_noalloc(const hy_moe_args* args, void* stream);

/* Bytes of DEVICE workspace hy_moe_forward_ex needs for this shape (for the
 * largest of the paths it may pick); 0 for invalid shapes. Alignment: 256 B. */
size_t hy_moe_workspace_size(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, hy_moe_wfmt expert_format);

/* Static text for a status code. */
const char* hy_moe_status_string(int status);

/*
 * hy_moe_sherry_pack_host — HOST helper: pack ternary values into the layout
 * above. tern: HOST int8 [rows][cols] in {-1,0,+1}, exactly one zero per group
 * of 4 along a row, cols % 128 == 0; packed: HOST uint32 [rows][cols/128*5].
 * Returns HY_MOE_ERR_INVALID_ARG (packed untouched) if a group breaks the rule.
 */
int hy_moe_sherry_pack_host(const int8_t* tern, int64_t rows, int64_t cols, uint32_t* packed);

/*
 * hy_moe_mxfp8_quantize — the activation quantization of HY_MOE_WEIGHTS_FP8_W8A8 on its
 * own (OCP Microscaling Formats v1.0, MXFP8): each row is cut into blocks of 32
 * consecutive values; a block shares the scale 2^e, e = floor(log2 max|v|) - 8 clamped
 * to [-127, 127] (-127 for a block of zeros), stored as the E8M0 byte e + 127; each
 * value becomes the E4M3 code (the encoding of HY_MOE_WEIGHTS_FP8_E4M3) of the value
 * nearest to v * 2^-e, ties to the even mantissa, saturated to +-448.
 *   x       DEVICE bf16 [rows][cols], 16-byte aligned; cols % 32 == 0
 *   codes   DEVICE uint8 [rows][cols], 16-byte aligned (out)
 *   scales  DEVICE uint8 [rows][cols / 32] (out)
 * Enqueued on `stream` without blocking. Returns HY_MOE_OK, HY_MOE_ERR_INVALID_ARG
 * (null or misaligned pointers, rows < 0, cols not a positive multiple of 32; nothing
 * enqueued), HY_MOE_ERR_UNSUPPORTED (rows * cols >= 2^40) or HY_MOE_ERR_HIP.
 * rows == 0 is a no-op.
 */
int hy_moe_mxfp8_quantize(const void* x, int64_t rows, int64_t cols, void* codes, void* scales, void* stream);

/*
 * hy_moe_block_bf16 — rewrites row-major bf16 matrices in the layout of
 * HY_MOE_WEIGHTS_BF16_BLOCKED (a one-time conversion of a model's expert weights).
 *   src    DEVICE bf16, `count` matrices of [rows][cols] back to back, 16-byte aligned
 *   dst    DEVICE bf16, the same size, 16-byte aligned, not overlapping src (out)
 *   count >= 0, rows % 16 == 0, cols % 64 == 0, rows > 0, cols > 0
 * Enqueued on `stream` without blocking. Returns HY_MOE_OK, HY_MOE_ERR_INVALID_ARG
 * (null or misaligned pointers, overlapping buffers, bad sizes; nothing enqueued) or
 * HY_MOE_ERR_HIP. count == 0 is a no-op.
 */
int hy_moe_block_bf16(const void* src, void* dst, int64_t count, int64_t rows, int64_t cols, void* stream);

/*
 * hy_moe_block_sherry — rewrites Sherry code matrices (the packing of
 * HY_MOE_WEIGHTS_SHERRY_TERNARY) in the layout of HY_MOE_WEIGHTS_SHERRY_BLOCKED.
 *   src    DEVICE, `count` code matrices of `rows` rows of cols / 128 * 20 bytes (cols
 *          weights per row) back to back, 16-byte aligned
 *   dst    DEVICE, the same size, 16-byte aligned, not overlapping src (out)
 *   count >= 0, rows % 16 == 0, cols % 512 == 0, rows > 0, cols > 0
 * Enqueued on `stream` without blocking. Returns HY_MOE_OK, HY_MOE_ERR_INVALID_ARG
 * (null or misaligned pointers, overlapping buffers, bad sizes; nothing enqueued) or
 * HY_MOE_ERR_HIP. count == 0 is a no-op.
 */
int hy_moe_block_sherry(const void* src, void* dst, int64_t count, int64_t rows, int64_t cols, void* stream);

/*
 * Machine-peak probes (not part of the layer): the rates this GPU reaches, for
 * reporting a layer's roofline fraction against measured as well as published
 * peaks. Each enqueues its kernels on `stream` (a hipStream_t, NULL = default),
 * waits for them, and returns HY_MOE_OK or HY_MOE_ERR_HIP; bad arguments give
 * HY_MOE_ERR_INVALID_ARG with nothing enqueued. They allocate nothing.
 *
 * hy_moe_probe_mfma_bf16: dense 32x32x16 bf16 MFMAs with fp32 accumulation on 4
 *   workgroups per CU for about 40 ms. operands: DEVICE, 16-byte aligned, at least
 *   HY_MOE_PROBE_OPERAND_BYTES of bf16 bit patterns filled by the caller (random
 *   values give the rate of real data: under the power cap the clock depends on
 *   operand bit activity). Writes TFLOP/s (2 flop per multiply-add) to *tflops
 *   (HOST).
 * hy_moe_probe_mfma_fp8: the same with 32x32x64 E4M3 MFMAs (block scales of 1.0) for
 *   about 40 ms at the FP8 rate. operands: as above, filled with E4M3 codes (finite
 *   values: random bytes include NaN codes). 2 flop per multiply-add.
 * hy_moe_probe_hbm_read: reads buf (DEVICE, 16-byte aligned, `bytes` >= 16; use
 *   much more than the 256 MB last-level cache) once untimed, then three times timed
 *   with non-temporal 16-byte loads, 1 KB in order per wave instruction. Writes the best
 *   pass's GB/s (1e9 B/s) to *gbps (HOST).
 */
#define HY_MOE_PROBE_OPERAND_BYTES 65536
int hy_moe_probe_mfma_bf16(const void* operands, size_t operand_bytes, float* tflops, void* stream);
int hy_moe_probe_mfma_fp8(const void* operands, size_t operand_bytes, float* tflops, void* stream);
int hy_moe_probe_hbm_read(const void* buf, size_t bytes, float* gbps, void* stream);

/*
 * hy_indexer_topk — sparse-attention indexer of the Hy4 preview configuration (Tencent
 * Hy4 preview model card, configuration summary: every layer uses DeepSeek-style sparse
 * attention with an indexer of 32 heads, head_dim 128 and top-k 2048, whose key per
 * token is shared by all heads; with IndexCache 57 of the 78 layers reuse the selection
 * of the layer before them, so only 21 layers run it). The pages give no score formula;
 * read here as score(s) = sum over heads h of w[h] * max(0, q[h] . k[s]).
 *   q       DEVICE bf16 [B][H][D]  one query per sequence (16-byte aligned)
 *   w       DEVICE fp32 [B][H]     per-head weights of each query
 *   keys    DEVICE bf16 [B][S][D]  each sequence's keys (16-byte aligned)
 *   idx     DEVICE int32 [B][min(K, S)]  out: the K highest-scoring keys of each
 *           query, ties to the lower key index, in ascending key order
 *   scores  DEVICE fp32 [B][S] or NULL: out, the scores (fp32 accumulation); when NULL
 *           they stay in the workspace
 *   workspace  DEVICE, 256-byte aligned, hy_indexer_workspace_size(B, S) bytes: the
 *           scores and the candidates of the two-stage selection (chunks of 8192 keys
 *           each keep their top K in parallel, then one merge per query)
 *   stage_events  NULL or 3 hipEvent_t (caller-created; NULL entries skipped) recorded
 *           before the scoring kernel, after it and after the selection kernel
 *   stream  hipStream_t; enqueued without blocking.
 * Supported: H == 32, D == 128, B <= 65535, B * S < 2^31. Returns HY_MOE_OK, INVALID_ARG
 * (null or misaligned pointers, negative sizes, K < 1), UNSUPPORTED, WORKSPACE or HIP;
 * B == 0 or S == 0 is a no-op. Checks run before anything is enqueued.
 */
size_t hy_indexer_workspace_size(int64_t B, int64_t S);
int hy_indexer_topk(const void* q, const float* w, const void* keys, int64_t B, int64_t H, int64_t D, int64_t S,
                    int64_t K, int32_t* idx, float* scores, void* workspace, size_t workspace_bytes,
                    void* const* stage_events, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HY_MOE_H */

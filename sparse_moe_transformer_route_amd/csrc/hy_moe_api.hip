// C ABI of the MoE layer: argument checks, workspace layout, launch sequence.
// The header (include/hy_moe.h) documents every entry point.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "hy_moe.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace hymoe;

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxK = 16;

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t part, topk_idx, topk_w, mask, blk_base, offs, meta, touched, tiles, perm_src, pos, h, y, xq, xs, hq, hs,
      total;
  int ks, nblk, max_tiles;
};

bool valid_format(int f) {
  return f == HY_MOE_WEIGHTS_BF16 || f == HY_MOE_WEIGHTS_SHERRY_TERNARY || f == HY_MOE_WEIGHTS_FP8_E4M3 ||
         f == HY_MOE_WEIGHTS_FP8_W8A8 || f == HY_MOE_WEIGHTS_BF16_BLOCKED || f == HY_MOE_WEIGHTS_SHERRY_BLOCKED;
}

// W8A8 runs on the grouped path only, whose y is bf16; it adds the MXFP8 codes and
// scales of the token rows and of the routed hidden rows.
Layout make_layout(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, int fmt) {
  Layout L{};
  L.ks = route_split_for((int)T, (int)d, (int)E);
  L.nblk = (int)((T + kMaskBlock - 1) / kMaskBlock);
  const int64_t Tk = T * k, rows = Tk + T;
  const int bm = grouped_gemm_bm();
  L.max_tiles = (int)((Tk + bm - 1) / bm + E + (T + bm - 1) / bm);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.part = take(sizeof(float) * (size_t)L.ks * T * E);
  L.topk_idx = take(sizeof(int32_t) * (size_t)Tk);
  L.topk_w = take(sizeof(float) * (size_t)Tk);
  L.mask = take(sizeof(unsigned long long) * (size_t)L.nblk * E);
  L.blk_base = take(sizeof(int32_t) * (size_t)L.nblk * E);
  L.offs = take(sizeof(int32_t) * (size_t)(E + 2));
  L.meta = take(sizeof(int32_t) * kMetaInts);
  L.touched = take(sizeof(int32_t) * (size_t)(E + 1));
  L.tiles = take(sizeof(int4) * (size_t)L.max_tiles);
  L.perm_src = take(sizeof(int32_t) * (size_t)Tk);
  L.pos = take(sizeof(int32_t) * (size_t)Tk);
  L.h = take(sizeof(uint16_t) * (size_t)rows * I);
  const bool a8 = fmt == HY_MOE_WEIGHTS_FP8_W8A8;
  L.y = take((a8 ? 2 : 4) * (size_t)rows * d);  // fp32 for the streaming path, bf16 for the grouped path
  if (a8) {
    L.xq = take((size_t)T * d);
    L.xs = take((size_t)T * (d / 32));
    L.hq = take((size_t)Tk * I);
    L.hs = take((size_t)Tk * (I / 32));
  }
  L.total = off;
  return L;
}

// The grouped GEMM addresses x and h with 32-bit byte offsets from their bases.
bool grouped_fits(int64_t T, int64_t d, int64_t k, int64_t I) {
  const int64_t lim = (int64_t)1 << 32;
  return T * d * 2 < lim && T * (k + 1) * I * 2 < lim;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_shape(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I) {
  if (T < 0 || d <= 0 || E <= 0 || I <= 0 || k < 1 || k > E) return HY_MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK || d % 128 != 0 || I % 128 != 0) return HY_MOE_ERR_UNSUPPORTED;
  if (d > (1 << 20) || I > (1 << 20)) return HY_MOE_ERR_UNSUPPORTED;
  if (T * (k + 1) >= ((int64_t)1 << 31)) return HY_MOE_ERR_UNSUPPORTED;
  return HY_MOE_OK;
}

int check_args(const hy_moe_args* a) {
  if (!a) return HY_MOE_ERR_INVALID_ARG;
  int rc = check_shape(a->T, a->d, a->E, a->k, a->I);
  if (rc != HY_MOE_OK) return rc;
  if (!valid_format(a->expert_format)) return HY_MOE_ERR_INVALID_ARG;
  if (a->path != HY_MOE_PATH_AUTO && a->path != HY_MOE_PATH_STREAM && a->path != HY_MOE_PATH_GROUPED)
    return HY_MOE_ERR_INVALID_ARG;
  // the shared expert: bf16 (Ws_*), or Sherry codes as expert E of the routed arrays
  const bool tshared = a->shared_format != HY_MOE_WEIGHTS_BF16;
  if (tshared && (a->shared_format != a->expert_format || (a->expert_format != HY_MOE_WEIGHTS_SHERRY_TERNARY &&
                                                          a->expert_format != HY_MOE_WEIGHTS_SHERRY_BLOCKED)))
    return HY_MOE_ERR_INVALID_ARG;
  if (a->T == 0) return HY_MOE_OK;
  const void* req[] = {a->x, a->W_router, a->out};
  for (const void* p : req)
    if (!p || !aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
  if (!tshared) {
    const void* sw[] = {a->Ws_gate, a->Ws_up, a->Ws_down};
    for (const void* p : sw)
      if (!p || !aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
  } else {
    // it runs in the LDS-staged decode kernels (16-byte code loads, 512-weight chunks)
    const void* q[] = {a->Wq_gate, a->Wq_up, a->Wq_down};
    for (const void* p : q)
      if (!p || !aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
    if (a->d % 512 != 0 || a->I % 512 != 0 || a->I * (a->d / 128 * 20) >= ((int64_t)1 << 31))
      return HY_MOE_ERR_UNSUPPORTED;
  }
  if (a->router_bias && !aligned(a->router_bias, 4)) return HY_MOE_ERR_INVALID_ARG;
  if (a->expert_format == HY_MOE_WEIGHTS_BF16 || a->expert_format == HY_MOE_WEIGHTS_BF16_BLOCKED) {
    const void* w[] = {a->W_gate, a->W_up, a->W_down};
    for (const void* p : w)
      if (!p || !aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
  } else if (a->expert_format == HY_MOE_WEIGHTS_SHERRY_TERNARY || a->expert_format == HY_MOE_WEIGHTS_SHERRY_BLOCKED) {
    const void* w[] = {a->Wq_gate, a->Wq_up, a->Wq_down, a->S_gate, a->S_up, a->S_down};
    for (const void* p : w)
      if (!p || !aligned(p, 4)) return HY_MOE_ERR_INVALID_ARG;
    if (a->expert_format == HY_MOE_WEIGHTS_SHERRY_BLOCKED) {
      // the blocked codes run in the LDS-staged kernels only: 512-weight slabs, 16-byte loads
      const void* q[] = {a->Wq_gate, a->Wq_up, a->Wq_down};
      for (const void* p : q)
        if (!aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
      if (a->d % 512 != 0 || a->I % 512 != 0) return HY_MOE_ERR_UNSUPPORTED;
      // and address one expert's code matrix (I d 20 / 128 bytes) with 32-bit offsets
      if (a->I * (a->d / 128 * 20) >= ((int64_t)1 << 31)) return HY_MOE_ERR_UNSUPPORTED;
    }
  } else {
    const void* q[] = {a->Wq_gate, a->Wq_up, a->Wq_down};
    for (const void* p : q)
      if (!p || !aligned(p, 16)) return HY_MOE_ERR_INVALID_ARG;
    const void* sc[] = {a->S_gate, a->S_up, a->S_down};
    for (const void* p : sc)
      if (!p || !aligned(p, 4)) return HY_MOE_ERR_INVALID_ARG;
  }
  if (a->path == HY_MOE_PATH_GROUPED && !grouped_fits(a->T, a->d, a->k, a->I)) return HY_MOE_ERR_UNSUPPORTED;
  if (a->expert_format == HY_MOE_WEIGHTS_FP8_W8A8) {
    // grouped path only, two 128-code k steps at least in both products
    if (a->path == HY_MOE_PATH_STREAM || !grouped_fits(a->T, a->d, a->k, a->I)) return HY_MOE_ERR_UNSUPPORTED;
    if (a->d % 256 != 0 || a->I % 256 != 0) return HY_MOE_ERR_UNSUPPORTED;
  }
  if ((a->hidden_codes == nullptr) != (a->hidden_scales == nullptr)) return HY_MOE_ERR_INVALID_ARG;
  if (a->hidden_codes && (a->expert_format != HY_MOE_WEIGHTS_FP8_W8A8 || !aligned(a->hidden_codes, 16)))
    return HY_MOE_ERR_INVALID_ARG;
  const void* opt4[] = {a->topk_idx, a->topk_w, a->counts, a->offsets, a->perm_src, a->margin};
  for (const void* p : opt4)
    if (p && !aligned(p, 4)) return HY_MOE_ERR_INVALID_ARG;
  if (a->workspace) {
    if (!aligned(a->workspace, 256)) return HY_MOE_ERR_INVALID_ARG;
    if (a->workspace_bytes < make_layout(a->T, a->d, a->E, a->k, a->I, a->expert_format).total)
      return HY_MOE_ERR_WORKSPACE;
  }
  return HY_MOE_OK;
}

}  // namespace

extern "C" int hy_moe_forward_ex(const hy_moe_args* a, void* stream) {
  const int rc = check_args(a);
  if (rc != HY_MOE_OK) return rc;
  if (a->T == 0) return HY_MOE_OK;

  hipStream_t s = (hipStream_t)stream;
  const Layout L = make_layout(a->T, a->d, a->E, a->k, a->I, a->expert_format);
  uint8_t* ws = (uint8_t*)a->workspace;
  bool owned = false;
  if (!ws) {
    void* p = nullptr;
    if (hipMallocAsync(&p, L.total, s) != hipSuccess) return HY_MOE_ERR_HIP;
    ws = (uint8_t*)p;
    owned = true;
  }

  Plan p{};
  p.T = (int)a->T; p.d = (int)a->d; p.E = (int)a->E; p.k = (int)a->k; p.I = (int)a->I;
  p.Tk = p.T * p.k;
  p.rows = p.Tk + p.T;
  p.nblk = L.nblk;
  p.ks = L.ks;
  p.gemm_bm = grouped_gemm_bm();
  p.max_tiles = L.max_tiles;
  p.part = (float*)(ws + L.part);
  p.topk_idx = a->topk_idx ? a->topk_idx : (int32_t*)(ws + L.topk_idx);
  p.topk_w = a->topk_w ? a->topk_w : (float*)(ws + L.topk_w);
  p.mask = (unsigned long long*)(ws + L.mask);
  p.blk_base = (int32_t*)(ws + L.blk_base);
  p.offs = (int32_t*)(ws + L.offs);
  p.meta = (int32_t*)(ws + L.meta);
  p.touched = (int32_t*)(ws + L.touched);
  p.tiles = (int4*)(ws + L.tiles);
  p.perm_src = a->perm_src ? a->perm_src : (int32_t*)(ws + L.perm_src);
  p.pos = (int32_t*)(ws + L.pos);
  p.h = (uint16_t*)(ws + L.h);
  p.y = (void*)(ws + L.y);
  const bool a8 = a->expert_format == HY_MOE_WEIGHTS_FP8_W8A8;
  if (a8) {
    p.xq = ws + L.xq;
    p.xs = ws + L.xs;
    p.hq = a->hidden_codes ? (uint8_t*)a->hidden_codes : ws + L.hq;
    p.hs = a->hidden_scales ? (uint8_t*)a->hidden_scales : ws + L.hs;
  }

  ExpertWeights w{};
  w.tblocked = a->expert_format == HY_MOE_WEIGHTS_SHERRY_BLOCKED;
  w.ternary = a->expert_format == HY_MOE_WEIGHTS_SHERRY_TERNARY || w.tblocked;
  w.blocked = a->expert_format == HY_MOE_WEIGHTS_BF16_BLOCKED;
  w.fp8 = a->expert_format == HY_MOE_WEIGHTS_FP8_E4M3 || a8;
  w.a8 = a8;
  w.f8gate = (const uint8_t*)a->Wq_gate;
  w.f8up = (const uint8_t*)a->Wq_up;
  w.f8down = (const uint8_t*)a->Wq_down;
  w.f8sgate = (const float*)a->S_gate;
  w.f8sup = (const float*)a->S_up;
  w.f8sdown = (const float*)a->S_down;
  w.gate = (const uint16_t*)a->W_gate;
  w.up = (const uint16_t*)a->W_up;
  w.down = (const uint16_t*)a->W_down;
  w.qgate = (const uint32_t*)a->Wq_gate;
  w.qup = (const uint32_t*)a->Wq_up;
  w.qdown = (const uint32_t*)a->Wq_down;
  w.sgate = (const uint16_t*)a->S_gate;
  w.sup = (const uint16_t*)a->S_up;
  w.sdown = (const uint16_t*)a->S_down;
  w.tshared = a->shared_format != HY_MOE_WEIGHTS_BF16;
  w.s_gate = (const uint16_t*)a->Ws_gate;
  w.s_up = (const uint16_t*)a->Ws_up;
  w.s_down = (const uint16_t*)a->Ws_down;

  bool stream_path;
  if (a->path == HY_MOE_PATH_STREAM)
    stream_path = true;
  else if (a->path == HY_MOE_PATH_GROUPED)
    stream_path = false;
  else
    stream_path = !a8 && ((int64_t)p.Tk <= 16 * (int64_t)p.E || !grouped_fits(p.T, p.d, p.k, p.I));

  const uint16_t* x = (const uint16_t*)a->x;
  Marks marks{a->stage_events, 0};
  hipError_t err = marks.mark(s);
  if (err == hipSuccess) err = launch_route(p, x, (const uint16_t*)a->W_router, a->router_bias, a->margin, a->counts,
                                              a->offsets, s, marks);
  if (err == hipSuccess) err = launch_permute(p, a->counts, a->offsets, s, marks);
  if (err == hipSuccess)
    err = stream_path ? launch_stream_experts(p, x, w, s, marks) : launch_grouped_experts(p, x, w, s, marks);
  if (err == hipSuccess) err = launch_combine(p, stream_path, (uint16_t*)a->out, s, marks);
  if (owned) {
    if (hipFreeAsync(ws, s) != hipSuccess && err == hipSuccess) err = hipErrorUnknown;
  }
  return err == hipSuccess ? HY_MOE_OK : HY_MOE_ERR_HIP;
}

// Scratch of hy_moe_forward_noalloc: a device global, one copy per device, resolved to
// its device address once per device. In host code `scratch` names a host-side stand-in,
// never the device memory: only the address from hipGetSymbolAddress is used.
static_assert(HY_MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[HY_MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` per device, NULL until resolved
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, resolved on the first call on that device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HY_MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HY_MOE_ERR_UNSUPPORTED;
  void* p = __atomic_load_n(&g_scratch_dev[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev];
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HY_MOE_ERR_HIP;
      __atomic_store_n(&g_scratch_dev[dev], p, __ATOMIC_RELEASE);
    }
  }
  *out = p;
  return HY_MOE_OK;
}

}  // namespace

extern "C" int hy_moe_forward_noalloc(const hy_moe_args* a, void* stream) {
  if (!a) return HY_MOE_ERR_INVALID_ARG;
  if (a->workspace || a->workspace_bytes) return HY_MOE_ERR_INVALID_ARG;
  int rc = check_args(a);
  if (rc != HY_MOE_OK) return rc;
  if (a->T == 0) return HY_MOE_OK;
  if (make_layout(a->T, a->d, a->E, a->k, a->I, a->expert_format).total > (size_t)HY_MOE_NOALLOC_SCRATCH_BYTES)
    return HY_MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != HY_MOE_OK) return rc;
  hy_moe_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = HY_MOE_NOALLOC_SCRATCH_BYTES;
  return hy_moe_forward_ex(&b, stream);
}

extern "C" int hy_moe_forward(const void* x, const void* W_router, const void* W_gate, const void* W_up,
                              const void* W_down, const void* Ws_gate, const void* Ws_up, const void* Ws_down,
                              int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, void* out, void* stream) {
  hy_moe_args a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.W_router = W_router;
  a.expert_format = HY_MOE_WEIGHTS_BF16;
  a.W_gate = W_gate;
  a.W_up = W_up;
  a.W_down = W_down;
  a.Ws_gate = Ws_gate;
  a.Ws_up = Ws_up;
  a.Ws_down = Ws_down;
  a.T = T; a.d = d; a.E = E; a.k = k; a.I = I;
  a.out = out;
  a.path = HY_MOE_PATH_AUTO;
  return hy_moe_forward_ex(&a, stream);
}

extern "C" size_t hy_moe_workspace_size(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                                        hy_moe_wfmt expert_format) {
  if (!valid_format(expert_format)) return 0;
  if (check_shape(T, d, E, k, I) != HY_MOE_OK) return 0;
  return make_layout(T, d, E, k, I, expert_format).total;
}

extern "C" const char* hy_moe_status_string(int status) {
  switch (status) {
    case HY_MOE_OK: return "ok";
    case HY_MOE_ERR_INVALID_ARG: return "invalid argument";
    case HY_MOE_ERR_UNSUPPORTED: return "shape or option outside the supported envelope";
    case HY_MOE_ERR_WORKSPACE: return "workspace too small";
    case HY_MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int hy_moe_sherry_pack_host(const int8_t* tern, int64_t rows, int64_t cols, uint32_t* packed) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return HY_MOE_ERR_INVALID_ARG;
  if (rows == 0) return HY_MOE_OK;
  if (!tern || !packed) return HY_MOE_ERR_INVALID_ARG;
  // validate every group first so that packed stays untouched on error
  for (int64_t i = 0; i < rows * cols; i += 4) {
    int zeros = 0;
    for (int q = 0; q < 4; ++q) {
      const int v = tern[i + q];
      if (v < -1 || v > 1) return HY_MOE_ERR_INVALID_ARG;
      zeros += v == 0;
    }
    if (zeros != 1) return HY_MOE_ERR_INVALID_ARG;
  }
  const int64_t words = cols / 128 * 5;
  for (int64_t r = 0; r < rows; ++r) {
    uint32_t* row = packed + r * words;
    for (int64_t i = 0; i < words; ++i) row[i] = 0u;
    for (int64_t gidx = 0; gidx < cols / 4; ++gidx) {
      const int8_t* v = tern + r * cols + 4 * gidx;
      uint32_t code = 0, nz = 0;
      for (uint32_t q = 0; q < 4; ++q) {
        if (v[q] == 0) {
          code |= q;
        } else {
          if (v[q] < 0) code |= 1u << (2 + nz);
          ++nz;
        }
      }
      uint32_t* blk = row + (gidx / 32) * 5;
      const int bit0 = 5 * (int)(gidx % 32);
      for (int b = 0; b < 5; ++b)
        if ((code >> b) & 1u) blk[(bit0 + b) >> 5] |= 1u << ((bit0 + b) & 31);
    }
  }
  return HY_MOE_OK;
}

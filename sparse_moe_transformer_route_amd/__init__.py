"""Python binding of libhy_moe.so, the MI355X (gfx950) forward pass of one
sparse-MoE FFN layer (router -> top-k -> dispatch -> SwiGLU experts + shared
expert -> weighted combine).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. The entry points carry
the C ABI's names (include/hy_moe.h documents each). There is no fallback: if
the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

# torch provides the device memory and streams, and brings its own HIP runtime
# (soname libamdhip64.so.7). It must be loaded before libhy_moe.so so that the
# library binds to that same runtime instead of loading a second copy.
import torch  # noqa: F401

__all__ = ["forward", "forward_ex", "forward_noalloc", "forward_layer", "workspace_size", "status_string",
           "sherry_pack_host", "HyMoeError", "lib", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhy_moe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
WEIGHTS_BF16, WEIGHTS_SHERRY_TERNARY, WEIGHTS_FP8_E4M3, WEIGHTS_FP8_W8A8 = 0, 1, 2, 3
WEIGHTS_BF16_BLOCKED, WEIGHTS_SHERRY_BLOCKED = 4, 5
PATH_AUTO, PATH_STREAM, PATH_GROUPED = 0, 1, 2
KERNELS = ["route_logits", "route_topk", "permute_scan", "permute_scatter", "expert_gateup", "expert_down",
           "combine"]
NUM_STAGE_EVENTS = len(KERNELS) + 1

EXPORTED = ["hy_moe_forward", "hy_moe_forward_ex", "hy_moe_forward_noalloc", "hy_moe_workspace_size",
            "hy_moe_status_string", "hy_moe_sherry_pack_host", "hy_moe_mxfp8_quantize", "hy_moe_block_bf16", "hy_moe_block_sherry", "hy_moe_probe_mfma_bf16", "hy_moe_probe_mfma_fp8", "hy_moe_probe_hbm_read",
            "hy_indexer_workspace_size", "hy_indexer_topk"]
PROBE_OPERAND_BYTES = 65536
NOALLOC_SCRATCH_BYTES = 64 << 20  # HY_MOE_NOALLOC_SCRATCH_BYTES


class HyMoeArgs(ctypes.Structure):
    """Mirror of struct hy_moe_args."""
    _fields_ = [
        ("x", ctypes.c_void_p), ("W_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
        ("expert_format", ctypes.c_int),
        ("W_gate", ctypes.c_void_p), ("W_up", ctypes.c_void_p), ("W_down", ctypes.c_void_p),
        ("Wq_gate", ctypes.c_void_p), ("Wq_up", ctypes.c_void_p), ("Wq_down", ctypes.c_void_p),
        ("S_gate", ctypes.c_void_p), ("S_up", ctypes.c_void_p), ("S_down", ctypes.c_void_p),
        ("Ws_gate", ctypes.c_void_p), ("Ws_up", ctypes.c_void_p), ("Ws_down", ctypes.c_void_p),
        ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64), ("k", ctypes.c_int64),
        ("I", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p), ("perm_src", ctypes.c_void_p), ("margin", ctypes.c_void_p),
        ("path", ctypes.c_int),
        ("stage_events", ctypes.c_void_p),
        ("hidden_codes", ctypes.c_void_p), ("hidden_scales", ctypes.c_void_p),
        ("shared_format", ctypes.c_int),
    ]


class HyMoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.hy_moe_forward.argtypes = [vp] * 8 + [i64] * 5 + [vp, vp]
    L.hy_moe_forward.restype = ctypes.c_int
    L.hy_moe_forward_ex.argtypes = [ctypes.POINTER(HyMoeArgs), vp]
    L.hy_moe_forward_ex.restype = ctypes.c_int
    L.hy_moe_forward_noalloc.argtypes = [ctypes.POINTER(HyMoeArgs), vp]
    L.hy_moe_forward_noalloc.restype = ctypes.c_int
    L.hy_moe_workspace_size.argtypes = [i64] * 5 + [ctypes.c_int]
    L.hy_moe_workspace_size.restype = ctypes.c_size_t
    L.hy_moe_status_string.argtypes = [ctypes.c_int]
    L.hy_moe_status_string.restype = ctypes.c_char_p
    L.hy_moe_sherry_pack_host.argtypes = [vp, i64, i64, vp]
    L.hy_moe_sherry_pack_host.restype = ctypes.c_int
    L.hy_moe_mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    L.hy_moe_mxfp8_quantize.restype = ctypes.c_int
    L.hy_moe_block_bf16.argtypes = [vp, vp, i64, i64, i64, vp]
    L.hy_moe_block_bf16.restype = ctypes.c_int
    L.hy_moe_block_sherry.argtypes = [vp, vp, i64, i64, i64, vp]
    L.hy_moe_block_sherry.restype = ctypes.c_int
    L.hy_moe_probe_mfma_bf16.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_float), vp]
    L.hy_moe_probe_mfma_bf16.restype = ctypes.c_int
    L.hy_moe_probe_mfma_fp8.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_float), vp]
    L.hy_moe_probe_mfma_fp8.restype = ctypes.c_int
    L.hy_moe_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_float), vp]
    L.hy_moe_probe_hbm_read.restype = ctypes.c_int
    L.hy_indexer_workspace_size.argtypes = [i64, i64]
    L.hy_indexer_workspace_size.restype = ctypes.c_size_t
    L.hy_indexer_topk.argtypes = [vp, vp, vp] + [i64] * 5 + [vp, vp, vp, ctypes.c_size_t, vp, vp]
    L.hy_indexer_topk.restype = ctypes.c_int
    return L


_lib = _load()


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.hy_moe_status_string(status).decode()


def workspace_size(T, d, E, k, I, expert_format=WEIGHTS_BF16) -> int:
    return int(_lib.hy_moe_workspace_size(T, d, E, k, I, expert_format))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def forward(x, W_router, W_gate, W_up, W_down, Ws_gate, Ws_up, Ws_down, k, out=None, stream=None):
    """hy_moe_forward on torch tensors (bf16, contiguous, on the GPU). Returns out [T][d]."""
    import torch
    T, d = x.shape
    E, I = W_gate.shape[0], W_gate.shape[1]
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=x.device)
    rc = _lib.hy_moe_forward(_ptr(x), _ptr(W_router), _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Ws_gate),
                             _ptr(Ws_up), _ptr(Ws_down), T, d, E, k, I, _ptr(out), _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_forward")
    return out


def forward_ex(args: HyMoeArgs, stream=None) -> int:
    """hy_moe_forward_ex; returns the status code unchanged."""
    return _lib.hy_moe_forward_ex(ctypes.byref(args), _stream(stream))


def forward_noalloc(args: HyMoeArgs, stream=None) -> int:
    """hy_moe_forward_noalloc (scratch from the library's static per-device buffer);
    returns the status code unchanged."""
    return _lib.hy_moe_forward_noalloc(ctypes.byref(args), _stream(stream))


def forward_layer(inp: dict, k: int, *, want_routing=False, path=PATH_AUTO, workspace=None, out=None,
                  stream=None, stage_events=None, noalloc=False, fp8_activations=False, want_hidden=False,
                  weights_blocked=False):
    """Runs hy_moe_forward_ex on a dict of device tensors as made by
    hy_inputs.dev_layer(): x, router, bias, shared{gate,up,down} and either
    gate/up/down (bf16), qgate/qup/qdown + sgate/sup/sdown (ternary) or
    fgate/fup/fdown + fsgate/fsup/fsdown (FP8 E4M3 codes and fp32 scales).
    Returns dict(out, and with want_routing: topk_idx, topk_w, counts, offsets,
    perm_src, margin). noalloc: call hy_moe_forward_noalloc (no workspace).
    fp8_activations (FP8 weights only): the W8A8 format, MXFP8 activations; with
    want_hidden also hidden_codes [T*k][I] and hidden_scales [T*k][I/32] (the routed
    hidden rows as the down projection reads them, dispatched-row order).
    weights_blocked: the weights are in the blocked layout (block_layer): bf16 gate/up/down
    and the shared expert's matrices (HY_MOE_WEIGHTS_BF16_BLOCKED), or the Sherry code
    matrices (HY_MOE_WEIGHTS_SHERRY_BLOCKED; the bf16 shared expert stays row-major).
    A ternary dict with shared_sherry true holds the shared expert Sherry-packed as
    expert E of qgate/qup/qdown and sgate/sup/sdown (E+1 experts; shared_format set to
    the expert format, "shared" not read)."""
    import torch
    x = inp["x"]
    T, d = x.shape
    E = inp["router"].shape[0]
    ternary, fp8 = "qgate" in inp, "fgate" in inp
    # the library reads raw memory: reject element types it would misread
    want = ({"fgate": torch.uint8, "fup": torch.uint8, "fdown": torch.uint8, "fsgate": torch.float32,
             "fsup": torch.float32, "fsdown": torch.float32} if fp8 else
            {"qgate": torch.int32, "qup": torch.int32, "qdown": torch.int32, "sgate": torch.bfloat16,
             "sup": torch.bfloat16, "sdown": torch.bfloat16} if ternary else
            {"gate": torch.bfloat16, "up": torch.bfloat16, "down": torch.bfloat16})
    want.update(x=torch.bfloat16, router=torch.bfloat16)
    for key, dt in want.items():
        if inp[key].dtype != dt or not inp[key].is_contiguous():
            raise TypeError(f"forward_layer: {key} must be a contiguous {dt} tensor, got {inp[key].dtype}")
    I = inp["sgate"].shape[1] if ternary else inp["fsgate"].shape[1] if fp8 else inp["gate"].shape[1]
    tshared = ternary and bool(inp.get("shared_sherry", False))
    first = "qgate" if ternary else "fgate" if fp8 else "gate"
    if inp[first].shape[0] != E + (1 if tshared else 0):  # the library reads E (or E+1) experts
        raise ValueError(f"forward_layer: {first} holds {inp[first].shape[0]} experts, expected "
                         f"{E + (1 if tshared else 0)}")
    dev = x.device
    a = HyMoeArgs()
    a.x, a.W_router, a.router_bias = _ptr(x), _ptr(inp["router"]), _ptr(inp.get("bias"))
    if fp8_activations and not fp8:
        raise ValueError("forward_layer: fp8_activations needs FP8 weights")
    if weights_blocked and fp8:
        raise ValueError("forward_layer: weights_blocked applies to bf16 and Sherry weights")
    a.expert_format = ((WEIGHTS_SHERRY_BLOCKED if weights_blocked else WEIGHTS_SHERRY_TERNARY) if ternary else
                       (WEIGHTS_FP8_W8A8 if fp8_activations else WEIGHTS_FP8_E4M3) if fp8 else
                       WEIGHTS_BF16_BLOCKED if weights_blocked else WEIGHTS_BF16)
    if ternary:
        a.Wq_gate, a.Wq_up, a.Wq_down = _ptr(inp["qgate"]), _ptr(inp["qup"]), _ptr(inp["qdown"])
        a.S_gate, a.S_up, a.S_down = _ptr(inp["sgate"]), _ptr(inp["sup"]), _ptr(inp["sdown"])
    elif fp8:
        a.Wq_gate, a.Wq_up, a.Wq_down = _ptr(inp["fgate"]), _ptr(inp["fup"]), _ptr(inp["fdown"])
        a.S_gate, a.S_up, a.S_down = _ptr(inp["fsgate"]), _ptr(inp["fsup"]), _ptr(inp["fsdown"])
    else:
        a.W_gate, a.W_up, a.W_down = _ptr(inp["gate"]), _ptr(inp["up"]), _ptr(inp["down"])
    if tshared:
        a.shared_format = a.expert_format
    else:
        sh = inp["shared"]
        a.Ws_gate, a.Ws_up, a.Ws_down = _ptr(sh["gate"]), _ptr(sh["up"]), _ptr(sh["down"])
    a.T, a.d, a.E, a.k, a.I = T, d, E, k, I
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    a.out = _ptr(out)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    res = {"out": out}
    if want_routing:
        i32, f32 = torch.int32, torch.float32
        res.update(topk_idx=torch.empty(T, k, dtype=i32, device=dev), topk_w=torch.empty(T, k, dtype=f32, device=dev),
                   counts=torch.empty(E, dtype=i32, device=dev), offsets=torch.empty(E + 1, dtype=i32, device=dev),
                   perm_src=torch.empty(T * k, dtype=i32, device=dev), margin=torch.empty(T, dtype=f32, device=dev))
        a.topk_idx, a.topk_w = _ptr(res["topk_idx"]), _ptr(res["topk_w"])
        a.counts, a.offsets = _ptr(res["counts"]), _ptr(res["offsets"])
        a.perm_src, a.margin = _ptr(res["perm_src"]), _ptr(res["margin"])
    if want_hidden:
        if not fp8_activations:
            raise ValueError("forward_layer: want_hidden needs fp8_activations")
        res.update(hidden_codes=torch.empty(T * k, I, dtype=torch.uint8, device=dev),
                   hidden_scales=torch.empty(T * k, I // 32, dtype=torch.uint8, device=dev))
        a.hidden_codes, a.hidden_scales = _ptr(res["hidden_codes"]), _ptr(res["hidden_scales"])
    a.path = path
    if stage_events is not None:
        a.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    if noalloc:
        if workspace is not None:
            raise ValueError("forward_layer: noalloc takes no workspace")
        rc = forward_noalloc(a, stream)
        if rc != OK:
            raise HyMoeError(rc, "hy_moe_forward_noalloc")
        return res
    rc = forward_ex(a, stream)
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_forward_ex")
    return res


def alloc_workspace(T, d, E, k, I, expert_format=WEIGHTS_BF16, device="cuda"):
    import torch
    n = workspace_size(T, d, E, k, I, expert_format)
    if n == 0:
        raise HyMoeError(ERR_INVALID_ARG, "hy_moe_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def sherry_pack_host(tern):
    """hy_moe_sherry_pack_host on a host int8 numpy array [rows][cols]."""
    import numpy as np
    tern = np.ascontiguousarray(tern, dtype=np.int8)
    rows, cols = tern.shape
    packed = np.zeros((rows, cols // 128 * 5), np.uint32)
    rc = _lib.hy_moe_sherry_pack_host(tern.ctypes.data, rows, cols, packed.ctypes.data)
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_sherry_pack_host")
    return packed


def mxfp8_quantize(x, stream=None):
    """hy_moe_mxfp8_quantize on a device bf16 tensor [rows][cols] (cols % 32 == 0).
    Returns (codes uint8 [rows][cols], scales uint8 [rows][cols / 32])."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() != 2:
        raise TypeError("mxfp8_quantize: x must be a contiguous 2-d bf16 tensor")
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, max(cols // 32, 1), dtype=torch.uint8, device=x.device)
    rc = _lib.hy_moe_mxfp8_quantize(x.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_mxfp8_quantize")
    return codes, scales


def block_bf16(t, stream=None):
    """hy_moe_block_bf16: a new device tensor holding the bf16 matrices of t (contiguous,
    [..., rows, cols], rows % 16 == 0, cols % 64 == 0) in the blocked layout."""
    import torch
    if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() < 2:
        raise TypeError("block_bf16: a contiguous bf16 tensor of at least 2 dimensions")
    rows, cols = t.shape[-2], t.shape[-1]
    count = t.numel() // (rows * cols) if rows * cols else 0
    out = torch.empty_like(t)
    rc = _lib.hy_moe_block_bf16(t.data_ptr(), out.data_ptr(), count, rows, cols, _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_block_bf16")
    return out


def block_sherry(q, stream=None):
    """hy_moe_block_sherry: a new device tensor holding the Sherry code matrices of q
    (contiguous int32, [..., rows, K/128*5], rows % 16 == 0, K % 512 == 0) blocked."""
    import torch
    if q.dtype != torch.int32 or not q.is_contiguous() or q.dim() < 2:
        raise TypeError("block_sherry: a contiguous int32 tensor of at least 2 dimensions")
    rows, words = q.shape[-2], q.shape[-1]
    count = q.numel() // (rows * words) if rows * words else 0
    out = torch.empty_like(q)
    rc = _lib.hy_moe_block_sherry(q.data_ptr(), out.data_ptr(), count, rows, words // 5 * 128, _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_block_sherry")
    return out


def block_layer(inp, stream=None):
    """A copy of a layer dict (hy_inputs.dev_layer) with its weights in the blocked
    layout: a bf16 layer's routed and shared expert matrices, or a Sherry layer's code
    matrices (the other entries are shared, not copied)."""
    out = dict(inp)
    if "qgate" in inp:
        for key in ("qgate", "qup", "qdown"):
            out[key] = block_sherry(inp[key], stream)
        return out
    for key in ("gate", "up", "down"):
        out[key] = block_bf16(inp[key], stream)
    out["shared"] = {key: block_bf16(v, stream) for key, v in inp["shared"].items()}
    return out


def probe_mfma_bf16(operands, stream=None) -> float:
    """hy_moe_probe_mfma_bf16: TFLOP/s of dense bf16 MFMAs on the given operand bits
    (a device tensor of at least PROBE_OPERAND_BYTES bytes)."""
    tf = ctypes.c_float()
    rc = _lib.hy_moe_probe_mfma_bf16(operands.data_ptr(), operands.numel() * operands.element_size(),
                                     ctypes.byref(tf), _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_probe_mfma_bf16")
    return tf.value


def probe_mfma_fp8(operands, stream=None) -> float:
    """hy_moe_probe_mfma_fp8: TFLOP/s of dense E4M3 MFMAs (32x32x64, block scales 1.0)
    on the given codes (a device tensor of at least PROBE_OPERAND_BYTES bytes)."""
    tf = ctypes.c_float()
    rc = _lib.hy_moe_probe_mfma_fp8(operands.data_ptr(), operands.numel() * operands.element_size(),
                                    ctypes.byref(tf), _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_probe_mfma_fp8")
    return tf.value


def probe_hbm_read(buf, stream=None) -> float:
    """hy_moe_probe_hbm_read: GB/s of one streaming read pass over a device tensor."""
    gb = ctypes.c_float()
    rc = _lib.hy_moe_probe_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), ctypes.byref(gb),
                                    _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_moe_probe_hbm_read")
    return gb.value


def indexer_topk(q, w, keys, K, *, scores=None, workspace=None, stream=None, stage_events=None):
    """hy_indexer_topk on device tensors q bf16 [B][H][D], w fp32 [B][H], keys bf16
    [B][S][D]. Returns (idx int32 [B][min(K, S)] ascending, scores fp32 [B][S] or None)."""
    import torch
    for name, t, dt in (("q", q, torch.bfloat16), ("w", w, torch.float32), ("keys", keys, torch.bfloat16)):
        if t.dtype != dt or not t.is_contiguous():
            raise TypeError(f"indexer_topk: {name} must be a contiguous {dt} tensor, got {t.dtype}")
    B, H, D = q.shape
    S = keys.shape[1]
    idx = torch.empty(B, min(K, S), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = torch.empty(int(_lib.hy_indexer_workspace_size(B, S)), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.hy_indexer_topk(q.data_ptr(), w.data_ptr(), keys.data_ptr(), B, H, D, S, K, idx.data_ptr(),
                              _ptr(scores), _ptr(workspace), ws_bytes,
                              None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p),
                              _stream(stream))
    if rc != OK:
        raise HyMoeError(rc, "hy_indexer_topk")
    return idx, scores

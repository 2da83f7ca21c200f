"""Seeded synthetic inputs for the MoE FFN layer, shared by the HIP path's tests,
the oracle's tests and the benchmark.

This module holds no arithmetic of the layer: it only draws inputs. Every
tensor is a Philox4x32-10 stream keyed by (seed, stream id), so any sub-range
can be regenerated on the host (``gen_host.c``) or filled on the device
(``gen_dev.hip``) with bit-identical values; the oracle regenerates one
expert's weights at a time on the host while the GPU path reads the same
weights generated in HBM.

Workloads (the layer shape of the Hy4 preview model: 256 routed experts with
top-8 plus one always-on shared expert and hidden size 6144, as stated on the
Tencent Hy4 preview model card and in the app.myzaker.com Hy4 Preview news,
section "770B 不是简单堆参数"). Value recipes:
  x ~ N(0, 1); router, gate, up ~ N(0, 1/sqrt(d)); down ~ N(0, 1/sqrt(I))
  (the second argument is a standard deviation). Ternary experts: uniform random
  5-bit codes (every 160-bit block of packed words is valid) and per-row scales
  ~ U(0.5, 1.5)/sqrt(fan_in). Skewed routing: a per-expert bias
  b_e = -alpha * s * ln(rank_e) with rank a seeded permutation of 1..E (s=1.2).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# One Philox stream per tensor.
S_X, S_WR, S_WG, S_WU, S_WD, S_WSG, S_WSU, S_WSD, S_BIAS = 1, 2, 3, 4, 5, 6, 7, 8, 9
S_QG, S_QU, S_QD, S_SG, S_SU, S_SD = 10, 11, 12, 13, 14, 15
S_FG, S_FU, S_FD, S_FSG, S_FSU, S_FSD = 16, 17, 18, 19, 20, 21
S_IQ, S_IK, S_IW = 22, 23, 24  # sparse-attention indexer: queries, keys, head weights

QBLOCK_WEIGHTS = 128  # weights per packed ternary block
QBLOCK_WORDS = 5      # uint32 words per packed ternary block (1.25 bits/weight)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    ternary: bool = False
    fp8: bool = False        # routed experts as E4M3 codes with fp32 row scales
    a8: bool = False         # with fp8: the routed experts' activations in MXFP8 (W8A8)
    tshared: bool = False    # with ternary: the shared expert Sherry-packed too, as expert E of the code arrays
    zipf_s: float = 0.0      # 0 => no router bias
    zipf_alpha: float = 1.0
    x_std: float = 1.0
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.T * self.k


CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, d=256, E=16, k=2, I=128),
    "decode": LayerConfig("decode", T=32, d=6144, E=256, k=8, I=2048),
    "prefill": LayerConfig("prefill", T=8192, d=6144, E=256, k=8, I=2048),
    "skewed": LayerConfig("skewed", T=4096, d=6144, E=256, k=8, I=2048, zipf_s=1.2),
    "ternary": LayerConfig("ternary", T=32, d=6144, E=256, k=8, I=2048, ternary=True),
    # routed experts as FP8 (E4M3 codes, fp32 row scales), decode batch
    "fp8": LayerConfig("fp8", T=32, d=6144, E=256, k=8, I=2048, fp8=True),
    "fp8_prefill": LayerConfig("fp8_prefill", T=8192, d=6144, E=256, k=8, I=2048, fp8=True),
    # FP8 weights with MXFP8 activations (W8A8) on the FP8 matrix cores
    "fp8_w8a8_prefill": LayerConfig("fp8_w8a8_prefill", T=8192, d=6144, E=256, k=8, I=2048, fp8=True, a8=True),
    "fp8_w8a8": LayerConfig("fp8_w8a8", T=32, d=6144, E=256, k=8, I=2048, fp8=True, a8=True),
    # the ternary experts at a prefill-sized batch (grouped GEMM on decoded codes)
    "ternary_prefill": LayerConfig("ternary_prefill", T=8192, d=6144, E=256, k=8, I=2048, ternary=True),
}


def _load_host():
    # HY_GEN_LIB: another build of gen_host.c (the sanitizer test loads an
    # AddressSanitizer/UBSan build through it)
    path = os.environ.get("HY_GEN_LIB") or os.path.join(_HERE, "libhy_gen.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    u64, u32, dbl, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
    lib.hy_gen_gauss_bf16.argtypes = [u64, u32, u64, u64, dbl, vp, ctypes.c_int]
    lib.hy_gen_uniform_bf16.argtypes = [u64, u32, u64, u64, dbl, dbl, vp, ctypes.c_int]
    lib.hy_gen_u32.argtypes = [u64, u32, u64, u64, vp, ctypes.c_int]
    lib.hy_gen_ln.restype = dbl
    lib.hy_gen_ln.argtypes = [dbl]
    lib.hy_gen_sqrt.restype = dbl
    lib.hy_gen_sqrt.argtypes = [dbl]
    lib.hy_gen_cossin_turn.argtypes = [dbl, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    lib.hy_gen_philox4x32_10.argtypes = [ctypes.POINTER(u32), ctypes.POINTER(u32), ctypes.POINTER(u32)]
    return lib


def _load_dev():
    import torch  # noqa: F401  (bind to torch's HIP runtime, loaded first)
    path = os.path.join(_HERE, "libhy_gen_dev.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    u64, u32, dbl, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
    lib.hy_gen_gauss_bf16_dev.argtypes = [u64, u32, u64, u64, dbl, vp, vp]
    lib.hy_gen_uniform_bf16_dev.argtypes = [u64, u32, u64, u64, dbl, dbl, vp, vp]
    lib.hy_gen_u32_dev.argtypes = [u64, u32, u64, u64, vp, vp]
    return lib


_host = None
_dev = None


def host_lib():
    global _host
    if _host is None:
        _host = _load_host()
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        _dev = _load_dev()
    return _dev


def _threads() -> int:
    return max(1, min(32, os.cpu_count() or 1))


# ---------------------------------------------------------------- host arrays
def gauss_bf16(seed: int, stream: int, count: int, std: float, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.uint16)
    if count:
        rc = host_lib().hy_gen_gauss_bf16(seed, stream, start, count, std, out.ctypes.data, _threads())
        if rc != 0:
            raise RuntimeError("hy_gen_gauss_bf16 failed")
    return out


def uniform_bf16(seed: int, stream: int, count: int, lo: float, width: float, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.uint16)
    if count:
        rc = host_lib().hy_gen_uniform_bf16(seed, stream, start, count, lo, width, out.ctypes.data, _threads())
        if rc != 0:
            raise RuntimeError("hy_gen_uniform_bf16 failed")
    return out


def words_u32(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.uint32)
    if count:
        rc = host_lib().hy_gen_u32(seed, stream, start, count, out.ctypes.data, _threads())
        if rc != 0:
            raise RuntimeError("hy_gen_u32 failed")
    return out


def zipf_bias(E: int, seed: int, s: float = 1.2, alpha: float = 1.0) -> np.ndarray:
    """b_e = -alpha*s*ln(rank_e); rank is a Fisher-Yates shuffle of 1..E driven by
    Philox words of the bias stream. Returned as fp32 (the boundary's bias type)."""
    w = words_u32(seed, S_BIAS, E)
    rank = np.arange(1, E + 1, dtype=np.int64)
    for i in range(E - 1, 0, -1):
        j = int(w[i]) % (i + 1)
        rank[i], rank[j] = rank[j], rank[i]
    return (-alpha * s * np.log(rank.astype(np.float64))).astype(np.float32)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ layer recipes
def weight_std(cfg: LayerConfig) -> dict:
    return {"x": cfg.x_std, "router": 1.0 / math.sqrt(cfg.d), "gate": 1.0 / math.sqrt(cfg.d),
            "up": 1.0 / math.sqrt(cfg.d), "down": 1.0 / math.sqrt(cfg.I)}


def host_x(cfg: LayerConfig, t0: int = 0, nt: int | None = None) -> np.ndarray:
    nt = cfg.T - t0 if nt is None else nt
    return gauss_bf16(cfg.seed, S_X, nt * cfg.d, cfg.x_std, start=t0 * cfg.d).reshape(nt, cfg.d)


def host_router(cfg: LayerConfig) -> np.ndarray:
    return gauss_bf16(cfg.seed, S_WR, cfg.E * cfg.d, 1.0 / math.sqrt(cfg.d)).reshape(cfg.E, cfg.d)


def host_bias(cfg: LayerConfig):
    if cfg.zipf_s == 0.0:
        return None
    return zipf_bias(cfg.E, cfg.seed, cfg.zipf_s, cfg.zipf_alpha)


def host_expert(cfg: LayerConfig, e: int) -> dict:
    """bf16 weights of routed expert e: gate, up [I][d]; down [d][I]."""
    d, I = cfg.d, cfg.I
    n = I * d
    sd, si = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    return {"gate": gauss_bf16(cfg.seed, S_WG, n, sd, start=e * n).reshape(I, d),
            "up": gauss_bf16(cfg.seed, S_WU, n, sd, start=e * n).reshape(I, d),
            "down": gauss_bf16(cfg.seed, S_WD, n, si, start=e * n).reshape(d, I)}


def host_shared(cfg: LayerConfig) -> dict:
    d, I = cfg.d, cfg.I
    n = I * d
    sd, si = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    return {"gate": gauss_bf16(cfg.seed, S_WSG, n, sd).reshape(I, d),
            "up": gauss_bf16(cfg.seed, S_WSU, n, sd).reshape(I, d),
            "down": gauss_bf16(cfg.seed, S_WSD, n, si).reshape(d, I)}


def qwords_per_row(cols: int) -> int:
    return cols // QBLOCK_WEIGHTS * QBLOCK_WORDS


def host_expert_ternary(cfg: LayerConfig, e: int) -> dict:
    """Packed ternary codes and bf16 per-row scales of routed expert e."""
    d, I = cfg.d, cfg.I
    wg, wd = qwords_per_row(d), qwords_per_row(I)
    sd, si = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    return {"qgate": words_u32(cfg.seed, S_QG, I * wg, start=e * I * wg).reshape(I, wg),
            "qup": words_u32(cfg.seed, S_QU, I * wg, start=e * I * wg).reshape(I, wg),
            "qdown": words_u32(cfg.seed, S_QD, d * wd, start=e * d * wd).reshape(d, wd),
            "sgate": uniform_bf16(cfg.seed, S_SG, I, 0.5 * sd, sd, start=e * I),
            "sup": uniform_bf16(cfg.seed, S_SU, I, 0.5 * sd, sd, start=e * I),
            "sdown": uniform_bf16(cfg.seed, S_SD, d, 0.5 * si, si, start=e * d)}


def fp8_codes_from_bytes(b):
    """Random bytes -> E4M3 codes: sign and mantissa bits kept, the exponent field
    forced into 4..7 (|value| in [1/8, 15/8], never NaN). numpy or torch uint8."""
    return (b & 0x87) | ((((b >> 3) & 3) + 4) << 3)


def fp8_scale_exponent(cols: int) -> int:
    """Row scales are m * 2^-(15 + p) with m in [0x6000, 0xE000) (mean 1.25 * 2^-p); the
    codes' mean |value| is 0.674, so p = round(log2(sqrt(cols) / 0.947)) makes the mean
    |weight| that of the bf16 weights (std 1/sqrt(cols)) within a factor of sqrt(2)."""
    return int(round(0.5 * math.log2(cols) + 0.078))


def fp8_scales_from_words(w, cols: int):
    """Random words -> fp32 row scales, exact on host and device: (w & 0x7FFF) + 0x6000
    (an integer below 2^16) times a power of two."""
    return ((w & 0x7FFF) + 0x6000) * (2.0 ** -(15 + fp8_scale_exponent(cols)))


def host_expert_fp8(cfg: LayerConfig, e: int) -> dict:
    """E4M3 codes (uint8 [rows][cols]) and fp32 row scales of routed expert e."""
    d, I = cfg.d, cfg.I
    def codes(stream, rows, cols):
        n = rows * cols // 4
        return fp8_codes_from_bytes(words_u32(cfg.seed, stream, n, start=e * n).view(np.uint8)).reshape(rows, cols)
    def scales(stream, rows, cols):
        return fp8_scales_from_words(words_u32(cfg.seed, stream, rows, start=e * rows), cols).astype(np.float32)
    return {"fgate": codes(S_FG, I, d), "fup": codes(S_FU, I, d), "fdown": codes(S_FD, d, I),
            "fsgate": scales(S_FSG, I, d), "fsup": scales(S_FSU, I, d), "fsdown": scales(S_FSD, d, I)}


def host_layer(cfg: LayerConfig) -> dict:
    """Every input of a (small) layer as host arrays: bf16 as uint16 bit patterns."""
    out = {"x": host_x(cfg), "router": host_router(cfg), "bias": host_bias(cfg),
           "shared": host_shared(cfg)}
    gen = host_expert_ternary if cfg.ternary else host_expert_fp8 if cfg.fp8 else host_expert
    # (a Sherry-packed shared expert continues the routed experts' streams as expert E)
    experts = [gen(cfg, e) for e in range(cfg.E + (1 if cfg.ternary and cfg.tshared else 0))]
    keys = experts[0].keys()
    for key in keys:
        out[key] = np.stack([ex[key] for ex in experts])
    return out


# ----------------------------------------------------------- device tensors
def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dev_gauss_(t, seed: int, stream_id: int, std: float, start: int = 0, stream=None):
    rc = dev_lib().hy_gen_gauss_bf16_dev(seed, stream_id, start, t.numel(), std, t.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError("hy_gen_gauss_bf16_dev failed")
    return t


def dev_uniform_(t, seed: int, stream_id: int, lo: float, width: float, start: int = 0, stream=None):
    rc = dev_lib().hy_gen_uniform_bf16_dev(seed, stream_id, start, t.numel(), lo, width, t.data_ptr(),
                                           _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError("hy_gen_uniform_bf16_dev failed")
    return t


def dev_words_(t, seed: int, stream_id: int, start: int = 0, stream=None):
    rc = dev_lib().hy_gen_u32_dev(seed, stream_id, start, t.numel(), t.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError("hy_gen_u32_dev failed")
    return t


def dev_layer(cfg: LayerConfig, device="cuda") -> dict:
    """Every input of a layer generated directly in device memory (bf16 tensors,
    int32 tensors holding packed ternary words). Values equal host_layer()'s."""
    import torch
    d, I, E, T = cfg.d, cfg.I, cfg.E, cfg.T
    sd, si = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    bf = torch.bfloat16
    out = {"x": dev_gauss_(torch.empty(T, d, dtype=bf, device=device), cfg.seed, S_X, cfg.x_std),
           "router": dev_gauss_(torch.empty(E, d, dtype=bf, device=device), cfg.seed, S_WR, sd)}
    b = host_bias(cfg)
    out["bias"] = None if b is None else torch.from_numpy(b).to(device)
    out["shared"] = {
        "gate": dev_gauss_(torch.empty(I, d, dtype=bf, device=device), cfg.seed, S_WSG, sd),
        "up": dev_gauss_(torch.empty(I, d, dtype=bf, device=device), cfg.seed, S_WSU, sd),
        "down": dev_gauss_(torch.empty(d, I, dtype=bf, device=device), cfg.seed, S_WSD, si)}
    if cfg.ternary:
        wg, wd = qwords_per_row(d), qwords_per_row(I)
        i32 = torch.int32
        EQ = E + 1 if cfg.tshared else E  # a Sherry-packed shared expert is expert E
        out["qgate"] = dev_words_(torch.empty(EQ, I, wg, dtype=i32, device=device), cfg.seed, S_QG)
        out["qup"] = dev_words_(torch.empty(EQ, I, wg, dtype=i32, device=device), cfg.seed, S_QU)
        out["qdown"] = dev_words_(torch.empty(EQ, d, wd, dtype=i32, device=device), cfg.seed, S_QD)
        out["sgate"] = dev_uniform_(torch.empty(EQ, I, dtype=bf, device=device), cfg.seed, S_SG, 0.5 * sd, sd)
        out["sup"] = dev_uniform_(torch.empty(EQ, I, dtype=bf, device=device), cfg.seed, S_SU, 0.5 * sd, sd)
        out["sdown"] = dev_uniform_(torch.empty(EQ, d, dtype=bf, device=device), cfg.seed, S_SD, 0.5 * si, si)
        out["shared_sherry"] = cfg.tshared
    elif cfg.fp8:
        i32 = torch.int32

        def codes(stream, rows, cols):
            w = dev_words_(torch.empty(E, rows, cols // 4, dtype=i32, device=device), cfg.seed, stream)
            b = w.view(torch.uint8).view(E, rows, cols)
            return fp8_codes_from_bytes(b)

        def scales(stream, rows, cols):
            w = dev_words_(torch.empty(E, rows, dtype=i32, device=device), cfg.seed, stream)
            return fp8_scales_from_words(w, cols).to(torch.float32)

        out["fgate"], out["fup"], out["fdown"] = codes(S_FG, I, d), codes(S_FU, I, d), codes(S_FD, d, I)
        out["fsgate"], out["fsup"], out["fsdown"] = scales(S_FSG, I, d), scales(S_FSU, I, d), scales(S_FSD, d, I)
    else:
        out["gate"] = dev_gauss_(torch.empty(E, I, d, dtype=bf, device=device), cfg.seed, S_WG, sd)
        out["up"] = dev_gauss_(torch.empty(E, I, d, dtype=bf, device=device), cfg.seed, S_WU, sd)
        out["down"] = dev_gauss_(torch.empty(E, d, I, dtype=bf, device=device), cfg.seed, S_WD, si)
    return out


# ------------------------------------------------------ sparse-attention indexer
@dataclass(frozen=True)
class IndexerConfig:
    """B queries (one per sequence), each scored against its own S keys by an H-head
    indexer of key dimension D; the K best keys are selected."""
    name: str
    B: int
    S: int
    H: int = 32
    D: int = 128
    K: int = 2048
    seed: int = 0


INDEXER_CONFIGS = {
    "indexer_tiny": IndexerConfig("indexer_tiny", B=4, S=3000, K=256),
    # 32 decoding sequences with 64K-token contexts (indexer of the Hy4 preview config:
    # 32 heads, head_dim 128, top-2048)
    "indexer_decode": IndexerConfig("indexer_decode", B=32, S=65536),
}


def host_indexer_queries(cfg: IndexerConfig):
    """(q bf16 bits [B][H][D], w fp32 [B][H]): q ~ N(0, 1/sqrt(D)), w ~ U(0.5, 1.5) / H."""
    q = gauss_bf16(cfg.seed, S_IQ, cfg.B * cfg.H * cfg.D, 1.0 / math.sqrt(cfg.D)).reshape(cfg.B, cfg.H, cfg.D)
    w = bf16_to_f32(uniform_bf16(cfg.seed, S_IW, cfg.B * cfg.H, 0.5 / cfg.H, 1.0 / cfg.H)).reshape(cfg.B, cfg.H)
    return q, w.astype(np.float32)


def host_indexer_keys(cfg: IndexerConfig, b: int) -> np.ndarray:
    """Keys of sequence b: bf16 bits [S][D], ~ N(0, 1)."""
    n = cfg.S * cfg.D
    return gauss_bf16(cfg.seed, S_IK, n, 1.0, start=b * n).reshape(cfg.S, cfg.D)


def dev_indexer(cfg: IndexerConfig, device="cuda") -> dict:
    """q bf16 [B][H][D], w fp32 [B][H], keys bf16 [B][S][D] in device memory (values
    equal the host generators')."""
    import torch
    bf = torch.bfloat16
    q = dev_gauss_(torch.empty(cfg.B, cfg.H, cfg.D, dtype=bf, device=device), cfg.seed, S_IQ, 1.0 / math.sqrt(cfg.D))
    w = dev_uniform_(torch.empty(cfg.B, cfg.H, dtype=bf, device=device), cfg.seed, S_IW, 0.5 / cfg.H, 1.0 / cfg.H)
    keys = dev_gauss_(torch.empty(cfg.B, cfg.S, cfg.D, dtype=bf, device=device), cfg.seed, S_IK, 1.0)
    return {"q": q, "w": w.float(), "keys": keys}

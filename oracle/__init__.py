"""fp64 CPU oracle of the sparse-MoE FFN layer (ctypes over ``libhy_oracle.so``).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path
(``sparse_moe_transformer_route_amd``) never loads it.

Every function wraps one step of ``hy_oracle.c``; the C file states, per step,
the passage of the pages it follows and the reading taken where they are
silent. Parity unpinned: none — each step is pinned in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        # HY_ORACLE_LIB: another build of hy_oracle.c (the sanitizer test loads an
        # AddressSanitizer/UBSan build through it)
        path = os.environ.get("HY_ORACLE_LIB") or os.path.join(_HERE, "libhy_oracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.hyo_logits.argtypes = [vp, vp, vp, i64, i64, i64, vp, ci]
        L.hyo_select.argtypes = [vp, i64, i64, i64, vp, vp]
        L.hyo_weights.argtypes = [vp, vp, i64, i64, i64, vp]
        L.hyo_permute.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
        L.hyo_ffn.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, ci]
        L.hyo_combine.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.hyo_sherry_decode.argtypes = [vp, vp, i64, i64, vp, vp]
        L.hyo_forward.argtypes = [vp] * 9 + [i64] * 5 + [vp] * 6 + [ci]
        L.hyo_fp8_decode.argtypes = [vp, vp, i64, i64, vp]
        L.hyo_ffn_w64.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, ci]
        L.hyo_forward_w64.argtypes = [vp] * 9 + [i64] * 5 + [vp] * 6 + [ci]
        L.hyo_mx_quantize.argtypes = [vp, i64, i64, vp, vp]
        L.hyo_ffn_w8a8.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, ci]
        L.hyo_ffn_w8a8_ex.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, vp, vp, vp, ci]
        L.hyo_forward_w8a8.argtypes = [vp] * 9 + [i64] * 5 + [vp] * 6 + [ci]
        L.hyo_indexer_scores.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.hyo_topk_indices.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        _lib = L
    return _lib


def _threads(n=None):
    return n if n is not None else max(1, min(32, os.cpu_count() or 1))


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


def logits(x, wr, bias=None, nthreads=None):
    x, wr, bias = _c(x, np.uint16), _c(wr, np.uint16), _c(bias, np.float32)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float64)
    _check(lib().hyo_logits(_p(x), _p(wr), _p(bias), T, d, E, _p(out), _threads(nthreads)), "hyo_logits")
    return out


def select(lg, k):
    lg = _c(lg, np.float64)
    T, E = lg.shape
    sets = np.empty((T, k), np.int32)
    margin = np.empty(T, np.float64)
    _check(lib().hyo_select(_p(lg), T, E, k, _p(sets), _p(margin)), "hyo_select")
    return sets, margin


def weights(lg, sets):
    lg, sets = _c(lg, np.float64), _c(sets, np.int32)
    T, E = lg.shape
    k = sets.shape[1]
    w = np.empty((T, k), np.float64)
    _check(lib().hyo_weights(_p(lg), _p(sets), T, E, k, _p(w)), "hyo_weights")
    return w


def permute(sets, E):
    sets = _c(sets, np.int32)
    T, k = sets.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_src = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    _check(lib().hyo_permute(_p(sets), T, E, k, _p(counts), _p(offsets), _p(perm_src), _p(pos)), "hyo_permute")
    return counts, offsets, perm_src, pos


def ffn(x_rows, wg, wu, wd, nthreads=None):
    x_rows = _c(np.atleast_2d(x_rows), np.uint16)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    n, d = x_rows.shape
    I = wg.shape[0]
    y = np.empty((n, d), np.float64)
    _check(lib().hyo_ffn(_p(x_rows), n, _p(wg), _p(wu), _p(wd), d, I, _p(y), _threads(nthreads)), "hyo_ffn")
    return y


def combine(ys, yr, w):
    ys, yr, w = _c(ys, np.float64), _c(yr, np.float64), _c(w, np.float64)
    T, d = ys.shape
    k = w.shape[1]
    out = np.empty((T, d), np.float64)
    _check(lib().hyo_combine(_p(ys), _p(yr), _p(w), T, k, d, _p(out)), "hyo_combine")
    return out


def sherry_decode(packed, scale=None, cols=None):
    """Returns (tern int8 [rows][cols], weights bf16-bits [rows][cols] or None)."""
    packed = _c(packed, np.uint32)
    rows, words = packed.shape
    cols = words // 5 * 128 if cols is None else cols
    tern = np.empty((rows, cols), np.int8)
    w = None
    if scale is not None:
        scale = _c(scale, np.uint16)
        w = np.empty((rows, cols), np.uint16)
    _check(lib().hyo_sherry_decode(_p(packed), _p(scale), rows, cols, _p(tern), _p(w)), "hyo_sherry_decode")
    return tern, w


def forward(x, wr, bias, wg, wu, wd, sg, su, sd, k, sets_in=None, nthreads=None):
    """Whole layer (bf16 routed experts). Returns dict(out, sets, w, margin, logits)."""
    x, wr, bias = _c(x, np.uint16), _c(wr, np.uint16), _c(bias, np.float32)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    sg, su, sd = _c(sg, np.uint16), _c(su, np.uint16), _c(sd, np.uint16)
    sets_in = _c(sets_in, np.int32)
    T, d = x.shape
    E = wr.shape[0]
    I = sg.shape[0]
    out = np.empty((T, d), np.float64)
    sets = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    margin = np.empty(T, np.float64)
    lg = np.empty((T, E), np.float64)
    _check(lib().hyo_forward(_p(x), _p(wr), _p(bias), _p(wg), _p(wu), _p(wd), _p(sg), _p(su), _p(sd),
                             T, d, E, k, I, _p(sets_in), _p(out), _p(sets), _p(w), _p(margin), _p(lg),
                             _threads(nthreads)), "hyo_forward")
    return {"out": out, "sets": sets, "w": w, "margin": margin, "logits": lg}


def fp8_decode(q, scale=None):
    """E4M3 codes uint8 [rows][cols] (and fp32 row scales) -> fp64 weights [rows][cols]."""
    q = _c(np.atleast_2d(q), np.uint8)
    rows, cols = q.shape
    scale = None if scale is None else _c(scale, np.float32)
    w = np.empty((rows, cols), np.float64)
    _check(lib().hyo_fp8_decode(_p(q), _p(scale), rows, cols, _p(w)), "hyo_fp8_decode")
    return w


def ffn_w64(x_rows, wg, wu, wd, nthreads=None):
    """Expert FFN with fp64 weights wg, wu [I][d], wd [d][I] on bf16 token rows."""
    x_rows = _c(np.atleast_2d(x_rows), np.uint16)
    wg, wu, wd = _c(wg, np.float64), _c(wu, np.float64), _c(wd, np.float64)
    n, d = x_rows.shape
    I = wg.shape[0]
    y = np.empty((n, d), np.float64)
    _check(lib().hyo_ffn_w64(_p(x_rows), n, _p(wg), _p(wu), _p(wd), d, I, _p(y), _threads(nthreads)),
           "hyo_ffn_w64")
    return y


def forward_w64(x, wr, bias, fg, fu, fd, sg, su, sd, k, sets_in=None, nthreads=None):
    """Whole layer with fp64 routed weights (fg, fu [E][I][d], fd [E][d][I]) and a bf16
    shared expert. Returns dict(out, sets, w, margin, logits)."""
    x, wr, bias = _c(x, np.uint16), _c(wr, np.uint16), _c(bias, np.float32)
    fg, fu, fd = _c(fg, np.float64), _c(fu, np.float64), _c(fd, np.float64)
    sg, su, sd = _c(sg, np.uint16), _c(su, np.uint16), _c(sd, np.uint16)
    sets_in = _c(sets_in, np.int32)
    T, d = x.shape
    E = wr.shape[0]
    I = sg.shape[0]
    out = np.empty((T, d), np.float64)
    sets = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    margin = np.empty(T, np.float64)
    lg = np.empty((T, E), np.float64)
    _check(lib().hyo_forward_w64(_p(x), _p(wr), _p(bias), _p(fg), _p(fu), _p(fd), _p(sg), _p(su), _p(sd),
                                 T, d, E, k, I, _p(sets_in), _p(out), _p(sets), _p(w), _p(margin), _p(lg),
                                 _threads(nthreads)), "hyo_forward_w64")
    return {"out": out, "sets": sets, "w": w, "margin": margin, "logits": lg}


def mx_quantize(v):
    """MXFP8 quantization (E4M3 codes, one E8M0 scale per 32 consecutive values along a
    row) of fp32 rows v [rows][cols]. Returns (codes uint8 [rows][cols], scales uint8
    [rows][cols / 32]); value = e4m3(code) * 2^(scale - 127)."""
    v = _c(np.atleast_2d(v), np.float32)
    rows, cols = v.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, max(cols // 32, 1)), np.uint8)
    _check(lib().hyo_mx_quantize(_p(v), rows, cols, _p(codes), _p(scales)), "hyo_mx_quantize")
    return codes, scales


def ffn_w8a8(x_rows, wg, wu, wd, nthreads=None):
    """Expert FFN with fp64 weights and MXFP8 activations (x and the hidden rows
    quantized) on bf16 token rows."""
    x_rows = _c(np.atleast_2d(x_rows), np.uint16)
    wg, wu, wd = _c(wg, np.float64), _c(wu, np.float64), _c(wd, np.float64)
    n, d = x_rows.shape
    I = wg.shape[0]
    y = np.empty((n, d), np.float64)
    _check(lib().hyo_ffn_w8a8(_p(x_rows), n, _p(wg), _p(wu), _p(wd), d, I, _p(y), _threads(nthreads)),
           "hyo_ffn_w8a8")
    return y


def ffn_w8a8_ex(x_rows, wg, wu, wd, hq=None, hs=None, want_hidden=False, nthreads=None):
    """ffn_w8a8 with the hidden rows' fp32 values returned (want_hidden) and, where hq, hs
    are given (E4M3 codes [n][I], E8M0 scales [n][I / 32]), those codes used as the hidden
    rows instead of the oracle's own quantization. Returns y or (y, h32)."""
    x_rows = _c(np.atleast_2d(x_rows), np.uint16)
    wg, wu, wd = _c(wg, np.float64), _c(wu, np.float64), _c(wd, np.float64)
    n, d = x_rows.shape
    I = wg.shape[0]
    hq, hs = _c(hq, np.uint8), _c(hs, np.uint8)
    y = np.empty((n, d), np.float64)
    h32 = np.empty((n, I), np.float32) if want_hidden else None
    _check(lib().hyo_ffn_w8a8_ex(_p(x_rows), n, _p(wg), _p(wu), _p(wd), d, I, _p(hq), _p(hs), _p(h32), _p(y),
                                 _threads(nthreads)), "hyo_ffn_w8a8_ex")
    return (y, h32) if want_hidden else y


def forward_w8a8(x, wr, bias, fg, fu, fd, sg, su, sd, k, sets_in=None, nthreads=None):
    """Whole layer with fp64 (decoded FP8) routed weights and MXFP8 activations in the
    routed experts; bf16 router and shared expert. Returns dict(out, sets, w, margin,
    logits)."""
    x, wr, bias = _c(x, np.uint16), _c(wr, np.uint16), _c(bias, np.float32)
    fg, fu, fd = _c(fg, np.float64), _c(fu, np.float64), _c(fd, np.float64)
    sg, su, sd = _c(sg, np.uint16), _c(su, np.uint16), _c(sd, np.uint16)
    sets_in = _c(sets_in, np.int32)
    T, d = x.shape
    E = wr.shape[0]
    I = sg.shape[0]
    out = np.empty((T, d), np.float64)
    sets = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    margin = np.empty(T, np.float64)
    lg = np.empty((T, E), np.float64)
    _check(lib().hyo_forward_w8a8(_p(x), _p(wr), _p(bias), _p(fg), _p(fu), _p(fd), _p(sg), _p(su), _p(sd),
                                  T, d, E, k, I, _p(sets_in), _p(out), _p(sets), _p(w), _p(margin), _p(lg),
                                  _threads(nthreads)), "hyo_forward_w8a8")
    return {"out": out, "sets": sets, "w": w, "margin": margin, "logits": lg}


def indexer_scores(q, w, keys):
    """Sparse-attention indexer scores: q bf16 [B][H][D], w fp32 [B][H], keys bf16
    [B][S][D] -> fp64 [B][S], score = sum_h w[h] * max(0, q[h] . k)."""
    q, w, keys = _c(q, np.uint16), _c(w, np.float32), _c(keys, np.uint16)
    B, H, D = q.shape
    S = keys.shape[1]
    out = np.empty((B, S), np.float64)
    _check(lib().hyo_indexer_scores(_p(q), _p(w), _p(keys), B, H, D, S, _p(out)), "hyo_indexer_scores")
    return out


def topk_indices(scores, K):
    """Per row: the K highest scores (ties to the lower index) as ascending indices,
    plus the K-th score and its margin over the (K+1)-th (+inf when S <= K)."""
    scores = _c(np.atleast_2d(scores), np.float64)
    B, S = scores.shape
    n = min(K, S)
    idx = np.empty((B, n), np.int32)
    kth = np.empty(B, np.float64)
    margin = np.empty(B, np.float64)
    _check(lib().hyo_topk_indices(_p(scores), B, S, K, _p(idx), _p(kth), _p(margin)), "hyo_topk_indices")
    return idx, kth, margin

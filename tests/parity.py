"""Comparison rules between the HIP path and the fp64 oracle (used by the GPU tests).

Routing: expert sets, counts, offsets and the permutation must be bit-exact for
every token whose oracle k-th/(k+1)-th logit margin exceeds NEAR_TIE. A token at
or below it may carry a different set only if that set is admissible (its
smallest logit is within NEAR_TIE of the largest logit left out, in the oracle's
fp64 logits); the oracle then recomputes weights, permutation and outputs with
the GPU's set substituted, and everything is compared for all tokens.
Weights: |w_gpu - w_ref| <= W_TOL. Outputs: |out - ref| <= OUT_TOL * (1 + |ref|).
"""
import numpy as np

import oracle

NEAR_TIE = 1e-4
W_TOL = 1e-5
OUT_TOL = 2e-2
TILE_ROWS = 256   # the grouped GEMM's largest M tile
BLOCK_ROWS = 32   # its row-block granularity


def f32_to_bf16_bits(a):
    """Round fp32 -> bf16 (nearest even) as uint16 bit patterns (input preparation)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_tensor_to_np(t):
    """bf16 torch tensor -> float64 numpy (exact)."""
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_tensor_bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_routing(sets_gpu, lg, k):
    """Returns (sets to use in the oracle, number of near-tie tokens, number substituted)."""
    sets_ref, margin = oracle.select(lg, k)
    T, E = lg.shape
    near = margin <= NEAR_TIE
    diff = ~(sets_gpu == sets_ref).all(axis=1)
    bad = diff & ~near
    assert not bad.any(), f"routing differs on {int(bad.sum())} tokens with margin > {NEAR_TIE}: " \
                          f"first {np.nonzero(bad)[0][:5]}"
    use = sets_ref.copy()
    for t in np.nonzero(diff)[0]:
        s = sets_gpu[t]
        assert len(set(s.tolist())) == k and (s >= 0).all() and (s < E).all()
        assert (np.diff(s) > 0).all(), "GPU set not in ascending expert order"
        out = np.setdiff1d(np.arange(E), s)
        worst_in = lg[t, s].min()
        best_out = lg[t, out].max() if out.size else -np.inf
        assert worst_in >= best_out - NEAR_TIE, f"inadmissible set for near-tie token {t}"
        use[t] = s
    return use, int(near.sum()), int(diff.sum())


def check_permutation(gpu, sets, E):
    counts, offsets, perm_src, _ = oracle.permute(sets, E)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], offsets)
    assert np.array_equal(gpu["perm_src"], perm_src)


def check_weights(w_gpu, lg, sets):
    w_ref = oracle.weights(lg, sets)
    err = np.abs(w_gpu.astype(np.float64) - w_ref).max() if w_ref.size else 0.0
    assert err <= W_TOL, f"routing weight error {err:.3e} > {W_TOL}"
    return err


def check_out(out_gpu, ref, extra=None):
    """|out - ref| <= OUT_TOL (1 + |ref|) (+ extra, a per-element allowance, where given)."""
    err = np.abs(out_gpu - ref)
    tol = OUT_TOL * (1.0 + np.abs(ref)) + (0.0 if extra is None else extra)
    rel = err / tol * OUT_TOL
    worst = float(rel.max()) if rel.size else 0.0
    assert np.isfinite(out_gpu).all()
    assert worst <= OUT_TOL, f"max |gpu-ref|/(1+|ref|) = {worst:.3e} > {OUT_TOL}"
    return worst, float(err.mean()) if rel.size else 0.0


# MXFP8 hidden rows (W8A8). The two sides quantize fp32 hidden values that differ by
# their sums' rounding, so a value lying that close to an E4M3 rounding boundary (or a
# block maximum that close to a power of two) may take the neighbouring code (scale) on
# the GPU: the quantization counterpart of a routing near tie. The GPU's hidden rows are
# read back (hy_moe_args.hidden_codes/hidden_scales) and checked to be admissible: every
# block scale is that of the block's largest oracle value moved by at most HID_REL, and
# every value lies within half an E4M3 step (at its size) plus HID_REL |h| + HID_ABS amax
# of the oracle's fp32 value. The oracle then recomputes the down projection from the
# GPU's admissible codes, and outputs are compared under the usual tolerance.
HID_REL = 2.0 ** -8
HID_ABS = 2.0 ** -10
HID_MAX_FLIP_FRACTION = 0.01


def _block_exp(amax):
    _, ex = np.frexp(amax)
    return np.where(amax > 0, np.clip(ex - 9, -127, 127), -127)


def check_hidden_rows(h32, gq, gs):
    """h32 fp32 [n][I] (oracle), gq uint8 [n][I], gs uint8 [n][I / 32] (GPU). Asserts
    admissibility; returns (codes differing from the oracle's own, blocks whose scale differs)."""
    n, I = h32.shape
    h = h32.astype(np.float64).reshape(n, I // 32, 32)
    amax = np.abs(h).max(axis=2)
    ge = gs.astype(np.int64) - 127
    lo, hi = _block_exp(amax * (1 - HID_REL)), _block_exp(amax * (1 + HID_REL))
    bad = ~((ge == lo) | (ge == hi))
    if bad.any():
        rows = np.argwhere(bad)
        info = "; ".join(f"row {r} block {b}: gpu e={ge[r, b]} oracle amax {amax[r, b]:.6g} -> e in [{lo[r, b]}, "
                         f"{hi[r, b]}]" for r, b in rows[:6])
        raise AssertionError(f"{len(rows)} hidden block scales inadmissible (rows {sorted(set(rows[:, 0].tolist()))[:20]}, "
                             f"blocks {sorted(set(rows[:, 1].tolist()))}): {info}")
    scale = np.exp2(ge.astype(np.float64))[:, :, None]
    vg = oracle.fp8_decode(gq.reshape(n, I)).reshape(n, I // 32, 32) * scale

    def step(v):  # E4M3 spacing at |v| (in the block's units), doubled at the top of a binade
        _, ex = np.frexp(np.minimum(np.abs(v) / scale, 448.0))
        return np.exp2(np.maximum(ex - 1, -6) - 3) * scale

    hc = np.clip(h, -448.0 * scale, 448.0 * scale)  # values past 448 saturate
    dev = np.abs(vg - hc) - 0.5 * np.maximum(step(hc), step(vg)) - HID_REL * np.abs(h) - HID_ABS * amax[:, :, None]
    sat = np.abs(h) >= 464.0 * scale * (1 + HID_REL)  # saturated on either side: exactly +-448
    dev = np.where(sat, np.abs(vg - np.sign(h) * 448.0 * scale), dev)
    worst = np.unravel_index(np.argmax(dev), dev.shape)
    assert dev.max() <= 0, f"hidden value inadmissible at row {worst[0]}, unit {32 * worst[1] + worst[2]}: " \
                           f"gpu {vg[worst]:.6g} oracle {h[worst]:.6g}"
    oq, osc = oracle.mx_quantize(h32)
    flips = int((oq != gq).sum())
    assert flips <= HID_MAX_FLIP_FRACTION * gq.size + 1, f"{flips} of {gq.size} hidden codes differ"
    return flips, int((osc != gs).sum())


def gpu_hidden_rows(res, t, j, k):
    """The GPU's hidden codes and scales of pair (token t, slot j) from a forward_layer
    result (dispatched-row order: row p holds the pair perm_src[p])."""
    perm = res["_perm_np"] if "_perm_np" in res else res["perm_src"].cpu().numpy()
    res["_perm_np"] = perm
    if "_pos_np" not in res:
        pos = np.empty_like(perm)
        pos[perm] = np.arange(perm.size, dtype=perm.dtype)
        res["_pos_np"] = pos
    p = res["_pos_np"][np.asarray(t) * k + np.asarray(j)]
    return res["_hq_np"][p], res["_hs_np"][p]


def hidden_to_np(res):
    res["_hq_np"] = res["hidden_codes"].cpu().numpy()
    res["_hs_np"] = res["hidden_scales"].cpu().numpy()


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def routing_to_np(res):
    return {key: res[key].cpu().numpy() for key in ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin")}


def m_tiles(n):
    """The grouped GEMM's M tiles of an expert with n rows: ceil(n/256) tiles of equal
    whole 32-row blocks, the last taking the rest. Returns [(first row, rows)]."""
    if n <= 0:
        return []
    nt = -(-n // TILE_ROWS)
    span = -(-(-(-n // BLOCK_ROWS)) // nt) * BLOCK_ROWS
    return [(i * span, min(span, n - i * span)) for i in range(nt)]


def tile_sample(cfg, g, extra=16, seed=0):
    """Tokens whose outputs are compared at prefill sizes, chosen from the GPU's
    (oracle-checked) counts and permutation so that they cover:
      * the first and last row of every M tile of the hottest routed expert,
      * the first and last row of the last tile of up to 8 two-tile experts,
      * the first and last rows of the shared expert's last tile (and first tile),
      * one tile from each eighth of the tile list (the persistent schedule deals
        items to the 8 XCDs in 8 contiguous ranges): its first, last and a middle row,
      * a 32-row block boundary inside a full tile,
    plus `extra` seeded random tokens. Returns (sorted tokens, description)."""
    counts, offsets, perm = g["counts"], g["offsets"], g["perm_src"]
    T, k, E = cfg.T, cfg.k, cfg.E
    tiles = []  # (expert, first row within expert, rows) in the library's order
    for e in range(E):
        for m0, rows in m_tiles(int(counts[e])):
            tiles.append((e, m0, rows))
    for m0, rows in m_tiles(T):
        tiles.append((E, m0, rows))

    def tok(e, r):
        return int(perm[offsets[e] + r]) // k if e < E else r

    chosen, why = set(), {}

    def add(e, r, reason):
        t = tok(e, r)
        chosen.add(t)
        why.setdefault(reason, 0)
        why[reason] += 1

    hot = int(np.argmax(counts))
    for m0, rows in m_tiles(int(counts[hot])):
        add(hot, m0, "hottest expert tile ends")
        add(hot, m0 + rows - 1, "hottest expert tile ends")
    two = [e for e in range(E) if len(m_tiles(int(counts[e]))) == 2]
    for e in two[:: max(1, len(two) // 8)][:8]:
        m0, rows = m_tiles(int(counts[e]))[-1]
        add(e, m0, "two-tile experts, last tile")
        add(e, m0 + rows - 1, "two-tile experts, last tile")
    sh = m_tiles(T)
    for m0, rows in (sh[0], sh[-1]):
        add(E, m0, "shared expert first/last tile")
        add(E, m0 + rows - 1, "shared expert first/last tile")
    for x in range(8):
        e, m0, rows = tiles[(2 * x + 1) * len(tiles) // 16]
        for r in (m0, m0 + rows // 2, m0 + rows - 1):
            add(e, r, "one tile per XCD range")
    full = [t for t in tiles if t[2] > BLOCK_ROWS and t[0] < E]
    if full:
        e, m0, rows = full[len(full) // 2]
        add(e, m0 + BLOCK_ROWS - 1, "32-row block boundary")
        add(e, m0 + BLOCK_ROWS, "32-row block boundary")
    rng = np.random.default_rng(seed)
    for t in rng.choice(T, size=extra, replace=False):
        chosen.add(int(t))
    why["random"] = extra
    return sorted(chosen), why

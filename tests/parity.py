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


def check_out(out_gpu, ref):
    rel = np.abs(out_gpu - ref) / (1.0 + np.abs(ref))
    worst = float(rel.max()) if rel.size else 0.0
    assert np.isfinite(out_gpu).all()
    assert worst <= OUT_TOL, f"max |gpu-ref|/(1+|ref|) = {worst:.3e} > {OUT_TOL}"
    return worst, float(np.abs(out_gpu - ref).mean()) if rel.size else 0.0


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

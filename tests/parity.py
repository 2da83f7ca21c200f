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

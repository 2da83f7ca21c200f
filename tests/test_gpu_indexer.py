"""GPU parity of the sparse-attention indexer (hy_indexer_topk, through the C ABI)
against the fp64 oracle.

Scores: fp32 on the GPU (exact bf16 products, fp32 sums) against fp64, within the
bound (D + H + 1) * 2^-24 * sum_h w_h sum_i |q_hi k_i| of that arithmetic.
Selection: the GPU's indices must equal the oracle's top-K (ties to the lower index)
of the GPU's own scores exactly, and the oracle's top-K of its fp64 scores exactly
wherever the K-th score leads the (K+1)-th by more than twice the score bound;
otherwise the GPU's set must be admissible (no unselected key scoring above a
selected one by more than that).
"""
import numpy as np
import pytest

import hy_inputs as hi
import oracle
from parity import bf16_tensor_bits

torch = pytest.importorskip("torch")
hm = pytest.importorskip("sparse_moe_transformer_route_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def say(msg):
    print(msg, flush=True)


def score_bound(q, w, keys, D, H):
    """Per-key bound of the fp32 scores' error: q bf16 bits [H][D], w [H], keys [S][D]."""
    aq = np.abs(hi.bf16_to_f32(q).astype(np.float64))
    ak = np.abs(hi.bf16_to_f32(keys).astype(np.float64))
    return (D + H + 1) * U * ((ak @ aq.T) @ w.astype(np.float64)) * 1.01


def check_row(idx, gpu_scores, q, w, keys, K, D, H, label):
    """One query: scores within the bound, selection exact on the GPU's scores and
    exact or admissible on the oracle's."""
    S = keys.shape[0]
    n = min(K, S)
    assert idx.shape == (n,)
    assert (np.diff(idx) > 0).all() and idx[0] >= 0 and idx[-1] < S, label
    own, _, _ = oracle.topk_indices(gpu_scores.astype(np.float64)[None], K)
    assert np.array_equal(idx, own[0]), f"{label}: not the top-{K} of its own scores"
    ref = oracle.indexer_scores(q[None], w[None], keys[None])[0]
    tol = score_bound(q, w, keys, D, H)
    err = np.abs(gpu_scores.astype(np.float64) - ref)
    assert (err <= tol).all(), f"{label}: score error {err.max():.3e} > bound {tol[err.argmax()]:.3e}"
    ridx, kth, margin = oracle.topk_indices(ref[None], K)
    tmax = 2 * tol.max()
    if margin[0] > tmax:
        assert np.array_equal(idx, ridx[0]), f"{label}: selection differs with margin {margin[0]:.3e}"
        near = False
    else:
        sel = np.zeros(S, bool)
        sel[idx] = True
        if n < S:
            assert ref[sel].min() >= ref[~sel].max() - tmax, f"{label}: inadmissible selection"
        near = True
    return err.max(), near


def run_case(cfg, keys_dev=None, keys_host=None):
    say(f"[case] indexer B={cfg.B} S={cfg.S} K={cfg.K}")
    inp = hi.dev_indexer(cfg, device=DEV)
    if keys_dev is not None:
        inp["keys"] = keys_dev
    scores = torch.empty(cfg.B, cfg.S, dtype=torch.float32, device=DEV)
    idx, _ = hm.indexer_topk(inp["q"], inp["w"], inp["keys"], cfg.K, scores=scores)
    torch.cuda.synchronize()
    q, w = hi.host_indexer_queries(cfg)
    idx, sc = idx.cpu().numpy(), scores.cpu().numpy()
    worst, nnear = 0.0, 0
    for b in range(cfg.B):
        kh = keys_host[b] if keys_host is not None else hi.host_indexer_keys(cfg, b)
        e, near = check_row(idx[b], sc[b], q[b], w[b], kh, cfg.K, cfg.D, cfg.H, f"b={b}")
        worst, nnear = max(worst, e), nnear + near
    say(f"       max score error {worst:.3e}, near-tie rows {nnear}")


@pytest.mark.parametrize("B,S,K", [
    (4, 3000, 256),    # the small workload
    (2, 1000, 64),     # last 128-key tile ragged (104 keys)
    (3, 100, 256),     # fewer keys than K: every key
    (1, 1, 1),
    (2, 5000, 2048),
    (5, 129, 128),     # one key past a tile
    (2, 70001, 2048),  # two-stage selection: 9 chunks of 8192 keys (the last one short), one merge
    (1, 65536, 4096),  # two stages with the larger merge (32K candidates)
    (1, 70001, 9000),  # K above a chunk: one pass over more keys than fit on chip (scores re-read)
    (2, 20000, 100),   # 3 chunks of 8192 (fewer than 4): one pass on chip
])
def test_indexer_small(B, S, K):
    run_case(hi.IndexerConfig("ix", B=B, S=S, K=K, seed=3))


def test_indexer_exact_ties_take_lower_keys():
    # keys repeat every 50 rows, so scores repeat exactly: the K-th falls inside a tie
    cfg = hi.IndexerConfig("ixtie", B=2, S=1000, K=70, seed=4)
    kh = np.stack([np.tile(hi.host_indexer_keys(cfg, b)[:50], (20, 1)) for b in range(cfg.B)])
    kd = torch.from_numpy(kh.view(np.int16)).to(DEV).view(torch.bfloat16)
    run_case(cfg, keys_dev=kd, keys_host=kh)


def test_indexer_device_keys_match_host_generator():
    cfg = hi.IndexerConfig("ixgen", B=3, S=700, K=16, seed=5)
    d = hi.dev_indexer(cfg, device=DEV)
    q, w = hi.host_indexer_queries(cfg)
    assert np.array_equal(bf16_tensor_bits(d["q"]), q)
    assert np.array_equal(d["w"].cpu().numpy(), w)
    for b in range(cfg.B):
        assert np.array_equal(bf16_tensor_bits(d["keys"][b]), hi.host_indexer_keys(cfg, b))


def test_indexer_full_size():
    # 32 sequences x 64K keys, top-2048: every row's selection is checked against its own
    # scores and against the oracle (keys copied from the generator's device tensor)
    cfg = hi.INDEXER_CONFIGS["indexer_decode"]
    say(f"[case] indexer full size B={cfg.B} S={cfg.S} K={cfg.K}")
    inp = hi.dev_indexer(cfg, device=DEV)
    scores = torch.empty(cfg.B, cfg.S, dtype=torch.float32, device=DEV)
    idx, _ = hm.indexer_topk(inp["q"], inp["w"], inp["keys"], cfg.K, scores=scores)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), scores.cpu().numpy()
    own, _, _ = oracle.topk_indices(sc.astype(np.float64), cfg.K)
    assert np.array_equal(idx, own)
    q, w = hi.host_indexer_queries(cfg)
    worst, nnear = 0.0, 0
    for b in range(cfg.B):
        e, near = check_row(idx[b], sc[b], q[b], w[b], bf16_tensor_bits(inp["keys"][b]), cfg.K, cfg.D, cfg.H,
                            f"b={b}")
        worst, nnear = max(worst, e), nnear + near
    say(f"       all {cfg.B} rows ok: max score error {worst:.3e}, near-tie rows {nnear}")
    del inp
    torch.cuda.empty_cache()


def test_indexer_workspace_path_matches_scores_path():
    cfg = hi.IndexerConfig("ixws", B=3, S=2000, K=100, seed=6)
    inp = hi.dev_indexer(cfg, device=DEV)
    a, _ = hm.indexer_topk(inp["q"], inp["w"], inp["keys"], cfg.K)  # scores in the workspace
    scores = torch.empty(cfg.B, cfg.S, dtype=torch.float32, device=DEV)
    b, _ = hm.indexer_topk(inp["q"], inp["w"], inp["keys"], cfg.K, scores=scores)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

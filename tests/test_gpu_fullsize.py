"""GPU parity at the full Hy4-preview layer shape (d=6144, E=256, k=8, I=2048)
in the launch configuration the benchmark times (hy_moe_forward_ex, automatic
path choice, caller workspace):
  decode   T=32,   bf16 experts
  prefill  T=8192, bf16 experts
  skewed   T=4096, bf16 experts, Zipf(1.2) router bias
  ternary  T=32,   Sherry ternary routed experts, bf16 shared expert
  ternary_prefill  T=8192, the same weights on the grouped path
  fp8      T=32,   FP8 (E4M3, fp32 row scales) routed experts, bf16 shared expert
  fp8_prefill  T=8192, the same weights on the grouped path
The routing of every token (sets, weights, counts, offsets, permutation) is
compared with the oracle; outputs are compared on sampled tokens, for which the
oracle regenerates the touched experts' weights on the host from the same
seeded streams. Rules and tolerances: tests/parity.py.
"""
import time

import numpy as np
import pytest

import hy_inputs as hi
import oracle
from parity import bf16_tensor_to_np, check_out, check_permutation, check_routing, check_weights, routing_to_np

torch = pytest.importorskip("torch")
hm = pytest.importorskip("sparse_moe_transformer_route_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def hy4_weights():
    """bf16 weights of the Hy4-shape layer (seed 0), shared by decode/prefill/skewed."""
    cfg = hi.CONFIGS["prefill"]
    say("[fixture] generating 19.3 GB of bf16 expert weights on the GPU")
    w = hi.dev_layer(cfg, device=DEV)
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()


def sampled_reference(cfg, x_host, sets, w, tokens, ternary=False, fp8=False):
    """Oracle outputs of the sampled tokens, one expert's weights at a time."""
    sh = hi.host_shared(cfg)
    ys = oracle.ffn(x_host[tokens], sh["gate"], sh["up"], sh["down"])
    yr = np.zeros((len(tokens), cfg.k, cfg.d))
    by_expert = {}
    for i, t in enumerate(tokens):
        for j, e in enumerate(sets[t]):
            by_expert.setdefault(int(e), []).append((i, j))
    for e, pairs in sorted(by_expert.items()):
        if fp8:
            f = hi.host_expert_fp8(cfg, e)
            rows = [tokens[i] for i, _ in pairs]
            y = oracle.ffn_w64(x_host[rows], oracle.fp8_decode(f["fgate"], f["fsgate"]),
                               oracle.fp8_decode(f["fup"], f["fsup"]), oracle.fp8_decode(f["fdown"], f["fsdown"]))
            for (i, j), yy in zip(pairs, y):
                yr[i, j] = yy
            continue
        if ternary:
            q = hi.host_expert_ternary(cfg, e)
            gate = oracle.sherry_decode(q["qgate"], q["sgate"])[1]
            up = oracle.sherry_decode(q["qup"], q["sup"])[1]
            down = oracle.sherry_decode(q["qdown"], q["sdown"])[1]
        else:
            ex = hi.host_expert(cfg, e)
            gate, up, down = ex["gate"], ex["up"], ex["down"]
        rows = [tokens[i] for i, _ in pairs]
        y = oracle.ffn(x_host[rows], gate, up, down)
        for (i, j), yy in zip(pairs, y):
            yr[i, j] = yy
    return oracle.combine(ys, yr, w[tokens])


def run_full(cfg, inp, sample):
    say(f"[case] {cfg.name} T={cfg.T} full-size, sampled tokens {sample}")
    fmt = hm.WEIGHTS_SHERRY_TERNARY if cfg.ternary else hm.WEIGHTS_FP8_E4M3 if cfg.fp8 else hm.WEIGHTS_BF16
    ws = hm.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, fmt, device=DEV)
    res = hm.forward_layer(inp, cfg.k, want_routing=True, workspace=ws)
    torch.cuda.synchronize()
    g = routing_to_np(res)
    out = bf16_tensor_to_np(res["out"])
    assert np.isfinite(out).all()
    t0 = time.time()
    x_host = hi.host_x(cfg)
    lg = oracle.logits(x_host, hi.host_router(cfg), hi.host_bias(cfg))
    sets, near, subst = check_routing(g["topk_idx"], lg, cfg.k)
    check_permutation(g, sets, cfg.E)
    werr = check_weights(g["topk_w"], lg, sets)
    assert g["counts"].sum() == cfg.T * cfg.k
    say(f"       routing of all {cfg.T} tokens ok: near-ties={near} substituted={subst} "
        f"max |dw|={werr:.2e} touched experts={int((g['counts'] > 0).sum())} ({time.time() - t0:.1f}s)")
    w_ref = oracle.weights(lg, sets)
    ref = sampled_reference(cfg, x_host, sets, w_ref, sample, ternary=cfg.ternary, fp8=cfg.fp8)
    worst, mean = check_out(out[sample], ref)
    say(f"       sampled outputs ok: max_rel_err={worst:.3e} mean_abs_err={mean:.3e} ({time.time() - t0:.1f}s)")
    return res, g


def with_x(cfg, weights):
    inp = dict(weights)
    inp["x"] = weights["x"][: cfg.T].contiguous()
    b = hi.host_bias(cfg)
    inp["bias"] = None if b is None else torch.from_numpy(b).to(DEV)
    return inp


def test_decode_full_size(hy4_weights):
    cfg = hi.CONFIGS["decode"]
    run_full(cfg, with_x(cfg, hy4_weights), sample=[0, 5, 17, 31])


def test_prefill_full_size(hy4_weights):
    cfg = hi.CONFIGS["prefill"]
    run_full(cfg, with_x(cfg, hy4_weights), sample=[0, 4095, 8191])


def test_skewed_full_size(hy4_weights):
    cfg = hi.CONFIGS["skewed"]
    res, g = run_full(cfg, with_x(cfg, hy4_weights), sample=[0, 2047, 4095])
    counts = g["counts"]
    say(f"       skew: hottest expert {int(counts.max())} rows, empty experts {int((counts == 0).sum())}")
    assert (counts == 0).any(), "the Zipf bias should leave some experts empty"


def test_skewed_paths_agree(hy4_weights):
    cfg = hi.CONFIGS["skewed"]
    say("[case] skewed T=4096: streaming path vs grouped path")
    inp = with_x(cfg, hy4_weights)
    a = hm.forward_layer(inp, cfg.k, path=hm.PATH_STREAM)
    b = hm.forward_layer(inp, cfg.k, path=hm.PATH_GROUPED)
    torch.cuda.synchronize()
    fa, fb = a["out"].float(), b["out"].float()
    assert ((fa - fb).abs() <= 2e-2 * (1 + fb.abs())).all()


def test_ternary_full_size():
    cfg = hi.CONFIGS["ternary"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample=[0, 9, 31])


def test_fp8_full_size():
    cfg = hi.CONFIGS["fp8"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample=[0, 13, 31])
    del inp
    torch.cuda.empty_cache()


def test_fp8_prefill_full_size():
    cfg = hi.CONFIGS["fp8_prefill"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample=[0, 4095, 8191])
    del inp
    torch.cuda.empty_cache()


def test_ternary_prefill_full_size():
    cfg = hi.CONFIGS["ternary_prefill"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample=[0, 4095, 8191])
    del inp
    torch.cuda.empty_cache()

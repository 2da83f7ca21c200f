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
  fp8_w8a8, fp8_w8a8_prefill  T=32 and T=8192, the same weights with MXFP8 activations
The routing of every token (sets, weights, counts, offsets, permutation) is
compared with the oracle. Outputs: every token of the decode batches; at
prefill sizes a sample chosen from the routing so that it covers the grouped
GEMM's schedule (tile_sample). The oracle's expert weights are copies of the
generator's device tensors (never a result of the HIP path), taken one expert at
a time. Rules and tolerances: tests/parity.py.
"""
import dataclasses
import time

import numpy as np
import pytest

import hy_inputs as hi
import oracle
from parity import (bf16_tensor_bits, bf16_tensor_to_np, check_out, check_permutation, check_routing,
                    check_weights, routing_to_np, tile_sample, check_hidden_rows, gpu_hidden_rows, hidden_to_np)

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


class DeviceExperts:
    """Routed experts' weights for the oracle, copied from the generator's device
    tensors one expert at a time (bf16 bits, or decoded Sherry / FP8 weights)."""

    def __init__(self, inp):
        self.inp = inp

    def get(self, e):
        inp = self.inp
        if "fgate" in inp:
            return tuple(oracle.fp8_decode(inp[q][e].cpu().numpy(), inp[s][e].cpu().numpy())
                         for q, s in (("fgate", "fsgate"), ("fup", "fsup"), ("fdown", "fsdown"))), True
        if "qgate" in inp:
            return tuple(oracle.sherry_decode(inp[q][e].cpu().numpy().view(np.uint32), bf16_tensor_bits(inp[s][e]))[1]
                         for q, s in (("qgate", "sgate"), ("qup", "sup"), ("qdown", "sdown"))), False
        return tuple(bf16_tensor_bits(inp[n][e]) for n in ("gate", "up", "down")), False


def reference_outputs(cfg, inp, x_host, sets, w, tokens, gpu_res=None):
    """Oracle outputs of `tokens`: the shared expert, then each routed expert the
    tokens use, one expert's weights at a time, combined in fp64."""
    if inp.get("shared_sherry"):  # expert E of the Sherry arrays
        (sg, su, sdn), _ = DeviceExperts(inp).get(cfg.E)
        ys = oracle.ffn(x_host[tokens], sg, su, sdn)
    else:
        sh = {n: bf16_tensor_bits(v) for n, v in inp["shared"].items()}
        ys = oracle.ffn(x_host[tokens], sh["gate"], sh["up"], sh["down"])
    yr = np.zeros((len(tokens), cfg.k, cfg.d))
    by_expert = {}
    for i, t in enumerate(tokens):
        for j, e in enumerate(sets[t]):
            by_expert.setdefault(int(e), []).append((i, j))
    src = DeviceExperts(inp)
    flips = [0, 0]
    for e, pairs in sorted(by_expert.items()):
        (gate, up, down), w64 = src.get(e)
        rows = x_host[[tokens[i] for i, _ in pairs]]
        if cfg.a8:
            # the GPU's hidden rows must be admissible; the oracle's down projection runs on
            # them (tests/parity.py)
            _, h32 = oracle.ffn_w8a8_ex(rows, gate, up, down, want_hidden=True)
            gq, gs = gpu_hidden_rows(gpu_res, [tokens[i] for i, _ in pairs], [j for _, j in pairs], cfg.k)
            f1, f2 = check_hidden_rows(h32, gq, gs)
            flips[0] += f1
            flips[1] += f2
            y = oracle.ffn_w8a8_ex(rows, gate, up, down, hq=gq, hs=gs)
        else:
            y = (oracle.ffn_w64 if w64 else oracle.ffn)(rows, gate, up, down)
        for (i, j), yy in zip(pairs, y):
            yr[i, j] = yy
    if cfg.a8:
        say(f"       hidden rows admissible: {flips[0]} codes and {flips[1]} block scales substituted")
    return oracle.combine(ys, yr, w[tokens])


def run_full(cfg, inp, sample="all"):
    say(f"[case] {cfg.name} T={cfg.T} full-size")
    fmt = (hm.WEIGHTS_SHERRY_TERNARY if cfg.ternary else
           (hm.WEIGHTS_FP8_W8A8 if cfg.a8 else hm.WEIGHTS_FP8_E4M3) if cfg.fp8 else hm.WEIGHTS_BF16)
    ws = hm.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, fmt, device=DEV)
    res = hm.forward_layer(inp, cfg.k, want_routing=True, workspace=ws, fp8_activations=cfg.a8, want_hidden=cfg.a8)
    torch.cuda.synchronize()
    if cfg.a8:
        hidden_to_np(res)
    g = routing_to_np(res)
    out = bf16_tensor_to_np(res["out"])
    assert np.isfinite(out).all()
    t0 = time.time()
    x_host = bf16_tensor_bits(inp["x"])
    bias = None if inp.get("bias") is None else inp["bias"].cpu().numpy()
    lg = oracle.logits(x_host, bf16_tensor_bits(inp["router"]), bias)
    sets, near, subst = check_routing(g["topk_idx"], lg, cfg.k)
    check_permutation(g, sets, cfg.E)
    werr = check_weights(g["topk_w"], lg, sets)
    assert g["counts"].sum() == cfg.T * cfg.k
    say(f"       routing of all {cfg.T} tokens ok: near-ties={near} substituted={subst} "
        f"max |dw|={werr:.2e} touched experts={int((g['counts'] > 0).sum())} ({time.time() - t0:.1f}s)")
    if sample == "all":
        tokens, why = list(range(cfg.T)), {"every token": cfg.T}
    else:
        tokens, why = tile_sample(cfg, g)
    say(f"       comparing {len(tokens)} tokens: {why}")
    w_ref = oracle.weights(lg, sets)
    ref = reference_outputs(cfg, inp, x_host, sets, w_ref, tokens, gpu_res=res)
    worst, mean = check_out(out[tokens], ref)
    say(f"       outputs ok: max_rel_err={worst:.3e} mean_abs_err={mean:.3e} ({time.time() - t0:.1f}s)")
    return res, g, tokens


def with_x(cfg, weights):
    inp = dict(weights)
    inp["x"] = weights["x"][: cfg.T].contiguous()
    b = hi.host_bias(cfg)
    inp["bias"] = None if b is None else torch.from_numpy(b).to(DEV)
    return inp


def test_decode_full_size(hy4_weights):
    cfg = hi.CONFIGS["decode"]
    run_full(cfg, with_x(cfg, hy4_weights))


def test_prefill_full_size(hy4_weights):
    cfg = hi.CONFIGS["prefill"]
    run_full(cfg, with_x(cfg, hy4_weights), sample="tiles")


def test_skewed_full_size(hy4_weights):
    cfg = hi.CONFIGS["skewed"]
    res, g, _ = run_full(cfg, with_x(cfg, hy4_weights), sample="tiles")
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


def test_blocked_weights_full_size(hy4_weights):
    """The blocked layout of the same weights gives bitwise the same outputs and routing
    as the row-major one at the decode, prefill and skewed sizes (the streaming path, the
    grouped path at every tile height, and the skewed hottest expert's 16 M tiles)."""
    blk = hm.block_layer(hy4_weights)
    for name in ("decode", "prefill", "skewed"):
        cfg = hi.CONFIGS[name]
        say(f"[case] {name} T={cfg.T}: blocked bf16 weights vs row-major")
        ref = hm.forward_layer(with_x(cfg, hy4_weights), cfg.k, want_routing=True)
        got = hm.forward_layer(with_x(cfg, blk), cfg.k, want_routing=True, weights_blocked=True)
        torch.cuda.synchronize()
        assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16)), name
        for key in ("topk_idx", "counts", "perm_src"):
            assert torch.equal(got[key], ref[key]), (name, key)
    del blk
    torch.cuda.empty_cache()


def test_ternary_full_size():
    cfg = hi.CONFIGS["ternary"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp)


def test_blocked_sherry_full_size():
    """Blocked Sherry codes give bitwise the same outputs and routing as row-major ones at
    the ternary decode (LDS-staged streaming kernels) and ternary prefill (grouped GEMM)
    sizes."""
    for name in ("ternary", "ternary_prefill"):
        cfg = hi.CONFIGS[name]
        say(f"[case] {name} T={cfg.T}: blocked Sherry codes vs row-major")
        inp = hi.dev_layer(cfg, device=DEV)
        ref = hm.forward_layer(inp, cfg.k, want_routing=True)
        blk = hm.block_layer(inp)
        got = hm.forward_layer(blk, cfg.k, want_routing=True, weights_blocked=True)
        torch.cuda.synchronize()
        assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16)), name
        for key in ("topk_idx", "counts", "perm_src"):
            assert torch.equal(got[key], ref[key]), (name, key)
        del inp, blk, ref, got
        torch.cuda.empty_cache()


def test_sherry_shared_expert_full_size():
    """A Sherry-packed shared expert at the ternary decode size (every token against the
    oracle) and the ternary prefill size (tile-covering sample)."""
    for name, sample in (("ternary", "all"), ("ternary_prefill", "tiles")):
        cfg = dataclasses.replace(hi.CONFIGS[name], tshared=True)
        inp = hi.dev_layer(cfg, device=DEV)
        run_full(cfg, inp, sample=sample)
        del inp
        torch.cuda.empty_cache()


def test_fp8_full_size():
    cfg = hi.CONFIGS["fp8"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp)
    del inp
    torch.cuda.empty_cache()


def test_fp8_prefill_full_size():
    cfg = hi.CONFIGS["fp8_prefill"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample="tiles")
    del inp
    torch.cuda.empty_cache()


def test_fp8_w8a8_full_size():
    # decode batch and prefill batch on the same FP8 weights with MXFP8 activations
    cfg = hi.CONFIGS["fp8_w8a8"]
    inp = hi.dev_layer(hi.CONFIGS["fp8_w8a8_prefill"], device=DEV)
    run_full(cfg, with_x(cfg, inp))
    run_full(hi.CONFIGS["fp8_w8a8_prefill"], inp, sample="tiles")
    del inp
    torch.cuda.empty_cache()


def test_ternary_prefill_full_size():
    cfg = hi.CONFIGS["ternary_prefill"]
    inp = hi.dev_layer(cfg, device=DEV)
    run_full(cfg, inp, sample="tiles")
    del inp
    torch.cuda.empty_cache()

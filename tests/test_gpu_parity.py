"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element over every token; the full-size
Hy4-shape workloads compare the routing of every token and the outputs of
sampled tokens (the oracle regenerates the sampled tokens' experts on the host
from the same seeded streams). Rules and tolerances: tests/parity.py.
"""
import math

import numpy as np
import pytest

import hy_inputs as hi
import oracle
from parity import (bf16_tensor_bits, bf16_tensor_to_np, check_out, check_permutation, check_routing, f32_to_bf16_bits,
                    check_hidden_rows, gpu_hidden_rows, hidden_to_np,
                    check_weights, routing_to_np)

torch = pytest.importorskip("torch")
hm = pytest.importorskip("sparse_moe_transformer_route_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def host_weights_bf16(cfg, L):
    """(gate, up, down) bf16 bit arrays for the oracle; ternary experts decoded."""
    if not cfg.ternary:
        return L["gate"], L["up"], L["down"]
    gate = np.stack([oracle.sherry_decode(L["qgate"][e], L["sgate"][e])[1] for e in range(cfg.E)])
    up = np.stack([oracle.sherry_decode(L["qup"][e], L["sup"][e])[1] for e in range(cfg.E)])
    down = np.stack([oracle.sherry_decode(L["qdown"][e], L["sdown"][e])[1] for e in range(cfg.E)])
    return gate, up, down


def host_shared_bf16(cfg, L):
    """The shared expert's (gate, up, down) bf16 bit arrays for the oracle: the bf16
    matrices, or expert E of the Sherry arrays decoded."""
    if not (cfg.ternary and cfg.tshared):
        return L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"]
    E = cfg.E
    return tuple(oracle.sherry_decode(L["q" + m][E], L["s" + m][E])[1] for m in ("gate", "up", "down"))


def run_small(cfg, path, bias=None, x_host=None, label="", fp8_codes=None):
    """Full element-by-element comparison on a small layer."""
    say(f"[case] {label or cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} "
        f"ternary={cfg.ternary} tshared={cfg.tshared} fp8={cfg.fp8} w8a8={cfg.a8} path={path}")
    L = hi.host_layer(cfg)
    inp = hi.dev_layer(cfg, device=DEV)
    if fp8_codes is not None:  # caller-chosen codes and scales
        for key, val in fp8_codes.items():
            L[key] = val
            inp[key] = torch.from_numpy(val).to(DEV)
    if bias is not None:
        L["bias"] = bias
        inp["bias"] = torch.from_numpy(bias).to(DEV)
    if x_host is not None:
        L["x"] = x_host
        inp["x"] = torch.from_numpy(x_host.view(np.int16)).to(DEV).view(torch.bfloat16)
    res = hm.forward_layer(inp, cfg.k, want_routing=True, path=path, fp8_activations=cfg.a8, want_hidden=cfg.a8)
    torch.cuda.synchronize()
    g = routing_to_np(res)
    lg = oracle.logits(L["x"], L["router"], L["bias"])
    sets, near, subst = check_routing(g["topk_idx"], lg, cfg.k)
    check_permutation(g, sets, cfg.E)
    check_weights(g["topk_w"], lg, sets)
    if cfg.fp8:
        fw = [np.stack([oracle.fp8_decode(L["f" + m][e], L["fs" + m][e]) for e in range(cfg.E)])
              for m in ("gate", "up", "down")]
        fwd = oracle.forward_w8a8 if cfg.a8 else oracle.forward_w64
        ref = fwd(L["x"], L["router"], L["bias"], *fw, L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"],
                  cfg.k, sets_in=sets)
    else:
        gate, up, down = host_weights_bf16(cfg, L)
        ref = oracle.forward(L["x"], L["router"], L["bias"], gate[:cfg.E], up[:cfg.E], down[:cfg.E],
                             *host_shared_bf16(cfg, L), cfg.k, sets_in=sets)
    if cfg.a8:
        # the GPU's hidden rows must be admissible quantizations of the oracle's; the
        # oracle's down projection then runs on them (tests/parity.py)
        hidden_to_np(res)
        yr = np.zeros((cfg.T, cfg.k, cfg.d))
        flips = sflips = 0
        for e in range(cfg.E):
            tk, slot = np.nonzero(sets == e)
            if not tk.size:
                continue
            _, h32 = oracle.ffn_w8a8_ex(L["x"][tk], fw[0][e], fw[1][e], fw[2][e], want_hidden=True)
            gq, gs = gpu_hidden_rows(res, tk, slot, cfg.k)
            f1, f2 = check_hidden_rows(h32, gq, gs)
            flips, sflips = flips + f1, sflips + f2
            yr[tk, slot] = oracle.ffn_w8a8_ex(L["x"][tk], fw[0][e], fw[1][e], fw[2][e], hq=gq, hs=gs)
        ys = oracle.ffn(L["x"], L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
        ref["out"] = oracle.combine(ys, yr, ref["w"])
        say(f"       hidden rows admissible: {flips} codes and {sflips} block scales substituted")
    worst, mean = check_out(bf16_tensor_to_np(res["out"]), ref["out"])
    # margins: fp32 GPU margin vs fp64 oracle margin
    fin = np.isfinite(ref["margin"])
    assert np.array_equal(np.isfinite(g["margin"]), fin)
    assert np.allclose(g["margin"][fin], ref["margin"][fin], atol=1e-4)
    say(f"       near-ties={near} substituted={subst} max_rel_err={worst:.3e} mean_abs_err={mean:.3e}")
    return res, ref


# ------------------------------------------------------------------ generator
def test_device_generator_matches_host():
    say("[case] generator twin")
    t = torch.empty(100_003, dtype=torch.bfloat16, device=DEV)
    hi.dev_gauss_(t, 5, 3, 0.25, start=777)
    assert np.array_equal(bf16_tensor_bits(t), hi.gauss_bf16(5, 3, 100_003, 0.25, start=777))
    w = torch.empty(4099, dtype=torch.int32, device=DEV)
    hi.dev_words_(w, 1, 10, start=3)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), hi.words_u32(1, 10, 4099, start=3))
    u = torch.empty(5001, dtype=torch.bfloat16, device=DEV)
    hi.dev_uniform_(u, 2, 13, 0.01, 0.02)
    assert np.array_equal(bf16_tensor_bits(u), hi.uniform_bf16(2, 13, 5001, 0.01, 0.02))
    cfg = hi.LayerConfig("f8", T=4, d=256, E=3, k=2, I=128, fp8=True, seed=4)
    dl, hl = hi.dev_layer(cfg, device=DEV), hi.host_layer(cfg)
    for key in ("fgate", "fup", "fdown", "fsgate", "fsup", "fsdown"):
        assert np.array_equal(dl[key].cpu().numpy(), hl[key]), key


# ------------------------------------------------------------ small layers
PATHS = [hm.PATH_STREAM, hm.PATH_GROUPED]


@pytest.mark.parametrize("path", [hm.PATH_AUTO] + PATHS)
def test_tiny_config(path):
    run_small(hi.CONFIGS["tiny"], path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [
    dict(T=1, d=256, E=16, k=2, I=128),
    dict(T=77, d=256, E=16, k=1, I=128),          # ragged token block, k=1
    dict(T=130, d=384, E=64, k=4, I=256),         # the pages' 64-expert / top-4 example
    dict(T=40, d=256, E=16, k=16, I=128),         # k = E: margin +inf
    dict(T=50, d=256, E=100, k=3, I=128),         # E not a multiple of 64
    dict(T=33, d=128, E=1024, k=16, I=128),       # largest E and k
    dict(T=600, d=256, E=4, k=2, I=128),          # ~300 rows per expert: several M tiles
    dict(T=300, d=512, E=8, k=8, I=384),          # every expert takes every token
    dict(T=1100, d=256, E=40, k=3, I=128),        # LDS-tiled router: ragged token tile, E < 256, 1 k step
    dict(T=1030, d=1024, E=300, k=2, I=128),      # LDS-tiled router: two expert tiles, 2 k steps per slice
])
def test_small_shapes(shape, path):
    cfg = hi.LayerConfig("shape", seed=1, **shape)
    run_small(cfg, path)


@pytest.mark.parametrize("path", PATHS)
def test_router_bias_and_empty_experts(path):
    cfg = hi.LayerConfig("bias", T=96, d=256, E=64, k=4, I=128, seed=2)
    run_small(cfg, path, bias=hi.zipf_bias(64, 2, 1.2))


@pytest.mark.parametrize("path", PATHS)
def test_all_tokens_on_one_expert(path):
    cfg = hi.LayerConfig("hot", T=300, d=256, E=16, k=2, I=128, seed=3)
    b = np.zeros(16, np.float32)
    b[11] = 1000.0
    res, _ = run_small(cfg, path, bias=b)
    counts = res["counts"].cpu().numpy()
    assert counts[11] == 300


@pytest.mark.parametrize("path", PATHS)
def test_all_logits_tied(path):
    cfg = hi.LayerConfig("ties", T=70, d=256, E=16, k=3, I=128, seed=4)
    x0 = np.zeros((70, 256), np.uint16)  # x = 0: every logit is 0, ties to the lowest indices
    res, ref = run_small(cfg, path, x_host=x0)
    assert (res["topk_idx"].cpu().numpy() == np.arange(3)).all()
    assert np.allclose(res["topk_w"].cpu().numpy(), 1.0 / 3.0, atol=1e-7)


@pytest.mark.parametrize("T", [1, 32, 100])
def test_ternary_small(T):
    cfg = hi.LayerConfig("tern", T=T, d=256, E=16, k=2, I=256, ternary=True, seed=5)
    run_small(cfg, hm.PATH_STREAM)


@pytest.mark.parametrize("shape", [
    dict(T=1, d=512, E=16, k=2, I=512),       # LDS-staged ternary kernels: one token
    dict(T=40, d=1024, E=16, k=4, I=512),     # ~10 tokens per expert, 2 k chunks per row in down
    dict(T=150, d=512, E=8, k=2, I=1024),     # ~38 tokens per expert: three 16-token passes
])
def test_ternary_lds_small(shape):
    cfg = hi.LayerConfig("tern", ternary=True, seed=5, **shape)
    run_small(cfg, hm.PATH_STREAM)


@pytest.mark.parametrize("shape", [
    # grouped GEMM on decoded Sherry codes; K / 64 mod 6 picks the k-loop tail (gate/up: d, down: I)
    dict(T=64, d=256, E=16, k=2, I=128),     # ~8 rows per expert (one 32-row block); tails 4 and 2
    dict(T=300, d=768, E=8, k=2, I=384),     # ~75 rows per expert, ragged; whole 6-step periods; 3 N tiles
    dict(T=1100, d=640, E=4, k=1, I=256),    # ~275 rows per expert: two M tiles; last down N tile half past d
    dict(T=200, d=512, E=16, k=4, I=512),    # ~50 rows per expert; tails 2 and 2
])
def test_ternary_grouped_small(shape):
    cfg = hi.LayerConfig("terng", ternary=True, seed=5, **shape)
    run_small(cfg, hm.PATH_GROUPED)


def test_ternary_paths_agree_mid_size():
    say("[case] ternary stream vs grouped at T=256 d=1024 E=32 k=4 I=512")
    cfg = hi.LayerConfig("ternmid", T=256, d=1024, E=32, k=4, I=512, ternary=True, seed=9)
    inp = hi.dev_layer(cfg, device=DEV)
    a = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_STREAM)
    b = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_GROUPED)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin"):
        assert torch.equal(a[key], b[key]), key
    fa, fb = a["out"].float(), b["out"].float()
    assert ((fa - fb).abs() <= 2e-2 * (1 + fb.abs())).all()


@pytest.mark.parametrize("shape", [
    dict(T=1, d=256, E=16, k=2, I=256),       # one token
    dict(T=32, d=512, E=16, k=4, I=256),      # ~8 tokens per expert
    dict(T=100, d=256, E=8, k=2, I=512),      # ~25 tokens per expert: two 16-token passes
    # 128-code chunks: gate/up d / 128, down I / 128; rings of 3 and 2 slots
    dict(T=40, d=768, E=16, k=2, I=1024),     # 6 and 8 chunks: both rings filled exactly
    dict(T=24, d=1024, E=8, k=2, I=384),      # 8 and 3 chunks: both ring loops guarded
])
def test_fp8_small(shape):
    cfg = hi.LayerConfig("fp8", fp8=True, seed=6, **shape)
    run_small(cfg, hm.PATH_STREAM)


@pytest.mark.parametrize("shape", [
    # grouped GEMM on FP8 codes; K / 64 mod 6 picks the k-loop tail (gate/up: d, down: I)
    dict(T=64, d=256, E=16, k=2, I=128),     # one 32-row block per expert; tails 4 and 2
    dict(T=300, d=768, E=8, k=2, I=384),     # ragged tiles; whole 6-step periods; 3 N tiles
    dict(T=1100, d=640, E=4, k=1, I=256),    # two M tiles per expert; last down N tile half past d
    dict(T=200, d=512, E=16, k=4, I=512),    # tails 2 and 2
])
def test_fp8_grouped_small(shape):
    cfg = hi.LayerConfig("fp8g", fp8=True, seed=8, **shape)
    run_small(cfg, hm.PATH_GROUPED)


def test_fp8_paths_agree_mid_size():
    say("[case] FP8 stream vs grouped at T=256 d=1024 E=32 k=4 I=512")
    cfg = hi.LayerConfig("fp8mid", T=256, d=1024, E=32, k=4, I=512, fp8=True, seed=9)
    inp = hi.dev_layer(cfg, device=DEV)
    a = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_STREAM)
    b = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_GROUPED)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin"):
        assert torch.equal(a[key], b[key]), key
    fa, fb = a["out"].float(), b["out"].float()
    assert ((fa - fb).abs() <= 2e-2 * (1 + fb.abs())).all()


@pytest.mark.parametrize("path", PATHS)
def test_fp8_every_code(path):
    # Expert e's weights are all E4M3 code e (the two NaN codes replaced by +-1), and
    # its row scales are 1 / |value|, so every expert computes +-1 weights: a wrong
    # conversion of any code (subnormals, zeros, 448) shows as a large error.
    cfg = hi.LayerConfig("fp8all", T=256, d=256, E=256, k=8, I=128, fp8=True, seed=7)
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x38, 0xB8
    val = np.abs(oracle.fp8_decode(codes[None, :])[0])
    scale = np.where(val > 0, 1.0 / np.where(val > 0, val, 1.0), 1.0).astype(np.float32)
    # gate/up sums over random activations grow like sqrt(d); the down sums add I equal
    # terms (every hidden unit of an expert is the same), so that row scale is 1 / I and
    # y stays O(1) (it is rounded to bf16 on the grouped path)
    sd, si = 1.0 / np.sqrt(cfg.d), 1.0 / cfg.I
    chosen = {}
    for m, rows, cols, s in (("gate", cfg.I, cfg.d, sd), ("up", cfg.I, cfg.d, sd), ("down", cfg.d, cfg.I, si)):
        chosen["f" + m] = np.ascontiguousarray(np.broadcast_to(codes[:, None, None], (cfg.E, rows, cols)))
        chosen["fs" + m] = np.ascontiguousarray(np.broadcast_to((scale * s)[:, None], (cfg.E, rows)), np.float32)
    res, _ = run_small(cfg, path, fp8_codes=chosen)
    touched = int((res["counts"] > 0).sum().item())
    say(f"       experts touched: {touched} of 256")
    assert touched >= 240


# ------------------------------------------------- FP8 W8A8 (MXFP8 activations)
def test_mxfp8_quantize_bit_exact():
    # codes and scales of the C-ABI quantizer against the oracle's, bit for bit, on rows
    # of very different magnitudes (subnormal codes, saturation, zero blocks, +-0)
    say("[case] hy_moe_mxfp8_quantize vs oracle")
    rng = np.random.default_rng(31)
    rows, cols = 257, 2048
    v = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-40, 40, (rows, 1)))
    v[5, :64] = 0.0
    v[6, :32] = -0.0
    v[7, :32] = np.exp2(-np.arange(32, dtype=np.float64))  # spans the subnormal range of its block
    v[8, 32:64] = [448.0, 449.0, 463.9, 464.0, 480.0, 500.0] + [1.0] * 26  # saturation ties
    xb = f32_to_bf16_bits(v.astype(np.float32))
    xt = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    codes, scales = hm.mxfp8_quantize(xt)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(hi.bf16_to_f32(xb))
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: gpu {got[tuple(bad[0])]:#x} " \
                          f"oracle {rq[tuple(bad[0])]:#x}"


W8A8_SHAPES = [
    # K / 128 mod 6 picks the k-loop tail (gate/up: d, down: I); d, I multiples of 256
    dict(T=64, d=256, E=16, k=2, I=256),      # one 32-row block per expert; 2 k steps each (tails 2, 2)
    dict(T=300, d=768, E=8, k=2, I=512),      # ragged tiles; 6 steps (a whole period) and 4
    dict(T=1100, d=512, E=4, k=1, I=256),     # two M tiles per expert (275 rows)
    dict(T=200, d=1536, E=16, k=4, I=768),    # 12 steps (two periods) and 6
]


W8A8_SHAPES += [
    dict(T=200, d=512, E=16, k=2, I=256),     # gate/up 4 steps (tail 4), one M tile per expert
    dict(T=1100, d=768, E=4, k=1, I=256),     # two M tiles per expert, gate/up 6 steps
]


@pytest.mark.parametrize("shape", W8A8_SHAPES)
def test_fp8_w8a8_small(shape):
    cfg = hi.LayerConfig("w8a8", fp8=True, a8=True, seed=10, **shape)
    run_small(cfg, hm.PATH_AUTO)


def test_fp8_w8a8_routes_like_weight_only_fp8():
    # the same FP8 weights with bf16 and MXFP8 activations: identical routing, outputs that
    # differ by the activation quantization only (a few percent, not more)
    cfg = hi.LayerConfig("w8a8cmp", T=256, d=1024, E=32, k=4, I=512, fp8=True, seed=11)
    inp = hi.dev_layer(cfg, device=DEV)
    a = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_GROUPED)
    b = hm.forward_layer(inp, cfg.k, want_routing=True, fp8_activations=True)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin"):
        assert torch.equal(a[key], b[key]), key
    fa, fb = a["out"].float(), b["out"].float()
    rel = ((fa - fb).abs() / (1 + fa.abs()))
    say(f"       W8A8 vs weight-only FP8: max rel difference {rel.max().item():.3e}, rms {rel.pow(2).mean().sqrt().item():.3e}")
    # E4M3 activations: about 2^-4 relative rounding per value, averaging over each sum
    assert 1e-4 < rel.pow(2).mean().sqrt().item() < 0.06 and rel.max().item() < 0.3


def test_fp8_w8a8_rejects_stream_path_and_odd_shapes():
    cfg = hi.LayerConfig("w8a8bad", T=16, d=384, E=8, k=2, I=256, fp8=True, seed=12)
    inp = hi.dev_layer(cfg, device=DEV)
    with pytest.raises(hm.HyMoeError) as e:
        hm.forward_layer(inp, cfg.k, fp8_activations=True)  # d % 256 != 0
    assert e.value.status == hm.ERR_UNSUPPORTED
    cfg = hi.LayerConfig("w8a8s", T=16, d=256, E=8, k=2, I=256, fp8=True, seed=12)
    inp = hi.dev_layer(cfg, device=DEV)
    with pytest.raises(hm.HyMoeError) as e:
        hm.forward_layer(inp, cfg.k, fp8_activations=True, path=hm.PATH_STREAM)
    assert e.value.status == hm.ERR_UNSUPPORTED


# ------------------------------------------------------------- determinism
@pytest.mark.parametrize("path", PATHS)
def test_bitwise_deterministic_and_workspace_independent(path):
    say(f"[case] determinism path={path}")
    cfg = hi.LayerConfig("det", T=200, d=512, E=32, k=4, I=256, seed=6)
    inp = hi.dev_layer(cfg, device=DEV)
    ws1 = hm.alloc_workspace(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, device=DEV)
    big = torch.empty(ws1.numel() + 4096, dtype=torch.uint8, device=DEV)
    ws2 = big[4096:]
    r1 = hm.forward_layer(inp, cfg.k, want_routing=True, path=path, workspace=ws1)
    r2 = hm.forward_layer(inp, cfg.k, want_routing=True, path=path, workspace=ws2)
    r3 = hm.forward_layer(inp, cfg.k, want_routing=True, path=path)
    torch.cuda.synchronize()
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
        assert torch.equal(r1[key], r3[key]), key


# ------------------------------------------------------------ blocked bf16 layout
def test_block_bf16_matches_layout_definition():
    """hy_moe_block_bf16 against the layout's definition, written out piece by piece: the
    8 values of row r in columns [64 c + 8 q, 64 c + 8 q + 8) start at element
    1024 ((r / 16) (K / 64) + c) + 8 (64 (q % 2) + 16 (q / 2) + r % 16) of its matrix."""
    say("[case] block_bf16 on 3 matrices of 48 x 192")
    g = torch.Generator(device=DEV).manual_seed(5)
    t = torch.randn(3, 48, 192, generator=g, device=DEV).to(torch.bfloat16)
    b = hm.block_bf16(t)
    torch.cuda.synchronize()
    src = t.view(torch.int16).cpu().numpy()
    got = b.view(torch.int16).cpu().numpy().reshape(3, -1)
    R, K = 48, 192
    exp = np.zeros_like(got)
    for m in range(3):
        for r in range(R):
            for c in range(K // 64):
                for q in range(8):
                    o = 1024 * ((r // 16) * (K // 64) + c) + 8 * (64 * (q % 2) + 16 * (q // 2) + r % 16)
                    exp[m, o:o + 8] = src[m, r, 64 * c + 8 * q:64 * c + 8 * q + 8]
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("path", PATHS)
# T=50: the shared expert's second pair of 16-token passes holds 16 + 2 valid tokens
@pytest.mark.parametrize("shape", [(40, 512, 16, 2, 256), (300, 768, 8, 2, 384), (33, 256, 4, 4, 128),
                                   (50, 256, 16, 4, 128)])
def test_blocked_weights_match_row_major(shape, path):
    T, d, E, k, I = shape
    say(f"[case] blocked bf16 weights T={T} d={d} E={E} k={k} I={I} path={path}")
    cfg = hi.LayerConfig("blk", T=T, d=d, E=E, k=k, I=I, seed=31)
    inp = hi.dev_layer(cfg, device=DEV)
    ref = hm.forward_layer(inp, k, want_routing=True, path=path)
    got = hm.forward_layer(hm.block_layer(inp), k, want_routing=True, path=path, weights_blocked=True)
    torch.cuda.synchronize()
    assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16))
    for key in ("topk_idx", "counts", "perm_src"):
        assert torch.equal(got[key], ref[key])


def test_block_sherry_matches_layout_definition():
    """hy_moe_block_sherry against the layout's definition, written out byte by byte: row
    r's 80-byte slab of weights [512 c, 512 c + 512) starts at byte
    1280 ((r / 16) (K / 512) + c) + 80 (r % 16) of its matrix."""
    say("[case] block_sherry on 3 matrices of 48 x 1536 weights")
    R, K = 48, 1536
    g = torch.Generator(device=DEV).manual_seed(6)
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (3, R, K // 128 * 5), generator=g, device=DEV, dtype=torch.int32)
    b = hm.block_sherry(q)
    torch.cuda.synchronize()
    src = q.cpu().numpy().view(np.uint8).reshape(3, R, K // 128 * 20)
    got = b.cpu().numpy().view(np.uint8).reshape(3, -1)
    exp = np.zeros_like(got)
    for m in range(3):
        for r in range(R):
            for c in range(K // 512):
                o = 1280 * ((r // 16) * (K // 512) + c) + 80 * (r % 16)
                exp[m, o:o + 80] = src[m, r, 80 * c:80 * c + 80]
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [(1, 512, 16, 2, 512), (40, 1024, 16, 4, 512), (300, 512, 8, 2, 1536)])
def test_blocked_sherry_match_row_major(shape, path):
    T, d, E, k, I = shape
    say(f"[case] blocked Sherry codes T={T} d={d} E={E} k={k} I={I} path={path}")
    cfg = hi.LayerConfig("tblk", T=T, d=d, E=E, k=k, I=I, ternary=True, seed=33)
    inp = hi.dev_layer(cfg, device=DEV)
    ref = hm.forward_layer(inp, k, want_routing=True, path=path)
    got = hm.forward_layer(hm.block_layer(inp), k, want_routing=True, path=path, weights_blocked=True)
    torch.cuda.synchronize()
    assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16))
    for key in ("topk_idx", "counts", "perm_src"):
        assert torch.equal(got[key], ref[key])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [
    dict(T=1, d=512, E=16, k=2, I=512),      # one token: one shared pass of 4
    dict(T=43, d=1024, E=16, k=4, I=512),    # ragged last shared pass (43 = 10 x 4 + 3)
    dict(T=300, d=512, E=8, k=2, I=1024),    # grouped: two shared M tiles
])
def test_sherry_shared_expert(shape, path):
    """The shared expert Sherry-packed as expert E of the code arrays (shared_format)."""
    cfg = hi.LayerConfig("tsh", ternary=True, tshared=True, seed=8, **shape)
    run_small(cfg, path)


@pytest.mark.parametrize("path", PATHS)
def test_sherry_shared_expert_blocked(path):
    T, d, E, k, I = 70, 512, 16, 2, 1536
    say(f"[case] blocked Sherry codes with a Sherry shared expert T={T} d={d} E={E} k={k} I={I} path={path}")
    cfg = hi.LayerConfig("tshb", T=T, d=d, E=E, k=k, I=I, ternary=True, tshared=True, seed=34)
    inp = hi.dev_layer(cfg, device=DEV)
    ref = hm.forward_layer(inp, k, want_routing=True, path=path)
    got = hm.forward_layer(hm.block_layer(inp), k, want_routing=True, path=path, weights_blocked=True)
    torch.cuda.synchronize()
    assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16))


# ------------------------------------------------- large cancelling expert outputs
def _bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("path", PATHS)
def test_large_cancelling_expert_outputs(path):
    """Experts in pairs (0, 1) and (2, 3) share router rows (so equal weights) and
    gate/up weights (so equal hidden rows), and the second's down projection is minus
    256 times the first's plus an ordinary matrix: each y row is ~256 times the output
    it sums to. The grouped path stores y rows in bf16 (RNE, relative error <= 2^-8),
    so its error may reach 2^-8 (sum_j w_j |y_j| + |y_shared|) on top of the usual
    tolerance; the streaming path keeps y in fp32 and meets the usual tolerance alone."""
    cfg = hi.LayerConfig("cancel", T=300, d=256, E=4, k=4, I=256, seed=21)
    say(f"[case] large cancelling outputs T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.I} path={path}")
    L = hi.host_layer(cfg)
    router, gate, up, down = L["router"].copy(), L["gate"].copy(), L["up"].copy(), L["down"].copy()
    for a, b in ((0, 1), (2, 3)):
        router[b], gate[b], up[b] = router[a], gate[a], up[a]
        big = _bits_to_f32(down[a]) * np.float32(256.0)  # exact: a power of two
        down[b] = f32_to_bf16_bits(-big + _bits_to_f32(down[b]))
        down[a] = f32_to_bf16_bits(big)
    def dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)
    inp = {"x": dev(L["x"]), "router": dev(router), "bias": None, "gate": dev(gate), "up": dev(up), "down": dev(down),
           "shared": {m: dev(L["shared"][m]) for m in ("gate", "up", "down")}}
    res = hm.forward_layer(inp, cfg.k, want_routing=True, path=path)
    torch.cuda.synchronize()
    assert (res["topk_idx"].cpu().numpy() == np.arange(4)).all()
    ref = oracle.forward(L["x"], router, None, gate, up, down, L["shared"]["gate"], L["shared"]["up"],
                         L["shared"]["down"], cfg.k)
    ys = oracle.ffn(L["x"], L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
    mag = np.abs(ys)
    for e in range(cfg.E):
        ye = oracle.ffn(L["x"], gate[e], up[e], down[e])
        mag += ref["w"][:, e:e + 1] * np.abs(ye)
    out = bf16_tensor_to_np(res["out"])
    plain = np.abs(out - ref["out"]) / (1.0 + np.abs(ref["out"]))
    say(f"       sum w|y| / |out| median {np.median(mag / (1e-3 + np.abs(ref['out']))):.0f}; "
        f"max |gpu-ref|/(1+|ref|) = {plain.max():.3e}")
    if path == hm.PATH_GROUPED:
        check_out(out, ref["out"], extra=2.0 ** -8 * mag)
    else:
        check_out(out, ref["out"])


def test_plain_entry_point_matches_ex():
    say("[case] hy_moe_forward vs hy_moe_forward_ex")
    cfg = hi.LayerConfig("plain", T=64, d=256, E=16, k=2, I=128, seed=7)
    inp = hi.dev_layer(cfg, device=DEV)
    out = hm.forward(inp["x"], inp["router"], inp["gate"], inp["up"], inp["down"], inp["shared"]["gate"],
                     inp["shared"]["up"], inp["shared"]["down"], cfg.k)
    r = hm.forward_layer(inp, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])


def test_paths_agree_mid_size():
    say("[case] stream vs grouped at T=256 d=1024 E=32 k=4 I=512")
    cfg = hi.LayerConfig("mid", T=256, d=1024, E=32, k=4, I=512, seed=8)
    inp = hi.dev_layer(cfg, device=DEV)
    a = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_STREAM)
    b = hm.forward_layer(inp, cfg.k, want_routing=True, path=hm.PATH_GROUPED)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "counts", "offsets", "perm_src", "margin"):
        assert torch.equal(a[key], b[key]), key
    fa, fb = a["out"].float(), b["out"].float()
    assert ((fa - fb).abs() <= 2e-2 * (1 + fb.abs())).all()

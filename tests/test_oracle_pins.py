"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each step of oracle/hy_oracle.c is checked against brute force on tiny inputs,
closed forms, invariants, hand-worked fixtures or an independent library
routine (numpy fp64), chosen so that a dropped term, a wrong sign or index, a
transposed operand or a wrong tie-break fails at least one test.
"""
import itertools
import math
import os

import numpy as np
import pytest

import hy_inputs as hi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16_ONE = 0x3F80


def f32_to_bf16_bits(a):
    """Round fp32 -> bf16 (nearest even) as uint16 bit patterns (test helper)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf(a):
    return hi.bf16_to_f32(np.asarray(a, np.uint16)).astype(np.float64)


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def np_swiglu(x, wg, wu, wd):
    """Dense SwiGLU with numpy fp64 matmuls: x [n][d] -> [n][d]."""
    g = x @ wg.T
    u = x @ wu.T
    return (np_silu(g) * u) @ wd.T


# ------------------------------------------------------------------ selection
def brute_force_sets(lg, k):
    """The k-subset with the largest logit sum; among equal sums the
    lexicographically smallest index tuple (== lower index wins ties)."""
    T, E = lg.shape
    combos = np.array(list(itertools.combinations(range(E), k)), dtype=np.int64)
    out = np.empty((T, k), np.int32)
    for t in range(T):
        sums = lg[t][combos].sum(axis=1)
        out[t] = combos[int(np.argmax(sums))]  # argmax returns the first maximum
    return out


@pytest.mark.parametrize("E,k,T", [(16, 2, 40), (10, 3, 40), (8, 4, 40), (64, 4, 6), (5, 5, 3), (7, 1, 30)])
@pytest.mark.parametrize("kind", ["integers", "continuous"])
def test_select_matches_brute_force(E, k, T, kind):
    rng = np.random.default_rng(E * 100 + k)
    if kind == "integers":
        lg = rng.integers(-3, 4, size=(T, E)).astype(np.float64)  # many exact ties
    else:
        lg = rng.standard_normal((T, E))
    sets, margin = oracle.select(lg, k)
    assert np.array_equal(sets, brute_force_sets(lg, k))
    srt = -np.sort(-lg, axis=1)
    expect_margin = np.full(T, np.inf) if k == E else srt[:, k - 1] - srt[:, k]
    assert np.array_equal(margin, expect_margin)
    # exactly k distinct experts, ascending
    assert (np.diff(sets, axis=1) > 0).all()


def test_select_all_equal_takes_lowest_indices():
    sets, margin = oracle.select(np.zeros((3, 16)), 4)
    assert (sets == np.arange(4)).all() and (margin == 0).all()


def test_routing_toy_example_from_pages():
    # tests/golden/routing_toy.txt: 64 experts, K=4 -> 4 active and 60 idle per token;
    # 256 experts, K=8 -> 8 active, 248 idle.
    rows = [l for l in open(os.path.join(GOLDEN, "routing_toy.txt")) if l[0] != "#" and l.strip()]
    for row in rows:
        f = dict(kv.split("=") for kv in row.split())
        E, K = int(f["E"]), int(f["K"])
        rng = np.random.default_rng(E)
        lg = rng.standard_normal((50, E))
        sets, _ = oracle.select(lg, K)
        counts, _, _, _ = oracle.permute(sets, E)
        for t in range(50):
            assert len(set(sets[t].tolist())) == int(f["active"])
            assert E - len(set(sets[t].tolist())) == int(f["idle"])
        assert counts.sum() == 50 * K


# -------------------------------------------------------------------- weights
def test_weights_closed_forms():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((20, 12)) * 3
    s1, _ = oracle.select(lg, 1)
    assert (oracle.weights(lg, s1) == 1.0).all()
    s2, _ = oracle.select(lg, 2)
    w2 = oracle.weights(lg, s2)
    for t in range(20):
        a, b = s2[t]
        sig = 1.0 / (1.0 + math.exp(-(lg[t, a] - lg[t, b])))
        assert abs(w2[t, 0] - sig) < 1e-15 and abs(w2[t, 1] - (1 - sig)) < 1e-15
    s4, _ = oracle.select(np.full((2, 9), 0.7), 4)
    assert np.allclose(oracle.weights(np.full((2, 9), 0.7), s4), 0.25, atol=0, rtol=1e-15)


def test_weights_are_softmax_renormalised_over_set():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((30, 32)) * 4
    sets, _ = oracle.select(lg, 8)
    w = oracle.weights(lg, sets)
    p = np.exp(lg) / np.exp(lg).sum(axis=1, keepdims=True)  # full softmax first
    ps = np.take_along_axis(p, sets.astype(np.int64), axis=1)
    assert np.allclose(w, ps / ps.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    # ordering: the largest logit in the set carries the largest weight
    lsel = np.take_along_axis(lg, sets.astype(np.int64), axis=1)
    assert (np.argmax(w, axis=1) == np.argmax(lsel, axis=1)).all()


# -------------------------------------------------------------------- permute
def test_permute_equals_stable_sort():
    rng = np.random.default_rng(3)
    T, E, k = 300, 24, 3
    lg = rng.standard_normal((T, E))
    sets, _ = oracle.select(lg, k)
    counts, offsets, perm_src, pos = oracle.permute(sets, E)
    flat = sets.ravel()
    assert np.array_equal(perm_src, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(pos[perm_src], np.arange(T * k))
    assert np.array_equal(np.sort(perm_src), np.arange(T * k))
    assert counts.sum() == T * k


def test_permute_empty_and_full_experts():
    sets = np.tile(np.array([[1, 4]], np.int32), (5, 1))
    counts, offsets, perm_src, _ = oracle.permute(sets, 6)
    assert counts.tolist() == [0, 5, 0, 0, 5, 0]
    assert offsets.tolist() == [0, 0, 5, 5, 5, 10, 10]
    assert perm_src.tolist() == [0, 2, 4, 6, 8, 1, 3, 5, 7, 9]


# --------------------------------------------------------------------- logits
def test_logits_unit_vectors_and_bias():
    rng = np.random.default_rng(4)
    E, d = 6, 10
    wr = f32_to_bf16_bits(rng.standard_normal((E, d)))
    x = np.zeros((d, d), np.uint16)
    x[np.arange(d), np.arange(d)] = BF16_ONE  # token t is the unit vector e_t
    bias = rng.standard_normal(E).astype(np.float32)
    lg = oracle.logits(x, wr, bias)
    assert np.array_equal(lg, bf(wr).T + bias.astype(np.float64)[None, :])
    assert np.array_equal(oracle.logits(x, wr), bf(wr).T)


def test_logits_match_numpy_matmul():
    rng = np.random.default_rng(5)
    x = f32_to_bf16_bits(rng.standard_normal((17, 96)))
    wr = f32_to_bf16_bits(rng.standard_normal((11, 96)) / 10)
    assert np.allclose(oracle.logits(x, wr), bf(x) @ bf(wr).T, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- expert FFN
def test_ffn_scalar_closed_form():
    for xv, g, u, dn in [(1.5, 0.75, -2.0, 0.5), (-3.0, 1.25, 1.0, -1.0), (0.0, 1.0, 1.0, 1.0)]:
        x = f32_to_bf16_bits([[xv]])
        y = oracle.ffn(x, f32_to_bf16_bits([[g]]), f32_to_bf16_bits([[u]]), f32_to_bf16_bits([[dn]]))
        z = g * xv
        assert y[0, 0] == pytest.approx(dn * (z / (1 + math.exp(-z))) * (u * xv), rel=1e-15, abs=0)


def test_ffn_index_order_with_one_hot_weights():
    # d != I so a transposed operand would address different entries.
    d, I = 12, 5
    a, g, u, v = 1.5, 0.5, -1.25, 2.0
    for j0, i0, m0 in [(0, 0, 0), (11, 4, 7), (3, 2, 11)]:
        x = np.zeros((1, d), np.uint16); x[0, j0] = f32_to_bf16_bits([a])[0]
        wg = np.zeros((I, d), np.uint16); wg[i0, j0] = f32_to_bf16_bits([g])[0]
        wu = np.zeros((I, d), np.uint16); wu[i0, j0] = f32_to_bf16_bits([u])[0]
        wd = np.zeros((d, I), np.uint16); wd[m0, i0] = f32_to_bf16_bits([v])[0]
        y = oracle.ffn(x, wg, wu, wd)
        expect = np.zeros(d)
        expect[m0] = v * (g * a / (1 + math.exp(-g * a))) * (u * a)
        assert np.array_equal(y[0], expect)


def test_ffn_matches_numpy():
    rng = np.random.default_rng(6)
    n, d, I = 5, 64, 48
    x = f32_to_bf16_bits(rng.standard_normal((n, d)))
    wg = f32_to_bf16_bits(rng.standard_normal((I, d)) / 8)
    wu = f32_to_bf16_bits(rng.standard_normal((I, d)) / 8)
    wd = f32_to_bf16_bits(rng.standard_normal((d, I)) / 7)
    y = oracle.ffn(x, wg, wu, wd, nthreads=3)
    assert np.allclose(y, np_swiglu(bf(x), bf(wg), bf(wu), bf(wd)), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- whole layer
def small_layer(seed=0, T=24, d=64, E=8, k=2, I=32, bias=False):
    cfg = hi.LayerConfig("t", T=T, d=d, E=E, k=k, I=I, seed=seed)
    L = hi.host_layer(cfg)
    if bias:
        L["bias"] = hi.zipf_bias(E, seed)
    return cfg, L


def run_forward(L, k, **kw):
    return oracle.forward(L["x"], L["router"], L["bias"], L["gate"], L["up"], L["down"],
                          L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"], k, **kw)


def dense_masked_reference(L, k):
    """Independent formulation: every expert on every token (numpy), top-k by a
    lexsort on (-logit, index), softmax renormalised, masked sum."""
    x = bf(L["x"]); wr = bf(L["router"])
    lg = x @ wr.T
    if L["bias"] is not None:
        lg = lg + L["bias"].astype(np.float64)
    T, E = lg.shape
    out = np_swiglu(x, bf(L["shared"]["gate"]), bf(L["shared"]["up"]), bf(L["shared"]["down"]))
    ys = np.stack([np_swiglu(x, bf(L["gate"][e]), bf(L["up"][e]), bf(L["down"][e])) for e in range(E)])
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t]))[:k]
        p = np.exp(lg[t, order] - lg[t, order].max())
        p /= p.sum()
        out[t] += (p[:, None] * ys[order, t]).sum(axis=0)
    return out


@pytest.mark.parametrize("bias", [False, True])
def test_forward_matches_dense_masked_numpy(bias):
    cfg, L = small_layer(bias=bias)
    ref = run_forward(L, cfg.k)
    assert np.allclose(ref["out"], dense_masked_reference(L, cfg.k), rtol=1e-11, atol=1e-11)


def test_tiny_config_forward_matches_dense_masked_numpy():
    cfg = hi.CONFIGS["tiny"]
    L = hi.host_layer(cfg)
    ref = run_forward(L, cfg.k)
    assert np.allclose(ref["out"], dense_masked_reference(L, cfg.k), rtol=1e-11, atol=1e-11)
    assert np.allclose(ref["w"].sum(axis=1), 1.0, atol=1e-15)


def test_identical_experts_reduce_to_dense_swiglu():
    cfg, L = small_layer(seed=1, bias=True)
    for key in ("gate", "up", "down"):
        L[key] = np.repeat(L[key][2:3], cfg.E, axis=0)
    ref = run_forward(L, cfg.k)
    x = bf(L["x"])
    dense = np_swiglu(x, bf(L["shared"]["gate"]), bf(L["shared"]["up"]), bf(L["shared"]["down"])) + \
        np_swiglu(x, bf(L["gate"][0]), bf(L["up"][0]), bf(L["down"][0]))
    assert np.allclose(ref["out"], dense, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_leaves_shared_expert():
    cfg, L = small_layer(seed=2)
    L["down"] = np.zeros_like(L["down"])
    ref = run_forward(L, cfg.k)
    shared = oracle.ffn(L["x"], L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
    assert np.array_equal(ref["out"], shared)


def test_linear_in_routed_down_projection():
    cfg, L = small_layer(seed=3)
    base = run_forward(L, cfg.k)["out"]
    shared = oracle.ffn(L["x"], L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"])
    L2 = dict(L)
    L2["down"] = f32_to_bf16_bits(bf(L["down"]) * 2.0)  # exact in bf16
    doubled = run_forward(L2, cfg.k)["out"]
    assert np.allclose(doubled - shared, 2.0 * (base - shared), rtol=1e-12, atol=1e-13)


def test_sets_override_substitutes_routing():
    cfg, L = small_layer(seed=4)
    ref = run_forward(L, cfg.k)
    alt = ref["sets"].copy()
    alt[0] = [e for e in range(cfg.E) if e not in ref["sets"][0]][: cfg.k]
    sub = run_forward(L, cfg.k, sets_in=alt)
    assert np.array_equal(sub["out"][1:], ref["out"][1:])
    assert not np.allclose(sub["out"][0], ref["out"][0])
    assert np.array_equal(sub["sets"], alt)


def test_combine_closed_form():
    ys = np.array([[1.0, 2.0]]); yr = np.array([[[10.0, 20.0], [100.0, 200.0]]])
    w = np.array([[0.25, 0.75]])
    assert np.array_equal(oracle.combine(ys, yr, w), np.array([[1 + 2.5 + 75, 2 + 5 + 150]]))


def test_invalid_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.select(np.zeros((2, 4)), 5)
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 9]], np.int32), 4)


# --------------------------------------------------------------------- Sherry
def pack_codes(codes):
    """Independent packer for the test: 32 codes -> 5 words (160-bit LE)."""
    B = 0
    for g, c in enumerate(codes):
        B |= int(c) << (5 * g)
    return np.array([(B >> (32 * i)) & 0xFFFFFFFF for i in range(5)], np.uint32)


def expected_group(code):
    z = code & 3
    vals, nz = [], 0
    for q in range(4):
        if q == z:
            vals.append(0)
        else:
            vals.append(-1 if (code >> (2 + nz)) & 1 else 1)
            nz += 1
    return vals


def test_sherry_all_32_codes():
    words = pack_codes(range(32))
    tern, _ = oracle.sherry_decode(words[None, :])
    groups = tern.reshape(32, 4)
    patterns = set()
    for c in range(32):
        g = groups[c].tolist()
        assert g.count(0) == 1, "exactly one zero per group"
        assert g.index(0) == (c & 3)
        nonzero = [v for v in g if v != 0]
        assert nonzero == [(-1 if (c >> (2 + i)) & 1 else 1) for i in range(3)]
        patterns.add(tuple(g))
    # bijection onto the 4 * 2^3 = 32 one-zero ternary groups
    every = {p for p in itertools.product([-1, 0, 1], repeat=4) if p.count(0) == 1}
    assert patterns == every and len(every) == 32


def test_sherry_hand_worked_blocks():
    for line in open(os.path.join(GOLDEN, "sherry_blocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        left, right = line.split("|")
        words = np.array([int(w, 16) for w in left.split()], np.uint32)
        tern, _ = oracle.sherry_decode(words[None, :])
        groups = tern.reshape(32, 4)
        listed = {}
        for item in right.split():
            g, vals = item.split(":")
            listed[int(g)] = [int(v) for v in vals.split(",")]
        for g in range(32):
            if g in listed:
                assert groups[g].tolist() == listed[g], (line, g)
            elif not (words == 0xFFFFFFFF).all():
                # groups not listed decode from code 0 unless their bits are set
                code = (sum(int(w) << (32 * i) for i, w in enumerate(words)) >> (5 * g)) & 31
                assert groups[g].tolist() == expected_group(code)


def test_sherry_random_round_trip_and_scales():
    rng = np.random.default_rng(7)
    rows, cols = 6, 384
    codes = rng.integers(0, 32, size=(rows, cols // 4))
    packed = np.stack([np.concatenate([pack_codes(codes[r, b * 32:(b + 1) * 32]) for b in range(cols // 128)])
                       for r in range(rows)])
    scale = f32_to_bf16_bits(rng.uniform(0.5, 1.5, rows) / 16)
    tern, w = oracle.sherry_decode(packed, scale)
    for r in range(rows):
        for g in range(cols // 4):
            assert tern[r, 4 * g:4 * g + 4].tolist() == expected_group(int(codes[r, g]))
    # repack from the decoded values: invert expected_group
    inv = {tuple(expected_group(c)): c for c in range(32)}
    recodes = np.array([[inv[tuple(tern[r, 4 * g:4 * g + 4])] for g in range(cols // 4)] for r in range(rows)])
    assert np.array_equal(recodes, codes)
    assert np.array_equal(bf(w), bf(scale)[:, None] * tern)
    # 1.25 bits per weight: 5 words of 32 bits per 128 weights
    assert packed.nbytes * 8 == 1.25 * rows * cols


def test_sherry_ternary_gemv_equals_dense_gemv():
    rng = np.random.default_rng(8)
    packed = hi.words_u32(0, 10, 4 * 10).reshape(4, 10)
    scale = f32_to_bf16_bits(rng.uniform(0.5, 1.5, 4) / 16)
    tern, w = oracle.sherry_decode(packed, scale)
    x = rng.standard_normal(256)
    dense = bf(w) @ x
    factored = bf(scale) * (tern.astype(np.float64) @ x)
    assert np.allclose(dense, factored, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------- FP8 E4M3
def test_fp8_hand_worked_codes():
    for line in open(os.path.join(GOLDEN, "fp8_e4m3.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        code, val = line.split()
        got = oracle.fp8_decode(np.array([[int(code, 16)]], np.uint8))[0, 0]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1.0, got) == math.copysign(1.0, float(val)), code


def test_fp8_all_codes_match_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = oracle.fp8_decode(codes[None, :])[0]
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert np.flatnonzero(np.isnan(got)).tolist() == [0x7F, 0xFF]


def test_fp8_row_scales():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 256, size=(5, 16), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38  # no NaN codes
    s = np.array([0.5, -2.0, 3.0e-3, 1.0, 7.25], np.float32)
    w1 = oracle.fp8_decode(q)
    w = oracle.fp8_decode(q, s)
    assert np.array_equal(w, w1 * s.astype(np.float64)[:, None])
    assert np.array_equal(w[3], w1[3]) and np.array_equal(w[1], -2.0 * w1[1])


def test_ffn_w64_equals_ffn_on_bf16_values():
    # the fp64-weight FFN must reproduce the pinned bf16 FFN bit for bit when the
    # weights are the same values (same sums in the same order)
    rng = np.random.default_rng(12)
    n, d, I = 3, 64, 40
    x = f32_to_bf16_bits(rng.standard_normal((n, d)))
    wg = f32_to_bf16_bits(rng.standard_normal((I, d)) / 8)
    wu = f32_to_bf16_bits(rng.standard_normal((I, d)) / 8)
    wd = f32_to_bf16_bits(rng.standard_normal((d, I)) / 7)
    a = oracle.ffn(x, wg, wu, wd, nthreads=2)
    b = oracle.ffn_w64(x, bf(wg), bf(wu), bf(wd), nthreads=2)
    assert np.array_equal(a, b)
    assert not np.array_equal(oracle.ffn_w64(x, bf(wu), bf(wg), bf(wd)), a)  # gate and up are not interchangeable


@pytest.mark.parametrize("bias", [False, True])
def test_forward_w64_equals_forward_on_bf16_values(bias):
    cfg, L = small_layer(seed=3, bias=bias)
    a = run_forward(L, cfg.k)
    b = oracle.forward_w64(L["x"], L["router"], L["bias"], bf(L["gate"]), bf(L["up"]), bf(L["down"]),
                           L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"], cfg.k)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_fp8_layer_matches_dense_masked_numpy():
    # FP8 experts decoded by the oracle, then the whole layer against the
    # independent dense formulation on the same (fp64) weights
    cfg, L = small_layer(seed=4, T=16, d=64, E=6, k=2, I=32, bias=True)
    rng = np.random.default_rng(13)
    fw = {}
    for key, rows, cols in (("gate", cfg.I, cfg.d), ("up", cfg.I, cfg.d), ("down", cfg.d, cfg.I)):
        q = rng.integers(0, 256, size=(cfg.E, rows, cols), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x30
        s = (rng.random((cfg.E, rows)) * 0.05 + 0.01).astype(np.float32)
        fw[key] = np.stack([oracle.fp8_decode(q[e], s[e]) for e in range(cfg.E)])
    ref = oracle.forward_w64(L["x"], L["router"], L["bias"], fw["gate"], fw["up"], fw["down"],
                             L["shared"]["gate"], L["shared"]["up"], L["shared"]["down"], cfg.k)
    x = bf(L["x"])
    lg = x @ bf(L["router"]).T + L["bias"].astype(np.float64)
    out = np_swiglu(x, bf(L["shared"]["gate"]), bf(L["shared"]["up"]), bf(L["shared"]["down"]))
    for t in range(cfg.T):
        order = np.lexsort((np.arange(cfg.E), -lg[t]))[:cfg.k]
        p = np.exp(lg[t, order] - lg[t, order].max())
        p /= p.sum()
        for pe, e in zip(p, order):
            out[t] += pe * np_swiglu(x[t:t + 1], fw["gate"][e], fw["up"][e], fw["down"][e])[0]
    assert np.allclose(ref["out"], out, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------- sparse-attention indexer
# --------------------------------------------------- MXFP8 activations (W8A8)
def read_mx_blocks():
    blocks, cur = [], None
    for line in open(os.path.join(GOLDEN, "mxfp8_blocks.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] == "block":
            cur = {"name": parts[1], "scale": int(parts[2]), "v": np.zeros(32, np.float32),
                   "codes": np.zeros(32, np.uint8)}
            blocks.append(cur)
        else:
            i, val, code = int(parts[0]), parts[1], int(parts[2], 16)
            cur["v"][i] = np.float32(float.fromhex(val) if "0x" in val else float(val))
            cur["codes"][i] = code
    return blocks


def mx_values(codes, scales):
    """Values of MXFP8 rows from the (separately pinned) E4M3 decoder and the scale bytes."""
    v = oracle.fp8_decode(codes)
    return v * np.exp2(np.repeat(scales.astype(np.float64) - 127.0, 32, axis=-1))


def test_mx_hand_worked_blocks():
    blocks = read_mx_blocks()
    assert len(blocks) == 6
    q, sc = oracle.mx_quantize(np.stack([b["v"] for b in blocks]))
    for i, b in enumerate(blocks):
        assert sc[i, 0] == b["scale"], b["name"]
        assert np.array_equal(q[i], b["codes"]), (b["name"], q[i][:8], b["codes"][:8])


def test_mx_codes_match_torch_float8_conversion():
    # the element rounding against torch's own float -> float8_e4m3fn conversion (round to
    # nearest even, an independent implementation), below the saturation threshold; the
    # block exponent from numpy's frexp
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    rows = (rng.standard_normal((64, 96)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    rows[3, :40] = 0.0
    q, sc = oracle.mx_quantize(rows)
    blk = rows.astype(np.float64).reshape(64, 3, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127)
    assert np.array_equal(sc.astype(np.int64), e + 127)
    scaled = blk * np.exp2(-e)[:, :, None]
    ref = torch.from_numpy(scaled.reshape(64, 96).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    ok = np.abs(scaled.reshape(64, 96)) < 448.0
    assert ok.mean() > 0.95
    assert np.array_equal(q[ok], ref[ok])
    assert np.all((q[~ok] & 0x7F) == 0x7E)  # at or beyond 448: saturated


def test_mx_error_bounds_and_round_trip():
    rng = np.random.default_rng(22)
    rows = (rng.standard_normal((40, 128)) * np.exp2(rng.integers(-12, 12, (40, 1)))).astype(np.float32)
    q, sc = oracle.mx_quantize(rows)
    v = mx_values(q, sc)
    x = rows.astype(np.float64)
    e = np.repeat(sc.astype(np.float64) - 127.0, 32, axis=1)
    # each value within half a step of the E4M3 grid at its own magnitude (steps are
    # 2^(E - 3) for normals, 2^-9 in the subnormal range, in units of the block scale)
    _, ex = np.frexp(np.abs(x) * np.exp2(-e))
    E = np.maximum(ex - 1, -6)
    step = np.exp2(E - 3 + e)
    scaled = np.abs(x) * np.exp2(-e)
    sat = scaled >= 464.0  # rounds past 448: saturated (the scale rule lets amax reach 2^9)
    assert np.all(np.abs(v - x)[~sat] <= 0.5 * step[~sat] * (1 + 1e-12))
    assert np.array_equal(np.abs(v)[sat], (448.0 * np.exp2(e))[sat]) and np.all(np.sign(v[sat]) == np.sign(x[sat]))
    assert sat.any()
    assert np.all(np.abs(v) <= 448.0 * np.exp2(e))
    # the largest value of each block lands in the top binade of E4M3 (field 15)
    blk_q = q.reshape(40, 4, 32)
    top = np.take_along_axis(blk_q, np.abs(x).reshape(40, 4, 32).argmax(axis=2)[:, :, None], axis=2)
    assert np.all(((top >> 3) & 15) == 15)
    # values already on the grid are reproduced: quantizing the read-back values is exact
    q2, sc2 = oracle.mx_quantize(v.astype(np.float32))
    assert np.array_equal(q2, q) and np.array_equal(sc2, sc)
    assert np.array_equal(mx_values(q2, sc2), v)


def _fp8_expert(rng, I, d, scale=0.05):
    def mat(rows, cols):
        q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x30
        s = (rng.random(rows) * scale + scale / 4).astype(np.float32)
        return oracle.fp8_decode(q, s)
    return mat(I, d), mat(I, d), mat(d, I)


def test_ffn_w8a8_composition():
    # the FFN's steps in their order, composed in numpy from the pinned quantizer: x
    # quantized along d, the hidden rows rounded to fp32 and quantized along I, fp64 sums
    rng = np.random.default_rng(23)
    n, d, I = 3, 96, 64
    x = f32_to_bf16_bits(rng.standard_normal((n, d)))
    wg, wu, wd = _fp8_expert(rng, I, d)
    got = oracle.ffn_w8a8(x, wg, wu, wd, nthreads=2)
    xq = mx_values(*oracle.mx_quantize(bf(x).astype(np.float32)))
    g, u = xq @ wg.T, xq @ wu.T
    h = (np_silu(g) * u).astype(np.float32)
    hq = mx_values(*oracle.mx_quantize(h))
    assert np.allclose(got, hq @ wd.T, rtol=1e-12, atol=1e-12)
    # the quantization is there: it differs from the FP8-weight FFN on bf16 activations, by
    # about the E4M3 rounding (relative 2^-4 per value)
    ref = oracle.ffn_w64(x, wg, wu, wd, nthreads=2)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert 1e-4 < err < 0.1
    # gate and up are not interchangeable, and the down input is the hidden row
    assert not np.allclose(oracle.ffn_w8a8(x, wu, wg, wd), got)


def test_ffn_w8a8_hidden_rows_and_substitution():
    rng = np.random.default_rng(25)
    n, d, I = 2, 64, 96
    x = f32_to_bf16_bits(rng.standard_normal((n, d)))
    wg, wu, wd = _fp8_expert(rng, I, d)
    y0 = oracle.ffn_w8a8(x, wg, wu, wd)
    y, h32 = oracle.ffn_w8a8_ex(x, wg, wu, wd, want_hidden=True)
    assert np.array_equal(y, y0) and h32.dtype == np.float32
    # the hidden rows are fp32 of the composition's silu(g) * u
    xq = mx_values(*oracle.mx_quantize(bf(x).astype(np.float32)))
    g, u = xq @ wg.T, xq @ wu.T
    assert np.allclose(h32, (np_silu(g) * u).astype(np.float32), rtol=1e-6, atol=1e-30)
    # substituting the oracle's own codes changes nothing; one code one step up moves the
    # output by that column of W_down times the step, exactly as the values say
    hq, hs = oracle.mx_quantize(h32)
    assert np.array_equal(oracle.ffn_w8a8_ex(x, wg, wu, wd, hq=hq, hs=hs), y)
    i = int(np.argmax(np.abs(h32[0]) < 400 * np.exp2(hs[0, 0] - 127.0)))  # a non-saturated code in block 0
    hq2 = hq.copy()
    hq2[0, i] = hq[0, i] + 1 if hq[0, i] & 0x7F < 0x7E else hq[0, i] - 1
    y2 = oracle.ffn_w8a8_ex(x, wg, wu, wd, hq=hq2, hs=hs)
    dv = (mx_values(hq2, hs) - mx_values(hq, hs))[0, i]
    assert dv != 0 and np.allclose(y2[0] - y[0], wd[:, i] * dv, rtol=1e-6, atol=1e-12 * np.abs(y).max())
    assert np.array_equal(y2[1], y[1])


def test_forward_w8a8_matches_dense_masked_numpy():
    cfg, L = small_layer(seed=5, T=12, d=64, E=6, k=2, I=32, bias=True)
    rng = np.random.default_rng(24)
    exp = [_fp8_expert(rng, cfg.I, cfg.d) for _ in range(cfg.E)]
    fg, fu, fd = (np.stack([e[i] for e in exp]) for i in range(3))
    ref = oracle.forward_w8a8(L["x"], L["router"], L["bias"], fg, fu, fd, L["shared"]["gate"],
                              L["shared"]["up"], L["shared"]["down"], cfg.k)
    x = bf(L["x"])
    lg = x @ bf(L["router"]).T + L["bias"].astype(np.float64)
    out = np_swiglu(x, bf(L["shared"]["gate"]), bf(L["shared"]["up"]), bf(L["shared"]["down"]))
    xq = mx_values(*oracle.mx_quantize(x.astype(np.float32)))
    for t in range(cfg.T):
        order = np.lexsort((np.arange(cfg.E), -lg[t]))[:cfg.k]
        p = np.exp(lg[t, order] - lg[t, order].max())
        p /= p.sum()
        for pe, e in zip(p, order):
            h = (np_silu(xq[t] @ fg[e].T) * (xq[t] @ fu[e].T)).astype(np.float32)
            out[t] += pe * (mx_values(*oracle.mx_quantize(h[None]))[0] @ fd[e].T)
    assert np.allclose(ref["out"], out, rtol=1e-11, atol=1e-11)
    # routing is that of the other formats
    w64 = oracle.forward_w64(L["x"], L["router"], L["bias"], fg, fu, fd, L["shared"]["gate"],
                             L["shared"]["up"], L["shared"]["down"], cfg.k)
    assert np.array_equal(ref["sets"], w64["sets"]) and np.array_equal(ref["w"], w64["w"])


def test_indexer_hand_worked():
    # H=2, D=2: q0=(1,2), q1=(-1,1), w=(0.5,2); key (3,-1): dots 1, -4 -> 0.5*1 + 2*0 = 0.5;
    # key (0,1): dots 2, 1 -> 0.5*2 + 2*1 = 3
    q = f32_to_bf16_bits(np.array([[[1.0, 2.0], [-1.0, 1.0]]]))
    w = np.array([[0.5, 2.0]], np.float32)
    keys = f32_to_bf16_bits(np.array([[[3.0, -1.0], [0.0, 1.0]]]))
    assert oracle.indexer_scores(q, w, keys).tolist() == [[0.5, 3.0]]


def test_indexer_unit_keys_read_the_query_through_relu():
    rng = np.random.default_rng(21)
    D = 16
    qv = rng.standard_normal(D)
    q = f32_to_bf16_bits(qv[None, None, :])
    keys = f32_to_bf16_bits(np.eye(D)[None])          # key s = e_s
    got = oracle.indexer_scores(q, np.ones((1, 1), np.float32), keys)[0]
    assert np.array_equal(got, np.maximum(bf(q)[0, 0], 0.0))
    assert (got[bf(q)[0, 0] < 0] == 0).all() and (got > 0).sum() == (bf(q)[0, 0] > 0).sum()


def test_indexer_heads_weights_and_batches():
    rng = np.random.default_rng(22)
    B, H, D, S = 3, 4, 32, 40
    q = f32_to_bf16_bits(rng.standard_normal((B, H, D)))
    keys = f32_to_bf16_bits(rng.standard_normal((B, S, D)))
    w = rng.random((B, H)).astype(np.float32)
    base = oracle.indexer_scores(q, w, keys)
    perm = np.array([2, 0, 3, 1])                       # heads are a sum: any order
    assert np.allclose(oracle.indexer_scores(q[:, perm], w[:, perm], keys), base, rtol=1e-14, atol=1e-14)
    per_head = [oracle.indexer_scores(q[:, h:h + 1], np.ones((B, 1), np.float32), keys) for h in range(H)]
    assert np.allclose(sum(w[:, h:h + 1].astype(np.float64) * per_head[h] for h in range(H)), base, rtol=1e-13)
    # each batch row scores only its own keys
    one = oracle.indexer_scores(q[1:2], w[1:2], keys[1:2])
    assert np.array_equal(one[0], base[1])
    assert not np.allclose(oracle.indexer_scores(q[1:2], w[1:2], keys[0:1])[0], base[1])


@pytest.mark.parametrize("S,K", [(50, 8), (300, 64), (20, 32), (64, 64)])
def test_topk_indices_brute_force(S, K):
    rng = np.random.default_rng(S + K)
    sc = np.round(rng.standard_normal((4, S)) * 4) / 4  # many ties
    idx, kth, margin = oracle.topk_indices(sc, K)
    for b in range(4):
        order = np.lexsort((np.arange(S), -sc[b]))      # score descending, index ascending
        want = np.sort(order[:min(K, S)])
        assert np.array_equal(idx[b], want)
        assert kth[b] == sc[b, order[min(K, S) - 1]]
        assert (margin[b] == np.inf) if S <= K else (margin[b] == sc[b, order[K - 1]] - sc[b, order[K]])


def test_topk_indices_all_equal_take_lowest():
    idx, _, margin = oracle.topk_indices(np.zeros((2, 100)), 10)
    assert (idx == np.arange(10)).all() and (margin == 0).all()

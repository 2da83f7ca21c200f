"""CPU checks of the seeded input generator (hy_inputs): it must be the published
Philox4x32-10, its Gaussians must have the stated moments, and any sub-range
must regenerate the same values (the oracle relies on regenerating one expert
at a time)."""
import ctypes
import math

import numpy as np
import pytest

import hy_inputs as hi


def philox(ctr, key):
    L = hi.host_lib()
    out = (ctypes.c_uint32 * 4)()
    L.hy_gen_philox4x32_10((ctypes.c_uint32 * 4)(*ctr), (ctypes.c_uint32 * 2)(*key), out)
    return list(out)


@pytest.mark.parametrize("ctr,key,expect", [
    # Known-answer vectors published with Random123 (Salmon et al., SC'11).
    ((0, 0, 0, 0), (0, 0), [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, expect):
    assert philox(ctr, key) == expect


def test_elementary_functions_accuracy():
    L = hi.host_lib()
    rng = np.random.default_rng(0)
    for u in np.concatenate([rng.random(3000), [2.0 ** -53, 0.5, 1.0 - 2.0 ** -53, 0.70710678]]):
        if u <= 0:
            continue
        ref = math.log(u)
        assert abs(L.hy_gen_ln(u) - ref) <= 4e-16 * max(1.0, abs(ref))
    for x in np.concatenate([rng.random(3000) * 75.0 + 1e-12, [2.0 ** -53, 1.0, 74.8]]):
        assert abs(L.hy_gen_sqrt(x) - math.sqrt(x)) <= 4e-16 * math.sqrt(x)
    c, s = ctypes.c_double(), ctypes.c_double()
    for a in np.concatenate([rng.random(3000), [0.0, 0.125, 0.25, 0.5, 0.75, 0.999999]]):
        L.hy_gen_cossin_turn(a, ctypes.byref(c), ctypes.byref(s))
        assert abs(c.value - math.cos(2 * math.pi * a)) < 2e-15
        assert abs(s.value - math.sin(2 * math.pi * a)) < 2e-15


def test_gaussian_moments():
    n = 4_000_000
    z = hi.bf16_to_f32(hi.gauss_bf16(0, 99, n, 1.0)).astype(np.float64)
    assert abs(z.mean()) < 5.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5e-3
    assert abs((z ** 4).mean() - 3.0) < 0.05
    # Tail mass beyond 3 sigma: 2(1 - Phi(3)) = 0.0026998
    assert abs((np.abs(z) > 3).mean() - 0.0026998) < 3e-4
    s = hi.bf16_to_f32(hi.gauss_bf16(0, 98, 200_000, 0.125)).astype(np.float64)
    assert abs(s.std() - 0.125) < 2e-3


def test_subrange_and_thread_independence():
    full = hi.gauss_bf16(7, 3, 100_001, 0.5)
    for start, cnt in [(0, 1), (1, 1), (12345, 777), (99_000, 1001)]:
        assert np.array_equal(hi.gauss_bf16(7, 3, cnt, 0.5, start=start), full[start:start + cnt])
    L = hi.host_lib()
    one = np.empty(50_001, np.uint16)
    L.hy_gen_gauss_bf16(7, 3, 0, 50_001, 0.5, one.ctypes.data, 1)
    assert np.array_equal(one, full[:50_001])
    w = hi.words_u32(7, 11, 4099)
    assert np.array_equal(hi.words_u32(7, 11, 100, start=3999), w[3999:])


def test_streams_and_seeds_differ():
    a = hi.gauss_bf16(0, 1, 1000, 1.0)
    assert not np.array_equal(a, hi.gauss_bf16(0, 2, 1000, 1.0))
    assert not np.array_equal(a, hi.gauss_bf16(1, 1, 1000, 1.0))


def test_uniform_scales_range():
    u = hi.bf16_to_f32(hi.uniform_bf16(0, 13, 100_000, 0.5, 1.0)).astype(np.float64)
    assert u.min() >= 0.5 and u.max() <= 1.5
    assert abs(u.mean() - 1.0) < 0.01


def test_random_words_give_uniform_codes():
    # Every 5-bit field of uniformly random words is uniform over 32 values.
    w = hi.words_u32(0, 10, 5 * 4000).reshape(-1, 5)
    B = [sum(int(x) << (32 * i) for i, x in enumerate(row)) for row in w[:2000]]
    codes = np.array([(b >> (5 * g)) & 31 for b in B for g in range(32)])
    hist = np.bincount(codes, minlength=32)
    assert hist.min() > 0.8 * codes.size / 32 and hist.max() < 1.2 * codes.size / 32


def test_zipf_bias_is_a_permutation_of_log_ranks():
    b = hi.zipf_bias(256, 0, 1.2)
    ranks = np.exp(-b.astype(np.float64) / 1.2)
    assert np.allclose(np.sort(ranks), np.arange(1, 257), rtol=1e-5)
    assert np.array_equal(b, hi.zipf_bias(256, 0, 1.2))


def test_layer_shapes():
    cfg = hi.CONFIGS["tiny"]
    L = hi.host_layer(cfg)
    assert L["x"].shape == (64, 256) and L["router"].shape == (16, 256)
    assert L["gate"].shape == (16, 128, 256) and L["down"].shape == (16, 256, 128)
    assert L["shared"]["down"].shape == (256, 128)
    e3 = hi.host_expert(cfg, 3)
    assert np.array_equal(e3["gate"], L["gate"][3]) and np.array_equal(e3["down"], L["down"][3])
    cfg5 = hi.LayerConfig("t5", T=4, d=256, E=4, k=2, I=128, ternary=True)
    q = hi.host_layer(cfg5)
    assert q["qgate"].shape == (4, 128, 10) and q["qdown"].shape == (4, 256, 5)
    assert q["sdown"].shape == (4, 256)

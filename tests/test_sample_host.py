"""Host logic of the full-size parity sample (tests/parity.py: m_tiles, tile_sample),
on the CPU."""
import numpy as np

import hy_inputs as hi
import oracle
from parity import m_tiles, tile_sample


def test_tile_sample_covers_schedule():
    # host logic of the sample, on a synthetic routing with a hot expert and two-tile experts
    cfg = hi.LayerConfig("t", T=4096, d=256, E=16, k=2, I=128)
    rng = np.random.default_rng(1)
    sets = np.stack([np.sort(rng.choice(16, 2, replace=False, p=np.r_[0.5, np.full(15, 0.5 / 15)]))
                     for _ in range(cfg.T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.permute(sets, cfg.E)
    g = {"counts": counts, "offsets": offsets, "perm_src": perm}
    tokens, why = tile_sample(cfg, g)
    hot = int(np.argmax(counts))
    hot_rows = perm[offsets[hot]:offsets[hot + 1]] // cfg.k
    for m0, rows in m_tiles(int(counts[hot])):
        assert hot_rows[m0] in tokens and hot_rows[m0 + rows - 1] in tokens
    assert cfg.T - 1 in tokens and len(tokens) >= 64


def test_m_tiles_match_library_rule():
    assert m_tiles(256) == [(0, 256)]
    assert m_tiles(257) == [(0, 160), (160, 97)]
    assert m_tiles(4000) == [(i * 256, 256) for i in range(15)] + [(3840, 160)]
    assert m_tiles(1) == [(0, 1)]
    assert m_tiles(0) == []


def test_hidden_row_admissibility_rule():
    # the W8A8 hidden-row check (tests/parity.py): the oracle's own codes pass; the
    # neighbouring code of a value sitting on a rounding midpoint passes as one
    # substitution; a neighbouring code elsewhere, or a wrong block scale, fails
    import pytest
    from parity import check_hidden_rows
    rng = np.random.default_rng(3)
    h = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    h[0, 5] = 0.0
    q, s = oracle.mx_quantize(h)
    assert check_hidden_rows(h, q, s) == (0, 0)
    # place h[1, 3] exactly on the midpoint between two E4M3 neighbours of its block
    blk_scale = 2.0 ** (int(s[1, 0]) - 127)
    h2 = h.copy()
    h2[1, 3] = np.float32(68.0 * blk_scale)  # the grid steps by 8 in [64, 128): 68 is the midpoint of 64 and 72
    q2, s2 = oracle.mx_quantize(h2)
    alt = q2.copy()
    alt[1, 3] = q2[1, 3] ^ 1  # the other neighbour (64 <-> 72 differ in the last mantissa bit)
    assert check_hidden_rows(h2, alt, s2) == (1, 0)
    # a neighbouring code of a value far from any midpoint is not admissible
    far = q.copy()
    i = int(np.argmax(np.abs(h[2, :32])))  # the block maximum sits well inside its interval or saturates
    far[2, (i + 1) % 32] ^= 0x04
    with pytest.raises(AssertionError):
        check_hidden_rows(h, far, s)
    # a block scale off by a factor of two is not admissible
    bad = s.copy()
    bad[3, 1] += 1
    with pytest.raises(AssertionError):
        check_hidden_rows(h, q, bad)

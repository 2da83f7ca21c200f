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

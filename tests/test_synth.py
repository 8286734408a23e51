"""The seeded input generator: properties the parity tests rely on."""
from __future__ import annotations

import numpy as np

from compressed_kv_cache_amd import synth


def test_residual_positions_distinct_in_range_and_unsorted():
    """Residual positions are distinct values in 1..255 per (slot, KV head), drawn
    in a seeded random order (the decode takes them in any order), so the GPU
    parity tests run positions that are not ascending."""
    wl = synth.make_config(1)
    pos = wl.layers[0].resid_pos.astype(np.int64)          # [slots][Hkv][R]
    assert pos.min() >= 1 and pos.max() <= 255
    flat = pos.reshape(-1, pos.shape[-1])
    assert all(len(set(row)) == len(row) for row in flat)
    ascending = np.all(np.diff(flat, axis=-1) > 0, axis=-1)
    assert not ascending.any()

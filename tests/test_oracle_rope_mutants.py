"""Planted mistakes in the un-rotated pools' oracle (on the CPU): each one must
be rejected by the parity checker's output bars when compared with the true
oracle, so that the GPU parity tests would catch the same mistake in the
kernels.  CPU only."""
import numpy as np
import pytest

import oracle
import parity
from oracle import dkv_oracle as D
from compressed_kv_cache_amd import synth

TRUE_ROPE = D.rope
TRUE_ROWS = D.block_rows


def _interleaved(x, pos, base):
    X = np.atleast_2d(np.asarray(x, np.float64))
    h = X.shape[1] // 2
    ang = np.asarray(pos, np.float64).reshape(-1)[:, None] * D.rope_theta(base, X.shape[1])[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = X[:, 0::2], X[:, 1::2]
    out = np.empty_like(X)
    out[:, 0::2], out[:, 1::2] = a * c - b * s, b * c + a * s
    return out


def _rows_residuals_unrotated(pool, slot, h):
    K, V = D.reconstruct_block(**D._slot_entry(pool, slot, h))
    Kr = TRUE_ROPE(K, int(pool["slot_pos"][slot]) + np.arange(D.BLOCK_SIZE), float(pool["rope_base"]))
    pos = np.asarray(pool["resid_pos"][slot, h], np.int64)
    Kr[pos] = K[pos]
    return Kr, V


def _rows_anchor_unrotated(pool, slot, h):
    K, V = TRUE_ROWS(pool, slot, h)
    K[0] = np.asarray(pool["anchor_k"][slot, h], np.float64)
    return K, V


MUTANTS = {
    "positions_off_by_one": ("rope", lambda x, pos, base: TRUE_ROPE(x, np.asarray(pos) + 1, base)),
    "interleaved_pairs": ("rope", _interleaved),
    "angle_sign_flipped": ("rope", lambda x, pos, base: TRUE_ROPE(x, -np.asarray(pos), base)),
    "base_1e4_for_1e6": ("rope", lambda x, pos, base: TRUE_ROPE(x, pos, 1e4)),
    "residual_rows_unrotated": ("block_rows", _rows_residuals_unrotated),
    "anchor_unrotated": ("block_rows", _rows_anchor_unrotated),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_checker_rejects_rotation_mistakes(monkeypatch, name):
    wl = synth.make_workload("mut", seed=71, batch=2, n_q_heads=4, n_kv_heads=2, window=16,
                             n_blocks=[6, 9], ranks=[16], n_resid=40, top_k=4, sigma0=2.0,
                             rope_base=synth.ROPE_BASE)
    lay = wl.layers[0]
    args = (lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len,
            wl.n_kv_heads, wl.top_k, wl.scale)
    ro, rl, idx = oracle.decode(*args)
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(D, attr, fn)
    mo, ml, _ = oracle.decode(*args, idx=idx)
    c = parity.check_outputs(mo.astype(np.float16), ml.astype(np.float32), ro, rl)
    assert not c.ok, f"{name}: max|d out| {c.max_out:.2e}, max|d lse| {c.max_lse:.2e} within the bars"


def test_control_passes():
    wl = synth.make_workload("mut", seed=71, batch=2, n_q_heads=4, n_kv_heads=2, window=16,
                             n_blocks=[6, 9], ranks=[16], n_resid=40, top_k=4, sigma0=2.0,
                             rope_base=synth.ROPE_BASE)
    lay = wl.layers[0]
    ro, rl, idx = oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len,
                                wl.n_kv_heads, wl.top_k, wl.scale)
    c = parity.check_outputs(ro.astype(np.float16), rl.astype(np.float32), ro, rl)
    assert c.ok, c.message

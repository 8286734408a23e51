"""Pins of the oracle's un-rotated pools (keys rotated to their absolute
positions at read) against things other than its own formulas: textbook values
of cos and sin, the complex-number form of the rotary embedding, its
relative-position and norm invariants, and the (separately pinned) rotated-pool
decode on keys rotated beforehand.  CPU only."""
import numpy as np
import pytest

import oracle
from compressed_kv_cache_amd import synth

COS1, SIN1 = 0.5403023058681398, 0.8414709848078965   # cos(1 rad), sin(1 rad)


def _unit(j, d=128):
    e = np.zeros(d)
    e[j] = 1.0
    return e


def _rope_complex(x, pos, base):
    """The rotary embedding as complex multiplication: z_j = x_j + i x_{j+64}
    is multiplied by exp(i pos theta_j)."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    h = x.shape[1] // 2
    theta = np.array([base ** (-j / h) for j in range(h)])
    z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.outer(np.asarray(pos, np.float64), theta))
    return np.hstack([z.real, z.imag])


def test_frequencies_closed_form():
    th = oracle.rope_theta(10000.0, 128)
    assert th[0] == 1.0
    assert abs(th[32] - 0.01) < 1e-17                    # 10000^(-1/2)
    assert abs(th[16] - 0.1) < 1e-16                     # 10000^(-1/4)
    assert np.all(np.diff(th) < 0) and th.shape == (64,)


def test_rotation_textbook_values():
    base = 10000.0
    # dimension 0 at position 1 turns by 1 rad into dimension 64
    r = oracle.rope(_unit(0), [1], base)[0]
    assert abs(r[0] - COS1) < 1e-15 and abs(r[64] - SIN1) < 1e-15
    assert np.count_nonzero(np.abs(r) > 1e-15) == 2
    # dimension 64 at position 1: (-sin, cos) in (0, 64)
    r = oracle.rope(_unit(64), [1], base)[0]
    assert abs(r[0] + SIN1) < 1e-15 and abs(r[64] - COS1) < 1e-15
    # dimension 32 (theta = 0.01) at position 100 also turns by 1 rad
    r = oracle.rope(_unit(32), [100], base)[0]
    assert abs(r[32] - COS1) < 1e-13 and abs(r[96] - SIN1) < 1e-13
    # position 0 is the identity
    x = np.random.default_rng(0).standard_normal((3, 128))
    assert np.array_equal(oracle.rope(x, [0, 0, 0], base), x)


@pytest.mark.parametrize("base", [10000.0, 1e6])
def test_matches_complex_form_at_large_positions(base):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 128))
    pos = np.array([0, 1, 255, 4096, 64511, 131071])
    np.testing.assert_allclose(oracle.rope(x, pos, base), _rope_complex(x, pos, base), atol=1e-9)


def test_relative_position_and_norm():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in ((7, 3), (70000, 65000), (12, 300)):
        a = oracle.rope(q, [m], 1e6)[0] @ oracle.rope(k, [n], 1e6)[0]
        b = oracle.rope(q, [m - n], 1e6)[0] @ k
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    x = rng.standard_normal((4, 128))
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(x, [5, 50, 500, 50000], 1e6), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-13)


def _small(n_resid, seed, **kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, window=20, n_blocks=[3, 5], ranks=[12],
                top_k=3, sigma0=2.0, win_len=[20, 9])
    base.update(kw)
    return synth.make_workload("rope", seed=seed, n_resid=n_resid, rope_base=1e6, **base)


def test_all_residual_block_equals_rotated_pool_on_rotated_keys():
    # every position but the anchor is a residual row: the un-rotated pool's
    # decode equals the rotated-pool decode of a pool whose anchor and residual
    # keys were rotated beforehand (anchor at the block's position, residual
    # row t at the block's position + resid_pos[t])
    wl = _small(255, 11)
    lay = wl.layers[0]
    pu = lay.pool()
    pr = {k: v for k, v in pu.items() if k not in ("rope_base", "slot_pos")}
    ak = np.asarray(lay.anchor_k, np.float64).copy()
    rk = np.asarray(lay.resid_k, np.float64).copy()
    for s in range(wl.n_slots):
        p0 = int(lay.slot_pos[s])
        for h in range(wl.n_kv_heads):
            ak[s, h] = _rope_complex(ak[s, h], [p0], 1e6)[0]
            rk[s, h] = _rope_complex(rk[s, h], p0 + lay.resid_pos[s, h].astype(np.int64), 1e6)
    pr["anchor_k"], pr["resid_k"] = ak, rk
    idx = np.array([[[0, 2, -1], [1, 2, -1]], [[0, 3, 4], [4, -1, -1]]])
    args = (lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len, wl.n_kv_heads,
            wl.top_k, wl.scale)
    ou, lu, _ = oracle.decode(pu, *args, idx=idx)
    orr, lr, _ = oracle.decode(pr, *args, idx=idx)
    np.testing.assert_allclose(ou, orr, atol=1e-12)
    np.testing.assert_allclose(lu, lr, atol=1e-12)


def test_lowrank_rows_rotated_to_their_positions():
    # no residual rows: decode equals plain softmax attention over the
    # reconstructed rows, each rotated (complex form) to block position + i
    wl = _small(0, 12)
    lay = wl.layers[0]
    idx = np.array([[[1, 2, -1], [0, -1, -1]], [[2, 4, 1], [3, -1, -1]]])
    out, lse, _ = oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                                wl.win_len, wl.n_kv_heads, wl.top_k, wl.scale, idx=idx)
    G = wl.group
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            Ks, Vs = [], []
            for j in idx[b, h]:
                if j < 0:
                    continue
                s = int(wl.block_table[b, j])
                assert lay.slot_pos[s] == 256 * j
                a_k = lay.anchor_k[s, h].astype(np.float64)
                a_v = lay.anchor_v[s, h].astype(np.float64)
                U = lay.u[s, h].astype(np.float64)
                K = np.vstack([a_k, a_k + U @ lay.vk[s, h].astype(np.float64)])
                V = np.vstack([a_v, a_v + U @ lay.vv[s, h].astype(np.float64)])
                Ks.append(_rope_complex(K, 256 * j + np.arange(256), 1e6))
                Vs.append(V)
            w = int(wl.win_len[b])
            Ks.append(lay.win_k[b, h, :w].astype(np.float64))      # the window arrives rotated
            Vs.append(lay.win_v[b, h, :w].astype(np.float64))
            K, V = np.vstack(Ks), np.vstack(Vs)
            for g in range(G):
                z = wl.scale * (K @ lay.q[b, h * G + g].astype(np.float64))
                p = np.exp(z - z.max())
                np.testing.assert_allclose(out[b, h * G + g], p @ V / p.sum(), atol=1e-12)
                assert abs(lse[b, h * G + g] - (z.max() + np.log(p.sum()))) < 1e-12


def test_route_key_is_mean_of_rotated_reconstructed_keys():
    wl = _small(16, 13)
    lay = wl.layers[0]
    for s in range(wl.n_slots):
        for h in range(wl.n_kv_heads):
            a_k = lay.anchor_k[s, h].astype(np.float64)
            K = a_k + lay.u[s, h].astype(np.float64) @ lay.vk[s, h].astype(np.float64)
            want = _rope_complex(K, int(lay.slot_pos[s]) + np.arange(1, 256), 1e6).mean(axis=0)
            got = oracle.block_route_key(lay.pool(), s, h)
            np.testing.assert_allclose(got, want, atol=1e-12)
    # the routing ranks blocks by q_bar . key, lowest index on ties
    idx, scores, keys = oracle.route_batch(lay.pool(), lay.q, wl.block_table, wl.n_blocks,
                                           wl.n_kv_heads, 2)
    qbar = lay.q[1, 0:2].astype(np.float64).mean(axis=0)
    sc = keys[(1, 0)] @ qbar
    assert list(idx[1, 0]) == sorted(np.argsort(-sc, kind="stable")[:2].tolist())


def test_block_partials_merge_to_the_block():
    wl = _small(40, 14)
    lay = wl.layers[0]
    pool = lay.pool()
    q = lay.q[0, 0:2]
    for s in (0, 3, 7):
        (lo, ll), (eo, el) = oracle.block_partials(pool, s, 1, q, wl.scale)
        mo, ml = oracle.lse_merge([lo, eo], [ll, el])
        K, V = oracle.block_rows(pool, s, 1)
        fo, fl = oracle.attend(q, K, V, wl.scale)
        np.testing.assert_allclose(mo, fo, atol=1e-12)
        np.testing.assert_allclose(ml, fl, atol=1e-12)

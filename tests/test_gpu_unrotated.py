"""GPU parity of un-rotated pools (keys stored before the rotary embedding and
rotated to their absolute positions at read) against the fp64 oracle, through
the C ABI: routing keys, routing, per-part partials, the fused decode, and the
layer-batched launch.  Same bars as the rotated pools."""
from __future__ import annotations

import numpy as np
import pytest

from compressed_kv_cache_amd import synth
import oracle
import parity
from test_gpu_parity import (DEV, _all_blocks_idx, _oracle_check, _run_layers, check_decode, lib,  # noqa: F401
                             say, upload)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _u(cfg, layers=None):
    return synth.make_config(cfg, layers=layers, variant="U")


@pytest.mark.parametrize("cfg", [0, 1])
def test_route_keys_unrotated(lib, cfg):
    wl = _u(cfg)
    say(f"[route_keys U] {wl.name}")
    pool, _ = upload(lib, wl)
    got = pool.route_key.cpu().numpy().astype(np.float64)
    P = wl.layers[0].pool()
    worst = 0.0
    for s in range(got.shape[0]):
        for h in range(got.shape[1]):
            ref = oracle.block_route_key(P, s, h)
            worst = max(worst, float(np.abs(got[s, h] - ref).max() / (np.abs(ref).max() + 1.0)))
    say(f"   max rel err {worst:.2e}")
    assert worst < 1e-5


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_route_topk_unrotated(lib, cfg):
    wl = _u(cfg)
    say(f"[route_topk U] {wl.name}")
    pool, batch = upload(lib, wl)
    idx = lib.route_topk(pool, batch, wl.top_k)
    torch.cuda.synchronize()
    _, scores, keys = oracle.route_batch(wl.layers[0].pool(), wl.layers[0].q, wl.block_table, wl.n_blocks,
                                         wl.n_kv_heads, wl.top_k)
    rc = parity.check_routing(idx.cpu().numpy(), scores, keys, wl.layers[0].q, wl.n_kv_heads, wl.top_k)
    say(f"   near-ties {rc.near_ties}")
    assert rc.ok, rc.message


@pytest.mark.parametrize("cfg", [0, 1])
def test_block_partials_unrotated(lib, cfg):
    wl = _u(cfg)
    say(f"[block partials U] {wl.name}")
    pool, batch = upload(lib, wl)
    idx = _all_blocks_idx(wl)
    K = idx.shape[-1]
    gi = torch.from_numpy(idx).to(DEV)
    lo, ll = lib.lowrank_attn(pool, batch, gi, K, wl.scale)
    eo, el = lib.exact_attn(pool, batch, gi, K, 0, wl.scale)
    torch.cuda.synchronize()
    lo, ll, eo, el = (t.cpu().numpy() for t in (lo, ll, eo, el))
    lay = wl.layers[0]
    G = wl.group
    ref = [np.zeros_like(x, dtype=np.float64) for x in (lo, ll, eo, el)]
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            for k in range(K):
                slot = int(wl.block_table[b, idx[b, h, k]])
                (o1, l1), (o2, l2) = oracle.block_partials(lay.pool(), slot, h, lay.q[b, h * G:(h + 1) * G],
                                                          wl.scale)
                rows = slice(b * wl.n_q_heads + h * G, b * wl.n_q_heads + (h + 1) * G)
                ref[0][rows, k], ref[1][rows, k], ref[2][rows, k], ref[3][rows, k] = o1, l1, o2, l2
    c1 = parity.check_partials(lo, ll, ref[0], ref[1])
    c2 = parity.check_partials(eo, el, ref[2], ref[3])
    say(f"   low-rank: rel {c1.rel_l2:.2e} lse {c1.max_lse:.2e}; residual: rel {c2.rel_l2:.2e} "
        f"lse {c2.max_lse:.2e}")
    assert c1.ok, c1.message
    assert c2.ok, c2.message


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_decode_unrotated(lib, cfg):
    check_decode(lib, _u(cfg), label="U")


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_decode_unrotated_stack_layers(lib, layer):
    """The 64k batch-4 stack read as un-rotated pools (positions up to 64511),
    one layer of each rank and the last layer, in the per-layer launch."""
    wl = _u(2, layers=[0, 9, 19, 27])
    check_decode(lib, wl, layer=layer, label=f"U rank {wl.layers[layer].rank}")


EDGE_U = {
    "rank1_R0": dict(ranks=[1], n_resid=0),
    "rank7": dict(ranks=[7]),
    "rank64": dict(ranks=[64], n_resid=4),
    "rank15_R255": dict(ranks=[15], n_resid=255),
    "group16": dict(n_q_heads=16, n_kv_heads=1),
    "window_only": dict(top_k=0),
    "permuted_pool": dict(permute_slots=True),
    "empty_sequence": dict(n_blocks=[3, 0, 5, 2], win_len=[64, 0, 64, 64]),
}


@pytest.mark.parametrize("case", sorted(EDGE_U))
def test_decode_unrotated_edge_cases(lib, case):
    kw = dict(seed=500 + len(case), batch=4, n_q_heads=6, n_kv_heads=2, window=64,
              n_blocks=[5, 3, 6, 4], ranks=[12], n_resid=20, top_k=3, sigma0=2.0)
    kw.update(EDGE_U[case])
    wl = synth.make_workload("U_" + case, rope_base=synth.ROPE_BASE, **kw)
    check_decode(lib, wl, label=case)


def test_decode_unrotated_far_positions(lib):
    """Blocks placed near the largest supported positions (2^24 - 256): the
    angle reduction keeps the rotation exact to fp32 rounding there too."""
    wl = synth.make_workload("U_far", seed=520, batch=2, n_q_heads=4, n_kv_heads=2, window=32,
                             n_blocks=[4, 6], ranks=[20], n_resid=16, top_k=3, sigma0=2.0,
                             rope_base=10000.0)
    for lay in wl.layers:
        lay.slot_pos = lay.slot_pos + np.int32((1 << 24) - 256 * 8)
    check_decode(lib, wl, label="far")


def test_decode_layers_unrotated(lib):
    """Four layers of the un-rotated 64k batch-4 stack in one layer-batched
    launch: routing equals the per-layer launch's and outputs match the oracle."""
    wl = _u(2, layers=[0, 9, 19, 27])
    say("[decode layers U] stack64k layers 0, 9, 19, 27")
    pools, batches = [], []
    for l in range(4):
        p_, b_ = upload(lib, wl, l)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    assert run.plan.unrotated == 1
    res = _run_layers(lib, run, reps=2)
    for l in range(4):
        _, _, i1 = lib.decode(pools[l], batches[l], wl.top_k, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(wl, wl.layers[l], *res[l], wl.top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


# ---------------------------------------------------------------------------
# Shared basis (blocks of an un-rotated pool reading one V_K, V_V entry)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,group", [(0, 2), (1, 2), (1, 4), (3, 3)])
def test_decode_shared_basis(lib, cfg, group):
    wl = synth.set_shared_basis(_u(cfg), group)
    pool, _ = upload(lib, wl)
    got = pool.route_key.cpu().numpy().astype(np.float64)
    P = wl.layers[0].pool()
    for s in range(0, got.shape[0], 7):
        for h in range(got.shape[1]):
            ref = oracle.block_route_key(P, s, h)
            assert np.abs(got[s, h] - ref).max() <= 1e-5 * (np.abs(ref).max() + 1.0)
    check_decode(lib, wl, label=f"shared basis, runs of {group}")


def test_decode_layers_shared_basis(lib):
    """Four layers of the un-rotated 64k batch-4 stack with pairs of blocks
    sharing a basis, in one layer-batched launch."""
    wl = synth.make_config(2, layers=[0, 9, 19, 27], variant="UB")
    say("[decode layers UB] stack64k layers 0, 9, 19, 27")
    pools, batches = [], []
    for l in range(4):
        p_, b_ = upload(lib, wl, l)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    res = _run_layers(lib, run, reps=2)
    for l in range(4):
        _, _, i1 = lib.decode(pools[l], batches[l], wl.top_k, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(wl, wl.layers[l], *res[l], wl.top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


@pytest.mark.parametrize("cfg,variant", [(0, "UC2"), (0, "UC4"), (1, "UC2"), (1, "UC4"), (3, "UC2"), (3, "UC4")])
def test_decode_compact_basis_store(lib, cfg, variant):
    """A basis store smaller than the pool (V_K, V_V in arrays of their own with
    about n_slots / 2 or n_slots / 4 entries, records without them): routing
    keys and the decode against the oracle."""
    wl = synth.make_config(cfg, variant=variant)
    lay = wl.layers[0]
    n_basis = lay.vk.shape[0]
    assert n_basis <= (wl.n_slots + int(variant[2]) * wl.batch) // int(variant[2])
    say(f"[compact basis] {wl.name}: {n_basis} entries for {wl.n_slots} slots")
    pool, _ = upload(lib, wl)
    assert pool.c.n_basis == n_basis and pool.tensors["vk"].shape[0] == n_basis
    got = pool.route_key.cpu().numpy().astype(np.float64)
    P = lay.pool()
    for s in range(0, got.shape[0], 5):
        for h in range(got.shape[1]):
            ref = oracle.block_route_key(P, s, h)
            assert np.abs(got[s, h] - ref).max() <= 1e-5 * (np.abs(ref).max() + 1.0)
    check_decode(lib, wl, label=f"compact basis store {variant}")


@pytest.mark.parametrize("variant", ["UC2", "UC4"])
def test_decode_layers_compact_basis_store(lib, variant):
    """Four layers of the un-rotated 64k batch-4 stack with compact basis
    stores, in one layer-batched launch and per layer."""
    wl = synth.make_config(2, layers=[0, 9, 19, 27], variant=variant)
    say(f"[decode layers {variant}] stack64k layers 0, 9, 19, 27: {wl.layers[0].vk.shape[0]} entries "
        f"for {wl.n_slots} slots")
    pools, batches = [], []
    for l in range(4):
        p_, b_ = upload(lib, wl, l)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    res = _run_layers(lib, run, reps=2)
    for l in range(4):
        o1, s1, i1 = lib.decode(pools[l], batches[l], wl.top_k, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(wl, wl.layers[l], *res[l], wl.top_k)
        c1 = _oracle_check(wl, wl.layers[l], o1, s1, i1, wl.top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} (per layer {c1.max_out:.3e})")


def test_decode_layers_unrotated_mixed_ranks(lib):
    """Un-rotated layers of every low-rank tile count (ranks 1..64, 0..255
    residual rows), ragged windows, an empty sequence and a shared basis in one
    layer-batched launch."""
    base = dict(batch=4, n_q_heads=6, n_kv_heads=2, window=48, n_blocks=[5, 0, 6, 3],
                win_len=[48, 0, 17, 30], top_k=3, sigma0=2.0, rope_base=synth.ROPE_BASE)
    specs = [dict(ranks=[1], n_resid=0), dict(ranks=[7], n_resid=20), dict(ranks=[24], n_resid=8),
             dict(ranks=[40], n_resid=33), dict(ranks=[64], n_resid=4), dict(ranks=[15], n_resid=255)]
    wls = [synth.make_workload(f"umix{i}", seed=600 + i, **base, **s) for i, s in enumerate(specs)]
    synth.set_shared_basis(wls[2], 2)
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, 3, wls[0].scale)
    assert run.plan.max_tiles >= 5 and run.plan.unrotated == 1
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        _, _, i1 = lib.decode(pools[l], batches[l], 3, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        _oracle_check(w, w.layers[0], *res[l], 3)


def test_decode_layers_unrotated_graph_replays(lib):
    """The un-rotated layer-batched launch captured in a graph replays to the
    eager bits, with eager launches and synchronisations between replays."""
    wl = synth.make_config(0, variant="UB")
    pools, batches = [], []
    for _ in range(3):
        p_, b_ = upload(lib, wl)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    run.run()
    torch.cuda.synchronize()
    ref = [(o.clone(), s.clone(), i.clone()) for o, s, i in zip(run.outs, run.lses, run.idxs)]
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        run.run(cs)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run.run(torch.cuda.current_stream())
    for _ in range(3):
        for o in run.outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for l, (o, s, i) in enumerate(ref):
            assert torch.equal(run.outs[l], o) and torch.equal(run.lses[l], s) and torch.equal(run.idxs[l], i)
        run.run()
        torch.cuda.synchronize()
        assert torch.equal(run.outs[0], ref[0][0])
    assert run.timeout_flag() == 0
    _oracle_check(wl, wl.layers[0], *ref[0], wl.top_k)


# ---------------------------------------------------------------------------
# Un-rotated pools with 8- and 4-bit residual rows (the pages' default preset
# stores keys un-rotated with 4-bit residual rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,variant", [(0, "Q8"), (0, "Q4"), (1, "Q4"), (1, "Q8")])
def test_decode_unrotated_quantised(lib, cfg, variant):
    wl = synth.set_unrotated(synth.make_config(cfg, variant=variant), synth.ROPE_BASE)
    check_decode(lib, wl, label=f"U {variant}")


@pytest.mark.parametrize("fmt,kw", [(2, dict(ranks=[7], n_resid=255)), (1, dict(ranks=[64], n_resid=4)),
                                    (2, dict(n_q_heads=16, n_kv_heads=1)), (1, dict(n_resid=0))])
def test_decode_unrotated_quantised_edges(lib, fmt, kw):
    base = dict(seed=540 + fmt, batch=4, n_q_heads=6, n_kv_heads=2, window=64, n_blocks=[5, 3, 6, 4],
                ranks=[12], n_resid=20, top_k=3, sigma0=2.0)
    base.update(kw)
    wl = synth.make_workload(f"UQ{fmt}", resid_format=fmt, rope_base=synth.ROPE_BASE, **base)
    check_decode(lib, wl, label=f"U fmt {fmt} {kw}")


def test_decode_layers_unrotated_mixed_formats(lib):
    """Un-rotated layers with fp16, 8-bit and 4-bit residual rows in one launch."""
    base = dict(batch=3, n_q_heads=6, n_kv_heads=2, window=40, n_blocks=[4, 6, 2], win_len=[40, 7, 33],
                top_k=3, sigma0=2.0, rope_base=synth.ROPE_BASE)
    wls = [synth.make_workload(f"umf{f}", seed=560 + f, ranks=[20 + 10 * f], n_resid=24, resid_format=f, **base)
           for f in (0, 1, 2)]
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, 3, wls[0].scale)
    assert run.plan.unrotated == 1 and run.plan.quantised == 1
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        _, _, i1 = lib.decode(pools[l], batches[l], 3, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        _oracle_check(w, w.layers[0], *res[l], 3)


def test_shared_basis_entry_out_of_range_is_empty(lib):
    """A block whose basis entry lies outside [0, n_basis) contributes no rows
    (its routing key is left as it was, zero here); every other block decodes
    as usual."""
    wl = synth.set_shared_basis(_u(0), 2)
    lay = wl.layers[0]
    bad_slot = int(wl.block_table[0, 3])
    lay.basis_of = lay.basis_of.copy()
    lay.basis_of[bad_slot] = lay.vk.shape[0] + 5
    pool, batch = upload(lib, wl)
    assert torch.all(pool.route_key[bad_slot] == 0)
    out, lse, idx = lib.decode(pool, batch, wl.top_k, wl.scale)
    torch.cuda.synchronize()
    g = idx.cpu().numpy().astype(np.int64)
    keep = g.copy()
    keep[0][keep[0] == 3] = -1
    P = lay.pool()
    P["basis_of"] = P["basis_of"].copy()
    P["basis_of"][bad_slot] = bad_slot            # never read: the block is dropped from the oracle's set
    ro, rl, _ = oracle.decode(P, lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len,
                              wl.n_kv_heads, wl.top_k, wl.scale, idx=keep)
    c = parity.check_outputs(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert c.ok, c.message

"""GPU parity: every C-ABI entry point against the fp64 oracle.

Bars (see parity.py): routing identical outside the near-tie band; decode
max |d out| <= 1e-2 and |d lse| <= 1e-3, compared on the GPU's accepted routed
set; per-part partials |d lse| <= 1e-3 and relative |d o| <= 1e-3.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest

from compressed_kv_cache_amd import synth
import oracle
import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_kv_cache_amd import lib as L
    L.load()                       # raises if the HIP library is not built
    return L


DEV = "cuda:0"


@functools.lru_cache(maxsize=None)
def config(cfg, variant=""):
    if cfg == 2:
        return synth.make_config(2, layers=[0, 9, 19, 27])
    return synth.make_config(cfg, variant=variant)


@functools.lru_cache(maxsize=None)
def planted_config1():
    """Config 1 with 8 outlier residual rows planted in a block the oracle routes
    for KV head 0 (planting residual rows does not move routing keys)."""
    wl = synth.make_config(1)
    L0 = wl.layers[0]
    idx, _, _ = oracle.route_batch(L0.pool(), L0.q, wl.block_table, wl.n_blocks, wl.n_kv_heads,
                                   wl.top_k)
    blk = int(idx[0, 0, 0])
    synth.plant_outlier_rows(wl, blk)
    wl.notes = f"planted block {blk}"
    wl.planted = blk
    return wl


def upload(L, wl, layer=0):
    lay = wl.layers[layer]
    pool = L.Pool.from_numpy(lay.pool(), DEV)
    batch = L.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                               wl.win_len, device=DEV)
    L.route_keys(pool)
    return pool, batch


def oracle_routing(wl, layer=0):
    lay = wl.layers[layer]
    return oracle.route_batch(lay.pool(), lay.q, wl.block_table, wl.n_blocks, wl.n_kv_heads,
                              wl.top_k)


def check_decode(L, wl, layer=0, label=""):
    say(f"[decode] {wl.name} {label} layer={layer}")
    pool, batch = upload(L, wl, layer)
    out, lse, idx = L.decode(pool, batch, wl.top_k, wl.scale)
    torch.cuda.synchronize()
    lay = wl.layers[layer]
    gidx = idx.cpu().numpy().astype(np.int64) if idx is not None else \
        np.full((wl.batch, wl.n_kv_heads, 0), -1)
    if wl.top_k > 0:
        _, scores, keys = oracle_routing(wl, layer)
        rc = parity.check_routing(gidx, scores, keys, lay.q, wl.n_kv_heads, wl.top_k)
        assert rc.ok, rc.message
    else:
        rc = parity.RouteCheck(True, 0)
    ref_o, ref_l, _ = oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table,
                                    wl.n_blocks, wl.win_len, wl.n_kv_heads, wl.top_k, wl.scale,
                                    idx=gidx)
    oc = parity.check_outputs(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l)
    say(f"   near-ties {rc.near_ties}; max|d out| {oc.max_out:.3e} max|d lse| {oc.max_lse:.3e} "
        f"rel {oc.rel_l2:.3e}")
    assert oc.ok, oc.message
    return gidx, out, lse


# ---------------------------------------------------------------------------
# Routing keys and routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,variant", [(0, ""), (0, "S1"), (1, ""), (2, "")])
def test_route_keys(lib, cfg, variant):
    wl = config(cfg, variant)
    say(f"[route_keys] {wl.name} {variant}")
    pool, _ = upload(lib, wl)
    got = pool.route_key.cpu().numpy().astype(np.float64)
    P = wl.layers[0].pool()
    S, H = got.shape[:2]
    worst = 0.0
    for s in range(S):
        for h in range(H):
            ref = oracle.route_key(P["anchor_k"][s, h], P["u"][s, h], P["vk"][s, h])
            worst = max(worst, float(np.abs(got[s, h] - ref).max() / (np.abs(ref).max() + 1.0)))
    say(f"   max rel err {worst:.2e}")
    assert worst < 2e-6


@pytest.mark.parametrize("cfg", [0, 1, 3, 4, 2])
def test_route_topk(lib, cfg):
    wl = config(cfg)
    for layer in range(len(wl.layers)):
        say(f"[route_topk] {wl.name} layer {layer}")
        pool, batch = upload(lib, wl, layer)
        idx, sc = lib.route_topk(pool, batch, wl.top_k, with_scores=True)
        torch.cuda.synchronize()
        _, scores, keys = oracle_routing(wl, layer)
        rc = parity.check_routing(idx.cpu().numpy(), scores, keys, wl.layers[layer].q,
                                  wl.n_kv_heads, wl.top_k)
        say(f"   near-ties {rc.near_ties}")
        assert rc.ok, rc.message
        g = idx.cpu().numpy()
        s = sc.cpu().numpy()
        for (b, h), ref in scores.items():
            sel = g[b, h][g[b, h] >= 0]
            assert np.allclose(s[b, h][:sel.size], ref[sel], rtol=1e-4, atol=1e-4)
            assert np.all(np.isneginf(s[b, h][sel.size:]))


def test_route_ties_go_to_lowest_index(lib):
    wl = synth.make_workload("ties", seed=5, batch=2, n_q_heads=4, n_kv_heads=2, window=16,
                             n_blocks=[40, 25], ranks=[16], n_resid=8, top_k=10)
    lay = wl.layers[0]
    for name in ("anchor_k", "u", "vk"):
        arr = getattr(lay, name)
        arr[:] = arr[0:1]                       # every block identical: all scores tie
    pool, batch = upload(lib, wl)
    idx = lib.route_topk(pool, batch, 10).cpu().numpy()
    assert np.array_equal(idx, np.broadcast_to(np.arange(10), idx.shape))
    # one dominant block is always chosen, the rest of the ties by lowest index
    G = wl.group
    for h in range(2):
        qbar = lay.q[0, h * G:(h + 1) * G].astype(np.float32).mean(axis=0)
        lay.anchor_k[int(wl.block_table[0, 30]), h] = (10 * qbar).astype(np.float16)
    pool, batch = upload(lib, wl)
    idx = lib.route_topk(pool, batch, 10).cpu().numpy()
    assert 30 in idx[0, 0] and 30 in idx[0, 1]


SPLIT_SHAPES = {
    # several 64-block score items per unit with a ragged last one, and units of different lengths
    # (up to 256 blocks: a wave holds 4 keys per lane; up to 512: 8; more: the selection in LDS)
    "ragged_items": dict(batch=4, n_q_heads=6, n_kv_heads=2, n_blocks=[300, 129, 64, 65], top_k=37),
    "long_unit": dict(batch=2, n_q_heads=4, n_kv_heads=2, n_blocks=[600, 37], top_k=12),
    "within_256": dict(batch=3, n_q_heads=6, n_kv_heads=2, n_blocks=[256, 255, 191], top_k=64),
    # top_k above some units' block counts, an empty unit, one block
    "topk_over_n": dict(batch=4, n_q_heads=6, n_kv_heads=2, n_blocks=[3, 0, 70, 1], top_k=5),
    # more units than XCD lists: 9 units, so list 0 holds two
    "nine_units": dict(batch=9, n_q_heads=2, n_kv_heads=1, n_blocks=[17, 64, 2, 130, 5, 66, 128, 1, 40],
                       top_k=9),
}


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("shape", sorted(SPLIT_SHAPES))
def test_decode_split_routing(lib, shape, gather):
    """dkv_decode's routing (score items of 64 blocks, each block part selecting
    its own block) routes exactly as dkv_route_topk does, from pool keys or a
    per-sequence key table, attends as the oracle does and never times out."""
    kw = dict(seed=40 + len(shape), window=40, ranks=[8], n_resid=8, sigma0=2.0, **SPLIT_SHAPES[shape])
    wl = synth.make_workload(shape, **kw)
    say(f"[split routing] {shape} gather={gather}")
    pool, batch = upload(lib, wl)
    if gather:
        lib.gather_route_keys(pool, batch)
    want = lib.route_topk(pool, batch, wl.top_k)
    ws = lib.alloc_workspace(pool, batch, wl.top_k)
    for rep in range(2):
        out, lse, idx = lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, want), rep
    assert int(ws[8:12].view(torch.int32).item()) == 0  # no part gave up waiting
    check_decode(lib, wl, label=shape)


def test_decode_split_routing_ties(lib):
    """All scores equal: every part of dkv_decode takes the lowest indices, as
    dkv_route_topk does."""
    wl = synth.make_workload("split_ties", seed=7, batch=2, n_q_heads=4, n_kv_heads=2, window=16,
                             n_blocks=[140, 25], ranks=[16], n_resid=8, top_k=10)
    lay = wl.layers[0]
    for name in ("anchor_k", "u", "vk"):
        arr = getattr(lay, name)
        arr[:] = arr[0:1]
    pool, batch = upload(lib, wl)
    _, _, idx = lib.decode(pool, batch, 10, wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.broadcast_to(np.arange(10), idx.shape))


def test_route_more_blocks_than_topk_and_padding(lib):
    wl = synth.make_workload("pad", seed=6, batch=3, n_q_heads=6, n_kv_heads=2, window=8,
                             n_blocks=[3, 0, 70], ranks=[8], n_resid=4, top_k=5, max_blocks=80)
    pool, batch = upload(lib, wl)
    idx = lib.route_topk(pool, batch, 5).cpu().numpy()
    _, scores, keys = oracle_routing(wl)
    rc = parity.check_routing(idx, scores, keys, wl.layers[0].q, 2, 5)
    assert rc.ok, rc.message
    assert np.array_equal(idx[0, 0], [0, 1, 2, -1, -1]) and np.all(idx[1] == -1)


# ---------------------------------------------------------------------------
# Per-part entry points (sensitivity variant S3: per-block partials)
# ---------------------------------------------------------------------------

def _all_blocks_idx(wl):
    K = int(wl.n_blocks.max())
    idx = np.full((wl.batch, wl.n_kv_heads, K), -1, dtype=np.int32)
    for b in range(wl.batch):
        idx[b, :, :wl.n_blocks[b]] = np.arange(wl.n_blocks[b])
    return idx


@pytest.mark.parametrize("cfg,variant", [(0, ""), (0, "S1"), (0, "S2"), (1, ""), (0, "Q8"), (0, "Q4"),
                                         (1, "Q8")])
def test_block_partials(lib, cfg, variant):
    wl = config(cfg, variant)
    say(f"[block partials] {wl.name} {variant}")
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
    ref_lo, ref_ll, ref_eo, ref_el = (np.zeros_like(lo, dtype=np.float64), np.zeros_like(ll, dtype=np.float64),
                                      np.zeros_like(eo, dtype=np.float64), np.zeros_like(el, dtype=np.float64))
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            for k in range(K):
                j = idx[b, h, k]
                slot = int(wl.block_table[b, j])
                (o1, l1), (o2, l2) = oracle.block_partials(lay.pool(), slot, h,
                                                          lay.q[b, h * G:(h + 1) * G], wl.scale)
                rows = slice(b * wl.n_q_heads + h * G, b * wl.n_q_heads + (h + 1) * G)
                ref_lo[rows, k], ref_ll[rows, k] = o1, l1
                ref_eo[rows, k], ref_el[rows, k] = o2, l2
    c1 = parity.check_partials(lo, ll, ref_lo, ref_ll)
    c2 = parity.check_partials(eo, el, ref_eo, ref_el)
    say(f"   low-rank: rel {c1.rel_l2:.2e} lse {c1.max_lse:.2e}; residual: rel {c2.rel_l2:.2e} "
        f"lse {c2.max_lse:.2e}")
    assert c1.ok, c1.message
    assert c2.ok, c2.message


@pytest.mark.parametrize("splits", [1, 3, 8, 37])
def test_window_partials(lib, splits):
    wl = synth.make_workload("win", seed=7, batch=3, n_q_heads=8, n_kv_heads=2, window=300,
                             n_blocks=[1, 1, 1], ranks=[8], n_resid=4, top_k=1,
                             win_len=[300, 17, 0])
    say(f"[window partials] splits={splits}")
    pool, batch = upload(lib, wl)
    po, pl = lib.exact_attn(pool, batch, None, 0, splits, wl.scale)
    torch.cuda.synchronize()
    lay = wl.layers[0]
    ro, rl = oracle.window_partials(lay.win_k, lay.win_v, wl.win_len, lay.q, 2, splits, wl.scale)
    c = parity.check_partials(po.cpu().numpy(), pl.cpu().numpy(),
                              ro.reshape(po.shape), rl.reshape(pl.shape))
    assert c.ok, c.message


def test_lse_merge(lib):
    rng = np.random.default_rng(3)
    rows, parts = 37, 23
    o = rng.standard_normal((rows, parts, 128)).astype(np.float32)
    l = (rng.standard_normal((rows, parts)) * 5).astype(np.float32)
    l[3, :5] = -np.inf
    o[3, :5] = 0
    l[7, :] = -np.inf                             # a row with no rows at all
    o[7, :] = 0
    out, lse = lib.lse_merge(torch.from_numpy(o).to(DEV), torch.from_numpy(l).to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(list(np.moveaxis(o, 1, 0)), list(np.moveaxis(l, 1, 0)))
    c = parity.check_outputs(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_out=2e-3, tol_lse=1e-5)
    assert c.ok, c.message
    assert np.all(out[7].cpu().numpy() == 0) and np.isneginf(lse[7].item())


# ---------------------------------------------------------------------------
# Fused decode on the five workloads and the sensitivity variants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,variant", [(0, ""), (0, "S1"), (0, "S2"), (3, ""), (4, ""),
                                         (0, "Q8"), (0, "Q4"), (1, "Q8"), (1, "Q4")])
def test_decode_configs(lib, cfg, variant):
    check_decode(lib, config(cfg, variant), label=variant)


def test_decode_config1_planted_outliers(lib):
    wl = planted_config1()
    gidx, out, lse = check_decode(lib, wl, label=wl.notes)
    assert wl.planted in gidx[0, 0]


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_decode_stack_layers(lib, layer):
    """The 28-layer 64k batch-4 stack, one layer of each rank (24, 48, 16) and the
    last layer, at full size in the per-layer launch the benchmark times."""
    check_decode(lib, config(2), layer=layer, label=f"rank {config(2).layers[layer].rank}")


EDGE = {
    "no_residuals": dict(n_resid=0),
    "rank1": dict(ranks=[1]),
    "odd_rank7": dict(ranks=[7]),
    "rank64": dict(ranks=[64]),
    "rank15_R255": dict(ranks=[15], n_resid=255),
    "group1": dict(n_q_heads=2, n_kv_heads=2),
    "group16": dict(n_q_heads=16, n_kv_heads=1),
    "ragged_window": dict(window=37, win_len=[37, 5, 0, 36]),
    "empty_sequence": dict(n_blocks=[3, 0, 5, 2], win_len=[64, 0, 64, 64]),
    "topk_over_n": dict(top_k=9, n_blocks=[3, 7, 1, 8]),
    "window_only": dict(top_k=0),
    "permuted_pool": dict(permute_slots=True),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_decode_edge_cases(lib, case):
    kw = dict(seed=100 + len(case), batch=4, n_q_heads=6, n_kv_heads=2, window=64,
              n_blocks=[5, 3, 6, 4], ranks=[12], n_resid=20, top_k=3, sigma0=2.0)
    kw.update(EDGE[case])
    wl = synth.make_workload(case, **kw)
    check_decode(lib, wl, label=case)


def test_decode_invalid_table_entries_are_empty(lib):
    wl = synth.make_workload("badslot", seed=9, batch=2, n_q_heads=4, n_kv_heads=2, window=32,
                             n_blocks=[4, 4], ranks=[8], n_resid=6, top_k=4)
    pool, batch = upload(lib, wl)
    bt = torch.from_numpy(wl.block_table.copy()).to(DEV)
    bt[0, 2] = -1
    bt[1, 1] = 10_000
    batch2 = lib.Batch(batch.tensors["q"], batch.tensors["win_k"], batch.tensors["win_v"], bt,
                       batch.tensors["n_blocks"], batch.tensors["win_len"])
    out, lse, idx = lib.decode(pool, batch2, 4, wl.scale)
    torch.cuda.synchronize()
    g = idx.cpu().numpy().astype(np.int64)
    lay = wl.layers[0]
    # reference: the bad blocks contribute no rows
    pool_np = lay.pool()
    keep = g.copy()
    keep[0][keep[0] == 2] = -1
    keep[1][keep[1] == 1] = -1
    ro, rl, _ = oracle.decode(pool_np, lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                              wl.win_len, 2, 4, wl.scale, idx=keep)
    c = parity.check_outputs(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert c.ok, c.message


def test_decode_is_deterministic(lib):
    wl = config(1)
    pool, batch = upload(lib, wl)
    ws = lib.alloc_workspace(pool, batch, wl.top_k)
    a = [t.clone() for t in lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws)]
    b = [t.clone() for t in lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_decode_graph_replays_match_eager(lib):
    """A captured decode replays correctly several times, with eager work and
    synchronisations between the replays (the workspace control words are
    left zeroed by every launch)."""
    wl = config(1)
    pool, batch = upload(lib, wl)
    ws = lib.alloc_workspace(pool, batch, wl.top_k)
    out = torch.empty((1, 12, 128), dtype=torch.float16, device=DEV)
    lse = torch.empty((1, 12), dtype=torch.float32, device=DEV)
    idx = torch.empty((1, 2, wl.top_k), dtype=torch.int32, device=DEV)
    lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws, out=out, out_lse=lse, out_idx=idx)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), idx.clone())
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws, out=out, out_lse=lse, out_idx=idx)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws, out=out, out_lse=lse, out_idx=idx)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(idx, ref[2]), rep
        # eager work between replays
        lib.decode(pool, batch, wl.top_k, wl.scale, workspace=ws, out=out, out_lse=lse, out_idx=idx)
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0])
    assert int(ws[8:12].view(torch.int32).item()) == 0      # no routing wait ever timed out


def test_decode_workspace_reused_across_shapes(lib):
    """One workspace, sized for the larger call, serves calls of different shapes."""
    big = config(1)
    small = synth.make_workload("small", seed=17, batch=2, n_q_heads=6, n_kv_heads=2, window=40,
                                n_blocks=[5, 3], ranks=[8], n_resid=10, top_k=4)
    pb, bb = upload(lib, big)
    ps, bs = upload(lib, small)
    ws = lib.alloc_workspace(pb, bb, big.top_k)
    for _ in range(2):
        o1, l1, i1 = lib.decode(pb, bb, big.top_k, big.scale, workspace=ws)
        o2, l2, i2 = lib.decode(ps, bs, small.top_k, small.scale, workspace=ws)
        torch.cuda.synchronize()
        r1, rl1, _ = oracle.decode(big.layers[0].pool(), big.layers[0].q, big.layers[0].win_k,
                                   big.layers[0].win_v, big.block_table, big.n_blocks, big.win_len, 2,
                                   big.top_k, big.scale, idx=i1.cpu().numpy().astype(np.int64))
        r2, rl2, _ = oracle.decode(small.layers[0].pool(), small.layers[0].q, small.layers[0].win_k,
                                   small.layers[0].win_v, small.block_table, small.n_blocks, small.win_len,
                                   2, small.top_k, small.scale, idx=i2.cpu().numpy().astype(np.int64))
        assert parity.check_outputs(o1.cpu().numpy(), l1.cpu().numpy(), r1, rl1).ok
        assert parity.check_outputs(o2.cpu().numpy(), l2.cpu().numpy(), r2, rl2).ok


@pytest.mark.parametrize("cfg,variant", [(1, ""), (0, "S1")])
def test_decode_pool_layouts(lib, cfg, variant):
    """The pool views may point into one record per (slot, KV head) or into one
    dense tensor per array: identical arithmetic, so identical bits."""
    wl = config(cfg, variant)
    lay = wl.layers[0]
    res = {}
    for layout in ("arrays", "records"):
        say(f"[decode layout] {wl.name} {variant} {layout}")
        pool = lib.Pool.from_numpy(lay.pool(), DEV, layout=layout)
        batch = lib.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                                     wl.win_len, device=DEV)
        lib.route_keys(pool)
        out, lse, idx = lib.decode(pool, batch, wl.top_k, wl.scale)
        torch.cuda.synchronize()
        res[layout] = (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy())
    for a, b in zip(res["arrays"], res["records"]):
        assert np.array_equal(a, b)
    gidx = res["records"][2].astype(np.int64)
    ref_o, ref_l, _ = oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table,
                                    wl.n_blocks, wl.win_len, wl.n_kv_heads, wl.top_k, wl.scale,
                                    idx=gidx)
    oc = parity.check_outputs(res["records"][0], res["records"][1], ref_o, ref_l)
    assert oc.ok, oc.message


@pytest.mark.parametrize("cfg,variant", [(1, ""), (3, ""), (0, "S2")])
def test_route_key_table(lib, cfg, variant):
    """dkv_gather_route_keys copies pool keys into block-table order (zero past
    n_blocks), and routing / decode read through it give the same bits as
    through the pool."""
    wl = config(cfg, variant)
    say(f"[route key table] {wl.name} {variant}")
    pool, batch = upload(lib, wl)
    tab = lib.gather_route_keys(pool, batch, attach=False)
    torch.cuda.synchronize()
    pk = pool.route_key.cpu().numpy()
    t = tab.cpu().numpy()
    want = np.zeros_like(t)
    for b in range(wl.batch):
        nb = int(wl.n_blocks[b])
        want[b, :, :nb] = pk[wl.block_table[b, :nb]].transpose(1, 0, 2)
    assert np.array_equal(t, want)
    idx0, sc0 = lib.route_topk(pool, batch, wl.top_k, with_scores=True)
    out0, lse0, oi0 = lib.decode(pool, batch, wl.top_k, wl.scale)
    batch.set_route_keys(tab)
    idx1, sc1 = lib.route_topk(pool, batch, wl.top_k, with_scores=True)
    out1, lse1, oi1 = lib.decode(pool, batch, wl.top_k, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx1) and torch.equal(sc0, sc1)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1) and torch.equal(oi0, oi1)


# ---------------------------------------------------------------------------
# Layer-batched decode: several layers' fused steps in one launch
# ---------------------------------------------------------------------------


def _upload_layers(L, wl, layers, route_table=True):
    pools, batches = [], []
    for l in layers:
        pool, batch = upload(L, wl, l)
        if route_table:
            L.gather_route_keys(pool, batch)
        pools.append(pool)
        batches.append(batch)
    return pools, batches


def _oracle_check(wl, lay, out, lse, idx, top_k):
    """The layer's outputs against the fp64 oracle at the routed blocks (routing
    itself checked against the oracle's scores, near ties allowed)."""
    gidx = idx.cpu().numpy().astype(np.int64) if idx is not None else \
        np.full((wl.batch, wl.n_kv_heads, 0), -1)
    if top_k > 0:
        _, scores, keys = oracle.route_batch(lay.pool(), lay.q, wl.block_table, wl.n_blocks, wl.n_kv_heads,
                                             top_k)
        rc = parity.check_routing(gidx, scores, keys, lay.q, wl.n_kv_heads, top_k)
        assert rc.ok, rc.message
    ro, rl, _ = oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                              wl.win_len, wl.n_kv_heads, top_k, wl.scale, idx=gidx)
    c = parity.check_outputs(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert c.ok, c.message
    return c


def _run_layers(L, run, reps=3):
    """Run a prepared layer-batched decode `reps` times; every run gives the same bits."""
    first = None
    for rep in range(reps):
        for o in run.outs:
            o.fill_(7)
        run.run()
        torch.cuda.synchronize()
        got = [(o.clone(), s.clone(), None if run.idxs is None else i.clone())
               for o, s, i in zip(run.outs, run.lses, run.idxs or [None] * len(run.outs))]
        if first is None:
            first = got
        else:
            for l, (a, b) in enumerate(zip(first, got)):
                assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (rep, l)
    assert run.timeout_flag() == 0
    return first


def test_decode_layers_stack_matches_oracle(lib):
    """Four layers of the 28-layer 64k batch-4 stack (ranks 24, 48, 16 and the
    last layer's) in one launch: each layer matches the oracle, routes exactly
    as the per-layer launch does, and three launches give the same bits."""
    wl = config(2)
    layers = list(range(len(wl.layers)))
    say(f"[decode layers] stack64k: layers {layers}")
    pools, batches = _upload_layers(lib, wl, layers)
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    res = _run_layers(lib, run)
    for l in layers:
        _, _, i1 = lib.decode(pools[l], batches[l], wl.top_k, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(wl, wl.layers[l], *res[l], wl.top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


def test_decode_layers_full_stack_sampled(lib):
    """The benchmark's launch: all 28 layers of the 64k batch-4 stack in one
    layer-batched launch.  Every layer routes exactly as its per-layer launch
    does, two launches give the same bits, and sampled layers (one of each
    rank) match the oracle."""
    layers = list(range(28))
    sampled = {3: None, 12: None, 22: None}
    say(f"[decode layers] stack64k, all {len(layers)} layers, oracle on layers {sorted(sampled)}")
    pools, batches = [], []
    scale = top_k = None
    for l in layers:
        w = synth.make_config(2, layers=[l])
        scale, top_k = w.scale, w.top_k
        pool, batch = upload(lib, w)
        lib.gather_route_keys(pool, batch)
        pools.append(pool)
        batches.append(batch)
        if l in sampled:
            sampled[l] = w
        del w
    run = lib.Layers(pools, batches, top_k, scale)
    res = _run_layers(lib, run, reps=2)
    assert run.timeout_flag() == 0
    for l in layers:
        _, _, i1 = lib.decode(pools[l], batches[l], top_k, scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1), l
    for l, w in sorted(sampled.items()):
        c = _oracle_check(w, w.layers[0], *res[l], w.top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


@pytest.mark.parametrize("variant", ["Q8", "Q4"])
def test_decode_layers_full_stack_quantised_sampled(lib, variant):
    """The 64k batch-4 stack with 8- or 4-bit residual rows, all 28 layers in
    the one streamed launch the benchmark times: every layer routes as its
    per-layer launch does, two launches give the same bits, and one layer of
    each rank matches the oracle."""
    sampled = {3: None, 12: None, 22: None}
    say(f"[decode layers] stack64k {variant}, 28 layers, oracle on layers {sorted(sampled)}")
    pools, batches = [], []
    scale = top_k = None
    for l in range(28):
        w = synth.make_config(2, layers=[l], variant=variant)
        scale, top_k = w.scale, w.top_k
        pool, batch = upload(lib, w)
        lib.gather_route_keys(pool, batch)
        pools.append(pool)
        batches.append(batch)
        if l in sampled:
            sampled[l] = w
        del w
    run = lib.Layers(pools, batches, top_k, scale)
    assert run.plan.stream == 1 and run.plan.quantised == 1
    res = _run_layers(lib, run, reps=2)
    for l in range(28):
        _, _, i1 = lib.decode(pools[l], batches[l], top_k, scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1), l
    for l, w in sorted(sampled.items()):
        c = _oracle_check(w, w.layers[0], *res[l], w.top_k)
        say(f"   layer {l} rank {w.layers[0].rank}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


def test_decode_layers_mixed_ranks_and_edges(lib):
    """Layers of every low-rank tile count (ranks 1..64, 0..255 residual rows),
    ragged windows and an empty sequence, in one launch."""
    base = dict(batch=4, n_q_heads=6, n_kv_heads=2, window=48, n_blocks=[5, 0, 6, 3],
                win_len=[48, 0, 17, 30], top_k=3, sigma0=2.0)
    specs = [dict(ranks=[1], n_resid=0), dict(ranks=[7], n_resid=20), dict(ranks=[24], n_resid=8),
             dict(ranks=[40], n_resid=33), dict(ranks=[64], n_resid=4), dict(ranks=[15], n_resid=255)]
    wls = [synth.make_workload(f"mix{i}", seed=300 + i, **base, **s) for i, s in enumerate(specs)]
    pools, batches = [], []
    for w in wls:
        p, b = upload(lib, w)
        pools.append(p)
        batches.append(b)
    run = lib.Layers(pools, batches, 3, wls[0].scale)
    assert run.plan.max_tiles >= 4           # rank 64 needs the largest instance
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        _, _, i1 = lib.decode(pools[l], batches[l], 3, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        _oracle_check(w, w.layers[0], *res[l], 3)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (10, 2), (16, 1)])
def test_decode_layers_query_groups(lib, hq, hkv):
    """One merge per unit combines G = 1, 5 and 16 query rows (16 takes two
    passes of the eight 32-lane slots), in a two-layer launch."""
    base = dict(batch=3, n_q_heads=hq, n_kv_heads=hkv, window=40, n_blocks=[4, 6, 2], win_len=[40, 7, 33],
                top_k=3, sigma0=2.0)
    wls = [synth.make_workload(f"group{hq // hkv}_{i}", seed=700 + 10 * i + hq, **base, ranks=[r], n_resid=n)
           for i, (r, n) in enumerate(((20, 16), (33, 40)))]
    say(f"[decode layers] G = {hq // hkv}")
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, 3, wls[0].scale)
    res = _run_layers(lib, run, reps=2)
    assert run.timeout_flag() == 0
    for l, w in enumerate(wls):
        _, _, i1 = lib.decode(pools[l], batches[l], 3, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(w, w.layers[0], *res[l], 3)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


def test_decode_layers_window_only(lib):
    base = dict(batch=3, n_q_heads=8, n_kv_heads=2, window=300, n_blocks=[2, 1, 2],
                win_len=[300, 129, 1], top_k=0, ranks=[8], n_resid=4)
    wls = [synth.make_workload(f"win{i}", seed=400 + i, **base) for i in range(3)]
    pools, batches = zip(*[upload(lib, w) for w in wls])
    run = lib.Layers(list(pools), list(batches), 0, wls[0].scale)
    assert run.idxs is None
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        _oracle_check(w, w.layers[0], res[l][0], res[l][1], None, 0)


def test_decode_layers_graph_replays(lib):
    """The layer-batched launch captured in a graph replays to the eager bits,
    with eager launches and synchronisations between replays."""
    wl = config(1)
    pools, batches = _upload_layers(lib, wl, [0, 0, 0])
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
    for rep in range(4):
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



# ---------------------------------------------------------------------------
# The layer-batched streams (plan.stream == 1): every pool qualifies
# ---------------------------------------------------------------------------

SEDGE = {
    "r8_no_residuals": dict(ranks=[8], n_resid=0),
    "r16_R252": dict(ranks=[16], n_resid=252),
    "r24_R68": dict(ranks=[24], n_resid=68),
    "r40_R4": dict(ranks=[40], n_resid=4),
    "r56_R128_G16": dict(ranks=[56], n_resid=128, n_q_heads=16, n_kv_heads=1),
    "r32_topk_over_blocks": dict(ranks=[32], n_resid=20, top_k=9),
    "r48_G1_long_ragged_window": dict(ranks=[48], n_resid=36, n_q_heads=2, n_kv_heads=2, window=300,
                                      win_len=[300, 129, 0, 17]),
    # residual rows of 8- and 4-bit codes: pages of 32 rows, items of 64 (ragged last pages and items)
    "q8_r16_R252": dict(ranks=[16], n_resid=252, resid_format=1),
    "q4_r24_R68": dict(ranks=[24], n_resid=68, resid_format=2),
    "q8_r40_R4": dict(ranks=[40], n_resid=4, resid_format=1),
    "q4_r56_R128_G16": dict(ranks=[56], n_resid=128, n_q_heads=16, n_kv_heads=1, resid_format=2),
    "q8_r8_no_residuals": dict(ranks=[8], n_resid=0, resid_format=1),
    "q4_r48_R36_G1_ragged": dict(ranks=[48], n_resid=36, n_q_heads=2, n_kv_heads=2, window=300,
                                 win_len=[300, 129, 0, 17], resid_format=2),
    "q8_r32_R96_topk_over_blocks": dict(ranks=[32], n_resid=96, top_k=9, resid_format=1),
}


@pytest.mark.parametrize("case", sorted(SEDGE))
def test_streams_edge_cases(lib, case):
    """Two layers of a shape the streams take (ranks 8..56 in steps of 8, 0..252
    residual rows in fp16 or 8- / 4-bit codes, G = 1..16, ragged and empty
    windows and sequences, top_k above the block count), in one step: the plan
    streams, both layers match the oracle, route as dkv_decode does and repeat
    bit for bit."""
    kw = dict(batch=4, n_q_heads=6, n_kv_heads=2, window=48, n_blocks=[5, 0, 6, 3],
              win_len=[48, 0, 17, 30], ranks=[16], n_resid=20, top_k=3, sigma0=2.0)
    kw.update(SEDGE[case])
    top_k = kw["top_k"]
    wls = [synth.make_workload(f"{case}_{i}", seed=900 + 7 * i + len(case), **kw) for i in range(2)]
    say(f"[streams] {case}")
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, top_k, wls[0].scale)
    assert run.plan.stream == 1 and run.plan.stream_waves > 0
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        _, _, i1 = lib.decode(pools[l], batches[l], top_k, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(res[l][2], i1)
        c = _oracle_check(w, w.layers[0], *res[l], top_k)
        say(f"   layer {l}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


def test_streams_mixed_ranks(lib):
    """Layers of ranks 8, 24, 40 and 56 with 4, 128 and 252 residual rows in one
    streamed step (each rank's U pages hold a different number of positions)."""
    base = dict(batch=2, n_q_heads=12, n_kv_heads=2, window=256, n_blocks=[9, 7], win_len=[256, 100],
                top_k=5, sigma0=2.0)
    specs = [(8, 4), (24, 128), (40, 252), (56, 128)]
    wls = [synth.make_workload(f"smix{i}", seed=950 + i, ranks=[r], n_resid=n, **base)
           for i, (r, n) in enumerate(specs)]
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, 5, wls[0].scale)
    assert run.plan.stream == 1
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        c = _oracle_check(w, w.layers[0], *res[l], 5)
        say(f"   rank {specs[l][0]} R {specs[l][1]}: max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


def test_streams_mixed_formats(lib):
    """fp16, 8-bit and 4-bit residual layers of different ranks in one streamed
    step, each against the oracle."""
    base = dict(batch=3, n_q_heads=8, n_kv_heads=2, window=160, n_blocks=[7, 2, 9], win_len=[160, 33, 90],
                top_k=4, sigma0=2.0)
    specs = [(24, 128, 0), (48, 128, 1), (16, 252, 2), (8, 60, 1), (40, 8, 2)]
    wls = [synth.make_workload(f"sfmt{i}", seed=970 + i, ranks=[r], n_resid=n, resid_format=f, **base)
           for i, (r, n, f) in enumerate(specs)]
    pools, batches = [], []
    for w in wls:
        p_, b_ = upload(lib, w)
        lib.gather_route_keys(p_, b_)
        pools.append(p_)
        batches.append(b_)
    run = lib.Layers(pools, batches, 4, wls[0].scale)
    assert run.plan.stream == 1
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        c = _oracle_check(w, w.layers[0], *res[l], 4)
        say(f"   rank {specs[l][0]} R {specs[l][1]} format {specs[l][2]}: "
            f"max|d out| {c.max_out:.3e} max|d lse| {c.max_lse:.3e}")


class _HipEvents:
    """Raw hipEvent_t handles (hipEventCreate through the HIP runtime torch loaded)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def make(self):
        e = self.ct.c_void_p()
        assert self.h.hipEventCreate(self.ct.byref(e)) == 0
        return e.value

    def ms(self, a, b):
        t = self.ct.c_float()
        assert self.h.hipEventElapsedTime(self.ct.byref(t), self.ct.c_void_p(a), self.ct.c_void_p(b)) == 0
        return t.value

    def free(self, e):
        self.h.hipEventDestroy(self.ct.c_void_p(e))


def test_decode_layers_profiled(lib):
    """dkv_decode_layers_profiled gives run()'s bits and four ordered events
    (before, after the routings, after the streams, after the merges)."""
    wl = config(1)
    pools, batches = _upload_layers(lib, wl, [0, 0])
    run = lib.Layers(pools, batches, wl.top_k, wl.scale)
    assert run.plan.stream == 1
    run.run()
    torch.cuda.synchronize()
    ref = [(o.clone(), s.clone()) for o, s in zip(run.outs, run.lses)]
    hip = _HipEvents()
    ev = [hip.make() for _ in range(4)]
    for o in run.outs:
        o.zero_()
    run.run_profiled(ev)
    torch.cuda.synchronize()
    for l, (o, s) in enumerate(ref):
        assert torch.equal(run.outs[l], o) and torch.equal(run.lses[l], s)
    gaps = [hip.ms(ev[k], ev[k + 1]) for k in range(3)]
    assert all(g >= 0.0 for g in gaps) and hip.ms(ev[0], ev[3]) > 0.0, gaps
    with pytest.raises(lib.DKVError):
        run.run_profiled([ev[0], 0, ev[2], ev[3]])
    for e in ev:
        hip.free(e)


@pytest.mark.parametrize("pages", [1, 3, 9])
def test_stream_read_probe(lib, pages):
    """The read-ceiling probe reads every byte once: each wave's 32-bit wrapping
    sum equals numpy's over its share; sizes it cannot take are refused."""
    n_waves = 40
    n = n_waves * pages * 4096 // 4
    g = torch.Generator(device="cpu").manual_seed(1234 + pages)
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, generator=g).to(DEV)
    sink = torch.zeros(n_waves, dtype=torch.int32, device=DEV)
    lib.read_probe(x, n_waves, sink)
    torch.cuda.synchronize()
    want = x.cpu().numpy().view(np.uint32).reshape(n_waves, -1).astype(np.uint64).sum(axis=1) % (1 << 32)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want.astype(np.uint32))
    with pytest.raises(lib.DKVError):
        lib.read_probe(x[:-4], n_waves, sink)


# ---------------------------------------------------------------------------
# Residual rows in the 8- and 4-bit group-quantised formats
# ---------------------------------------------------------------------------

QEDGE = {
    "q8_R255_rank15": dict(ranks=[15], n_resid=255, resid_format=1),
    "q4_R255_rank7": dict(ranks=[7], n_resid=255, resid_format=2),
    "q8_no_residuals": dict(n_resid=0, resid_format=1),
    "q4_rank64_ragged": dict(ranks=[64], resid_format=2, window=37, win_len=[37, 5, 0, 36]),
    "q8_group16": dict(n_q_heads=16, n_kv_heads=1, resid_format=1),
}


@pytest.mark.parametrize("case", sorted(QEDGE))
def test_decode_quantised_edge_cases(lib, case):
    kw = dict(seed=500 + len(case), batch=4, n_q_heads=6, n_kv_heads=2, window=64,
              n_blocks=[5, 3, 6, 4], ranks=[12], n_resid=20, top_k=3, sigma0=2.0)
    kw.update(QEDGE[case])
    wl = synth.make_workload(case, **kw)
    check_decode(lib, wl, label=case)


@pytest.mark.parametrize("variant", ["Q8", "Q4"])
def test_decode_quantised_pool_layouts(lib, variant):
    """Records and dense per-array tensors give the same bits for quantised pools."""
    wl = config(1, variant)
    lay = wl.layers[0]
    res = {}
    for layout in ("arrays", "records"):
        pool = lib.Pool.from_numpy(lay.pool(), DEV, layout=layout)
        batch = lib.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                                     wl.win_len, device=DEV)
        lib.route_keys(pool)
        out, lse, idx = lib.decode(pool, batch, wl.top_k, wl.scale)
        torch.cuda.synchronize()
        res[layout] = (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy())
    for a, b in zip(res["arrays"], res["records"]):
        assert np.array_equal(a, b)


def test_decode_layers_mixed_formats(lib):
    """fp16, 8-bit and 4-bit layers in one layer-batched launch, each against the oracle."""
    base = dict(batch=4, n_q_heads=6, n_kv_heads=2, window=48, n_blocks=[5, 2, 6, 3],
                win_len=[48, 9, 17, 30], top_k=3, sigma0=2.0, n_resid=24)
    specs = [dict(ranks=[24], resid_format=0), dict(ranks=[48], resid_format=1),
             dict(ranks=[16], resid_format=2), dict(ranks=[9], resid_format=1)]
    wls = [synth.make_workload(f"fmt{i}", seed=610 + i, **base, **sp) for i, sp in enumerate(specs)]
    pools, batches = [], []
    for w in wls:
        p, b = upload(lib, w)
        pools.append(p)
        batches.append(b)
    run = lib.Layers(pools, batches, 3, wls[0].scale)
    assert run.plan.quantised == 1
    res = _run_layers(lib, run, reps=2)
    for l, w in enumerate(wls):
        say(f"[layers mixed formats] layer {l} format {specs[l]['resid_format']}")
        _oracle_check(w, w.layers[0], *res[l], 3)

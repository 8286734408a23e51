"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status codes before
enqueueing anything.  No call here reaches a kernel launch, so these run
without a GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from compressed_kv_cache_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dkv_attn.h")


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(L.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return L.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(clib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(clib, n), f"{n} declared in dkv_attn.h but not exported"
    assert set(names) == set(L.EXPORTED)


def test_abi_version_and_status_strings(clib):
    m = re.search(r"#define DKV_ABI_VERSION (\d+)", open(HEADER).read())
    assert clib.dkv_abi_version() == int(m.group(1))
    for code, name in [(0, "DKV_OK"), (1, "DKV_ERR_INVALID_ARG"), (2, "DKV_ERR_UNSUPPORTED"),
                       (3, "DKV_ERR_WORKSPACE"), (4, "DKV_ERR_HIP")]:
        assert clib.dkv_status_string(code).decode() == name


FAKE = 0x10000  # 64 KiB-aligned dummy address: never dereferenced on the host


def _pool(**kw):
    v = L.View(FAKE, 4096, 1024)
    p = L.PoolC(128, 256, 32, 16, 2, 10, v, v, L.View(FAKE, 16320, 8160), v, v, v, v,
                L.View(FAKE, 32, 16), L.View(FAKE, 256, 128))
    for k, val in kw.items():
        setattr(p, k, val)
    return p


def _batch(**kw):
    b = L.BatchC(2, 12, 64, 8, FAKE, FAKE, None, FAKE, FAKE, FAKE)
    for k, val in kw.items():
        setattr(b, k, val)
    return b


def _decode(clib, pool, batch, top_k=4, ws=FAKE, ws_bytes=1 << 30, out=FAKE):
    return clib.dkv_decode(ctypes.byref(pool) if pool is not None else None,
                           ctypes.byref(batch) if batch is not None else None, top_k,
                           0.088, ws, ws_bytes, out, FAKE, None, None)


@pytest.mark.parametrize("pool_kw,batch_kw,top_k,code", [
    ({"head_dim": 64}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"block_size": 128}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"rank": 0}, {}, 4, L.DKV_ERR_INVALID_ARG),
    ({"rank": 65}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"n_resid": 256}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"n_resid": -1}, {}, 4, L.DKV_ERR_INVALID_ARG),
    ({"n_kv_heads": 0}, {}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {"n_q_heads": 13}, 4, L.DKV_ERR_INVALID_ARG),
    ({"n_kv_heads": 1}, {"n_q_heads": 17}, 4, L.DKV_ERR_UNSUPPORTED),
    ({}, {"window": -1}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {"q": None}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {"q": FAKE + 2}, 4, L.DKV_ERR_UNSUPPORTED),
    ({}, {"block_table": None}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {"win_k": None}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {"max_blocks": 20000}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"vk": L.View(FAKE + 8, 4096, 1024)}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"vk": L.View(FAKE, 4100, 1024)}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"u": L.View(None, 0, 0)}, {}, 4, L.DKV_ERR_INVALID_ARG),
    ({}, {}, -1, L.DKV_ERR_INVALID_ARG),
    ({"rope_freq": FAKE}, {}, 4, L.DKV_ERR_INVALID_ARG),                    # no slot_pos
    ({"rope_freq": FAKE + 4, "slot_pos": FAKE}, {}, 4, L.DKV_ERR_UNSUPPORTED),
    ({"basis_of": FAKE, "n_basis": 4}, {}, 4, L.DKV_ERR_UNSUPPORTED),       # shared basis, rotated pool
    ({"rope_freq": FAKE, "slot_pos": FAKE, "basis_of": FAKE, "n_basis": 0}, {}, 4, L.DKV_ERR_INVALID_ARG),
    ({"rope_freq": FAKE, "slot_pos": FAKE, "basis_of": FAKE + 2, "n_basis": 4}, {}, 4, L.DKV_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_arguments(clib, pool_kw, batch_kw, top_k, code):
    st = _decode(clib, _pool(**pool_kw), _batch(**batch_kw), top_k=top_k)
    assert st == code, (st, clib.dkv_last_error().decode())
    assert clib.dkv_last_error().decode() != ""


def test_decode_null_structs_and_workspace(clib):
    assert _decode(clib, None, _batch()) == L.DKV_ERR_INVALID_ARG
    assert _decode(clib, _pool(), None) == L.DKV_ERR_INVALID_ARG
    need = clib.dkv_decode_workspace_size(ctypes.byref(_pool()), ctypes.byref(_batch()), 4)
    assert _decode(clib, _pool(), _batch(), ws_bytes=need - 1) == L.DKV_ERR_WORKSPACE
    assert _decode(clib, _pool(), _batch(), ws=None) == L.DKV_ERR_WORKSPACE
    assert _decode(clib, _pool(), _batch(), ws=FAKE + 16) == L.DKV_ERR_WORKSPACE
    assert _decode(clib, _pool(), _batch(), out=None) == L.DKV_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(clib):
    assert _decode(clib, _pool(), _batch(batch=0)) == L.DKV_OK
    p, b = _pool(), _batch(batch=0)
    assert clib.dkv_route_topk(ctypes.byref(p), ctypes.byref(b), 4, FAKE, None, None) == L.DKV_OK


def test_workspace_size_formula(clib):
    def a256(x):
        return (x + 255) // 256 * 256
    p = _pool()
    for window in (0, 64, 300):
        b = _batch(window=window)
        for top_k in (0, 1, 16, 64):
            # the fused launch's parts: routed-block parts each with a share of the
            # window, or (no routed blocks) window chunks of 512 rows
            n_parts = top_k if top_k > 0 else max(1, (window + 511) // 512)
            rows, units, max_blocks = 2 * 12, 2 * 2, 8
            # counters/queues, per-unit counts (a 256-byte line each), routed slots, and (top_k > 0) the
            # 8-byte (slot, score) word of every block-table entry
            ctrl = 4096 + a256(units * 256) + a256(units * top_k * 4) \
                + (a256(units * max_blocks * 8) if top_k > 0 else 0)
            want = ctrl + a256(units * top_k * 4) + a256(rows * n_parts * 4) \
                + a256(rows * n_parts * 128 * 4)
            assert clib.dkv_decode_workspace_size(ctypes.byref(p), ctypes.byref(b), top_k) == want
    assert clib.dkv_decode_workspace_size(None, ctypes.byref(_batch()), 4) == 0


def test_workspace_init_validates(clib):
    p, b = _pool(), _batch()
    need = clib.dkv_decode_workspace_size(ctypes.byref(p), ctypes.byref(b), 4)
    assert clib.dkv_decode_workspace_init(ctypes.byref(p), ctypes.byref(b), 4, FAKE, need - 1, None) \
        == L.DKV_ERR_WORKSPACE
    assert clib.dkv_decode_workspace_init(ctypes.byref(p), ctypes.byref(b), 4, None, need, None) \
        == L.DKV_ERR_WORKSPACE
    assert clib.dkv_decode_workspace_init(ctypes.byref(p), ctypes.byref(b), -2, FAKE, need, None) \
        == L.DKV_ERR_INVALID_ARG


def test_other_entry_points_validate(clib):
    p, b = _pool(), _batch()
    P, B = ctypes.byref(p), ctypes.byref(b)
    assert clib.dkv_route_topk(P, B, 0, FAKE, None, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_route_topk(P, B, 4, None, None, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_lowrank_attn(P, B, FAKE, 4, 0.1, FAKE, FAKE, 3, 0, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_lowrank_attn(P, B, FAKE, 0, 0.1, FAKE, FAKE, 3, 0, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_exact_attn(P, B, None, 2, 1, 0.1, FAKE, FAKE, 3, 0, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_exact_attn(P, B, FAKE, 2, 2, 0.1, FAKE, FAKE, 3, 0, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_exact_attn(P, B, FAKE, 0, -1, 0.1, FAKE, FAKE, 3, 0, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_lse_merge(FAKE, FAKE, 4, 8, 64, FAKE, FAKE, None) == L.DKV_ERR_UNSUPPORTED
    assert clib.dkv_lse_merge(FAKE, FAKE, -1, 8, 128, FAKE, FAKE, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_lse_merge(FAKE, FAKE, 4, 0, 128, FAKE, FAKE, None) == L.DKV_OK
    assert clib.dkv_route_keys(P, FAKE, -1, None) == L.DKV_ERR_INVALID_ARG
    q = _pool(route_key=L.View(FAKE + 4, 256, 128))
    assert clib.dkv_route_keys(ctypes.byref(q), None, 0, None) == L.DKV_ERR_UNSUPPORTED


def test_route_key_table_validates(clib):
    p, b = _pool(), _batch()
    P, B = ctypes.byref(p), ctypes.byref(b)
    assert clib.dkv_gather_route_keys(P, B, None, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_gather_route_keys(P, B, FAKE + 8, None) == L.DKV_ERR_UNSUPPORTED
    assert clib.dkv_gather_route_keys(P, ctypes.byref(_batch(batch=0)), None, None) == L.DKV_OK
    q = _pool(route_key=L.View(None, 0, 0))
    assert clib.dkv_gather_route_keys(ctypes.byref(q), B, FAKE, None) == L.DKV_ERR_INVALID_ARG
    # a misaligned per-sequence table is refused by routing and decode alike
    bad = _batch(route_keys=FAKE + 4)
    assert clib.dkv_route_topk(P, ctypes.byref(bad), 4, FAKE, None, None) == L.DKV_ERR_UNSUPPORTED
    assert _decode(clib, _pool(), bad) == L.DKV_ERR_UNSUPPORTED
    # with the table, routing needs no pool routing keys
    ok = _batch(route_keys=FAKE)
    assert clib.dkv_decode_workspace_size(ctypes.byref(q), ctypes.byref(ok), 4) > 0


def test_layer_batched_entry_points_validate(clib):
    p, b = _pool(), _batch()
    PA = (L.PoolC * 2)(p, p)
    BA = (L.BatchC * 2)(b, b)
    assert clib.dkv_decode_layers_table_size(0) == 0
    assert clib.dkv_decode_layers_table_size(3) > 0
    need = clib.dkv_decode_layers_workspace_size(PA, BA, 2, 4)
    one = clib.dkv_decode_workspace_size(ctypes.byref(p), ctypes.byref(b), 4)
    assert need >= 2 * one
    assert clib.dkv_decode_layers_workspace_size(PA, BA, 0, 4) == 0
    plan = L.LayersPlanC()
    outs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    tsz = clib.dkv_decode_layers_table_size(2)
    # bad counts and sizes are refused before anything touches the device
    assert clib.dkv_decode_layers_prepare(PA, BA, 0, 4, 0.1, outs, outs, None, FAKE, tsz, FAKE, need,
                                          ctypes.byref(plan)) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_decode_layers_prepare(PA, BA, 2, 4, 0.1, outs, outs, None, FAKE, tsz - 1, FAKE, need,
                                          ctypes.byref(plan)) == L.DKV_ERR_WORKSPACE
    assert clib.dkv_decode_layers_prepare(PA, BA, 2, 4, 0.1, outs, outs, None, FAKE, tsz, FAKE, need - 1,
                                          ctypes.byref(plan)) == L.DKV_ERR_WORKSPACE
    b2 = _batch(n_q_heads=16)
    BB = (L.BatchC * 2)(b, b2)
    need2 = clib.dkv_decode_layers_workspace_size(PA, BB, 2, 4)
    assert clib.dkv_decode_layers_prepare(PA, BB, 2, 4, 0.1, outs, outs, None, FAKE, tsz, FAKE, need2,
                                          ctypes.byref(plan)) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_decode_layers(None, None) == L.DKV_ERR_INVALID_ARG


# Shapes the streams' schedule builder runs on (host code: sizing a workspace
# builds the whole schedule).  Each must come back at once with a size that
# covers the classic layout's per-layer regions.
SCHED_SHAPES = [
    # (ranks per layer, residual rows, residual format, window, top_k, batch, q heads, kv heads, max_blocks)
    ([8], 0, 0, 0, 1, 1, 2, 2, 4),
    ([16], 252, 0, 37, 3, 4, 6, 2, 6),
    ([24], 68, 2, 300, 9, 4, 2, 2, 5),
    ([56], 128, 1, 1024, 32, 1, 16, 1, 252),
    ([40], 4, 2, 4096, 32, 2, 8, 2, 512),
    ([24] * 9 + [48] * 10 + [16] * 9, 128, 0, 1024, 32, 4, 12, 2, 252),
    ([24] * 9 + [48] * 10 + [16] * 9, 128, 1, 1024, 32, 4, 12, 2, 252),
    ([24] * 9 + [48] * 10 + [16] * 9, 128, 2, 1024, 32, 4, 12, 2, 252),
    ([32] * 4, 40, 0, 4096, 32, 32, 32, 8, 128),
]


@pytest.mark.timeout(60)
@pytest.mark.parametrize("shape", range(len(SCHED_SHAPES)))
def test_stream_schedule_sizes(clib, shape):
    ranks, R, fmt, W, top_k, B, hq, hkv, mb = SCHED_SHAPES[shape]
    sb = L.View(FAKE, 4096, 2048)
    pools = [_pool(rank=r, n_resid=R, n_kv_heads=hkv, resid_format=fmt, resid_k_sb=sb, resid_v_sb=sb)
             for r in ranks]
    b = _batch(batch=B, n_q_heads=hq, window=W, max_blocks=mb)
    n = len(ranks)
    PA = (L.PoolC * n)(*pools)
    BA = (L.BatchC * n)(*([b] * n))
    need = clib.dkv_decode_layers_workspace_size(PA, BA, n, top_k)
    one = sum(clib.dkv_decode_workspace_size(ctypes.byref(p), ctypes.byref(b), top_k) for p in pools)
    assert need > 0 and need >= one // 2


def test_seal_blocks_validates(clib):
    p = _pool()
    src = L.View(FAKE, 2 * 256 * 128, 256 * 128)
    omega = FAKE

    def seal(pool=p, width=40, iters=2, n=2, slots=FAKE, om=omega, sk=src):
        return clib.dkv_seal_blocks(ctypes.byref(pool) if pool is not None else None, sk, src, slots, n, om,
                                    width, iters, None)
    assert seal(pool=None) == L.DKV_ERR_INVALID_ARG
    assert seal(width=31) == L.DKV_ERR_INVALID_ARG          # width below the rank (32)
    assert seal(width=81) == L.DKV_ERR_UNSUPPORTED          # test matrix wider than 80 columns
    assert seal(iters=-1) == L.DKV_ERR_INVALID_ARG
    assert seal(iters=9) == L.DKV_ERR_INVALID_ARG
    assert seal(n=-1) == L.DKV_ERR_INVALID_ARG
    assert seal(n=0) == L.DKV_OK                            # nothing to do, nothing enqueued
    assert seal(slots=None) == L.DKV_ERR_INVALID_ARG
    assert seal(om=None) == L.DKV_ERR_INVALID_ARG
    assert seal(sk=L.View(FAKE + 2, 0, 0)) == L.DKV_ERR_UNSUPPORTED   # source rows not 16-byte aligned
    assert seal(pool=_pool(resid_format=L.RESID_INT8)) == L.DKV_ERR_INVALID_ARG   # codes without (scale, bias)
    assert seal(pool=_pool(resid_format=7)) == L.DKV_ERR_INVALID_ARG
    assert seal(pool=_pool(head_dim=64)) == L.DKV_ERR_UNSUPPORTED
    assert seal(width=81) == L.DKV_ERR_UNSUPPORTED and b"width" in clib.dkv_last_error()


def test_rope_freqs_table(clib):
    # host-only: theta_j / (2 pi) = base^(-j/64) / (2 pi) as hi + lo floats
    import numpy as np
    out = np.zeros(128, dtype=np.float32)
    assert clib.dkv_rope_freqs(1e6, 128, out.ctypes.data) == L.DKV_OK
    hi, lo = out[:64].astype(np.float64), out[64:].astype(np.float64)
    assert hi[0] == np.float32(1 / (2 * np.pi))                 # theta_0 = 1
    assert abs(hi[32] + lo[32] - 1e-3 / (2 * np.pi)) < 1e-18     # theta_32 = base^(-1/2)
    want = np.array([1e6 ** (-j / 64) for j in range(64)]) / (2 * np.pi)
    assert np.all(np.abs(hi + lo - want) <= 1e-14 * want)
    assert np.all(np.abs(lo) <= np.spacing(out[:64]).astype(np.float64))
    assert clib.dkv_rope_freqs(1e6, 64, out.ctypes.data) == L.DKV_ERR_UNSUPPORTED
    assert clib.dkv_rope_freqs(1.0, 128, out.ctypes.data) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_rope_freqs(1e4, 128, None) == L.DKV_ERR_INVALID_ARG


def test_layer_batched_rejects_mixed_rotation(clib):
    p, q, b = _pool(), _pool(rope_freq=FAKE, slot_pos=FAKE), _batch()
    PA, BA = (L.PoolC * 2)(p, q), (L.BatchC * 2)(b, b)
    plan = L.LayersPlanC()
    outs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    tsz = clib.dkv_decode_layers_table_size(2)
    need = clib.dkv_decode_layers_workspace_size(PA, BA, 2, 4)
    st = clib.dkv_decode_layers_prepare(PA, BA, 2, 4, 0.088, outs, outs, None, FAKE, tsz, FAKE, need,
                                        ctypes.byref(plan))
    assert st == L.DKV_ERR_UNSUPPORTED and "rotated" in clib.dkv_last_error().decode()


def test_join_basis_validates(clib):
    p = _pool()
    P = ctypes.byref(p)
    assert clib.dkv_join_basis(None, FAKE, FAKE, 1, 1, FAKE, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_join_basis(P, FAKE, FAKE, -1, 1, FAKE, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_join_basis(P, FAKE, FAKE, 0, 1, FAKE, None) == L.DKV_OK          # nothing to do
    assert clib.dkv_join_basis(P, None, FAKE, 2, 1, FAKE, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_join_basis(P, FAKE, FAKE, 2, 1, None, None) == L.DKV_ERR_INVALID_ARG
    assert clib.dkv_join_basis(P, FAKE + 2, FAKE, 2, 1, FAKE, None) == L.DKV_ERR_UNSUPPORTED
    q = _pool(rank=65)
    assert clib.dkv_join_basis(ctypes.byref(q), FAKE, FAKE, 2, 1, FAKE, None) == L.DKV_ERR_UNSUPPORTED
    q = _pool(basis_of=FAKE, n_basis=0)
    assert clib.dkv_join_basis(ctypes.byref(q), FAKE, FAKE, 2, 1, FAKE, None) == L.DKV_ERR_INVALID_ARG

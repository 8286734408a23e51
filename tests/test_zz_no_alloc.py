"""dkv_decode_noalloc (the entry point for callers that cannot allocate)
against dkv_decode on the same inputs, through the C ABI: two calls in a row,
the second with a smaller input, each identical to dkv_decode's results."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from compressed_kv_cache_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_kv_cache_amd import lib as L
    L.load()
    return L


def _upload(L, wl, layer=0):
    lay = wl.layers[layer]
    pool = L.Pool.from_numpy(lay.pool(), DEV)
    batch = L.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len,
                               device=DEV)
    L.route_keys(pool)
    return pool, batch


def _both(L, wl, layer=0):
    pool, batch = _upload(L, wl, layer)
    ref = L.decode(pool, batch, wl.top_k, wl.scale)
    got = L.decode_noalloc(pool, batch, wl.top_k, wl.scale)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_decode_two_calls_second_smaller(lib):
    """The 16k single layer (12 query heads, 60 blocks), then the 4k single head:
    the second call reuses the scratch the first one left behind."""
    for wl in (synth.make_config(1), synth.make_config(0)):
        say(f"[noalloc] {wl.name}")
        (ro, rl, ri), (go, gl, gi) = _both(lib, wl)
        assert torch.equal(ri, gi)
        assert torch.equal(ro, go) and torch.equal(rl, gl)


def test_noalloc_refuses_a_decode_larger_than_its_scratch(lib):
    """A decode whose workspace exceeds the fixed scratch is refused before
    anything is enqueued, with DKV_ERR_WORKSPACE."""
    import ctypes
    c = lib.load()
    cap = int(c.dkv_decode_noalloc_max_bytes())
    assert cap == 16 << 20
    wl = synth.make_config(0)
    pool, batch = _upload(lib, wl)
    big = lib.Batch.from_numpy(wl.layers[0].q, wl.layers[0].win_k, wl.layers[0].win_v, wl.block_table,
                               wl.n_blocks, wl.win_len, device=DEV)
    need = c.dkv_decode_workspace_size(ctypes.byref(pool.c), ctypes.byref(big.c), 100000)
    assert need > cap
    with pytest.raises(lib.DKVError) as err:
        lib.decode_noalloc(pool, big, 100000, wl.scale)
    assert "scratch" in str(err.value)

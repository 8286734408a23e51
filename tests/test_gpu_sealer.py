"""GPU parity of block sealing (dkv_seal_blocks) against the fp64 oracle
(oracle/dkv_sealer.py), on the same seeded blocks and test matrix.

Bars:
- anchors and residual rows are bit-exact copies of the source rows;
- the reconstruction from the stored fp16 factors, U V_K and U V_V, matches the
  oracle's within 5e-4 of the delta's Frobenius norm (each side rounds its
  factors to fp16, 2^-11 relative per entry, which moves the product by about
  1e-4 of |A|; the fp32 and fp64 subspace iterations agree to ~1e-6);
- the singular values (column norms of U) within 2e-3 relative, for those
  above 1e-3 of the largest;
- the basis rows [V_K | V_V] orthonormal within 4e-3 (fp16 entries);
- residual positions equal to the oracle's outside a near-tie band of the key
  errors (a position may swap only with one whose oracle error is within 2% of
  the cut), and every planted row selected;
- routing keys within 1e-3 (relative to their norm) of the oracle's.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from compressed_kv_cache_amd import synth
import oracle
from oracle import dkv_sealer as S

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
    L.load()                       # raises if the HIP library is not built
    return L


def _seal_gpu(L, inp, rank, n_resid, power_iters, slots=None, n_slots=None, layout="records", resid_format=0):
    nb, H = inp.k.shape[:2]
    slots = np.arange(nb, dtype=np.int32) if slots is None else np.asarray(slots, np.int32)
    n_slots = nb if n_slots is None else n_slots
    pool = L.Pool.empty(n_slots, H, rank, n_resid, DEV, layout, resid_format)
    k = torch.from_numpy(inp.k).to(DEV)
    v = torch.from_numpy(inp.v).to(DEV)
    om = torch.from_numpy(np.ascontiguousarray(inp.omega)).to(DEV)
    L.seal_blocks(pool, k, v, torch.from_numpy(slots).to(DEV), om, power_iters)
    torch.cuda.synchronize()
    out = {n: t.cpu().numpy() for n, t in pool.tensors.items() if t is not None and not n.startswith("_")}
    return out, om.cpu().numpy()


def _check_selection(gpu_pos, err, n_resid, planted=()):
    order = sorted(range(255), key=lambda i: (-err[i], i))
    cut = err[order[n_resid - 1]]
    tau = 0.02 * cut
    g = set(int(p) - 1 for p in gpu_pos)
    o = set(order[:n_resid])
    assert len(g) == n_resid and list(gpu_pos) == sorted(gpu_pos)
    for i in g - o:
        assert err[i] >= cut - tau, f"position {i + 1} chosen with error {err[i]:.4g}, cut {cut:.4g}"
    for i in o - g:
        assert err[i] <= cut + tau, f"position {i + 1} dropped with error {err[i]:.4g}, cut {cut:.4g}"
    for p in planted:
        assert int(p) - 1 in g
    return len(g - o)


def _compare_block(out, b, h, k, v, ref, rank, n_resid, planted=()):
    assert out["anchor_k"][b, h].tobytes() == k[0].tobytes()
    assert out["anchor_v"][b, h].tobytes() == v[0].tobytes()
    u = out["u"][b, h].astype(np.float64)
    vk = out["vk"][b, h].astype(np.float64)
    vv = out["vv"][b, h].astype(np.float64)
    _, _, a = S.joint_delta(k, v)
    scale = np.linalg.norm(a)
    ru = ref["u"].astype(np.float64)
    rec_g = np.hstack([u @ vk, u @ vv])
    rec_o = np.hstack([ru @ ref["vk"].astype(np.float64), ru @ ref["vv"].astype(np.float64)])
    rel = np.linalg.norm(rec_g - rec_o) / scale
    assert rel <= 5e-4, f"reconstruction differs by {rel:.3g} of |A|"
    s_g = np.linalg.norm(u, axis=0)
    s_o = ref["fp64"]["s"]
    big = s_o > 1e-3 * s_o[0]
    np.testing.assert_allclose(s_g[big], s_o[big], rtol=2e-3)
    w = np.hstack([vk, vv])
    gram = w[big] @ w[big].T
    assert np.max(np.abs(gram - np.eye(int(big.sum())))) <= 4e-3
    swaps = 0
    if n_resid > 0:
        pos = out["resid_pos"][b, h].astype(np.int64)
        swaps = _check_selection(pos, ref["err"], n_resid, planted)
        assert out["resid_k"][b, h].tobytes() == k[pos].tobytes()
        assert out["resid_v"][b, h].tobytes() == v[pos].tobytes()
    # routing key of the sealed block against the oracle's, from the oracle's factors
    rk_o = oracle.route_key(ref["anchor_k"], ref["u"], ref["vk"])
    rk_g = out["route_key"][b, h].astype(np.float64)
    assert np.linalg.norm(rk_g - rk_o) <= 1e-3 * np.linalg.norm(rk_o)
    return rel, swaps


@pytest.mark.parametrize("rank,n_resid,iters", [(16, 40, 2), (24, 128, 2), (32, 128, 2), (48, 128, 2),
                                                 (64, 64, 2), (32, 40, 0), (32, 40, 1), (8, 0, 3)])
def test_seal_matches_oracle(lib, rank, n_resid, iters):
    say(f"[seal] rank {rank} R {n_resid} power iterations {iters}")
    width = rank + 8
    inp = synth.make_seal_input(2000 + rank, 3, 2, width=width)
    out, om = _seal_gpu(lib, inp, rank, n_resid, iters)
    worst, swaps = 0.0, 0
    for b in range(3):
        for h in range(2):
            k, v = inp.k[b, h], inp.v[b, h]
            ref = S.seal_block(k, v, rank, n_resid, om, iters)
            planted = inp.outliers[b, h] if n_resid >= 8 and rank <= 32 else ()
            rel, sw = _compare_block(out, b, h, k, v, ref, rank, n_resid, planted)
            worst, swaps = max(worst, rel), swaps + sw
    say(f"[seal]   worst reconstruction difference {worst:.2e} of |A|; near-tie swaps {swaps}")


def test_seal_slots_layouts_and_skips(lib):
    # blocks go to permuted slots of a larger pool; a slot of -1 skips its
    # block and leaves the pool untouched; both pool layouts give the same bytes
    say("[seal] slot permutation, skipped block, pool layouts")
    inp = synth.make_seal_input(2100, 4, 2, width=40)
    slots = [5, -1, 0, 3]
    outs = [_seal_gpu(lib, inp, 32, 40, 2, slots=slots, n_slots=6, layout=lay)[0] for lay in ("records", "arrays")]
    for name in ("anchor_k", "u", "vk", "vv", "resid_k", "resid_v", "resid_pos", "route_key"):
        assert outs[0][name].tobytes() == outs[1][name].tobytes(), name
    out = outs[0]
    for s in (1, 2, 4):
        assert not out["u"][s].any() and not out["anchor_k"][s].any() and not out["resid_pos"][s].any()
    om = inp.omega
    for b, s in ((0, 5), (2, 0), (3, 3)):
        for h in range(2):
            ref = S.seal_block(inp.k[b, h], inp.v[b, h], 32, 40, om, 2)
            _compare_block(out, s, h, inp.k[b, h], inp.v[b, h], ref, 32, 40, inp.outliers[b, h])


def test_seal_degenerate_blocks(lib):
    say("[seal] exactly low-rank, constant and fully residual blocks")
    rng = np.random.default_rng(2200)
    inp = synth.make_seal_input(2200, 3, 1, width=24, n_outliers=0, noise=0.0, true_rank=6)
    # block 1: every row equal (A = 0); block 2: keep it, sealed with R = 255 below
    inp.k[1, 0] = inp.k[1, 0, :1]
    inp.v[1, 0] = inp.v[1, 0, :1]
    out, om = _seal_gpu(lib, inp, 16, 0, 2)
    # exactly rank-6 delta (up to the fp16 rounding of the rows): reproduced
    _, _, a = S.joint_delta(inp.k[0, 0], inp.v[0, 0])
    u = out["u"][0, 0].astype(np.float64)
    rec = np.hstack([u @ out["vk"][0, 0].astype(np.float64), u @ out["vv"][0, 0].astype(np.float64)])
    assert np.linalg.norm(rec - a) <= 3e-3 * np.linalg.norm(a)
    ref = S.seal_block(inp.k[0, 0], inp.v[0, 0], 16, 0, om, 2)
    _compare_block(out, 0, 0, inp.k[0, 0], inp.v[0, 0], ref, 16, 0)
    # constant block: zero delta, zero factors
    assert not out["u"][1, 0].astype(np.float64).any()
    assert out["anchor_k"][1, 0].tobytes() == inp.k[1, 0, 0].tobytes()
    # every position residual: the block is reproduced exactly
    full, _ = _seal_gpu(lib, synth.make_seal_input(2201, 1, 1, width=24), 16, 255, 2)
    src = synth.make_seal_input(2201, 1, 1, width=24)
    sealed = {k2: full[k2][0, 0] for k2 in ("anchor_k", "anchor_v", "u", "vk", "vv", "resid_k", "resid_v",
                                            "resid_pos")}
    assert list(sealed["resid_pos"]) == list(range(1, 256))
    rk, rv = S.reconstruct(sealed)
    assert np.array_equal(rk, src.k[0, 0].astype(np.float64)) and np.array_equal(rv, src.v[0, 0].astype(np.float64))
    del rng


def test_sealed_blocks_decode_like_the_oracle(lib):
    # a sequence of 14 blocks sealed on the GPU and decoded on the GPU, against
    # the oracle's decode of the oracle's sealing (every block routed, K = 14)
    say("[seal] seal 14 blocks, then decode them")
    nb, H, G, W = 14, 2, 6, 64
    inp = synth.make_seal_input(2300, nb, H, width=40)
    rank, R = 32, 40
    out, om = _seal_gpu(lib, inp, rank, R, 2)
    ref_pool = {n: np.zeros_like(out[n]) for n in ("anchor_k", "anchor_v", "u", "vk", "vv", "resid_k",
                                                     "resid_v", "resid_pos")}
    for b in range(nb):
        for h in range(H):
            r = S.seal_block(inp.k[b, h], inp.v[b, h], rank, R, om, 2)
            for n in ref_pool:
                ref_pool[n][b, h] = r[n]
    rng = np.random.default_rng(2301)
    q = rng.standard_normal((1, H * G, 128)).astype(np.float16)
    win_k = rng.standard_normal((1, H, W, 128)).astype(np.float16)
    win_v = rng.standard_normal((1, H, W, 128)).astype(np.float16)
    table = np.arange(nb, dtype=np.int32)[None]
    nblk = np.array([nb], np.int32)
    wlen = np.array([W], np.int32)
    scale = 128 ** -0.5
    o_ref, lse_ref, _ = oracle.decode(ref_pool, q, win_k, win_v, table, nblk, wlen, H, nb, scale)
    gpu_pool = lib.Pool.from_numpy({n: out[n] for n in ref_pool}, DEV)
    batch = lib.Batch.from_numpy(q, win_k, win_v, table, nblk, wlen, device=DEV)
    lib.route_keys(gpu_pool)
    o, lse, _ = lib.decode(gpu_pool, batch, nb, scale)
    torch.cuda.synchronize()
    d_o = np.max(np.abs(o.cpu().numpy().astype(np.float64) - o_ref))
    d_l = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref))
    say(f"[seal]   decode max |d out| {d_o:.2e}, max |d lse| {d_l:.2e}")
    assert d_o <= 1e-2 and d_l <= 1e-3


def test_seal_full_layer_sampled(lib):
    # the benchmark's sealing launch: one layer's 1008 blocks x 2 KV heads of
    # the 64k batch-4 stack at rank 48 (R = 128, q = 2); sampled blocks against
    # the oracle, every block's anchor and residual rows checked as copies
    say("[seal] one layer of the 64k stack (2016 block-heads), sampled against the oracle")
    nb, H, rank, R = 4 * 252, 2, 48, 128
    inp = synth.make_seal_input(3000, nb, H, width=rank + 8)
    out, om = _seal_gpu(lib, inp, rank, R, 2)
    assert np.array_equal(out["anchor_k"], inp.k[:, :, 0]) and np.array_equal(out["anchor_v"], inp.v[:, :, 0])
    pos = out["resid_pos"].astype(np.int64)
    assert np.all(np.diff(pos, axis=-1) > 0) and pos.min() >= 1 and pos.max() <= 255
    rows = np.take_along_axis(inp.k, pos[..., None], axis=2)
    assert np.array_equal(out["resid_k"], rows)
    for b in (0, 333, 777, nb - 1):
        for h in range(H):
            ref = S.seal_block(inp.k[b, h], inp.v[b, h], rank, R, om, 2)
            _compare_block(out, b, h, inp.k[b, h], inp.v[b, h], ref, rank, R)


@pytest.mark.parametrize("variant", ["U", "UB"])
def test_join_basis(lib, variant):
    """dkv_join_basis against the oracle's join: U' = U V_cur V_g^T and the
    retained energy, scored first without writing, then written; an item out of
    range changes nothing."""
    from compressed_kv_cache_amd import synth
    wl = synth.make_config(1, variant=variant)
    lay = wl.layers[0]
    P = lay.pool()
    pool = lib.Pool.from_numpy(P, DEV)
    n_entries = P["vk"].shape[0]
    slots = np.array([0, 1, 2, 3, 4, 5, 6], dtype=np.int32)
    entries = np.array([7, 9, 2, 11, 13, 20, n_entries], dtype=np.int32)   # the last one is out of range
    ts, te = torch.from_numpy(slots).to(DEV), torch.from_numpy(entries).to(DEV)
    u0 = pool.tensors["u"].clone()
    e0 = lib.join_basis(pool, ts, te, write=False)
    torch.cuda.synchronize()
    assert torch.equal(pool.tensors["u"], u0)
    e1 = lib.join_basis(pool, ts, te, write=True)
    torch.cuda.synchronize()
    assert torch.equal(e0, e1)
    e1 = e1.cpu().numpy()
    u1 = pool.tensors["u"].cpu().numpy()
    for i, (s, g) in enumerate(zip(slots, entries)):
        for h in range(wl.n_kv_heads):
            if g >= n_entries:
                assert e1[i, h] == -1.0
                assert np.array_equal(u1[s, h], u0[s, h].cpu().numpy())
                continue
            cur = int(P["basis_of"][s]) if "basis_of" in P else int(s)
            ref_u, ref_e = S.join_basis(P["u"][s, h], P["vk"][cur, h], P["vv"][cur, h], P["vk"][g, h],
                                                 P["vv"][g, h])
            got = u1[s, h].astype(np.float64)
            assert np.all(np.abs(got - ref_u) <= 1e-3 * np.abs(ref_u) + 1e-5 * np.abs(ref_u).max()), (i, h)
            assert abs(e1[i, h] - ref_e) <= 1e-4, (i, h, e1[i, h], ref_e)
            if g == cur:
                # its own basis (joint rows of V_K, V_V not orthonormal here: the
                # synthetic bases are orthonormal in K and in V separately)
                assert abs(e1[i, h] - 1.0) <= 1e-4, (i, h, e1[i, h])


def _related_pool(seed, n, H, r, related):
    """n blocks of H KV heads with random orthonormal joint bases [V_K | V_V],
    except that block i in `related` takes block i - 1's subspace (a random
    rotation of its basis plus a little noise): fp16 pool arrays."""
    rng = np.random.default_rng(seed)
    u = (rng.standard_normal((n, H, 255, r)) * np.linspace(2.0, 0.5, r)).astype(np.float16)
    W = np.zeros((n, H, r, 256))
    for i in range(n):
        for h in range(H):
            if i in related:
                Qr, _ = np.linalg.qr(rng.standard_normal((r, r)))
                w = Qr @ W[i - 1, h] + 1e-3 * rng.standard_normal((r, 256))
            else:
                w = rng.standard_normal((r, 256))
            W[i, h] = np.linalg.qr(w.T)[0].T
    W = W.astype(np.float16)
    z = np.zeros((n, H, 128), np.float16)
    return dict(anchor_k=z, anchor_v=z.copy(), u=u, vk=np.ascontiguousarray(W[..., :128]),
                vv=np.ascontiguousarray(W[..., 128:]), resid_k=np.zeros((n, H, 0, 128), np.float16),
                resid_v=np.zeros((n, H, 0, 128), np.float16), resid_pos=np.zeros((n, H, 0), np.uint8))


@pytest.mark.parametrize("capacity,threshold", [(12, 0.9), (5, 0.9), (3, 0.5), (1, 2.0)])
def test_share_bases_against_oracle(lib, capacity, threshold):
    """dkv_share_bases against the oracle's policy (assign_bases) on blocks in a
    shuffled seal order, some of which can join an earlier block's basis almost
    losslessly: the same kinds and entries (a forced join may pick another entry
    only within 1e-4 of the best energy), the energies, the joined U, and the
    store holding each opener's basis bit for bit."""
    n, H, r = 12, 2, 16
    related = {1, 2, 5, 8, 11}
    P = _related_pool(2024, n, H, r, related)
    order = np.random.default_rng(7).permutation(n).astype(np.int32)      # seal order (blocks)
    slot_of = np.random.default_rng(8).permutation(n).astype(np.int32)    # block i lives in slot slot_of[i]
    arrays = {k: (v[np.argsort(slot_of)] if v.shape[0] == n else v) for k, v in P.items()}
    pool = lib.Pool.from_numpy(arrays, DEV)
    slots = slot_of[order]
    store_vk, store_vv, entry, opener, energy, kind = lib.share_bases(pool, slots, capacity, threshold)
    torch.cuda.synchronize()
    blocks = [(P["u"][i].astype(np.float64), P["vk"][i].astype(np.float64), P["vv"][i].astype(np.float64))
              for i in order]
    e_ref, op_ref, us_ref, en_ref, kd_ref = S.assign_bases(blocks, capacity, threshold)
    say(f"[share bases] capacity {capacity} threshold {threshold}: kinds {list(kind)} entries {len(opener)}")
    assert list(kind) == list(kd_ref)
    assert list(opener) == list(slots[op_ref])
    u_gpu = pool.tensors["u"].cpu().numpy()
    for i in range(n):
        if kind[i] == 2 and entry[i] != e_ref[i]:
            _, e_alt = zip(*[S.join_basis(blocks[i][0][h], blocks[i][1][h], blocks[i][2][h],
                                          blocks[op_ref[entry[i]]][1][h], blocks[op_ref[entry[i]]][2][h])
                             for h in range(H)])
            assert abs(np.mean(e_alt) - en_ref[i]) <= 1e-4, (i, entry[i], e_ref[i])
            continue
        assert entry[i] == e_ref[i], (i, entry[i], e_ref[i])
        assert abs(energy[i] - en_ref[i]) <= 1e-4, (i, energy[i], en_ref[i])
        got = u_gpu[slots[i]].astype(np.float64)
        ref = us_ref[i]
        assert np.all(np.abs(got - ref) <= 2e-3 * np.abs(ref) + 2e-3 * np.abs(ref).max()), i
    # the store: entry j holds its opener's basis, bit for bit
    svk, svv = store_vk.cpu().numpy(), store_vv.cpu().numpy()
    for j, s in enumerate(opener):
        blk = int(np.where(slot_of == s)[0][0])
        assert np.array_equal(svk[j], P["vk"][blk]) and np.array_equal(svv[j], P["vv"][blk])
    assert len(opener) <= capacity


@pytest.mark.parametrize("fmt,bits", [(1, 8), (2, 4)])
def test_seal_quantised_residuals(lib, fmt, bits):
    """Sealing into a pool of 8- or 4-bit residual rows: the positions are the
    fp16 sealing's (same kernel path), and the codes and (scale, bias) pairs
    equal the oracle's quantisation of those rows bit for bit; the sealed blocks
    then decode like the oracle's."""
    say(f"[seal] {bits}-bit residual rows")
    nb, H, G, W = 14, 2, 6, 64
    inp = synth.make_seal_input(2400 + bits, nb, H, width=40)
    rank, R = 32, 40
    ref16, om = _seal_gpu(lib, inp, rank, R, 2)
    out, _ = _seal_gpu(lib, inp, rank, R, 2, resid_format=fmt)
    assert np.array_equal(out["resid_pos"], ref16["resid_pos"]) and np.array_equal(out["u"], ref16["u"])
    for b in range(nb):
        for h in range(H):
            pos = out["resid_pos"][b, h].astype(np.int64)
            for n, src in (("k", inp.k), ("v", inp.v)):
                codes, sb = S.quantize_rows(src[b, h][pos], bits)
                assert np.array_equal(out[f"resid_{n}"][b, h], codes), (b, h, n)
                assert out[f"resid_{n}_sb"][b, h].tobytes() == sb.tobytes(), (b, h, n)
    # decode the quantised pool against the oracle's decode of the same arrays
    rng = np.random.default_rng(2401)
    q = rng.standard_normal((1, H * G, 128)).astype(np.float16)
    win_k = rng.standard_normal((1, H, W, 128)).astype(np.float16)
    win_v = rng.standard_normal((1, H, W, 128)).astype(np.float16)
    table = np.arange(nb, dtype=np.int32)[None]
    nblk = np.array([nb], np.int32)
    wlen = np.array([W], np.int32)
    scale = 128 ** -0.5
    P = {n: out[n] for n in ("anchor_k", "anchor_v", "u", "vk", "vv", "resid_k", "resid_v", "resid_pos",
                             "resid_k_sb", "resid_v_sb")}
    P["resid_format"] = fmt
    o_ref, lse_ref, _ = oracle.decode(P, q, win_k, win_v, table, nblk, wlen, H, nb, scale)
    gpu_pool = lib.Pool.from_numpy(P, DEV)
    batch = lib.Batch.from_numpy(q, win_k, win_v, table, nblk, wlen, device=DEV)
    lib.route_keys(gpu_pool)
    o, lse, _ = lib.decode(gpu_pool, batch, nb, scale)
    torch.cuda.synchronize()
    d_o = np.max(np.abs(o.cpu().numpy().astype(np.float64) - o_ref))
    d_l = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref))
    say(f"[seal]   decode max |d out| {d_o:.2e}, max |d lse| {d_l:.2e}")
    assert d_o <= 1e-2 and d_l <= 1e-3

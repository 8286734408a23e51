"""Pins of the block-sealing oracle (oracle/dkv_sealer.py) against things other
than itself: numpy's exact SVD and the Eckart-Young theorem, exact recovery of
low-rank inputs, brute force on small cases, and the planted structure of the
synthetic blocks.  CPU only."""
import numpy as np
import pytest

from compressed_kv_cache_amd import synth
from oracle import dkv_sealer as S


def _rank_k(rng, k, shape=(255, 256)):
    return rng.standard_normal((shape[0], k)) @ rng.standard_normal((k, shape[1]))


def test_exact_low_rank_input_is_recovered():
    # a rank-10 matrix lies in the range of A omega for any Gaussian omega of
    # width >= 10, so the rank-12 factors reproduce it exactly
    rng = np.random.default_rng(1)
    a = _rank_k(rng, 10)
    for q in (0, 1, 2):
        us, s, wt = S.randomized_svd(a, 12, rng.standard_normal((256, 20)), q)
        assert np.max(np.abs(us @ wt - a)) < 1e-10 * np.max(np.abs(a))
        assert np.all(s[10:] < 1e-9 * s[0])


def test_singular_values_and_eckart_young():
    # on the synthetic blocks (decaying spectrum), q = 2 power iterations give
    # the top singular values of numpy's exact SVD and a truncation error
    # within 1% of the optimal one, sum of sigma_j^2 over j >= r
    inp = synth.make_seal_input(7, 2, 2, width=40)
    for b in range(2):
        for h in range(2):
            _, _, a = S.joint_delta(inp.k[b, h], inp.v[b, h])
            sig = np.linalg.svd(a, compute_uv=False)
            us, s, wt = S.randomized_svd(a, 32, inp.omega, 2)
            # the singular values of Q^T A interlace those of A: never above
            # them; near r the spectrum is flat (sigma_31 / sigma_40 ~ 1.4), so
            # q = 2 leaves them within 3e-2, and q = 4 within 1e-3
            assert np.all(s <= sig[:32] * (1 + 1e-12)) and np.all(s >= sig[:32] * (1 - 3e-2))
            opt = np.sum(sig[32:] ** 2)
            err = np.sum((a - us @ wt) ** 2)
            assert opt <= err <= 1.01 * opt
            _, s4, _ = S.randomized_svd(a, 32, inp.omega, 4)
            assert np.all(s4 <= sig[:32] * (1 + 1e-12)) and np.all(s4 >= sig[:32] * (1 - 1e-3))


def test_power_iterations_do_not_hurt():
    inp = synth.make_seal_input(8, 1, 1, width=24)
    _, _, a = S.joint_delta(inp.k[0, 0], inp.v[0, 0])
    errs = []
    for q in (0, 1, 2):
        us, _, wt = S.randomized_svd(a, 16, inp.omega, q)
        errs.append(np.sum((a - us @ wt) ** 2))
    assert errs[2] <= errs[1] * (1 + 1e-9) and errs[1] <= errs[0] * (1 + 1e-9)


def test_basis_rows_are_orthonormal_and_us_carries_the_singular_values():
    inp = synth.make_seal_input(9, 1, 1, width=40)
    _, _, a = S.joint_delta(inp.k[0, 0], inp.v[0, 0])
    us, s, wt = S.randomized_svd(a, 32, inp.omega, 2)
    np.testing.assert_allclose(wt @ wt.T, np.eye(32), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(us, axis=0), s, rtol=1e-12)
    # the columns of U S are orthogonal (left singular vectors times sigma)
    g = us.T @ us
    assert np.max(np.abs(g - np.diag(np.diag(g)))) < 1e-9 * s[0] ** 2


def test_anchor_delta_and_copies():
    inp = synth.make_seal_input(10, 1, 1, width=40)
    k, v = inp.k[0, 0], inp.v[0, 0]
    a_k, a_v, a = S.joint_delta(k, v)
    assert np.array_equal(a_k, k[0].astype(np.float64)) and np.array_equal(a_v, v[0].astype(np.float64))
    assert np.array_equal(a[:, :128], k[1:].astype(np.float64) - k[0].astype(np.float64))
    assert np.array_equal(a[:, 128:], v[1:].astype(np.float64) - v[0].astype(np.float64))
    out = S.seal_block(k, v, 32, 40, inp.omega)
    assert out["anchor_k"].tobytes() == k[0].tobytes() and out["anchor_v"].tobytes() == v[0].tobytes()
    pos = out["resid_pos"].astype(np.int64)
    assert np.all(np.diff(pos) > 0) and pos[0] >= 1 and pos[-1] <= 255
    assert out["resid_k"].tobytes() == k[pos].tobytes() and out["resid_v"].tobytes() == v[pos].tobytes()
    assert out["u"].dtype == np.float16 and out["u"].shape == (255, 32)
    assert out["vk"].shape == (32, 128) and out["vv"].shape == (32, 128)


def test_residual_errors_and_selection_by_brute_force():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((256, 128)).astype(np.float16)
    a_k = k[0]
    u = (rng.standard_normal((255, 3)) * 0.3).astype(np.float16)
    vk = rng.standard_normal((3, 128)).astype(np.float16)
    err = S.residual_errors(k, a_k, u, vk)
    for i in (1, 17, 255):
        tot = 0.0
        for c in range(128):
            rec = float(a_k[c]) + sum(float(u[i - 1, j]) * float(vk[j, c]) for j in range(3))
            tot += (float(k[i, c]) - rec) ** 2
        assert abs(err[i - 1] - tot ** 0.5) < 1e-12 * max(1.0, tot ** 0.5)
    # selection: the largest errors, equal errors to the lower position
    e = np.array([1.0, 5.0, 3.0, 5.0, 2.0, 5.0])
    assert list(S.select_residuals(e, 2)) == [2, 4]
    assert list(S.select_residuals(e, 4)) == [2, 3, 4, 6]
    e = rng.random(255)
    want = sorted(np.argsort(-e, kind="stable")[:40] + 1)
    assert list(S.select_residuals(e, 40)) == want


def test_planted_outliers_become_residuals():
    # the planted rows carry N(0, 0.35^2) noise of their own, less energy than
    # any of the top 32 components: a rank-32 basis leaves them out, so they
    # are the worst-reconstructed keys
    inp = synth.make_seal_input(11, 2, 2, width=40)
    for b in range(2):
        for h in range(2):
            out = S.seal_block(inp.k[b, h], inp.v[b, h], 32, 16, inp.omega)
            assert set(inp.outliers[b, h].tolist()) <= set(out["resid_pos"].tolist())


def test_full_residual_budget_reproduces_the_block():
    inp = synth.make_seal_input(12, 1, 1, width=24)
    k, v = inp.k[0, 0], inp.v[0, 0]
    out = S.seal_block(k, v, 16, 255, inp.omega)
    rk, rv = S.reconstruct(out)
    assert np.array_equal(rk, k.astype(np.float64)) and np.array_equal(rv, v.astype(np.float64))


@pytest.mark.parametrize("rank", [8, 24, 48])
def test_reconstruction_error_matches_the_truncation(rank):
    # the stored (fp16) factors reconstruct the non-residual rows about as well
    # as the exact rank-r truncation (fp16 storage adds ~1e-3 relative)
    inp = synth.make_seal_input(13, 1, 1, width=rank + 8)
    k, v = inp.k[0, 0], inp.v[0, 0]
    _, _, a = S.joint_delta(k, v)
    sig = np.linalg.svd(a, compute_uv=False)
    out = S.seal_block(k, v, rank, 0, inp.omega)
    rk, rv = S.reconstruct(out)
    x = np.hstack([k, v]).astype(np.float64)
    err = np.sum((x - np.hstack([rk, rv])) ** 2)
    opt = np.sum(sig[rank:] ** 2)
    assert opt <= err <= 1.02 * opt + 1e-3 * np.sum(a ** 2) * 1e-3


def _orth_rows(rng, r, n=256):
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q.T


def test_join_to_own_or_rotated_basis_keeps_everything():
    rng = np.random.default_rng(21)
    V = _orth_rows(rng, 12)
    U = rng.standard_normal((255, 12))
    up, e = S.join_basis(U, V[:, :128], V[:, 128:], V[:, :128], V[:, 128:])
    np.testing.assert_allclose(up, U, atol=1e-12)
    assert abs(e - 1.0) < 1e-12
    Q, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    Vg = Q @ V                                    # another basis of the same subspace
    up, e = S.join_basis(U, V[:, :128], V[:, 128:], Vg[:, :128], Vg[:, 128:])
    np.testing.assert_allclose(up @ Vg, U @ V, atol=1e-11)
    assert abs(e - 1.0) < 1e-12


def test_join_is_the_least_squares_projection():
    rng = np.random.default_rng(22)
    V, Vg = _orth_rows(rng, 10), _orth_rows(rng, 10)
    U = rng.standard_normal((255, 10))
    up, e = S.join_basis(U, V[:, :128], V[:, 128:], Vg[:, :128], Vg[:, 128:])
    # the best X with X Vg ~ U V in the least-squares sense (numpy's solver)
    X = np.linalg.lstsq(Vg.T, (U @ V).T, rcond=None)[0].T
    np.testing.assert_allclose(up, X, atol=1e-10)
    # orthogonal subspaces keep nothing; random ones about r / 256 of the energy
    W = _orth_rows(rng, 20)
    up0, e0 = S.join_basis(U, W[:10, :128], W[:10, 128:], W[10:, :128], W[10:, 128:])
    assert np.abs(up0).max() < 1e-12 and e0 < 1e-24
    assert 0.0 < e < 0.2


def test_join_energy_closed_form_at_interior_values():
    """V_g shares the first k of the block's basis rows and replaces the rest by
    rows orthogonal to all of V: the join keeps exactly the first k columns of
    U, so the retained energy is their share of |U|^2 (V orthonormal)."""
    rng = np.random.default_rng(23)
    r, k = 12, 5
    W = _orth_rows(rng, 2 * r)                 # 24 orthonormal rows
    V = W[:r]
    Vg = np.vstack([W[:k], W[r:r + (r - k)]])
    U = rng.standard_normal((255, r)) * (0.9 ** np.arange(r))
    up, e = S.join_basis(U, V[:, :128], V[:, 128:], Vg[:, :128], Vg[:, 128:])
    want = np.sum(U[:, :k] ** 2) / np.sum(U ** 2)
    assert 0.5 < want < 0.9                    # an interior value
    assert abs(e - want) < 1e-12
    np.testing.assert_allclose(up[:, :k], U[:, :k], atol=1e-12)
    np.testing.assert_allclose(up[:, k:], 0.0, atol=1e-12)


def test_join_energy_is_the_pages_trace_ratio():
    """For V_g with orthonormal rows the energy equals tr(G C C^T) / tr(G V V^T)
    with G = U^T U and C = V V_g^T (README "3. Shared Low-Rank Bases"), at
    interior values: V_g mixes the block's rows with new directions."""
    rng = np.random.default_rng(24)
    r = 10
    V = _orth_rows(rng, r)
    for t in (0.2, 0.5, 0.8):
        N = _orth_rows(rng, r)
        # rows of V_g: orthonormal rows spanning a mix of V and N
        Vg = np.linalg.qr((np.sqrt(1 - t) * V + np.sqrt(t) * N).T)[0].T
        U = rng.standard_normal((255, r)) * (0.8 ** np.arange(r))
        _, e = S.join_basis(U, V[:, :128], V[:, 128:], Vg[:, :128], Vg[:, 128:])
        G = U.T @ U
        C = V @ Vg.T
        want = np.trace(G @ C @ C.T) / np.trace(G @ V @ V.T)
        assert 0.05 < want < 0.98
        assert abs(e - want) < 1e-10


def test_join_with_a_basis_whose_rows_are_not_orthonormal():
    """V_K and V_V orthonormal each (joint Gram 2 I), or V_g any full-rank r x 256
    matrix: U' is numpy's least-squares solution of X V_g = U V, and joining to
    the block's own basis keeps U and all of the energy."""
    rng = np.random.default_rng(25)
    r = 8
    vk, vv = _orth_rows(rng, r, 128), _orth_rows(rng, r, 128)
    U = rng.standard_normal((255, r))
    up, e = S.join_basis(U, vk, vv, vk, vv)
    np.testing.assert_allclose(up, U, atol=1e-12)
    assert abs(e - 1.0) < 1e-12
    V = np.hstack([vk, vv])
    Vg = rng.standard_normal((r, 256))
    up, e = S.join_basis(U, vk, vv, Vg[:, :128], Vg[:, 128:])
    X = np.linalg.lstsq(Vg.T, (U @ V).T, rcond=None)[0].T
    np.testing.assert_allclose(up, X, atol=1e-10)
    assert abs(e - np.sum((X @ Vg) ** 2) / np.sum((U @ V) ** 2)) < 1e-12


# ---------------------------------------------------------------------------
# Shared bases under a budget (assign_bases)
# ---------------------------------------------------------------------------

def _blocks(seed, n, H=2, r=6, related=()):
    """n random blocks (orthonormal joint basis rows); block i in `related`
    takes block i - 1's subspace (its basis turned by a random rotation, plus
    a little noise), so that it can join that block's entry almost losslessly."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        u = rng.standard_normal((H, 255, r))
        if i in related:
            _, vk0, vv0 = out[i - 1]
            vk, vv = [], []
            for h in range(H):
                Qr, _ = np.linalg.qr(rng.standard_normal((r, r)))
                W = Qr @ np.hstack([vk0[h], vv0[h]]) + 1e-3 * rng.standard_normal((r, 256))
                W = np.linalg.qr(W.T)[0].T
                vk.append(W[:, :128])
                vv.append(W[:, 128:])
            vk, vv = np.stack(vk), np.stack(vv)
        else:
            W = np.stack([np.linalg.qr(rng.standard_normal((256, r)))[0].T for _ in range(H)])
            vk, vv = W[:, :, :128], W[:, :, 128:]
        out.append((u, vk, vv))
    return out


def _energy_lstsq(b, g):
    """Retained energy of block b on block g's basis, by numpy's least squares
    (an independent route to join_basis's U'), mean over heads."""
    u, vk, vv = b
    _, vkg, vvg = g
    es = []
    for h in range(len(u)):
        V = np.hstack([vk[h], vv[h]])
        Vg = np.hstack([vkg[h], vvg[h]])
        X = np.linalg.lstsq(Vg.T, (u[h] @ V).T, rcond=None)[0].T
        es.append(np.sum((X @ Vg) ** 2) / np.sum((u[h] @ V) ** 2))
    return float(np.mean(es))


def test_assign_bases_brute_force():
    """Every decision against a brute-force replay: the energies of each block
    to every entry open at that time by least squares, the best entry, and the
    rule (voluntary at or above the threshold, a new entry while there is room,
    else forced); the store never exceeds its capacity."""
    blocks = _blocks(5, 9, related=(1, 2, 5, 8))
    for capacity, thr in ((9, 0.9), (3, 0.9), (2, 0.5), (1, 0.99), (4, 1.5)):
        entry, opener, us, energy, kind = S.assign_bases(blocks, capacity, thr)
        assert len(opener) <= capacity
        open_now = []
        for i, b in enumerate(blocks):
            es = [_energy_lstsq(b, blocks[o]) for o in open_now]
            best = int(np.argmax(es)) if es else -1
            if es and es[best] >= thr:
                assert kind[i] == 1 and entry[i] == best and abs(energy[i] - es[best]) < 1e-9
            elif len(open_now) < capacity:
                assert kind[i] == 0 and entry[i] == len(open_now) and opener[len(open_now)] == i
                open_now.append(i)
                assert np.array_equal(us[i], b[0])
            else:
                assert kind[i] == 2 and entry[i] == best and abs(energy[i] - es[best]) < 1e-9
            if kind[i] != 0:
                # the joined U reproduces the least-squares projection onto the entry's basis
                _, vkg, vvg = blocks[opener[entry[i]]]
                for h in range(2):
                    Vg = np.hstack([vkg[h], vvg[h]])
                    V = np.hstack([b[1][h], b[2][h]])
                    X = np.linalg.lstsq(Vg.T, (b[0][h] @ V).T, rcond=None)[0].T
                    assert np.allclose(us[i][h], X, atol=1e-9)


def test_assign_bases_special_cases():
    blocks = _blocks(11, 6, related=(3,))
    # room for everyone and a threshold no energy reaches: every block opens an entry
    entry, opener, _, energy, kind = S.assign_bases(blocks, 6, 1.01)
    assert list(kind) == [0] * 6 and list(entry) == list(range(6)) and list(opener) == list(range(6))
    # one entry: every later block joins it (forced unless related enough)
    entry, opener, _, _, kind = S.assign_bases(blocks, 1, 2.0)
    assert list(opener) == [0] and list(entry) == [0] * 6 and list(kind) == [0] + [2] * 5
    # the related block joins its parent voluntarily, keeping almost all its energy
    entry, opener, _, energy, kind = S.assign_bases(blocks, 6, 0.9)
    assert kind[3] == 1 and entry[3] == entry[2] and energy[3] > 0.99
    assert all(kind[i] == 0 for i in (0, 1, 2, 4, 5))
    # an exact copy of a block keeps all its energy
    copy = [blocks[0], (blocks[0][0] * 1.5, blocks[0][1], blocks[0][2])]
    entry, _, us, energy, kind = S.assign_bases(copy, 2, 0.999)
    assert kind[1] == 1 and abs(energy[1] - 1.0) < 1e-12 and np.allclose(us[1], copy[1][0])
    with pytest.raises(ValueError):
        S.assign_bases(blocks, 0, 0.5)


# ---------------------------------------------------------------------------
# Writing residual rows in the 8- and 4-bit group-quantised format
# ---------------------------------------------------------------------------

from oracle.dkv_oracle import dequantize_rows   # noqa: E402  (the read side, pinned in test_oracle_pins)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_round_trip_within_half_step(bits):
    """Dequantised (by the read side) rows are within half a scale step of the
    fp16 rows, for rows of every spread and sign; the grid spans each group."""
    rng = np.random.default_rng(60 + bits)
    rows = np.vstack([rng.standard_normal((40, 128)) * sc + off
                      for sc, off in ((1, 0), (0.01, 3), (30, -100), (1e-3, 0))]).astype(np.float16)
    codes, sb = S.quantize_rows(rows, bits)
    assert codes.shape == (rows.shape[0], 128 if bits == 8 else 64) and sb.shape == (rows.shape[0], 2, 2)
    back = dequantize_rows(codes, sb, bits)
    step = np.repeat(sb[:, :, 0].astype(np.float64), 64, axis=1)
    assert np.all(np.abs(back - rows.astype(np.float64)) <= step / 2 * (1 + 1e-5) + 1e-12)
    L = (1 << bits) - 1
    x = rows.astype(np.float64)
    for g in range(2):
        lo, hi = x[:, 64 * g:64 * g + 64].min(1), x[:, 64 * g:64 * g + 64].max(1)
        assert np.array_equal(sb[:, g, 1].astype(np.float64), lo)               # bias: the group's minimum
        assert np.all(sb[:, g, 0].astype(np.float64) * L >= hi - lo)            # the grid reaches the maximum


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_codes_are_nearest(bits):
    """Each code is a nearest grid point: no neighbouring code reconstructs the
    value better (up to the fp32 rounding the decision is taken in)."""
    rng = np.random.default_rng(70 + bits)
    rows = (rng.standard_normal((64, 128)) * 2).astype(np.float16)
    codes, sb = S.quantize_rows(rows, bits)
    L = (1 << bits) - 1
    c = codes.astype(np.int64) if bits == 8 else np.stack([codes & 15, codes >> 4], -1).reshape(64, 128).astype(np.int64)
    s_ = np.repeat(sb[:, :, 0].astype(np.float64), 64, axis=1)
    b_ = np.repeat(sb[:, :, 1].astype(np.float64), 64, axis=1)
    x = rows.astype(np.float64)
    err = np.abs(x - (b_ + c * s_))
    for d in (-1, 1):
        cn = np.clip(c + d, 0, L)
        assert np.all(err <= np.abs(x - (b_ + cn * s_)) + 1e-6 * s_)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_rows_on_the_grid_are_exact(bits):
    """Rows that lie on a grid (fp16 bias, a power-of-two scale, codes 0 and L
    present) come back with that grid's scale, bias and codes exactly, and
    ties between two grid points go to the even code."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(80 + bits)
    s, b = 2.0 ** -6, -1.0
    c = rng.integers(0, L + 1, size=(8, 128))
    c[:, 0], c[:, 1], c[:, 64], c[:, 65] = 0, L, 0, L
    rows = (b + c * s).astype(np.float16)
    assert np.array_equal(rows.astype(np.float64), b + c * s)
    codes, sb = S.quantize_rows(rows, bits)
    assert np.all(sb[:, :, 0] == np.float16(s)) and np.all(sb[:, :, 1] == np.float16(b))
    got = codes.astype(np.int64) if bits == 8 else np.stack([codes & 15, codes >> 4], -1).reshape(8, 128)
    assert np.array_equal(got, c)
    # ties: halfway values round to the even code
    t = np.zeros((1, 128))
    t[0, :64] = b + np.array([0, L] + [2.5, 3.5, 4.5] * 20 + [1.0, 1.5])[:64] * s
    t[0, 64:] = b
    codes, sb = S.quantize_rows(t.astype(np.float16), bits)
    got = codes.astype(np.int64) if bits == 8 else np.stack([codes & 15, codes >> 4], -1).reshape(1, 128)
    assert list(got[0, 2:5]) == [2, 4, 4] and got[0, 63] == 2 and got[0, 62] == 1
    assert np.all(got[0, 64:] == 0) and sb[0, 1, 0] == 0                      # a constant group: scale 0


def test_quantize_nibble_order():
    """4-bit codes: dimension 2j in the low nibble of byte j, 2j + 1 in the high
    one (the read side's order), on a row whose codes are d mod 16."""
    d = np.arange(128)
    rows = (-2.0 + (d % 16) * 0.25)[None, :].astype(np.float16)
    codes, sb = S.quantize_rows(rows, 4)
    assert np.all(sb[0, :, 0] == np.float16(0.25)) and np.all(sb[0, :, 1] == np.float16(-2.0))
    want = ((2 * np.arange(64)) % 16) | (((2 * np.arange(64) + 1) % 16) << 4)
    assert np.array_equal(codes[0], want.astype(np.uint8))


def test_seal_block_quantised_residuals():
    """A block sealed with 8- or 4-bit residual rows stores the quantised fp16
    residual rows of the fp16 seal (same positions), and reconstructs within
    half a step of them."""
    inp = synth.make_seal_input(91, 1, 1, width=40)
    k, v = inp.k[0, 0], inp.v[0, 0]
    om = inp.omega[:, :40]
    ref = S.seal_block(k, v, 32, 24, om)
    for bits in (8, 4):
        q = S.seal_block(k, v, 32, 24, om, resid_bits=bits)
        assert np.array_equal(q["resid_pos"], ref["resid_pos"]) and np.array_equal(q["u"], ref["u"])
        ck, sk = S.quantize_rows(ref["resid_k"], bits)
        assert np.array_equal(q["resid_k"], ck) and np.array_equal(q["resid_k_sb"], sk)
        kk, _ = S.reconstruct(q)
        pos = ref["resid_pos"].astype(np.int64)
        step = np.repeat(q["resid_k_sb"][:, :, 0].astype(np.float64), 64, axis=1)
        assert np.all(np.abs(kk[pos] - ref["resid_k"].astype(np.float64)) <= step / 2 * (1 + 1e-5))

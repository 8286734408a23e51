"""fp64 CPU oracle for sealing a DKV block (the write side of the compressed cache).

TEST INFRASTRUCTURE ONLY.  Only tests, the package's smoke() check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never sees its outputs.

What it computes (sources are the pages on DKV, cited by title and section):

* Block layout -- "DKV: Anchor + Low-Rank Differential KV-Cache Compression for
  Scalable Long-Context Inference" (Zenodo record, abstract) and the
  Differential-KV README, "Core Architecture & Paper Overview", items 1-3: the
  first token of a 256-token block is the anchor (a_k, a_v), kept exact; the
  other 255 tokens are represented by a rank-r truncated SVD of the joint K|V
  delta, U in R^{255 x r} and V_K, V_V in R^{r x d}; a budget of R tokens is
  kept exact as residual rows.
* Residual selection -- README "Content-Aware / Rarity-Aware Residual
  Selection": plain DKV picks the residual tokens by the L2 reconstruction
  error of their key, the largest errors first (the content-aware boosts
  need token text and are not built).
* The SVD is randomised and seeded -- README "Key Environment Knobs"
  (DKV_SVD_SEED, the random state of the SVD) and the note on A/B method
  (the randomised SVD's seed is the axis to vary).  The steps are those of a
  randomised subspace iteration (Halko, Martinsson and Tropp, "Finding
  structure with randomness", the range finder with power iterations followed
  by the SVD of the small projected matrix).  The Gaussian test matrix is an
  input: the caller draws it from its seeded generator.

Readings where the pages are silent (listed in the design notes):
  the delta is taken relative to the anchor, A = [K[1:] - a_k | V[1:] - a_v]
  (255 x 256), and the singular values are folded into U; the oversampling p
  (test-matrix width r + p) and the number of power iterations q are
  arguments, with defaults p = 8 and q = 2; each orthonormalisation is a QR
  factorisation (any orthonormal basis of the same range gives the same
  result); the factors are stored as fp16 (round to nearest even) and the
  residual errors are measured against the reconstruction from those stored
  factors; equal errors go to the lower position; positions are stored in
  ascending order.

Every function is plain numpy in float64: inputs are upcast exactly from fp16.
Pins against things other than this code live in tests/test_oracle_sealer.py.
"""
from __future__ import annotations

import numpy as np

BLOCK = 256
D = 128
ROWS = BLOCK - 1

DEFAULT_OVERSAMPLE = 8
DEFAULT_POWER_ITERS = 2


def joint_delta(k: np.ndarray, v: np.ndarray):
    """Anchor and joint delta of one block: a_k = k[0], a_v = v[0] and
    A = [k[1:] - a_k | v[1:] - a_v] (README "Core Architecture", items 1-2)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    assert k.shape == (BLOCK, D) and v.shape == (BLOCK, D)
    a_k, a_v = k[0].copy(), v[0].copy()
    return a_k, a_v, np.hstack([k[1:] - a_k, v[1:] - a_v])


def _orth(x: np.ndarray) -> np.ndarray:
    q, _ = np.linalg.qr(x)
    return q


def randomized_svd(a: np.ndarray, rank: int, omega: np.ndarray, power_iters: int = DEFAULT_POWER_ITERS):
    """Rank-`rank` factors of `a` by randomised subspace iteration with the
    test matrix `omega` (n x l): Y = A omega, Q = orth(Y); q times Z =
    orth(A^T Q), Q = orth(A Z); then B = Q^T A = Ub S W^T (a small exact SVD)
    and A ~ (Q Ub_r) S_r W_r^T.  Returns (U S, singular values, W^T rows)."""
    a = np.asarray(a, np.float64)
    omega = np.asarray(omega, np.float64)
    assert omega.shape[0] == a.shape[1] and omega.shape[1] >= rank
    q = _orth(a @ omega)
    for _ in range(power_iters):
        z = _orth(a.T @ q)
        q = _orth(a @ z)
    b = q.T @ a
    ub, s, wt = np.linalg.svd(b, full_matrices=False)
    us = (q @ ub[:, :rank]) * s[:rank]
    return us, s[:rank], wt[:rank]


def _f16(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float16)


def residual_errors(k: np.ndarray, a_k: np.ndarray, u: np.ndarray, vk: np.ndarray) -> np.ndarray:
    """L2 error of each reconstructed key, e_i = |k_i - (a_k + U_{i-1} V_K)|
    for positions i = 1..255 (README, residual selection by reconstruction
    error), from the given (stored) factors."""
    k = np.asarray(k, np.float64)
    rec = np.asarray(a_k, np.float64) + np.asarray(u, np.float64) @ np.asarray(vk, np.float64)
    return np.sqrt(np.sum((k[1:] - rec) ** 2, axis=1))


def select_residuals(err: np.ndarray, n_resid: int) -> np.ndarray:
    """The n_resid positions (1-based in-block, 1..255) with the largest error,
    equal errors to the lower position, in ascending order."""
    err = np.asarray(err, np.float64)
    order = sorted(range(err.shape[0]), key=lambda i: (-err[i], i))
    return np.sort(np.array(order[:n_resid], dtype=np.int64) + 1)


def quantize_rows(rows, bits: int):
    """Residual rows into the 8- or 4-bit group-quantised format (README "2.
    Physical 4-Bit Group-Quantized Residual Buffers (INT4)" and "Tunable
    Quantization Dials": asymmetric groups of 64 dimensions, a half-precision
    scale and bias per group and row, unsigned codes; the layout
    dequantize_rows reads).  rows: fp16 [R][128].  Per row and group, with
    L = 2^bits - 1 and the group's smallest and largest values lo, hi:
        bias  = lo (an fp16 value already);
        scale = (hi - lo) / L in fp32, rounded up to fp16 (so the grid reaches
                hi);
        code  = round((x - bias) / scale) in fp32 (ties to even), clamped to
                [0, L]; 0 when the scale is 0 (a constant group).
    The codes are decided in fp32 (IEEE subtract and divide, as the kernel
    computes them), so both sides find the same integers.  Returns (codes uint8
    [R][128] for 8 bits, or [R][64] with dimension 2j in the low nibble of
    byte j for 4 bits; scale_bias fp16 [R][2][2] holding (scale, bias) per
    group)."""
    x = np.asarray(rows, np.float16).astype(np.float32)
    R = x.shape[0]
    L = np.float32((1 << bits) - 1)
    codes = np.zeros((R, D), np.uint8)
    sb = np.zeros((R, D // 64, 2), np.float16)
    for g in range(D // 64):
        xs = x[:, 64 * g:64 * (g + 1)]
        lo = xs.min(axis=1) if R else np.zeros(0, np.float32)
        hi = xs.max(axis=1) if R else np.zeros(0, np.float32)
        s32 = (hi - lo) / L                                   # fp32 subtract and divide
        s16 = s32.astype(np.float16)                          # nearest even ...
        up = s16.astype(np.float32) < s32                     # ... then up to the next fp16
        s16[up] = np.nextafter(s16[up], np.float16(np.inf))
        b16 = lo.astype(np.float16)
        sf, bf = s16.astype(np.float32), b16.astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (xs - bf[:, None]) / sf[:, None]             # fp32
        c = np.where(sf[:, None] > 0, np.clip(np.rint(q), 0, L), 0)
        codes[:, 64 * g:64 * (g + 1)] = c.astype(np.uint8)
        sb[:, g, 0], sb[:, g, 1] = s16, b16
    if bits == 8:
        return codes, sb
    if bits != 4:
        raise ValueError(f"bits {bits}")
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8), sb


def seal_block(k: np.ndarray, v: np.ndarray, rank: int, n_resid: int, omega: np.ndarray,
               power_iters: int = DEFAULT_POWER_ITERS, resid_bits: int = 16) -> dict:
    """One block (256 x 128 keys and values, fp16 values) sealed into the pool
    arrays of one slot and KV head: anchors, U (255 x r), V_K, V_V (r x 128),
    residual positions and rows (fp16, or with resid_bits 8 / 4 in the
    group-quantised format: codes in resid_k / resid_v, (scale, bias) in
    resid_k_sb / resid_v_sb).  Stored factors are fp16; `fp64` holds the
    unrounded factors and the singular values."""
    assert 1 <= rank <= min(ROWS, 2 * D) and 0 <= n_resid <= ROWS
    a_k, a_v, a = joint_delta(k, v)
    us, s, wt = randomized_svd(a, rank, omega, power_iters)
    u16, vk16, vv16 = _f16(us), _f16(wt[:, :D]), _f16(wt[:, D:])
    err = residual_errors(k, a_k, u16, vk16)
    pos = select_residuals(err, n_resid)
    k16, v16 = np.asarray(k, np.float16), np.asarray(v, np.float16)
    out = {
        "anchor_k": k16[0].copy(), "anchor_v": v16[0].copy(),
        "u": u16, "vk": vk16, "vv": vv16,
        "resid_pos": pos.astype(np.uint8),
        "resid_k": k16[pos].copy(), "resid_v": v16[pos].copy(),
        "err": err,
        "fp64": {"us": us, "s": s, "wt": wt},
    }
    if resid_bits in (8, 4):
        out["resid_k"], out["resid_k_sb"] = quantize_rows(k16[pos], resid_bits)
        out["resid_v"], out["resid_v_sb"] = quantize_rows(v16[pos], resid_bits)
    elif resid_bits != 16:
        raise ValueError(f"resid_bits {resid_bits}")
    return out


def reconstruct(sealed: dict):
    """Keys and values a sealed block stands for: the anchor, a + U V for the
    other positions, and the residual rows in place of their twins."""
    u = np.asarray(sealed["u"], np.float64)
    k = np.vstack([sealed["anchor_k"], np.asarray(sealed["anchor_k"], np.float64) + u @ np.asarray(sealed["vk"], np.float64)])
    v = np.vstack([sealed["anchor_v"], np.asarray(sealed["anchor_v"], np.float64) + u @ np.asarray(sealed["vv"], np.float64)])
    pos = np.asarray(sealed["resid_pos"], np.int64)
    if "resid_k_sb" in sealed:
        from .dkv_oracle import dequantize_rows
        bits = 8 if np.asarray(sealed["resid_k"]).shape[-1] == D else 4
        k[pos] = dequantize_rows(sealed["resid_k"], sealed["resid_k_sb"], bits)
        v[pos] = dequantize_rows(sealed["resid_v"], sealed["resid_v_sb"], bits)
    else:
        k[pos] = np.asarray(sealed["resid_k"], np.float64)
        v[pos] = np.asarray(sealed["resid_v"], np.float64)
    return k, v


def join_basis(u, vk, vv, vk_g, vv_g):
    """Join a block to a shared basis (README "Key Environment Knobs",
    DKV_SHARED_BASIS, and "3. Shared Low-Rank Bases": a joined block reads the
    group's basis instead of its own V, and keeps the part of its delta that
    the group's subspace can express).  With V = [V_K | V_V] and V_g = [V_K,g |
    V_V,g] (r x 256, linearly independent rows), U' is the least-squares
    solution of U' V_g = U V:

        U' = U V V_g^T (V_g V_g^T)^-1,

    which for rows of V_g that are orthonormal (a basis written by the sealer)
    is the pages' U' = U (V V_g^T).  The retained energy is |U' V_g|^2 /
    |U V|^2, the pages' tr(G C C^T) / tr(G V V^T) (G = U^T U, C = V V_g^T) for
    such a V_g; 1 when the subspaces agree.  Returns (U' [255 x r], retained
    energy), float64."""
    U = np.asarray(u, np.float64)
    V = np.hstack([np.asarray(vk, np.float64), np.asarray(vv, np.float64)])
    Vg = np.hstack([np.asarray(vk_g, np.float64), np.asarray(vv_g, np.float64)])
    M = V @ Vg.T
    up = np.linalg.solve(Vg @ Vg.T, (U @ M).T).T
    num = np.sum((up @ Vg) ** 2)
    den = np.sum((U @ V) ** 2)
    return up, (num / den if den > 0 else 1.0)


def assign_bases(blocks, capacity, threshold):
    """Shared bases under a budget (README "Key Environment Knobs",
    DKV_SHARED_BASIS and DKV_SHARED_BASIS_FRAC: the basis store is allocated
    as a fraction of the block slots; "3. Shared Low-Rank Bases": a block
    joins a basis voluntarily when the retained energy is high enough, and is
    forced to join once the store is full).  blocks: sealed blocks in seal
    order, each (u [H][255][r], vk [H][r][128], vv [H][r][128]) for its H KV
    heads, with its own basis.  Block i is scored against every entry of the
    store so far: the retained energy of joining entry j is the mean over the
    KV heads of join_basis's energy against the basis of the block that opened
    entry j.  With the best entry (largest energy, ties to the lower entry):
      - energy >= threshold: a voluntary join (block i reads entry j);
      - else, while the store holds fewer than `capacity` entries: block i
        opens a new entry holding its own basis;
      - else: a forced join to the best entry.
    A joined block's U becomes join_basis's U' (per head).  Returns (entry
    [n] (the store entry each block reads), opener [m] (the block that opened
    each entry), U list (per block, [H][255][r], U' for joined blocks),
    energy [n] (1 for a block that opened an entry), kind [n] (0 opened, 1
    voluntary, 2 forced))."""
    if capacity < 1:
        raise ValueError("capacity must be at least 1")
    n = len(blocks)
    entry = np.zeros(n, np.int64)
    energy = np.ones(n, np.float64)
    kind = np.zeros(n, np.int64)
    opener = []
    us = []
    for i, (u, vk, vv) in enumerate(blocks):
        H = len(u)
        best, best_e, best_u = -1, -np.inf, None
        for j, o in enumerate(opener):
            _, vk_g, vv_g = blocks[o]
            ups, es = [], []
            for h in range(H):
                up, e = join_basis(u[h], vk[h], vv[h], vk_g[h], vv_g[h])
                ups.append(up)
                es.append(e)
            e = float(np.mean(es))
            if e > best_e:
                best, best_e, best_u = j, e, ups
        if best >= 0 and best_e >= threshold:
            entry[i], energy[i], kind[i] = best, best_e, 1
            us.append(np.stack(best_u))
        elif len(opener) < capacity:
            entry[i] = len(opener)
            opener.append(i)
            us.append(np.asarray(u, np.float64))
        else:
            entry[i], energy[i], kind[i] = best, best_e, 2
            us.append(np.stack(best_u))
    return entry, np.asarray(opener, np.int64), us, energy, kind

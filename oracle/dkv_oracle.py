"""fp64 CPU oracle for DKV decode attention over a compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Only tests, the package's smoke() check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never sees its outputs.

What it computes (sources are the pages on DKV, cited by title and section):

* Block storage -- "DKV: Anchor + Low-Rank Differential KV-Cache Compression
  for Scalable Long-Context Inference" (Zenodo record, abstract) and the
  Differential-KV README, "Core Architecture & Paper Overview", items 1-3:
  a 256-token block keeps its first token exact as the anchor (a_k, a_v); the
  other 255 tokens are the anchor plus a row of a joint K|V low-rank delta,
  k_i = a_k + U_i V_K and v_i = a_v + U_i V_V with U in R^{255 x r}; R exact
  residual tokens are kept uncompressed at recorded in-block positions.
  Residual rows REPLACE their reconstructed twin (README, "Physical 4-Bit
  Group-Quantized Residual Buffers": the lossy SVD twin of a residual token is
  dropped).
* Decode -- Zenodo abstract and README "Decode & Prefill Innovations": route to
  the top-K blocks, score in low-rank space (the result equals attention over
  the reconstructed rows, which is what is written out here), attend residual
  rows and the dense recency window exactly, and merge the parts with an fp32
  log-sum-exp ("Flash-Style LSE Combine").
* Routing -- README "Key Environment Knobs": DKV_TOPK_BLOCKS picks the number of
  routed blocks; DKV_CB_GQA_ROUTE averages the query heads of one GQA group;
  DKV_CB_ROUTE_ALL scores every resident block.  The per-block routing key is
  the block's centroid key c = a_k + mean_i(U_i) V_K over all 255 rows of U
  (the pages keep per-block decode-router metadata, README "Per-Block Memory
  Breakdown"); ties go to the lowest logical block index.

* Residual storage formats -- README "Physical 4-Bit Group-Quantized Residual
  Buffers" and its "Tunable Quantization Dials": residual keys and values may
  be stored with asymmetric group quantisation, groups of 64 dimensions, 8 or
  4 bits, with a half-precision scale and bias per group; the decode attends
  the dequantised rows x = scale * code + bias.

* Un-rotated pools -- README "Key Environment Knobs" (DKV_ROTATED_POOL) and
  the preset ladder ("keys stored" column): a pool may hold the keys as they
  were before the rotary position embedding and rotate them to their absolute
  positions when they are read; values are never rotated, and the query and
  the dense window arrive rotated as usual.  A pool dict that carries
  "rope_base" and "slot_pos" (absolute position of token 0 of the block held
  in each slot) is such a pool.
* Shared basis -- README "Key Environment Knobs" (DKV_SHARED_BASIS and
  DKV_SHARED_BASIS_FRAC) and "3. Shared Low-Rank Bases": several blocks may
  use one stored V_K, V_V pair in place of one each; the pages allow this only
  for pools of un-rotated keys.  A pool dict that carries "basis_of" (per slot, the entry
  of vk / vv that holds the block's V_K and V_V) is such a pool; the block's
  own anchor, U and residual rows stay per slot.

Readings where the pages are silent (listed in the design notes):
  the anchor is attended as its own row at position 0; the delta is relative to
  the anchor with the singular values folded into U; the LSE is the natural log
  of the sum of exp of scaled scores z = scale * q.k; a sequence with no rows
  at all gives o = 0 and lse = -inf; routing scores are unscaled (scale does not
  change the order); quantised codes are unsigned (0 .. 2^bits - 1), 4-bit
  codes are packed two per byte with the even dimension in the low nibble (the
  little-endian order of the pages' uint32 words), and each row stores
  (scale, bias) for dimensions 0..63 then for 64..127; the rotary embedding
  pairs dimension j with j + d/2 (the half-split pairing of the Qwen and Llama
  models the pages run) at angular frequency base^(-2j/d); in an un-rotated
  pool the anchor sits at the block's position, row i at position + i, and a
  residual row at position + its in-block position, and the routing key is the
  mean of the 255 reconstructed keys each rotated to its own position.

Every function is plain numpy in float64: inputs are upcast exactly from fp16.
Pins against things other than this code live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 256
LOWRANK_ROWS = BLOCK_SIZE - 1


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Residual storage formats (README "Physical 4-Bit Group-Quantized Residual
# Buffers", "Tunable Quantization Dials")
# ---------------------------------------------------------------------------

RESID_FP16, RESID_INT8, RESID_INT4 = 0, 1, 2
QUANT_GROUP = 64
RESID_BITS = {RESID_INT8: 8, RESID_INT4: 4}


def dequantize_rows(codes, scale_bias, bits: int) -> np.ndarray:
    """Rows stored with asymmetric group quantisation: x[d] = scale[g] * code[d] +
    bias[g] with g = d // 64 and unsigned codes.  codes: uint8 [R][d] (8 bits)
    or [R][d / 2] (4 bits, dimension 2j in the low nibble of byte j and 2j + 1
    in the high nibble); scale_bias: fp16 [R][d / 64][2] holding (scale, bias).
    Returns float64 [R][d]."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        q = c.astype(np.float64)
    elif bits == 4:
        q = np.empty(c.shape[:-1] + (2 * c.shape[-1],))
        q[..., 0::2] = (c & 0x0F).astype(np.float64)
        q[..., 1::2] = (c >> 4).astype(np.float64)
    else:
        raise ValueError(f"bits {bits}")
    sb = _f64(scale_bias)
    n_groups = sb.shape[-2]
    assert q.shape[-1] == n_groups * QUANT_GROUP
    scale = np.repeat(sb[..., 0], QUANT_GROUP, axis=-1)
    bias = np.repeat(sb[..., 1], QUANT_GROUP, axis=-1)
    return scale * q + bias


def residual_rows(pool: Dict[str, np.ndarray], slot: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """Residual K and V rows of one block and KV head as float64 [R][d], in any
    of the storage formats."""
    fmt = int(pool.get("resid_format", RESID_FP16))
    if fmt == RESID_FP16:
        return _f64(pool["resid_k"][slot, h]), _f64(pool["resid_v"][slot, h])
    bits = RESID_BITS[fmt]
    return (dequantize_rows(pool["resid_k"][slot, h], pool["resid_k_sb"][slot, h], bits),
            dequantize_rows(pool["resid_v"][slot, h], pool["resid_v_sb"][slot, h], bits))


# ---------------------------------------------------------------------------
# Block reconstruction (README "Core Architecture & Paper Overview", items 1-3)
# ---------------------------------------------------------------------------

def route_key(anchor_k, u, vk) -> np.ndarray:
    """Routing key of one block and KV head: c = a_k + mean over the 255 rows of U,
    times V_K.  Shapes: a_k [d], U [255, r], V_K [r, d] -> [d]."""
    return _f64(anchor_k) + _f64(u).mean(axis=0) @ _f64(vk)


def rope_theta(base: float, d: int) -> np.ndarray:
    """Angular frequencies theta_j = base^(-2j/d) of the rotary embedding, j < d/2."""
    return float(base) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rope(x, pos, base: float) -> np.ndarray:
    """Rows x [n, d] rotated to absolute positions pos [n]: each pair
    (x_j, x_{j+d/2}) is turned by the angle pos * theta_j,
    x'_j = x_j cos - x_{j+d/2} sin and x'_{j+d/2} = x_{j+d/2} cos + x_j sin."""
    X = np.atleast_2d(_f64(x))
    h = X.shape[1] // 2
    ang = np.asarray(pos, dtype=np.float64).reshape(-1)[:, None] * rope_theta(base, X.shape[1])[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = X[:, :h], X[:, h:]
    return np.hstack([a * c - b * s, b * c + a * s])


def route_key_unrotated(anchor_k, u, vk, block_pos: int, base: float) -> np.ndarray:
    """Routing key of a block of an un-rotated pool: the mean over positions
    i = 1..255 of the reconstructed key a_k + U_i V_K rotated to block_pos + i."""
    K = _f64(anchor_k)[None, :] + _f64(u) @ _f64(vk)
    return rope(K, int(block_pos) + np.arange(1, BLOCK_SIZE), base).mean(axis=0)


def reconstruct_block(anchor_k, anchor_v, u, vk, vv, resid_k, resid_v, resid_pos
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Explicit K, V rows [256, d] of one block and KV head, in position order.

    Position 0 is the anchor; position i in 1..255 is a + U[i-1] V; each residual
    row t replaces position resid_pos[t].  Positions must be distinct in 1..255."""
    ak, av = _f64(anchor_k), _f64(anchor_v)
    U, VK, VV = _f64(u), _f64(vk), _f64(vv)
    K = np.empty((BLOCK_SIZE, ak.shape[0]))
    V = np.empty_like(K)
    K[0], V[0] = ak, av
    K[1:] = ak[None, :] + U @ VK
    V[1:] = av[None, :] + U @ VV
    pos = np.asarray(resid_pos, dtype=np.int64)
    if pos.size:
        if pos.min() < 1 or pos.max() > LOWRANK_ROWS or np.unique(pos).size != pos.size:
            raise ValueError("residual positions must be distinct values in 1..255")
        K[pos] = _f64(resid_k)
        V[pos] = _f64(resid_v)
    return K, V


def lowrank_rows(anchor_k, anchor_v, u, vk, vv, resid_pos) -> Tuple[np.ndarray, np.ndarray]:
    """The anchor row plus the reconstructed rows that are NOT residual positions
    (the low-rank part of a block), in position order."""
    ak, av = _f64(anchor_k), _f64(anchor_v)
    keep = np.ones(BLOCK_SIZE, dtype=bool)
    keep[np.asarray(resid_pos, dtype=np.int64)] = False
    K = np.concatenate([ak[None], ak[None] + _f64(u) @ _f64(vk)])
    V = np.concatenate([av[None], av[None] + _f64(u) @ _f64(vv)])
    return K[keep], V[keep]


# ---------------------------------------------------------------------------
# Attention and the log-sum-exp combine (README "Flash-Style LSE Combine")
# ---------------------------------------------------------------------------

def attend(q, k_rows, v_rows, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows q [G, d] over (k_rows, v_rows) [n, d].

    z = scale * q k^T; lse = log sum exp z (natural log); o = softmax(z) v.
    With n = 0: o = 0 and lse = -inf."""
    Q = np.atleast_2d(_f64(q))
    K, V = _f64(k_rows), _f64(v_rows)
    if K.shape[0] == 0:
        return np.zeros((Q.shape[0], V.shape[1] if V.ndim == 2 else Q.shape[1])), \
            np.full(Q.shape[0], -np.inf)
    z = scale * (Q @ K.T)                          # [G, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    o = (e @ V) / s
    lse = (m + np.log(s))[:, 0]
    return o, lse


def lse_merge(parts_o: Sequence[np.ndarray], parts_lse: Sequence[np.ndarray]
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Merge partials (o_j normalised, lse_j) of disjoint row sets.

    lse = M + log sum_j exp(lse_j - M) with M = max_j lse_j;
    o = sum_j exp(lse_j - lse) o_j.  Parts with lse = -inf carry no weight; if
    every part is empty the result is o = 0, lse = -inf."""
    O = np.stack([_f64(o) for o in parts_o])        # [P, ..., d]
    L = np.stack([_f64(x) for x in parts_lse])      # [P, ...]
    M = L.max(axis=0)
    empty = ~np.isfinite(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(L - Ms[None])
    s = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, s)))
    o = np.einsum("p...,p...d->...d", w, O) / np.where(empty, 1.0, s)[..., None]
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


# ---------------------------------------------------------------------------
# Routing (README "Key Environment Knobs": TOPK_BLOCKS, CB_GQA_ROUTE, CB_ROUTE_ALL)
# ---------------------------------------------------------------------------

def route(q_group, keys, top_k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Route one GQA group.  q_group [G, d], keys [N, d] (logical block order).

    The group's query heads are averaged, every block is scored by q_bar . c_j,
    and the K_eff = min(top_k, N) highest scores are kept; equal scores go to
    the lower block index.  Returns (indices ascending, all N scores)."""
    qbar = _f64(q_group).mean(axis=0)
    C = _f64(keys)
    n = C.shape[0]
    s = C @ qbar if n else np.zeros(0)
    k_eff = min(int(top_k), n)
    order = np.lexsort((np.arange(n), -s))         # score descending, then index ascending
    return np.sort(order[:k_eff]), s


# ---------------------------------------------------------------------------
# Whole decode step for one layer
# ---------------------------------------------------------------------------

def basis_entry(pool: Dict[str, np.ndarray], slot: int) -> int:
    """Entry of vk / vv holding the basis of the block in `slot` (the slot itself
    unless the pool shares bases)."""
    b = pool.get("basis_of")
    return int(slot) if b is None else int(b[slot])


def _slot_entry(pool: Dict[str, np.ndarray], slot: int, h: int) -> Dict[str, np.ndarray]:
    e = {k: pool[k][slot, h] for k in ("anchor_k", "anchor_v", "u", "resid_pos")}
    g = basis_entry(pool, slot)
    e["vk"], e["vv"] = pool["vk"][g, h], pool["vv"][g, h]
    e["resid_k"], e["resid_v"] = residual_rows(pool, slot, h)
    return e


def is_unrotated(pool: Dict[str, np.ndarray]) -> bool:
    return pool.get("rope_base") is not None


def block_route_key(pool: Dict[str, np.ndarray], slot: int, h: int) -> np.ndarray:
    """Routing key of the block in `slot`, KV head h, for either kind of pool."""
    vk = pool["vk"][basis_entry(pool, slot), h]
    if is_unrotated(pool):
        return route_key_unrotated(pool["anchor_k"][slot, h], pool["u"][slot, h], vk,
                                   int(pool["slot_pos"][slot]), float(pool["rope_base"]))
    return route_key(pool["anchor_k"][slot, h], pool["u"][slot, h], vk)


def block_rows(pool: Dict[str, np.ndarray], slot: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """Explicit K, V rows [256, d] of a block as attention sees them: in an
    un-rotated pool the keys are rotated to their absolute positions."""
    K, V = reconstruct_block(**_slot_entry(pool, slot, h))
    if is_unrotated(pool):
        K = rope(K, int(pool["slot_pos"][slot]) + np.arange(BLOCK_SIZE), float(pool["rope_base"]))
    return K, V


def route_batch(pool, q, block_table, n_blocks, n_kv_heads: int, top_k: int):
    """Routing of every (sequence, KV head).  Returns (idx [B][Hkv][top_k] padded
    with -1, list of per-(b, h) score vectors, list of per-(b, h) key matrices)."""
    B, Hq, _ = q.shape
    G = Hq // n_kv_heads
    idx = np.full((B, n_kv_heads, top_k), -1, dtype=np.int64)
    scores, keys_all = {}, {}
    for b in range(B):
        for h in range(n_kv_heads):
            nb = int(n_blocks[b])
            keys = np.stack([block_route_key(pool, int(block_table[b, j]), h) for j in range(nb)]) \
                if nb else np.zeros((0, q.shape[-1]))
            sel, s = route(q[b, h * G:(h + 1) * G], keys, top_k)
            idx[b, h, :sel.size] = sel
            scores[(b, h)] = s
            keys_all[(b, h)] = keys
    return idx, scores, keys_all


def decode(pool, q, win_k, win_v, block_table, n_blocks, win_len, n_kv_heads: int,
           top_k: int, scale: float, idx: Optional[np.ndarray] = None):
    """One decode step of one layer.

    For each sequence b and KV head h: route (unless `idx` [B][Hkv][>=K] is given,
    -1 entries ignored), reconstruct every routed block explicitly, append the
    first win_len[b] window rows, and attend each of the G query heads over all
    of these rows.  Returns (out [B][Hq][d], lse [B][Hq], idx used)."""
    B, Hq, d = q.shape
    G = Hq // n_kv_heads
    if idx is None:
        idx, _, _ = route_batch(pool, q, block_table, n_blocks, n_kv_heads, top_k)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(n_kv_heads):
            Ks: List[np.ndarray] = []
            Vs: List[np.ndarray] = []
            for j in idx[b, h]:
                if j < 0:
                    continue
                K, V = block_rows(pool, int(block_table[b, j]), h)
                Ks.append(K)
                Vs.append(V)
            w = int(win_len[b])
            Ks.append(_f64(win_k[b, h, :w]))
            Vs.append(_f64(win_v[b, h, :w]))
            o, l = attend(q[b, h * G:(h + 1) * G], np.concatenate(Ks), np.concatenate(Vs), scale)
            out[b, h * G:(h + 1) * G] = o
            lse[b, h * G:(h + 1) * G] = l
    return out, lse, idx


# ---------------------------------------------------------------------------
# Per-part partials (the split used by the library's per-kernel entry points)
# ---------------------------------------------------------------------------

def block_partials(pool, slot: int, h: int, q_group, scale: float):
    """(o, lse) of one block's low-rank part (anchor + unmasked reconstructed rows)
    and of its residual rows, for the query rows q_group [G, d]."""
    e = _slot_entry(pool, slot, h)
    Klr, Vlr = lowrank_rows(e["anchor_k"], e["anchor_v"], e["u"], e["vk"], e["vv"], e["resid_pos"])
    Kex = e["resid_k"]
    if is_unrotated(pool):
        base, p0 = float(pool["rope_base"]), int(pool["slot_pos"][slot])
        keep = np.ones(BLOCK_SIZE, dtype=bool)
        keep[np.asarray(e["resid_pos"], dtype=np.int64)] = False
        Klr = rope(Klr, p0 + np.flatnonzero(keep), base)
        Kex = rope(Kex, p0 + np.asarray(e["resid_pos"], dtype=np.int64), base)
    lr = attend(q_group, Klr, Vlr, scale)
    ex = attend(q_group, Kex, e["resid_v"], scale)
    return lr, ex


def window_partials(win_k, win_v, win_len, q, n_kv_heads: int, splits: int, scale: float):
    """Window partials: rows [s * c, min((s+1) * c, win_len)) with c = ceil(W / splits).
    Returns o [B][Hq][splits][d], lse [B][Hq][splits]."""
    B, Hq, d = q.shape
    W = win_k.shape[2]
    G = Hq // n_kv_heads
    c = -(-W // splits)
    o = np.zeros((B, Hq, splits, d))
    l = np.full((B, Hq, splits), -np.inf)
    for b in range(B):
        for h in range(n_kv_heads):
            for s in range(splits):
                a, e = s * c, min((s + 1) * c, int(win_len[b]))
                if e <= a:
                    continue
                oo, ll = attend(q[b, h * G:(h + 1) * G], win_k[b, h, a:e], win_v[b, h, a:e], scale)
                o[b, h * G:(h + 1) * G, s] = oo
                l[b, h * G:(h + 1) * G, s] = ll
    return o, l


def bytes_per_block(rank: int, n_resid: int, head_dim: int = 128, elem: int = 2,
                    resid_format: int = RESID_FP16) -> int:
    """Algorithmic bytes one routed block of one KV head streams at decode:
    anchors (2d), U (255 r), V_K and V_V (2 r d) in fp16, residual K and V rows
    (fp16, or codes plus an fp16 scale and bias per 64-dimension group), and one
    byte per residual position."""
    if resid_format == RESID_FP16:
        row = elem * head_dim
    else:
        row = head_dim * RESID_BITS[resid_format] // 8 + 4 * (head_dim // QUANT_GROUP)
    return elem * (2 * head_dim + LOWRANK_ROWS * rank + 2 * rank * head_dim) + 2 * n_resid * row + n_resid

"""Seeded synthetic compressed KV caches.

This module only draws random data in the storage format of a DKV cache
(anchor + rank-r joint K|V delta + exact residual rows per 256-token block,
plus a dense recency window and one decode query per sequence).  It holds
none of the method's arithmetic: no reconstruction, scoring, routing or
softmax.  Both the fp64 oracle (through the tests) and the GPU path read the
identical fp16 arrays produced here.

Storage format (per layer), following the DKV paper page (Zenodo record,
abstract) and the Differential-KV README ("Core Architecture & Paper
Overview"): each block of B_s = 256 tokens keeps its first token exact as the
anchor (a_k, a_v), a rank-r joint delta U in R^{255 x r} with bases V_K, V_V
in R^{r x d}, and R exact residual rows at recorded in-block positions.

Array shapes (S = pool slots, Hkv = KV heads, d = 128):
  anchor_k, anchor_v  fp16 [S][Hkv][d]
  u                   fp16 [S][Hkv][255][r]
  vk, vv              fp16 [S][Hkv][r][d]
  resid_k, resid_v    fp16 [S][Hkv][R][d]
  resid_pos           uint8 [S][Hkv][R], distinct values in 1..255, ascending
  q                   fp16 [B][Hq][d]
  win_k, win_v        fp16 [B][Hkv][W][d]
  block_table         int32 [B][max_blocks], pool slot of each logical block
  n_blocks            int32 [B]
  win_len             int32 [B]

Distributions (the workloads' stated recipe): anchors, queries, residual and
window rows ~ N(0, 1); U[:, j] ~ N(0, sigma_j^2) with sigma_j = s0 * decay^j;
V_K and V_V have orthonormal rows (transposed Q factor of a d x r Gaussian).
All values are drawn in float32 and rounded once to fp16 (round to nearest
even).

Quantised residual formats (README "Physical 4-Bit Group-Quantized Residual
Buffers", "Tunable Quantization Dials": groups of 64 dimensions, 8 or 4 bits,
an fp16 scale and bias per group).  The stored bytes are drawn directly:
  resid_k, resid_v        uint8 [S][Hkv][R][d] codes (8 bits), or
                          uint8 [S][Hkv][R][d/2], two 4-bit codes per byte
  resid_k_sb, resid_v_sb  fp16 [S][Hkv][R][d/64][2] = (scale, bias)
Codes are uniform; scales uniform in [0.012, 0.020] (8 bits) or [0.20, 0.30]
(4 bits) and biases ~ N(-2.0, 0.3) or N(-1.9, 0.2), so that the rows they
stand for span roughly [-2, 2].
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

HEAD_DIM = 128
BLOCK_SIZE = 256
LOWRANK_ROWS = BLOCK_SIZE - 1
QUANT_GROUP = 64
RESID_FP16, RESID_INT8, RESID_INT4 = 0, 1, 2


@dataclasses.dataclass
class Layer:
    rank: int
    anchor_k: np.ndarray
    anchor_v: np.ndarray
    u: np.ndarray
    vk: np.ndarray
    vv: np.ndarray
    resid_k: np.ndarray
    resid_v: np.ndarray
    resid_pos: np.ndarray
    q: np.ndarray
    win_k: np.ndarray
    win_v: np.ndarray
    resid_format: int = RESID_FP16
    resid_k_sb: Optional[np.ndarray] = None
    resid_v_sb: Optional[np.ndarray] = None
    # un-rotated pools: the rotary base and each slot's absolute position
    rope_base: Optional[float] = None
    slot_pos: Optional[np.ndarray] = None
    # shared basis: the vk / vv entry each slot reads (vk, vv then hold the bases)
    basis_of: Optional[np.ndarray] = None

    def pool(self) -> dict:
        """The block-store arrays as a plain dict (the oracle's input form)."""
        d = {k: getattr(self, k) for k in
             ("anchor_k", "anchor_v", "u", "vk", "vv", "resid_k", "resid_v", "resid_pos")}
        if self.resid_format != RESID_FP16:
            d["resid_format"] = self.resid_format
            d["resid_k_sb"] = self.resid_k_sb
            d["resid_v_sb"] = self.resid_v_sb
        if self.rope_base is not None:
            d["rope_base"] = self.rope_base
            d["slot_pos"] = self.slot_pos
        if self.basis_of is not None:
            d["basis_of"] = self.basis_of
        return d


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    n_resid: int
    top_k: int
    scale: float
    block_table: np.ndarray
    n_blocks: np.ndarray
    win_len: np.ndarray
    layers: List[Layer]
    seed: int
    notes: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_slots(self) -> int:
        return int(self.layers[0].anchor_k.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def _f16(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x.astype(np.float16))


_CHUNK = 1 << 22          # values per independently seeded chunk of a large draw


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:       # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(rng: np.random.Generator, shape, fill) -> np.ndarray:
    """Fill a float32 array of `shape` in fixed chunks along axis 0, each from its
    own child stream of `rng`, so the result does not depend on the thread count."""
    out = np.empty(shape, dtype=np.float32)
    if out.size == 0:
        return out
    per = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    rows = max(1, _CHUNK // max(per, 1))
    starts = list(range(0, shape[0], rows))
    kids = rng.spawn(len(starts))
    flat = out.reshape(shape[0], -1)

    def work(i):
        a = starts[i]
        b = min(shape[0], a + rows)
        fill(np.random.Generator(kids[i].bit_generator), flat[a:b])

    if len(starts) == 1:
        work(0)
    else:
        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def _normal(rng: np.random.Generator, shape, std=1.0) -> np.ndarray:
    def fill(g, view):
        g.standard_normal(dtype=np.float32, out=view)
    a = _chunked(rng, tuple(shape), fill)
    if std != 1.0:
        a *= np.asarray(std, dtype=np.float32)
    return a


def _orthonormal_rows(rng: np.random.Generator, lead: tuple, r: int, d: int) -> np.ndarray:
    """[..., r, d] with orthonormal rows: transposed Q factor of a d x r Gaussian."""
    n = int(np.prod(lead, dtype=np.int64))
    g = _normal(rng, (n, d, r))
    out = np.empty((n, r, d), dtype=np.float32)
    step = 512

    def work(a):
        qf, _ = np.linalg.qr(g[a:a + step])      # [k, d, r], orthonormal columns
        out[a:a + step] = np.swapaxes(qf, -1, -2)

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, n, step)))
    return out.reshape(lead + (r, d))


def _positions(rng: np.random.Generator, lead: tuple, n_resid: int, ascending: bool = False) -> np.ndarray:
    """n_resid distinct in-block positions from 1..255 per entry, in the seeded
    random order of the draw (the decode takes them in any order), or ascending."""
    if n_resid == 0:
        return np.zeros(lead + (0,), dtype=np.uint8)
    keys = rng.random(size=lead + (LOWRANK_ROWS,))
    pos = np.argsort(keys, axis=-1, kind="stable")[..., :n_resid] + 1
    if ascending:
        pos = np.sort(pos, axis=-1)
    return pos.astype(np.uint8)


def _quantised_residuals(rng: np.random.Generator, lead: tuple, n_resid: int, d: int, fmt: int):
    """Codes and (scale, bias) pairs of the K and V residual rows, drawn directly."""
    kids = rng.spawn(6)
    width = d if fmt == RESID_INT8 else d // 2
    lo, hi, mu, sd = (0.012, 0.020, -2.0, 0.3) if fmt == RESID_INT8 else (0.20, 0.30, -1.9, 0.2)
    out = []
    for i in range(2):
        codes = kids[3 * i].integers(0, 256, size=lead + (n_resid, width), dtype=np.uint8)
        sb = np.empty(lead + (n_resid, d // QUANT_GROUP, 2), dtype=np.float32)
        sb[..., 0] = kids[3 * i + 1].uniform(lo, hi, size=sb.shape[:-1])
        sb[..., 1] = kids[3 * i + 2].normal(mu, sd, size=sb.shape[:-1])
        out.append((np.ascontiguousarray(codes), _f16(sb)))
    return out


def make_layer(rng: np.random.Generator, *, n_slots: int, batch: int, n_q_heads: int,
               n_kv_heads: int, window: int, rank: int, n_resid: int,
               sigma0: float = 0.5, decay: float = 0.9, zero_anchor: bool = False,
               head_dim: int = HEAD_DIM, resid_format: int = RESID_FP16) -> Layer:
    """Draw one layer's pool, query and window with child streams in a fixed order."""
    d = head_dim
    streams = rng.spawn(9)
    lead = (n_slots, n_kv_heads)
    ak = _normal(streams[0], lead + (d,))
    av = _normal(streams[1], lead + (d,))
    if zero_anchor:
        ak[:] = 0.0
        av[:] = 0.0
    sig = (sigma0 * decay ** np.arange(rank)).astype(np.float32)
    u = _normal(streams[2], lead + (LOWRANK_ROWS, rank)) * sig
    vk = _orthonormal_rows(streams[3], lead, rank, d)
    vv = _orthonormal_rows(streams[4], lead, rank, d)
    ksb = vsb = None
    if resid_format == RESID_FP16:
        rk = _f16(_normal(streams[5], lead + (n_resid, d)))
        rv = _f16(_normal(streams[5], lead + (n_resid, d)))
    else:
        (rk, ksb), (rv, vsb) = _quantised_residuals(rng.spawn(1)[0], lead, n_resid, d, resid_format)
    pos = _positions(streams[6], lead, n_resid)
    q = _normal(streams[7], (batch, n_q_heads, d))
    wk = _normal(streams[8], (batch, n_kv_heads, window, d))
    wv = _normal(streams[8], (batch, n_kv_heads, window, d))
    return Layer(rank=rank, anchor_k=_f16(ak), anchor_v=_f16(av), u=_f16(u), vk=_f16(vk),
                 vv=_f16(vv), resid_k=rk, resid_v=rv, resid_pos=pos,
                 q=_f16(q), win_k=_f16(wk), win_v=_f16(wv), resid_format=resid_format,
                 resid_k_sb=ksb, resid_v_sb=vsb)


def make_workload(name: str, *, seed: int, batch: int, n_q_heads: int, n_kv_heads: int,
                  window: int, n_blocks: Sequence[int], ranks: Sequence[int], n_resid: int,
                  top_k: int, sigma0: float = 0.5, decay: float = 0.9,
                  permute_slots: bool = False, zero_anchor: bool = False,
                  win_len: Optional[Sequence[int]] = None, max_blocks: Optional[int] = None,
                  head_dim: int = HEAD_DIM, only_layers: Optional[Sequence[int]] = None,
                  notes: str = "", resid_format: int = RESID_FP16,
                  rope_base: Optional[float] = None) -> Workload:
    """Generic seeded workload: one Layer per entry of `ranks`.

    With `rope_base`, every layer's pool is an un-rotated one: its keys are
    read as pre-rotation keys, and slot_pos holds the absolute position of
    token 0 of each slot's block, BLOCK_SIZE times its logical index (the
    arrays drawn are the same either way).

    Sequence b owns n_blocks[b] logical blocks; their pool slots are
    consecutive (b-major) or a seeded permutation of all slots.  Every layer
    has its own child seed, so `only_layers` (a subset of layer indices)
    yields exactly the same arrays for those layers as the full stack.
    """
    ss = np.random.SeedSequence(seed)
    top, layer_seq = ss.spawn(2)
    trng = np.random.Generator(np.random.PCG64(top))
    nb = np.asarray(n_blocks, dtype=np.int32)
    assert nb.shape == (batch,)
    total = int(nb.sum())
    mb = int(max_blocks if max_blocks is not None else max(1, int(nb.max(initial=0))))
    slots = np.arange(total, dtype=np.int32)
    if permute_slots:
        slots = trng.permutation(total).astype(np.int32)
    table = np.full((batch, mb), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :nb[b]] = slots[off:off + nb[b]]
        off += int(nb[b])
    wl = np.full((batch,), window, dtype=np.int32) if win_len is None else np.asarray(win_len, np.int32)
    layers = []
    children = layer_seq.spawn(len(ranks))
    sel = range(len(ranks)) if only_layers is None else list(only_layers)
    for li in sel:
        lrng = np.random.Generator(np.random.PCG64(children[li]))
        layers.append(make_layer(lrng, n_slots=max(total, 1), batch=batch, n_q_heads=n_q_heads,
                                 n_kv_heads=n_kv_heads, window=window, rank=int(ranks[li]),
                                 n_resid=n_resid, sigma0=sigma0, decay=decay,
                                 zero_anchor=zero_anchor, head_dim=head_dim,
                                 resid_format=resid_format))
    out = Workload(name=name, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                   head_dim=head_dim, window=window, n_resid=n_resid, top_k=top_k,
                   scale=float(1.0 / np.sqrt(head_dim)), block_table=table, n_blocks=nb,
                   win_len=wl, layers=layers, seed=seed, notes=notes)
    if rope_base is not None:
        set_unrotated(out, rope_base)
    return out


def set_shared_basis(wl: Workload, group: int, seed: int = 0, compact: bool = False) -> Workload:
    """Let runs of `group` consecutive logical blocks of each sequence read one
    basis: the first block's V_K, V_V entry serves the run, so about 1/group of
    the entries are read, the pages' sharing fraction.  compact=False keeps
    every slot's entry in the arrays (the others unread); compact=True keeps
    only the entries that are read, so vk / vv shrink to n_basis entries (a
    basis store of its own, smaller than the slot count).  A seeded shuffle of
    the entries' order keeps a run's entry away from its own slots."""
    S = max(wl.n_slots, 1)
    pos = np.arange(S, dtype=np.int32)
    for b in range(wl.batch):
        nb = int(wl.n_blocks[b])
        for j in range(nb):
            pos[wl.block_table[b, j]] = wl.block_table[b, (j // group) * group]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 91, seed])))
    if compact:
        used = np.unique(pos)                                  # slots whose basis some block reads
        order = rng.permutation(used.size)
        keep = used[order]                                     # entry e holds slot keep[e]'s basis
        entry_of = np.full(S, -1, dtype=np.int64)
        entry_of[keep] = np.arange(keep.size)
        for lay in wl.layers:
            lay.vk = np.ascontiguousarray(lay.vk[keep])
            lay.vv = np.ascontiguousarray(lay.vv[keep])
            lay.basis_of = entry_of[pos].astype(np.int32)
        return wl
    perm = rng.permutation(S).astype(np.int32)
    for lay in wl.layers:
        lay.vk = np.ascontiguousarray(lay.vk[np.argsort(perm)])
        lay.vv = np.ascontiguousarray(lay.vv[np.argsort(perm)])
        lay.basis_of = perm[pos]
    return wl


def set_unrotated(wl: Workload, rope_base: float) -> Workload:
    """Read the workload's pools as un-rotated ones: record the rotary base and
    each slot's absolute position (BLOCK_SIZE times its logical block index)."""
    pos = np.zeros(max(wl.n_slots, 1), dtype=np.int32)
    for b in range(wl.batch):
        nb = int(wl.n_blocks[b])
        pos[wl.block_table[b, :nb]] = BLOCK_SIZE * np.arange(nb, dtype=np.int32)
    for lay in wl.layers:
        lay.rope_base = float(rope_base)
        lay.slot_pos = pos
    return wl


def plant_outlier_rows(wl: Workload, logical_block: int, n_rows: int = 8, rms: float = 4.0,
                       seq: int = 0, layer: int = 0) -> List[int]:
    """Rescale n_rows residual rows (K and V) of one block, in every KV head, to an
    l2 norm of rms * sqrt(d).  The rows are a seeded choice among the block's R
    residual rows.  Returns the chosen residual-row indices."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 77])))
    L = wl.layers[layer]
    slot = int(wl.block_table[seq, logical_block])
    rows = sorted(int(x) for x in rng.choice(wl.n_resid, size=n_rows, replace=False))
    target = rms * np.sqrt(wl.head_dim)
    for arr in (L.resid_k, L.resid_v):
        blk = arr[slot].astype(np.float32)               # [Hkv][R][d]
        for t in rows:
            nrm = np.linalg.norm(blk[:, t, :], axis=-1, keepdims=True)
            blk[:, t, :] = blk[:, t, :] * (target / nrm)
        arr[slot] = blk.astype(np.float16)
    return rows


# ---------------------------------------------------------------------------
# The five workloads and the sensitivity variants.  Seeds are 1000 + id.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "ctx4k_1head_r32_R40",
    1: "qwen2.5-1.5b_layer_ctx16k",
    2: "qwen2.5-1.5b_28layers_ctx64k_b4",
    3: "ragged_b32_ctx8k-32k",
    4: "llama3-8b_layer_ctx128k_b8",
}

# Rotary base of the un-rotated variants (the Qwen2.5 models' value).
ROPE_BASE = 1_000_000.0

# Layer-adaptive rank of the 28-layer stack: 0.75r early, 1.5r mid, 0.5r late (r = 32).
STACK_RANKS = [24] * 9 + [48] * 10 + [16] * 9


def ragged_lengths(seed: int, batch: int = 32, lo: int = 8192, hi: int = 32768) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    raw = rng.uniform(lo, hi, size=batch)
    return (BLOCK_SIZE * np.round(raw / BLOCK_SIZE)).astype(np.int64)


def make_config(cfg: int, seed: Optional[int] = None, layers: Optional[Sequence[int]] = None,
                variant: str = "") -> Workload:
    """Build configuration `cfg` (0..4).  `layers` selects a subset of the
    28-layer stack (config 2) to bound host memory; `variant` is one of
    "", "S1" (sigma_j = 4 * 0.9^j) or "S2" (zero anchors) for config 0, or
    "Q8" / "Q4" (residual rows in the 8- or 4-bit group-quantised format) for
    configs 0, 1 and 2, or "U" (the same arrays read as an un-rotated pool with
    rotary base ROPE_BASE) for any configuration, or "UB" (the U variant with
    pairs of consecutive blocks sharing one basis, a sharing fraction of 0.5),
    or "UC2" / "UC4" (the U variant with runs of 2 or 4 blocks sharing one
    basis, kept in a compact basis store of about n_slots / 2 or n_slots / 4
    entries)."""
    seed = 1000 + cfg if seed is None else seed
    if variant == "U":
        wl = make_config(cfg, seed, layers)
        wl.name += "_U"
        return set_unrotated(wl, ROPE_BASE)
    if variant == "UB":
        wl = make_config(cfg, seed, layers, "U")
        wl.name += "B"
        return set_shared_basis(wl, 2)
    if variant in ("UC2", "UC4"):
        wl = make_config(cfg, seed, layers, "U")
        wl.name += variant[1:]
        return set_shared_basis(wl, int(variant[2]), compact=True)
    if variant in ("Q8", "Q4"):
        fmt = RESID_INT8 if variant == "Q8" else RESID_INT4
        base = {0: dict(batch=1, n_q_heads=1, n_kv_heads=1, window=512, n_blocks=[14], ranks=[32],
                        n_resid=40, top_k=14),
                1: dict(batch=1, n_q_heads=12, n_kv_heads=2, window=1024, n_blocks=[60], ranks=[32],
                        n_resid=128, top_k=16),
                2: dict(batch=4, n_q_heads=12, n_kv_heads=2, window=1024, n_blocks=[252] * 4,
                        ranks=STACK_RANKS, n_resid=128, top_k=32, only_layers=layers)}[cfg]
        return make_workload(CONFIG_NAMES[cfg] + "_" + variant, seed=seed, resid_format=fmt, **base)
    if cfg == 0:
        sigma0 = 4.0 if variant == "S1" else 0.5
        return make_workload(CONFIG_NAMES[0] + (("_" + variant) if variant else ""), seed=seed,
                             batch=1, n_q_heads=1, n_kv_heads=1, window=512, n_blocks=[14],
                             ranks=[32], n_resid=40, top_k=14, sigma0=sigma0,
                             zero_anchor=(variant == "S2"))
    assert variant == ""
    if cfg == 1:
        return make_workload(CONFIG_NAMES[1], seed=seed, batch=1, n_q_heads=12, n_kv_heads=2,
                             window=1024, n_blocks=[60], ranks=[32], n_resid=128, top_k=16)
    if cfg == 2:
        return make_workload(CONFIG_NAMES[2], seed=seed, batch=4, n_q_heads=12, n_kv_heads=2,
                             window=1024, n_blocks=[252] * 4, ranks=STACK_RANKS, n_resid=128,
                             top_k=32, only_layers=layers)
    if cfg == 3:
        lens = ragged_lengths(seed)
        nb = (lens - 1024) // BLOCK_SIZE
        return make_workload(CONFIG_NAMES[3], seed=seed, batch=32, n_q_heads=12, n_kv_heads=2,
                             window=1024, n_blocks=nb.tolist(), ranks=[32], n_resid=128, top_k=32,
                             permute_slots=True)
    if cfg == 4:
        return make_workload(CONFIG_NAMES[4], seed=seed, batch=8, n_q_heads=32, n_kv_heads=8,
                             window=2048, n_blocks=[504] * 8, ranks=[32], n_resid=128, top_k=64,
                             decay=0.93)
    raise ValueError(f"unknown config {cfg}")


# ---------------------------------------------------------------------------
# Blocks to seal (the write side of the cache): the raw keys and values of
# 256-token blocks, and the Gaussian test matrix of the randomised SVD.
#
# Each (block, KV head) holds X = [K | V] (256 x 256): a per-block offset row
# ~ N(0, 1), plus a planted rank-`true_rank` part C W with C[:, j] ~
# N(0, sigma_j^2), sigma_j = s0 * decay^j, and W with orthonormal rows, plus
# N(0, noise^2) noise, plus N(0, outlier_std^2) added to `n_outliers`
# distinct rows among 1..255: tokens the low-rank part cannot hold (with the
# defaults a planted row carries less energy, 256 * 0.35^2 = 31, than the
# 32nd planted component, about 46, so a rank-32 basis does not spend a
# component on it, while its key error, about 4, is far above the others').  The
# test matrix is N(0, 1) in float32, [256][width].  Keys and values are
# rounded once to fp16.

@dataclasses.dataclass
class SealInput:
    k: np.ndarray          # fp16 [n_blocks][Hkv][256][128]
    v: np.ndarray          # fp16 [n_blocks][Hkv][256][128]
    omega: np.ndarray      # float32 [256][width]
    outliers: np.ndarray   # uint8 [n_blocks][Hkv][n_outliers], the planted rows


def make_seal_input(seed: int, n_blocks: int, n_kv_heads: int, *, width: int, true_rank: int = 48,
                    s0: float = 4.0, decay: float = 0.93, noise: float = 0.05, n_outliers: int = 8,
                    outlier_std: float = 0.35) -> SealInput:
    rng = np.random.default_rng(seed)
    streams = rng.spawn(6)
    lead = (n_blocks, n_kv_heads)
    two_d = 2 * HEAD_DIM
    x = _normal(streams[0], lead + (1, two_d)) + np.zeros(lead + (BLOCK_SIZE, two_d), np.float32)
    sig = (s0 * decay ** np.arange(true_rank)).astype(np.float32)
    c = _normal(streams[1], lead + (BLOCK_SIZE, true_rank)) * sig
    w = _orthonormal_rows(streams[2], lead, true_rank, two_d)
    x += np.matmul(c, w)
    x += _normal(streams[3], lead + (BLOCK_SIZE, two_d), noise)
    pos = _positions(streams[4], lead, n_outliers, ascending=True)
    bump = _normal(streams[5], lead + (n_outliers, two_d), outlier_std)
    for idx in np.ndindex(*lead):
        x[idx][pos[idx].astype(np.int64)] += bump[idx]
    omega = np.random.default_rng([seed, 1]).standard_normal((two_d, width), dtype=np.float32)
    return SealInput(k=_f16(x[..., :HEAD_DIM]), v=_f16(x[..., HEAD_DIM:]), omega=omega, outliers=pos)

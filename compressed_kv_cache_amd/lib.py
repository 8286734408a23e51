"""Thin Python binding of libdkv_attn (argument marshalling only).

Every computation runs in the HIP library; this module only fills the C structs
from torch tensors (device pointers, element strides), allocates output tensors
with torch, and passes torch's current HIP stream.  If the built library is
missing it raises instead of falling back to anything else.

Entry points mirror include/dkv_attn.h: route_keys, route_topk, lowrank_attn,
exact_attn, lse_merge, decode_workspace_size, decode.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdkv_attn.so")

HEAD_DIM = 128
BLOCK_SIZE = 256

DKV_OK = 0
DKV_ERR_INVALID_ARG = 1
DKV_ERR_UNSUPPORTED = 2
DKV_ERR_WORKSPACE = 3
DKV_ERR_HIP = 4

EXPORTED = ("dkv_status_string", "dkv_last_error", "dkv_abi_version", "dkv_route_keys",
            "dkv_route_topk", "dkv_lowrank_attn", "dkv_exact_attn", "dkv_lse_merge",
            "dkv_decode_workspace_size", "dkv_decode_workspace_init", "dkv_decode",
            "dkv_decode_profiled", "dkv_gather_route_keys", "dkv_decode_layers_table_size",
            "dkv_decode_layers_workspace_size", "dkv_decode_layers_prepare", "dkv_decode_layers",
            "dkv_seal_blocks", "dkv_rope_freqs", "dkv_join_basis", "dkv_decode_noalloc",
            "dkv_decode_noalloc_max_bytes", "dkv_decode_layers_profiled", "dkv_stream_read_probe",
            "dkv_share_bases")


class DKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("slot_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class PoolC(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("n_resid", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("anchor_k", View), ("anchor_v", View), ("u", View), ("vk", View), ("vv", View),
                ("resid_k", View), ("resid_v", View), ("resid_pos", View), ("route_key", View),
                ("resid_format", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("resid_k_sb", View), ("resid_v_sb", View),
                ("rope_freq", ctypes.c_void_p), ("slot_pos", ctypes.c_void_p),
                ("basis_of", ctypes.c_void_p), ("n_basis", ctypes.c_int32), ("reserved2", ctypes.c_int32)]

RESID_FP16, RESID_INT8, RESID_INT4 = 0, 1, 2


class BatchC(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("n_blocks", ctypes.c_void_p),
                ("win_len", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("win_k", ctypes.c_void_p), ("win_v", ctypes.c_void_p),
                ("route_keys", ctypes.c_void_p)]


class LayersPlanC(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_units", ctypes.c_int32), ("routes", ctypes.c_int32),
                ("parts", ctypes.c_int32), ("win_parts", ctypes.c_int32),
                ("group", ctypes.c_int32), ("n_items", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("max_tiles", ctypes.c_int32), ("quantised", ctypes.c_int32), ("unrotated", ctypes.c_int32),
                ("stream", ctypes.c_int32), ("stream_top_k", ctypes.c_int32),
                ("stream_items", ctypes.c_int32), ("stream_waves", ctypes.c_int32),
                ("stream_sched", ctypes.c_int32),
                ("table", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(PoolC)
    Bp = ctypes.POINTER(BatchC)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.dkv_status_string.argtypes = [i32]
    lib.dkv_status_string.restype = ctypes.c_char_p
    lib.dkv_last_error.argtypes = []
    lib.dkv_last_error.restype = ctypes.c_char_p
    lib.dkv_abi_version.argtypes = []
    lib.dkv_abi_version.restype = i32
    lib.dkv_route_keys.argtypes = [P, vp, i32, vp]
    lib.dkv_route_keys.restype = i32
    lib.dkv_rope_freqs.argtypes = [ctypes.c_double, i32, vp]
    lib.dkv_rope_freqs.restype = i32
    lib.dkv_join_basis.argtypes = [P, vp, vp, i32, i32, vp, vp]
    lib.dkv_join_basis.restype = i32
    lib.dkv_share_bases.argtypes = [P, vp, i32, i32, f32, View, View, vp, vp, vp, vp, vp, vp]
    lib.dkv_share_bases.restype = i32
    lib.dkv_route_topk.argtypes = [P, Bp, i32, vp, vp, vp]
    lib.dkv_gather_route_keys.argtypes = [P, Bp, vp, vp]
    lib.dkv_decode_layers_table_size.argtypes = [i32]
    lib.dkv_decode_layers_table_size.restype = ctypes.c_size_t
    lib.dkv_decode_layers_workspace_size.argtypes = [P, Bp, i32, i32]
    lib.dkv_decode_layers_workspace_size.restype = ctypes.c_size_t
    lib.dkv_decode_layers_prepare.argtypes = [P, Bp, i32, i32, f32, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                              ctypes.c_size_t, ctypes.POINTER(LayersPlanC)]
    lib.dkv_decode_layers_prepare.restype = i32
    lib.dkv_decode_layers.argtypes = [ctypes.POINTER(LayersPlanC), vp]
    lib.dkv_decode_layers.restype = i32
    lib.dkv_decode_layers_profiled.argtypes = [ctypes.POINTER(LayersPlanC), vp, vp]
    lib.dkv_decode_layers_profiled.restype = i32
    lib.dkv_stream_read_probe.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    lib.dkv_stream_read_probe.restype = i32
    lib.dkv_seal_blocks.argtypes = [P, View, View, vp, i32, vp, i32, i32, vp]
    lib.dkv_seal_blocks.restype = i32
    lib.dkv_gather_route_keys.restype = i32
    lib.dkv_route_topk.restype = i32
    lib.dkv_lowrank_attn.argtypes = [P, Bp, vp, i32, f32, vp, vp, i32, i32, vp]
    lib.dkv_lowrank_attn.restype = i32
    lib.dkv_exact_attn.argtypes = [P, Bp, vp, i32, i32, f32, vp, vp, i32, i32, vp]
    lib.dkv_exact_attn.restype = i32
    lib.dkv_lse_merge.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.dkv_lse_merge.restype = i32
    lib.dkv_decode_workspace_size.argtypes = [P, Bp, i32]
    lib.dkv_decode_workspace_size.restype = ctypes.c_size_t
    lib.dkv_decode_workspace_init.argtypes = [P, Bp, i32, vp, ctypes.c_size_t, vp]
    lib.dkv_decode_workspace_init.restype = i32
    lib.dkv_decode.argtypes = [P, Bp, i32, f32, vp, ctypes.c_size_t, vp, vp, vp, vp]
    lib.dkv_decode.restype = i32
    lib.dkv_decode_profiled.argtypes = [P, Bp, i32, f32, vp, ctypes.c_size_t, vp, vp, vp,
                                        ctypes.POINTER(ctypes.c_void_p), vp]
    lib.dkv_decode_profiled.restype = i32
    lib.dkv_decode_noalloc.argtypes = [P, Bp, i32, f32, vp, vp, vp, vp]
    lib.dkv_decode_noalloc.restype = i32
    lib.dkv_decode_noalloc_max_bytes.argtypes = []
    lib.dkv_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != DKV_OK:
        lib = load()
        raise DKVError(status, f"{what}: {lib.dkv_status_string(status).decode()}: "
                               f"{lib.dkv_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _torch_dtypes():
    import torch
    return {"<f2": torch.float16, "<f4": torch.float32, "|u1": torch.uint8, "<i4": torch.int32}


class _LazyDtypes(dict):
    def __missing__(self, key):
        self.update(_torch_dtypes())
        return dict.__getitem__(self, key)


_TORCH_DTYPE = _LazyDtypes()


def _view(t, dims_inside: int) -> View:
    """View of a tensor shaped [slots][heads][...inside...] (strides in elements)."""
    if t is None:
        return View(None, 0, 0)
    st = t.stride()
    return View(t.data_ptr(), st[0], st[1])


class Pool:
    """One layer's block pool on the device (torch tensors kept alive here).

    anchor_k, anchor_v fp16 [S][Hkv][128]; u fp16 [S][Hkv][255][r];
    vk, vv fp16 [S][Hkv][r][128]; resid_k, resid_v fp16 [S][Hkv][R][128], or
    uint8 codes [S][Hkv][R][128] (8-bit) / [S][Hkv][R][64] (4-bit) with
    resid_k_sb, resid_v_sb fp16 [S][Hkv][R][2][2]; resid_pos uint8 [S][Hkv][R];
    route_key fp32 [S][Hkv][128].
    Inner dimensions must be packed; outer (slot, head) strides are free."""

    def __init__(self, anchor_k, anchor_v, u, vk, vv, resid_k, resid_v, resid_pos, route_key,
                 resid_format: int = RESID_FP16, resid_k_sb=None, resid_v_sb=None):
        self.tensors = dict(anchor_k=anchor_k, anchor_v=anchor_v, u=u, vk=vk, vv=vv,
                            resid_k=resid_k, resid_v=resid_v, resid_pos=resid_pos,
                            route_key=route_key, resid_k_sb=resid_k_sb, resid_v_sb=resid_v_sb)
        S, Hkv = anchor_k.shape[0], anchor_k.shape[1]
        self.rank = int(u.shape[-1])
        self.n_resid = int(resid_k.shape[2])
        self.n_kv_heads = int(Hkv)
        self.n_slots = int(S)
        self.resid_format = int(resid_format)
        self.c = PoolC(HEAD_DIM, BLOCK_SIZE, self.rank, self.n_resid, self.n_kv_heads, self.n_slots,
                       _view(anchor_k, 1), _view(anchor_v, 1), _view(u, 2), _view(vk, 2),
                       _view(vv, 2), _view(resid_k, 2), _view(resid_v, 2), _view(resid_pos, 1),
                       _view(route_key, 1), self.resid_format, 0, _view(resid_k_sb, 3),
                       _view(resid_v_sb, 3))

    # per-(slot, head) record order: what a block's attention reads first comes first
    RECORD_ORDER = ("resid_pos", "vv", "anchor_v", "vk", "anchor_k", "u", "resid_k", "resid_v")
    RECORD_ORDER_Q = ("resid_pos", "vv", "anchor_v", "vk", "anchor_k", "u", "resid_k_sb", "resid_k",
                      "resid_v_sb", "resid_v")

    @classmethod
    def from_numpy(cls, arrays: dict, device="cuda", layout: str = "records"):
        """Upload one layer's pool.

        layout "records": all compressed arrays of one (slot, KV head) share one
        contiguous record (each piece 256-byte aligned), so a routed block is
        one contiguous read and one or two address translations.
        layout "arrays": one dense tensor per array.
        The routing key is a dense fp32 [S][Hkv][128] array in both layouts
        (routing reads it for every block of a sequence)."""
        import torch
        S, Hkv, d = arrays["anchor_k"].shape
        rk = torch.zeros((S, Hkv, d), dtype=torch.float32, device=device)
        fmt = int(arrays.get("resid_format", RESID_FP16))
        names = ("anchor_k", "anchor_v", "u", "vk", "vv", "resid_k", "resid_v", "resid_pos")
        order = cls.RECORD_ORDER
        if fmt != RESID_FP16:
            names = names + ("resid_k_sb", "resid_v_sb")
            order = cls.RECORD_ORDER_Q
        # a basis store smaller than the slot count (shared bases): V_K and V_V
        # live in arrays of their own, [n_basis][Hkv][r][128]; the records hold
        # the rest
        store = arrays.get("basis_of") is not None and arrays["vk"].shape[0] != S
        if store:
            order = tuple(k for k in order if k not in ("vk", "vv"))
        if layout == "arrays":
            t = {k: torch.from_numpy(arrays[k]).to(device) for k in names}
        elif layout == "records":
            offs, rec = {}, 0
            for k in order:
                offs[k] = rec
                nbytes = arrays[k][0, 0].nbytes if arrays[k].size else 0
                rec += (nbytes + 255) // 256 * 256
            rec = max(rec, 256)
            host = np.zeros((S, Hkv, rec), dtype=np.uint8)
            for k in order:
                a = np.ascontiguousarray(arrays[k])
                nb = a[0, 0].nbytes if a.size else 0
                if nb:
                    host[:, :, offs[k]:offs[k] + nb] = a.reshape(S, Hkv, -1).view(np.uint8).reshape(S, Hkv, nb)
            buf = torch.from_numpy(host).to(device)
            t = {}
            for k in names:
                a = arrays[k]
                if store and k in ("vk", "vv"):
                    t[k] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
                    continue
                dt = _TORCH_DTYPE[a.dtype.str]
                nb = a[0, 0].nbytes if a.size else 0
                if nb == 0:
                    t[k] = torch.empty(a.shape, dtype=dt, device=device)
                else:
                    t[k] = buf[:, :, offs[k]:offs[k] + nb].view(dt).unflatten(2, a.shape[2:])
            t["_record"] = buf
        else:
            raise ValueError(f"unknown pool layout {layout!r}")
        pool = cls(t["anchor_k"], t["anchor_v"], t["u"], t["vk"], t["vv"], t["resid_k"],
                   t["resid_v"], t["resid_pos"], rk, fmt, t.get("resid_k_sb"), t.get("resid_v_sb"))
        if "_record" in t:
            pool.tensors["_record"] = t["_record"]
        if arrays.get("rope_base") is not None:
            pool.set_unrotated(float(arrays["rope_base"]), arrays["slot_pos"])
        if arrays.get("basis_of") is not None:
            pool.set_shared_basis(arrays["basis_of"], int(arrays["vk"].shape[0]))
        return pool

    def set_shared_basis(self, basis_of, n_basis: int) -> None:
        """Let slot s read its V_K, V_V from entry basis_of[s] of vk / vv (an
        un-rotated pool only).  basis_of: int32 [n_slots], numpy or a device tensor."""
        import torch
        dev = self.tensors["anchor_k"].device
        b = basis_of if isinstance(basis_of, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(basis_of, dtype=np.int32))
        b = b.to(device=dev, dtype=torch.int32).contiguous()
        if b.numel() < self.n_slots:
            raise ValueError(f"basis_of has {b.numel()} entries for {self.n_slots} slots")
        self.tensors["basis_of"] = b
        self.c.basis_of, self.c.n_basis = b.data_ptr(), int(n_basis)

    def set_unrotated(self, rope_base: float, slot_pos) -> None:
        """Read this pool as an un-rotated one: keys are rotated at read to the
        absolute positions slot_pos[s] (+ in-block position), with the rotary
        frequencies of `rope_base` (table from dkv_rope_freqs).  slot_pos:
        int32 [n_slots], numpy or a device tensor."""
        import torch
        table = np.zeros(HEAD_DIM, dtype=np.float32)
        _check(load().dkv_rope_freqs(float(rope_base), HEAD_DIM, table.ctypes.data), "dkv_rope_freqs")
        dev = self.tensors["anchor_k"].device
        freq = torch.from_numpy(table).to(dev)
        pos = slot_pos if isinstance(slot_pos, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(slot_pos, dtype=np.int32))
        pos = pos.to(device=dev, dtype=torch.int32).contiguous()
        if pos.numel() < self.n_slots:
            raise ValueError(f"slot_pos has {pos.numel()} entries for {self.n_slots} slots")
        self.tensors["rope_freq"], self.tensors["slot_pos"] = freq, pos
        self.c.rope_freq, self.c.slot_pos = freq.data_ptr(), pos.data_ptr()

    @classmethod
    def empty(cls, n_slots: int, n_kv_heads: int, rank: int, n_resid: int, device="cuda",
              layout: str = "records", resid_format: int = RESID_FP16):
        """A zero-filled pool for dkv_seal_blocks to write into (residual rows
        fp16, or 8- / 4-bit codes with their (scale, bias) pairs)."""
        S, H, d = n_slots, n_kv_heads, HEAD_DIM
        arrays = dict(anchor_k=np.zeros((S, H, d), np.float16), anchor_v=np.zeros((S, H, d), np.float16),
                      u=np.zeros((S, H, BLOCK_SIZE - 1, rank), np.float16),
                      vk=np.zeros((S, H, rank, d), np.float16), vv=np.zeros((S, H, rank, d), np.float16),
                      resid_k=np.zeros((S, H, n_resid, d), np.float16),
                      resid_v=np.zeros((S, H, n_resid, d), np.float16),
                      resid_pos=np.zeros((S, H, n_resid), np.uint8))
        if resid_format != RESID_FP16:
            w = d if resid_format == RESID_INT8 else d // 2
            arrays.update(resid_k=np.zeros((S, H, n_resid, w), np.uint8), resid_v=np.zeros((S, H, n_resid, w), np.uint8),
                          resid_k_sb=np.zeros((S, H, n_resid, 2, 2), np.float16),
                          resid_v_sb=np.zeros((S, H, n_resid, 2, 2), np.float16), resid_format=resid_format)
        return cls.from_numpy(arrays, device, layout)

    @property
    def route_key(self):
        return self.tensors["route_key"]


class Batch:
    """One decode step's batch on the device.

    q fp16 [B][Hq][128]; win_k, win_v fp16 [B][Hkv][W][128]; block_table int32
    [B][max_blocks]; n_blocks int32 [B]; win_len int32 [B] or None."""

    def __init__(self, q, win_k, win_v, block_table, n_blocks, win_len=None, route_keys=None):
        self.tensors = dict(q=q, win_k=win_k, win_v=win_v, block_table=block_table,
                            n_blocks=n_blocks, win_len=win_len, route_keys=route_keys)
        B, Hq = int(q.shape[0]), int(q.shape[1])
        W = int(win_k.shape[2]) if win_k is not None else 0
        mb = int(block_table.shape[1]) if block_table is not None else 0
        self.batch, self.n_q_heads, self.window, self.max_blocks = B, Hq, W, mb
        self.c = BatchC(B, Hq, W, mb, _ptr(block_table), _ptr(n_blocks), _ptr(win_len), _ptr(q),
                        _ptr(win_k), _ptr(win_v), _ptr(route_keys))

    def set_route_keys(self, route_keys) -> None:
        """Attach (or with None detach) the per-sequence routing-key table
        fp32 [B][Hkv][max_blocks][128]."""
        self.tensors["route_keys"] = route_keys
        self.c.route_keys = _ptr(route_keys)

    @classmethod
    def from_numpy(cls, q, win_k, win_v, block_table, n_blocks, win_len=None, device="cuda"):
        import torch

        def up(a):
            return None if a is None else torch.from_numpy(a).to(device)
        return cls(up(q), up(win_k), up(win_v), up(block_table), up(n_blocks), up(win_len))


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def gather_route_keys(pool: Pool, batch: Batch, out=None, attach: bool = True, stream=None):
    """Per-sequence routing-key table (dkv_gather_route_keys); attached to the
    batch unless attach is False.  Returns the fp32 [B][Hkv][max_blocks][128] tensor."""
    import torch
    lib = load()
    if out is None:
        dev = batch.tensors["q"].device
        out = torch.empty((batch.batch, pool.n_kv_heads, batch.max_blocks, HEAD_DIM),
                          dtype=torch.float32, device=dev)
    saved = batch.c.route_keys
    batch.c.route_keys = None
    try:
        _check(lib.dkv_gather_route_keys(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(out),
                                         _stream(stream)), "dkv_gather_route_keys")
    finally:
        batch.c.route_keys = saved
    if attach:
        batch.set_route_keys(out)
    return out


def seal_blocks(pool: Pool, k, v, slots, omega, power_iters: int = 2, stream=None) -> None:
    """Seal blocks into pool slots (dkv_seal_blocks).  k, v: fp16 [n_blocks][Hkv][256][128]
    with contiguous rows; slots: int32 [n_blocks] on the device; omega: fp32 [256][width]."""
    import torch
    lib = load()
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.float16 or t.dim() != 4 or tuple(t.shape[2:]) != (BLOCK_SIZE, HEAD_DIM) \
                or t.stride(3) != 1 or t.stride(2) != HEAD_DIM:
            raise ValueError(f"{name} must be fp16 [n_blocks][Hkv][256][128] with contiguous rows")
    if slots.dtype != torch.int32 or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("slots must be int32, omega contiguous fp32 [256][width]")
    n = int(k.shape[0])
    _check(lib.dkv_seal_blocks(ctypes.byref(pool.c), _view(k, 2), _view(v, 2), _ptr(slots), n, _ptr(omega),
                               int(omega.shape[1]), int(power_iters), _stream(stream)), "dkv_seal_blocks")


def join_basis(pool: Pool, slots, entries, write: bool = True, stream=None):
    """Join the blocks in `slots` to the basis entries `entries` (dkv_join_basis):
    U' = U V V_g^T written in place when `write`; returns the retained energies,
    fp32 [n][Hkv] on the device.  slots, entries: int32 [n] device tensors."""
    import torch
    lib = load()
    if slots.dtype != torch.int32 or entries.dtype != torch.int32 or slots.numel() != entries.numel() \
            or not slots.is_contiguous() or not entries.is_contiguous():
        raise ValueError("slots and entries must be contiguous int32 tensors of one length")
    n = int(slots.numel())
    energy = torch.empty((n, pool.n_kv_heads), dtype=torch.float32, device=slots.device)
    _check(lib.dkv_join_basis(ctypes.byref(pool.c), _ptr(slots), _ptr(entries), n,
                              1 if write else 0, _ptr(energy), _stream(stream)), "dkv_join_basis")
    return energy


def share_bases(pool: Pool, slots, capacity: int, threshold: float, stream=None):
    """dkv_share_bases: assign the blocks in `slots` (host int sequence, seal
    order) to a basis store of `capacity` entries.  Returns (store_vk, store_vv
    device tensors [entries][Hkv][r][128], entry, opener, energy, kind numpy
    arrays).  The pool's U of joined blocks is rewritten in place."""
    import torch
    lib = load()
    dev = pool.tensors["vk"].device
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
    n = int(sl.size)
    cap = max(1, min(int(capacity), n))
    store_vk = torch.empty((cap, pool.n_kv_heads, pool.rank, HEAD_DIM), dtype=torch.float16, device=dev)
    store_vv = torch.empty_like(store_vk)
    entry = np.zeros(n, np.int32)
    opener = np.zeros(cap, np.int32)
    energy = np.zeros(n, np.float32)
    kind = np.zeros(n, np.int32)
    n_entries = ctypes.c_int32(0)
    _check(lib.dkv_share_bases(ctypes.byref(pool.c), sl.ctypes.data, n, int(capacity), float(threshold),
                               _view(store_vk, 2), _view(store_vv, 2), entry.ctypes.data, opener.ctypes.data,
                               energy.ctypes.data, kind.ctypes.data, ctypes.byref(n_entries), _stream(stream)),
           "dkv_share_bases")
    m = int(n_entries.value)
    return store_vk[:m], store_vv[:m], entry, opener[:m], energy, kind


def route_keys(pool: Pool, slots=None, stream=None) -> None:
    lib = load()
    n = 0 if slots is None else int(slots.numel())
    _check(lib.dkv_route_keys(ctypes.byref(pool.c), _ptr(slots), n, _stream(stream)), "dkv_route_keys")


def route_topk(pool: Pool, batch: Batch, top_k: int, with_scores: bool = False, stream=None):
    import torch
    lib = load()
    dev = batch.tensors["q"].device
    idx = torch.empty((batch.batch, pool.n_kv_heads, top_k), dtype=torch.int32, device=dev)
    sc = torch.empty((batch.batch, pool.n_kv_heads, top_k), dtype=torch.float32, device=dev) \
        if with_scores else None
    _check(lib.dkv_route_topk(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k, _ptr(idx),
                              _ptr(sc), _stream(stream)), "dkv_route_topk")
    return (idx, sc) if with_scores else idx


def _parts(batch: Batch, n_parts: int, part_o, part_lse, dev):
    import torch
    rows = batch.batch * batch.n_q_heads
    if part_o is None:
        part_o = torch.empty((rows, n_parts, HEAD_DIM), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((rows, n_parts), dtype=torch.float32, device=dev)
    return part_o, part_lse


def lowrank_attn(pool: Pool, batch: Batch, idx, top_k: int, scale: float, part_o=None,
                 part_lse=None, n_parts: Optional[int] = None, part_offset: int = 0, stream=None):
    lib = load()
    n_parts = top_k + part_offset if n_parts is None else n_parts
    part_o, part_lse = _parts(batch, n_parts, part_o, part_lse, batch.tensors["q"].device)
    _check(lib.dkv_lowrank_attn(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(idx), top_k,
                                scale, _ptr(part_o), _ptr(part_lse), n_parts, part_offset,
                                _stream(stream)), "dkv_lowrank_attn")
    return part_o, part_lse


def exact_attn(pool: Pool, batch: Batch, idx, top_k: int, window_splits: int, scale: float,
               part_o=None, part_lse=None, n_parts: Optional[int] = None, part_offset: int = 0,
               stream=None):
    lib = load()
    n_parts = top_k + window_splits + part_offset if n_parts is None else n_parts
    part_o, part_lse = _parts(batch, n_parts, part_o, part_lse, batch.tensors["q"].device)
    _check(lib.dkv_exact_attn(ctypes.byref(pool.c), ctypes.byref(batch.c), _ptr(idx), top_k,
                              window_splits, scale, _ptr(part_o), _ptr(part_lse), n_parts,
                              part_offset, _stream(stream)), "dkv_exact_attn")
    return part_o, part_lse


def lse_merge(part_o, part_lse, stream=None):
    import torch
    lib = load()
    rows, n_parts = int(part_lse.shape[0]), int(part_lse.shape[1])
    out = torch.empty((rows, HEAD_DIM), dtype=torch.float16, device=part_o.device)
    lse = torch.empty((rows,), dtype=torch.float32, device=part_o.device)
    _check(lib.dkv_lse_merge(_ptr(part_o), _ptr(part_lse), n_parts, rows, HEAD_DIM, _ptr(out),
                             _ptr(lse), _stream(stream)), "dkv_lse_merge")
    return out, lse


def decode_workspace_size(pool: Pool, batch: Batch, top_k: int) -> int:
    return int(load().dkv_decode_workspace_size(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k))


def alloc_workspace(pool: Pool, batch: Batch, top_k: int, stream=None):
    """A decode workspace, zero-filled and prepared by dkv_decode_workspace_init."""
    import torch
    n = max(decode_workspace_size(pool, batch, top_k), 256)
    ws = torch.zeros((n,), dtype=torch.uint8, device=batch.tensors["q"].device)
    _check(load().dkv_decode_workspace_init(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k, _ptr(ws), n,
                                            _stream(stream)), "dkv_decode_workspace_init")
    return ws


def decode(pool: Pool, batch: Batch, top_k: int, scale: float, workspace=None, out=None,
           out_lse=None, out_idx=None, return_idx: bool = True, stream=None):
    """One fused decode step.  Returns (out fp16 [B][Hq][128], lse fp32 [B][Hq], idx or None)."""
    import torch
    lib = load()
    dev = batch.tensors["q"].device
    if workspace is None:
        workspace = alloc_workspace(pool, batch, top_k)
    if out is None:
        out = torch.empty((batch.batch, batch.n_q_heads, HEAD_DIM), dtype=torch.float16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((batch.batch, batch.n_q_heads), dtype=torch.float32, device=dev)
    if out_idx is None and return_idx and top_k > 0:
        out_idx = torch.empty((batch.batch, pool.n_kv_heads, top_k), dtype=torch.int32, device=dev)
    _check(lib.dkv_decode(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k, scale,
                          _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                          _ptr(out), _ptr(out_lse), _ptr(out_idx), _stream(stream)), "dkv_decode")
    return out, out_lse, out_idx


def decode_noalloc(pool: Pool, batch: Batch, top_k: int, scale: float, out=None, out_lse=None, out_idx=None,
                   return_idx: bool = True, stream=None):
    """dkv_decode_noalloc: one fused decode step with the library's fixed scratch
    as its workspace.  Returns (out, lse, idx or None)."""
    import torch
    lib = load()
    dev = batch.tensors["q"].device
    if out is None:
        out = torch.empty((batch.batch, batch.n_q_heads, HEAD_DIM), dtype=torch.float16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((batch.batch, batch.n_q_heads), dtype=torch.float32, device=dev)
    if out_idx is None and return_idx and top_k > 0:
        out_idx = torch.empty((batch.batch, pool.n_kv_heads, top_k), dtype=torch.int32, device=dev)
    _check(lib.dkv_decode_noalloc(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k, scale, _ptr(out),
                                  _ptr(out_lse), _ptr(out_idx), _stream(stream)), "dkv_decode_noalloc")
    return out, out_lse, out_idx


def decode_profiled(pool: Pool, batch: Batch, top_k: int, scale: float, workspace, out, out_lse,
                    events, out_idx=None, stream=None) -> None:
    """dkv_decode plus two hipEvent_t records around its kernel (raw handles as ints)."""
    lib = load()
    arr = (ctypes.c_void_p * 2)(*events)
    _check(lib.dkv_decode_profiled(ctypes.byref(pool.c), ctypes.byref(batch.c), top_k, scale,
                                   _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                   _ptr(out), _ptr(out_lse), _ptr(out_idx), arr, _stream(stream)),
           "dkv_decode_profiled")


def read_probe(src, n_waves: int, sink, stream=None) -> None:
    """dkv_stream_read_probe over the bytes of device tensor `src` (a multiple of
    4096 * n_waves); sink: int32 or uint32 device tensor of n_waves words."""
    assert sink.numel() >= n_waves
    _check(load().dkv_stream_read_probe(_ptr(src), src.numel() * src.element_size(), n_waves, _ptr(sink),
                                        _stream(stream)), "dkv_stream_read_probe")


class Layers:
    """A prepared layer-batched decode (dkv_decode_layers_prepare): the fused
    decode steps of several layers in one launch per run().  Holds the device
    argument table, the workspace and the per-layer outputs."""

    def __init__(self, pools: Sequence[Pool], batches: Sequence[Batch], top_k: int, scale: float,
                 with_idx: bool = True):
        import torch
        lib = load()
        n = len(pools)
        assert n == len(batches) and n > 0
        self.pools, self.batches, self.top_k = list(pools), list(batches), top_k
        dev = batches[0].tensors["q"].device
        PA = (PoolC * n)(*[p.c for p in pools])
        BA = (BatchC * n)(*[b.c for b in batches])
        self.outs = [torch.empty((b.batch, b.n_q_heads, HEAD_DIM), dtype=torch.float16, device=dev)
                     for b in batches]
        self.lses = [torch.empty((b.batch, b.n_q_heads), dtype=torch.float32, device=dev) for b in batches]
        self.idxs = [torch.empty((b.batch, p.n_kv_heads, top_k), dtype=torch.int32, device=dev)
                     for p, b in zip(pools, batches)] if (with_idx and top_k > 0) else None
        tsz = lib.dkv_decode_layers_table_size(n)
        wsz = lib.dkv_decode_layers_workspace_size(PA, BA, n, top_k)
        self.table = torch.empty((max(tsz, 16),), dtype=torch.uint8, device=dev)
        self.workspace = torch.empty((max(wsz, 256),), dtype=torch.uint8, device=dev)
        vpa = ctypes.c_void_p * n
        outs = vpa(*[o.data_ptr() for o in self.outs])
        lses = vpa(*[x.data_ptr() for x in self.lses])
        idxs = vpa(*[x.data_ptr() for x in self.idxs]) if self.idxs is not None else None
        self.plan = LayersPlanC()
        _check(lib.dkv_decode_layers_prepare(PA, BA, n, top_k, scale, outs, lses, idxs, _ptr(self.table),
                                             self.table.numel(), _ptr(self.workspace), self.workspace.numel(),
                                             ctypes.byref(self.plan)), "dkv_decode_layers_prepare")

    def run(self, stream=None) -> None:
        _check(load().dkv_decode_layers(ctypes.byref(self.plan), _stream(stream)), "dkv_decode_layers")

    def run_profiled(self, events, stream=None) -> None:
        """run() plus four hipEvent_t records (raw handles as ints): before the
        step, after the routings, after the streams, after the merges."""
        arr = (ctypes.c_void_p * 4)(*events)
        _check(load().dkv_decode_layers_profiled(ctypes.byref(self.plan), arr, _stream(stream)),
               "dkv_decode_layers_profiled")

    def timeout_flag(self) -> int:
        """The workspace's sticky wait-timeout word (0 in every correct run)."""
        return int(self.workspace[8:12].view(__import__("torch").int32).item())

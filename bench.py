#!/usr/bin/env python3
"""Decode-attention benchmark over a compressed KV cache on one MI355X.

Headline workload: the Qwen2.5-1.5B-shaped 28-layer stack at 64k context,
batch 4 (12 query heads over 2 KV heads, d = 128, 252 compressed blocks of 256
tokens plus a 1024-token exact window per sequence, 128 residual rows per
block, top-K = 32 routed blocks, layer ranks 24 / 48 / 16).  Synthetic seeded
caches of that shape stand in for model-derived KV (no weights or datasets
are used).

One step = one decode query for each of the 4 sequences in each of the 28
layers (112 queries): routing, block and window attention and the
log-sum-exp merge of every layer, with every input resident in HBM.  The step
is timed in four launch modes:
  per_layer_eager         28 dkv_decode calls (one fused launch per layer);
  per_layer_hipgraph      the same 28 calls captured once as a hipGraph;
  layer_batched_eager     one dkv_decode_layers step for all 28 layers (three
                          launches: routings, streams, merges);
  layer_batched_hipgraph  that step captured as a hipGraph.
The per-layer modes are the schedule one token's decode runs (layer l+1's
query needs layer l's output); the layer-batched modes need all the layers'
queries at once (micro-batches in flight at different layers, or layers
evaluated on given queries).  `value` is the queries/s of the fastest mode,
named in config.timed_mode; every mode is in ms_per_step_by_mode, with the
median and p10 / p90 over the timed steps.

Roofline: the dominant kernel of the timed mode.  For the layer-batched modes
that is k_blocks (the streams): its algorithmic bytes per launch are the K_eff
routed blocks of P(r, R) = 2*(2d + 255 r + 2 r d) + 2 R (row bytes) + R bytes
each, the window rows (2 * 2 * d bytes each) and the fp16 queries (each read
once per unit), and its duration comes from events around that launch alone
(dkv_decode_layers_profiled) in the timed eager steps.  For the per-layer
modes it is k_decode, one launch per layer, over the whole layer's bytes
(routing keys, 512 bytes per block, included).  `traffic` is the committed
rocprofv3 PMC summary for that kernel, null when the kernel sources changed
since it was taken.

Beside the headline (not part of `value`):
  configs         every configuration (4k, 16k, the stack, ragged batch 32,
                  131k batch 8), each in its per-layer and streamed launch,
                  graph-replayed, cycling over enough cache copies (>= 512 MB
                  per cycle) that no step finds its data in the 256 MB
                  Infinity Cache, with its own CPU oracle baseline;
  read_ceiling    dkv_stream_read_probe over 2 GiB: the box's streaming-read
                  bandwidth for the loads the streams use;
  the stack with 8- / 4-bit residual rows (quantised_residuals), read as
  un-rotated pools (unrotated_pool), with pairs of blocks sharing one basis in
  a compact basis store (shared_basis, with its resident bytes), and the write side, dkv_seal_blocks sealing one layer's
  1008 blocks x 2 KV heads at each of the stack's ranks (sealing).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
METRIC = "decode attention queries/sec + achieved HBM GB/s over compressed KV at 64k ctx"
D = 128
CACHE_DEFEAT_BYTES = 512 * 10 ** 6   # >= 2 x the 256 MB Infinity Cache per cycle over copies
MAX_COPIES = 512

RESID_ROW_BYTES = {0: 2 * D, 1: D + 8, 2: D // 2 + 8}   # fp16; 8- / 4-bit codes + fp16 scale, bias per 64


def bytes_per_block(rank: int, n_resid: int, resid_format: int = 0) -> int:
    """Algorithmic bytes of one routed block of one KV head (fp16 low-rank state,
    residual rows in their storage format, u8 positions)."""
    return 2 * (2 * D + 255 * rank + 2 * rank * D) + 2 * n_resid * RESID_ROW_BYTES[resid_format] + n_resid


def step_bytes(batch, hq, hkv, top_k, n_blocks, win_len, layers):
    """Algorithmic bytes of one decode step by part.  n_blocks, win_len: per
    sequence; layers: (rank, n_resid, resid_format) per layer.  Parts: route
    (the routing keys, fp32, every block of every unit), blocks (K_eff routed
    blocks per unit), window (the unit's window rows), q (fp16 queries, once),
    merge (fp16 outputs, fp32 lse, int32 routed indices)."""
    nb = [max(0, int(n)) for n in n_blocks]
    wl = [max(0, int(w)) for w in win_len]
    out = dict(route=0, blocks=0, window=0, q=0, merge=0)
    for rank, n_resid, fmt in layers:
        out["route"] += hkv * sum(nb) * D * 4
        out["blocks"] += hkv * sum(min(top_k, n) for n in nb) * bytes_per_block(rank, n_resid, fmt)
        out["window"] += hkv * sum(wl) * 2 * 2 * D
        out["q"] += batch * hq * D * 2
        out["merge"] += batch * hq * (D * 2 + 4) + batch * hkv * top_k * 4
    out["step"] = sum(out.values())
    out["streams"] = out["blocks"] + out["window"] + out["q"]
    return out


def workload_bytes(wl, layers=None):
    lays = wl.layers if layers is None else layers
    return step_bytes(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.top_k, wl.n_blocks,
                      [min(int(w), wl.window) for w in wl.win_len],
                      [(l.rank, wl.n_resid, l.resid_format) for l in lays])


def stack_bytes(n_layers: int, resid_format: int = 0):
    """step_bytes of the first n_layers layers of the 64k batch-4 stack."""
    from compressed_kv_cache_amd import synth
    return step_bytes(4, 12, 2, 32, [252] * 4, [1024] * 4,
                      [(synth.STACK_RANKS[i], 128, resid_format) for i in range(n_layers)])


def pct(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "n": int(a.size)}


def source_digest() -> str:
    """sha256[:16] over every kernel source of the library and its header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_kv_cache_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "dkv_attn.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, digest: str):
    """HBM bytes per launch of `kernel` (read + written, scaled by the
    copy-kernel calibration) from the committed rocprofv3 PMC summary, or None
    when the kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_traffic_stack64k_b4.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != digest:
        return None
    return t.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:                                   # pragma: no cover
        return len(os.sched_getaffinity(0))


class Hip:
    """hipEvent helpers through the HIP runtime torch already loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.h.hipEventDestroy(ctypes.c_void_p(e))


def graph_steps(torch, np, step, n_steps: int, reps: int, warmup: int):
    """Capture step(i, stream) for i in range(n_steps) as one hipGraph and replay
    it warmup + reps times; per-step milliseconds of each timed replay."""
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for i in range(n_steps):
            step(i, cs)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n_steps):
            step(i, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for r in range(reps):
        e0[r].record()
        g.replay()
        e1[r].record()
    torch.cuda.synchronize()
    return [e0[r].elapsed_time(e1[r]) / n_steps for r in range(reps)], g


def measure_ceiling(lib, torch, np, log, n_waves: int = 2048, per_wave: int = 1 << 20, reps: int = 7):
    """The streams' read ceiling: dkv_stream_read_probe over n_waves x per_wave bytes."""
    dev = torch.device("cuda:0")
    n = n_waves * per_wave
    x = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(n_waves, dtype=torch.int32, device=dev)
    lib.read_probe(x, n_waves, sink)
    torch.cuda.synchronize()
    assert int(sink.sum().item()) == n // 4, "read probe checksum"
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.read_probe(x, n_waves, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    p = pct(ts)
    gbps = n / (p["median"] * 1e-3) / 1e9
    log(f"read ceiling: {gbps:.0f} GB/s ({n_waves} one-wave workgroups x {per_wave >> 10} KiB)")
    del x, sink
    torch.cuda.empty_cache()
    return {"GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS, "bytes": n, "ms": p,
            "method": f"dkv_stream_read_probe: {n_waves} one-wave workgroups each streaming {per_wave >> 10} KiB "
                      "through a four-page LDS ring with 16-byte buffer loads into LDS (the streams' loads); "
                      f"median of {reps} launches"}


def oracle_sample(wl, b0: int, b1: int):
    """The oracle's inputs for sequences b0 .. b1 - 1 of a one-layer workload."""
    lay = wl.layers[0]
    return (lay.pool(), lay.q[b0:b1], lay.win_k[b0:b1], lay.win_v[b0:b1], wl.block_table[b0:b1],
            wl.n_blocks[b0:b1], wl.win_len[b0:b1], wl.n_kv_heads, wl.top_k, wl.scale)


def cpu_decode_rate(samples, seconds: float, log, what: str):
    """Queries/s of the fp64 oracle (as it stands) over `samples` ((args,
    queries) pairs), cycled until about `seconds` of wall time are spent."""
    import oracle
    runs, spent, queries = 0, 0.0, 0
    while spent < seconds or runs == 0:
        args, nq = samples[runs % len(samples)]
        t0 = time.perf_counter()
        oracle.decode(*args)
        spent += time.perf_counter() - t0
        runs += 1
        queries += nq
    log(f"cpu baseline ({what}): {runs} decodes, {queries} queries in {spent:.1f} s")
    return queries / spent, runs, spent


def measure_config(cfg: int, lib, synth, torch, np, steps: int, warmup: int, cpu_seconds: float, log,
                   want_cpu: bool):
    """One single-layer configuration in its per-layer (dkv_decode) and streamed
    (dkv_decode_layers over the one layer) launch: enough cache copies that a
    cycle over them moves >= 512 MB, one graph holding one step per copy,
    replayed `steps` times; per-step median and p10 / p90."""
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    wl = synth.make_config(cfg)
    by = workload_bytes(wl)
    copies = max(1, min(MAX_COPIES, math.ceil(CACHE_DEFEAT_BYTES / by["step"])))
    lay = wl.layers[0]
    arrays = lay.pool()
    pools, batches, runs = [], [], []
    for c in range(copies):
        p = lib.Pool.from_numpy(arrays, dev)
        b = lib.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks, wl.win_len, device=dev)
        lib.route_keys(p)
        lib.gather_route_keys(p, b)
        pools.append(p)
        batches.append(b)
    torch.cuda.synchronize()
    log(f"{wl.name}: {copies} cache copies of {by['step'] / 1e6:.2f} MB per step "
        f"({time.perf_counter() - t0:.0f} s to build)")
    queries = wl.batch * wl.n_q_heads
    ws = lib.alloc_workspace(pools[0], batches[0], wl.top_k)
    out = torch.empty((wl.batch, wl.n_q_heads, D), dtype=torch.float16, device=dev)
    lse = torch.empty((wl.batch, wl.n_q_heads), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.batch, wl.n_kv_heads, wl.top_k), dtype=torch.int32, device=dev)

    def per_layer(i, st):
        c = i % copies
        lib.decode(pools[c], batches[c], wl.top_k, wl.scale, workspace=ws, out=out, out_lse=lse, out_idx=idx,
                   stream=st)
    per_layer(0, None)
    torch.cuda.synchronize()
    ref_out, ref_idx = out.clone(), idx.clone()
    layers = [lib.Layers([pools[c]], [batches[c]], wl.top_k, wl.scale) for c in range(copies)]
    layers[0].run()
    torch.cuda.synchronize()
    assert torch.equal(layers[0].idxs[0], ref_idx), f"{wl.name}: streamed step routes differently"
    d_out = (layers[0].outs[0].float() - ref_out.float()).abs().max().item()
    assert d_out <= 2e-3, f"{wl.name}: streamed and per-layer outputs differ by {d_out:.2e}"

    def streamed(i, st):
        layers[i % copies].run(st)
    modes = {}
    for name, fn in (("per_layer_hipgraph", per_layer), ("layer_batched_hipgraph", streamed)):
        ms, g = graph_steps(torch, np, fn, copies, max(steps, 10), warmup)
        del g
        p = pct(ms)
        modes[name] = {"ms_per_step": p, "queries_per_s": queries / (p["median"] * 1e-3),
                       "GBps": by["step"] / (p["median"] * 1e-3) / 1e9,
                       "hbm_frac": by["step"] / (p["median"] * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        log(f"{wl.name} {name}: {p['median'] * 1e3:.1f} us/step (p10 {p['p10'] * 1e3:.1f}, p90 {p['p90'] * 1e3:.1f}), "
            f"{modes[name]['GBps']:.0f} GB/s")
    best = min(modes, key=lambda k: modes[k]["ms_per_step"]["median"])
    plan = layers[0].plan
    entry = {"config": wl.name, "queries_per_step": queries, "algorithmic_bytes_per_step": by["step"],
             "bytes_by_part": {k: by[k] for k in ("route", "blocks", "window", "q", "merge")},
             "cache_copies": copies, "streamed": bool(plan.stream), "modes": modes, "best_mode": best,
             "queries_per_s": modes[best]["queries_per_s"], "GBps": modes[best]["GBps"],
             "hbm_frac": modes[best]["hbm_frac"]}
    del layers, pools, batches, ws
    torch.cuda.empty_cache()
    if want_cpu:
        # a bounded sample: whole batch for the small configs, a slice for the large ones
        nb = {0: wl.batch, 1: wl.batch, 3: 2, 4: 1}[cfg]
        samples = [(oracle_sample(wl, b, b + nb), nb * wl.n_q_heads) for b in range(0, wl.batch, nb)][:4]
        qps, runs, spent = cpu_decode_rate(samples, cpu_seconds, log, wl.name)
        entry["cpu_baseline"] = {"value": qps, "unit": "queries/s", "cores": oracle_threads(),
                                 "cpu_model": cpu_model(), "kind": "oracle",
                                 "sample": f"{runs} oracle decodes of {nb} sequence(s) each ({spent:.1f} s)"}
    del wl
    return entry


def seal_flops(width: int, rank: int, power_iters: int, passes: int = 2) -> int:
    """Main arithmetic of sealing one (block, KV head), an FMA counted as 2:
    the 2 + 2q products of A (255 x 256) with a 256 x w or 255 x w factor, the
    Gram matrices and triangular solves of the (1 + 2q) x passes Cholesky QR
    steps and the final Gram of B^T, the factors U S and W, and the residual
    errors.  The Jacobi sweeps (data-dependent count) are not counted."""
    w, q = width, power_iters
    products = (2 + 2 * q) * 255 * 256 * w * 2
    orth = (1 + 2 * q) * passes * (256 * w * w + 256 * w * w)
    final = 256 * w * w + (255 + 256) * rank * w * 2 + 255 * rank * 128 * 2
    return products + orth + final


def measure_sealing(lib, synth, torch, np, log, repeats: int = 3, power_iters: int = 2):
    """dkv_seal_blocks over the blocks of one layer of the 64k batch-4 stack
    (4 sequences x 252 blocks x 2 KV heads, R = 128) at each of the stack's
    ranks, test-matrix width r + 8; timed with events, checked repeat-equal."""
    dev = torch.device("cuda:0")
    nb, H, R = 4 * 252, 2, 128
    inp = synth.make_seal_input(3000, nb, H, width=max(synth.STACK_RANKS) + 8)
    k = torch.from_numpy(inp.k).to(dev)
    v = torch.from_numpy(inp.v).to(dev)
    slots = torch.arange(nb, dtype=torch.int32, device=dev)
    out = []
    for rank in sorted(set(synth.STACK_RANKS)):
        w = rank + 8
        om = torch.from_numpy(np.ascontiguousarray(inp.omega[:, :w])).to(dev)
        pool = lib.Pool.empty(nb, H, rank, R, dev)
        lib.seal_blocks(pool, k, v, slots, om, power_iters)
        torch.cuda.synchronize()
        ref = pool.tensors["_record"].clone()
        ts = []
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.seal_blocks(pool, k, v, slots, om, power_iters)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        assert torch.equal(ref, pool.tensors["_record"])
        ms = float(np.median(ts))
        items = nb * H
        in_bytes = items * 2 * 256 * 128 * 2
        fl = items * seal_flops(w, rank, power_iters)
        log(f"sealing rank {rank}: {ms:.2f} ms for {items} block-heads ({items / ms * 1e3:.0f} per s), "
            f"{fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        out.append({"rank": rank, "width": w, "power_iters": power_iters, "block_heads": items,
                    "ms": ms, "block_heads_per_s": items / (ms * 1e-3),
                    "input_GBps": in_bytes / (ms * 1e-3) / 1e9, "flops_per_block_head": seal_flops(w, rank, power_iters),
                    "achieved_TFLOPs": fl / (ms * 1e-3) / 1e12})
        del pool
    del k, v
    torch.cuda.empty_cache()
    return out


def measure_joins(lib, synth, torch, np, log, repeats: int = 3):
    """dkv_join_basis scoring every block of one un-rotated layer of the 64k
    batch-4 stack (rank 48, 1008 blocks x 2 KV heads) against the basis of its
    neighbour (the candidate evaluation of a join; no write), timed with events."""
    dev = torch.device("cuda:0")
    wl = synth.make_config(2, layers=[9], variant="U")
    pool = lib.Pool.from_numpy(wl.layers[0].pool(), dev)
    n = wl.n_slots
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    entries = (slots ^ 1).clamp(max=n - 1).contiguous()
    lib.join_basis(pool, slots, entries, write=False)
    torch.cuda.synchronize()
    ts = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.join_basis(pool, slots, entries, write=False)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    items = n * wl.n_kv_heads
    log(f"joins (scored) rank {wl.layers[0].rank}: {ms:.3f} ms for {items} block-heads")
    del pool
    torch.cuda.empty_cache()
    return {"rank": wl.layers[0].rank, "block_heads": items, "ms": ms, "block_heads_per_s": items / (ms * 1e-3)}


def pmc_summary(args) -> int:
    """Per-launch HBM traffic of one kernel from two rocprofv3 --pmc runs of
    this benchmark (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each
    scaled by what the same counter reads for the benchmark's copy probe
    (torch.mul over --copy-probe-mib MiB of fp32: that many bytes read and
    written).  Writes profiles/<kernel>_traffic_stack64k_b4.{json,md}."""
    import csv
    import collections

    def per_dispatch(path, counter):
        vals = collections.defaultdict(float)
        names = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                d = row["Dispatch_Id"]
                vals[d] += float(row["Counter_Value"])
                names[d] = row["Kernel_Name"]
        return vals, names

    copy_bytes = args.copy_probe_mib * (1 << 20)
    if copy_bytes <= 0:
        print("--pmc-summary needs --copy-probe-mib (the probe size of the profiled runs)", file=sys.stderr)
        return 2
    out = {}
    for key, path, counter in (("fetch", args.pmc_summary[0], "FETCH_SIZE"),
                               ("write", args.pmc_summary[1], "WRITE_SIZE")):
        vals, names = per_dispatch(path, counter)
        probe = [v for d, v in vals.items() if "MulFunctor" in names[d]]  # the torch.mul copy probe only
        pat = re.compile(r"(^|[\s:])" + re.escape(args.pmc_kernel) + r"[(<]")
        kern = [v for d, v in vals.items() if pat.search(names[d])]
        if not probe or not kern:
            print(f"{path}: no copy-probe or {args.pmc_kernel} dispatches", file=sys.stderr)
            return 2
        probe_kib = max(probe)
        scale = copy_bytes / (probe_kib * 1024.0)
        out[key] = {"counter": counter, "probe_KiB": probe_kib, "scale": scale, "dispatches": len(kern),
                    "bytes_per_launch": sum(kern) / len(kern) * 1024.0 * scale}
    n_layers = max(1, min(28, args.layers))
    sb = stack_bytes(n_layers)
    alg = sb["streams"] if args.pmc_kernel == "k_blocks" else sb["step"]
    if args.pmc_kernel == "k_decode":
        alg /= n_layers
    total = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    res = {
        "kernel": args.pmc_kernel,
        "workload": f"qwen2.5-1.5b 64k ctx, batch 4, layers 0-{n_layers - 1}",
        "kernel_source_sha256_16": source_digest(),
        "dispatches": out["fetch"]["dispatches"],
        "fetch_bytes_per_launch": out["fetch"]["bytes_per_launch"],
        "write_bytes_per_launch": out["write"]["bytes_per_launch"],
        "bytes_per_launch": total,
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": total / alg,
        "calibration": {"copy_kernel": f"torch.mul(a, 1.0, out=b) over {args.copy_probe_mib} MiB fp32",
                        "FETCH_SIZE_KiB": out["fetch"]["probe_KiB"], "WRITE_SIZE_KiB": out["write"]["probe_KiB"],
                        "fetch_scale": out["fetch"]["scale"], "write_scale": out["write"]["scale"]},
    }
    base = os.path.join(ROOT, "profiles", f"{args.pmc_kernel}_traffic_stack64k_b4")
    with open(base + ".json", "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write(f"# {args.pmc_kernel} HBM traffic — 64k-context stack, batch 4, layers 0-{n_layers - 1}\n\n")
        f.write(f"Kernel source sha256[:16] = `{res['kernel_source_sha256_16']}`. "
                f"Numbers in `{os.path.basename(base)}.json`, written by `python bench.py --pmc-summary`.\n\n")
        f.write("Commands (from the repository root, `TMPDIR=/tmp`):\n\n```\n" + args.pmc_command.strip() + "\n```\n\n")
        c = res["calibration"]
        f.write(f"Calibration: the copy probe reads and writes {copy_bytes // 1024:,} KiB. FETCH_SIZE reports "
                f"{c['FETCH_SIZE_KiB']:,.0f} KiB for it (scale {c['fetch_scale']:.3f}), WRITE_SIZE "
                f"{c['WRITE_SIZE_KiB']:,.0f} KiB (scale {c['write_scale']:.3f}).\n\n")
        f.write(f"| per {args.pmc_kernel} launch (mean of {res['dispatches']}) | bytes |\n|---|---|\n")
        f.write(f"| FETCH_SIZE x {c['fetch_scale']:.3f} | {res['fetch_bytes_per_launch'] / 1e6:.2f} MB |\n")
        f.write(f"| WRITE_SIZE x {c['write_scale']:.3f} | {res['write_bytes_per_launch'] / 1e6:.2f} MB |\n")
        f.write(f"| total HBM traffic | {total / 1e6:.2f} MB |\n")
        f.write(f"| algorithmic bytes | {alg / 1e6:.2f} MB |\n")
        f.write(f"| traffic / algorithmic | {res['traffic_over_algorithmic']:.3f} |\n")
    print(json.dumps(res))
    return 0


def measure_variant(lib, synth, torch, np, variant: str, n_layers: int, steps: int, warmup: int, log):
    """The same 64k batch-4 stack with its residual rows stored in the 8- or
    4-bit group-quantised format (variant "Q8" / "Q4"), or read as un-rotated
    pools whose keys are rotated to their positions at read (variant "U"), or
    those with pairs of blocks sharing one basis in a compact basis store
    ("UC2"): one layer-batched step
    per step, timed eagerly with events and as a graph replay."""
    dev = torch.device("cuda:0")
    pools, batches = [], []
    for li in range(n_layers):
        wl = synth.make_config(2, layers=[li], variant=variant)
        lay = wl.layers[0]
        pool = lib.Pool.from_numpy(lay.pool(), dev)
        batch = lib.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                                     wl.win_len, device=dev)
        lib.route_keys(pool)
        lib.gather_route_keys(pool, batch)
        pools.append(pool)
        batches.append(batch)
        del wl, lay
    pool_bytes = {}
    for p_ in pools:
        for t in p_.tensors.values():
            if t is not None:
                st = t.untyped_storage()
                pool_bytes[st.data_ptr()] = st.nbytes()
    resident_pool = sum(pool_bytes.values())
    run = lib.Layers(pools, batches, 32, float(1.0 / np.sqrt(D)))
    for _ in range(warmup):
        run.run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in run.outs]
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda._sleep(int(2e-3 * 2.4e9))
    for s in range(steps):
        e0[s].record()
        run.run()
        e1[s].record()
    torch.cuda.synchronize()
    eager = pct([e0[s].elapsed_time(e1[s]) for s in range(steps)])
    assert run.timeout_flag() == 0 and all(torch.equal(a, b) for a, b in zip(ref, run.outs))
    ms, g = graph_steps(torch, np, lambda i, st: run.run(st), 1, steps, warmup)
    assert all(torch.equal(a, b) for a, b in zip(ref, run.outs))
    p = pct(ms)
    fmt = {"Q8": 1, "Q4": 2, "U": 0, "UC2": 0}[variant]
    alg = stack_bytes(n_layers, fmt)["step"]
    log(f"{variant} variant, layer-batched: {p['median']:.4f} ms/step (graph); eager {eager['median'] * 1e3:.1f} us; "
        f"{alg / 1e6:.1f} MB per step; streamed {bool(run.plan.stream)}")
    res = {"resid_format": {"Q8": "int8", "Q4": "int4", "U": "fp16", "UC2": "fp16"}[variant],
           "keys": "unrotated, rotated at read" if variant in ("U", "UC2") else "rotated",
           "shared_basis": ("pairs of consecutive blocks, a compact basis store of about n_slots / 2 entries"
                            if variant == "UC2" else None),
           "resident_pool_bytes": resident_pool,
           "streamed": bool(run.plan.stream), "ms_per_step": p["median"], "ms_per_step_pct": p,
           "queries_per_s": 4 * n_layers / (p["median"] * 1e-3), "algorithmic_bytes_per_step": alg,
           "eager_us_per_step": eager["median"] * 1e3, "achieved_GBps": alg / (p["median"] * 1e-3) / 1e9}
    del run, pools, batches, g
    torch.cuda.empty_cache()
    return res


CPU_SAMPLE_LAYERS = (0, 9, 19, 27)      # one layer of each rank (24, 48, 16) and the last


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=28, help="layers of the stack to use (default all 28)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="CPU oracle time per configuration of the configs list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--configs", default="0,1,3,4",
                    help="configurations measured beside the stack (comma list of 0,1,3,4; '' for none)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--no-unrotated", action="store_true",
                    help="skip the stack read as un-rotated pools (keys rotated at read)")
    ap.add_argument("--no-sealing", action="store_true",
                    help="skip the block-sealing measurement (dkv_seal_blocks, reported beside the decode)")
    ap.add_argument("--quantised", choices=("none", "int8", "int4", "both"), default="both",
                    help="also time the stack with its residual rows in the 8- / 4-bit format "
                         "(layer-batched step; reported beside the fp16 value)")
    ap.add_argument("--mode", choices=("all", "per-layer", "layer-batched"), default="all",
                    help="which launch modes of the stack to time (default: all)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this benchmark "
                         "into profiles/<kernel>_traffic_stack64k_b4.{json,md} and exit")
    ap.add_argument("--pmc-kernel", default="k_blocks", help="kernel the PMC summary is for")
    ap.add_argument("--pmc-command", default="", help="the rocprofv3 command lines, recorded in the summary")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this size (PMC scaling reference)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.pmc_summary:
        return pmc_summary(args)

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from compressed_kv_cache_amd import lib, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    lib.load()

    if args.copy_probe_mib:
        # a plain device copy of known size: the reference for HBM counter scaling
        # (an elementwise kernel, so that it is a dispatch the counters see)
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"copy probe: {n * 4} bytes read and {n * 4} bytes written per dispatch")
        del a, b

    ceiling = None if args.no_ceiling else measure_ceiling(lib, torch, np, log)

    hip = Hip()
    n_layers = max(1, min(28, args.layers))
    layer_ids = list(range(n_layers))
    # ---- build the resident cache: one layer at a time on the host
    pools, batches, wss, outs, lses, idxs = [], [], [], [], [], []
    meta = None
    cpu_sample = {}
    t0 = time.perf_counter()
    for li in layer_ids:
        wl = synth.make_config(2, layers=[li])
        lay = wl.layers[0]
        pool = lib.Pool.from_numpy(lay.pool(), dev)
        batch = lib.Batch.from_numpy(lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                                     wl.win_len, device=dev)
        lib.route_keys(pool)                      # once per sealed block, not per query
        lib.gather_route_keys(pool, batch)        # per-sequence key table: refreshed with the block table
        pools.append(pool)
        batches.append(batch)
        wss.append(lib.alloc_workspace(pool, batch, wl.top_k))
        outs.append(torch.empty((wl.batch, wl.n_q_heads, D), dtype=torch.float16, device=dev))
        lses.append(torch.empty((wl.batch, wl.n_q_heads), dtype=torch.float32, device=dev))
        idxs.append(torch.empty((wl.batch, wl.n_kv_heads, wl.top_k), dtype=torch.int32, device=dev))
        meta = wl
        if li in CPU_SAMPLE_LAYERS and not args.no_cpu_baseline:
            cpu_sample[li] = wl
        del wl, lay
        if li % 7 == 6:
            log(f"uploaded {li + 1} layers ({time.perf_counter() - t0:.0f} s)")
    torch.cuda.synchronize()
    wl = meta
    storages = {}
    for holder in pools + batches:
        for t in holder.tensors.values():
            if t is not None:
                st = t.untyped_storage()
                storages[st.data_ptr()] = st.nbytes()
    resident = sum(storages.values())
    log(f"resident cache {resident / 1e9:.2f} GB in {time.perf_counter() - t0:.0f} s")

    B, Hq, Hkv, K, R, W, N = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.top_k, wl.n_resid, wl.window, 252
    by = stack_bytes(n_layers)
    queries_per_step = B * n_layers

    def step_eager(stream=None):
        for i in range(n_layers):
            lib.decode(pools[i], batches[i], K, wl.scale, workspace=wss[i], out=outs[i],
                       out_lse=lses[i], out_idx=idxs[i], stream=stream)

    per_layer_modes = args.mode in ("all", "per-layer")
    hold = int(2e-3 * 2.4e9)                              # ~2 ms of shader clock
    # ---- per-layer: eager, with hipEvents around every layer's decode kernel
    for _ in range(args.warmup if per_layer_modes else 1):
        step_eager()
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in outs]
    ref_lse = [x.clone() for x in lses]
    modes, kern_by_mode = {}, {}
    kernel_ms = None
    streamed_parts = None
    if per_layer_modes:
        ev = [[[hip.event() for _ in range(2)] for _ in range(n_layers)] for _ in range(args.steps)]
        s_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        s_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        # Each step is enqueued while a spin kernel holds the GPU, so that its 28
        # kernels then run back to back, as they do in a graph replay: host launch
        # gaps would otherwise leave the GPU idle between layers.
        for s in range(args.steps):
            torch.cuda._sleep(hold)
            s_start[s].record()
            for i in range(n_layers):
                lib.decode_profiled(pools[i], batches[i], K, wl.scale, wss[i], outs[i], lses[i],
                                    ev[s][i], out_idx=idxs[i])
            s_end[s].record()
        torch.cuda.synchronize()
        modes["per_layer_eager"] = pct([s_start[s].elapsed_time(s_end[s]) for s in range(args.steps)])
        kern = [hip.elapsed_ms(ev[s][i][0], ev[s][i][1]) for s in range(args.steps) for i in range(n_layers)]
        kernel_ms = pct(kern)
        for s in ev:
            for e2 in s:
                for e in e2:
                    hip.destroy(e)
        log(f"per-layer eager: {modes['per_layer_eager']['median']:.4f} ms/step; k_decode "
            f"{kernel_ms['median'] * 1e3:.2f} us per layer (p10 {kernel_ms['p10'] * 1e3:.2f}, "
            f"p90 {kernel_ms['p90'] * 1e3:.2f})")
        for i in range(n_layers):
            assert torch.equal(outs[i], ref_out[i]) and torch.equal(lses[i], ref_lse[i]), \
                "eager steps are not bit-identical"
        if not args.no_graph:
            ms, g = graph_steps(torch, np, lambda i, st: step_eager(st), 1, args.steps, args.warmup)
            for i in range(n_layers):
                assert torch.equal(outs[i], ref_out[i]) and torch.equal(lses[i], ref_lse[i]), \
                    "graph replays differ from eager"
            del g
            modes["per_layer_hipgraph"] = pct(ms)
            log(f"per-layer hipGraph: {modes['per_layer_hipgraph']['median']:.4f} ms/step")
        # ---- per layer, streamed: a one-layer dkv_decode_layers step (routings,
        # streams, merges) per layer, in layer order
        runs1 = [lib.Layers([pools[i]], [batches[i]], K, wl.scale) for i in range(n_layers)]
        if all(r.plan.stream for r in runs1):
            def step_streamed(stream=None):
                for r in runs1:
                    r.run(stream)
            for _ in range(args.warmup):
                step_streamed()
            torch.cuda.synchronize()
            for i in range(n_layers):
                assert torch.equal(runs1[i].idxs[0], idxs[i]), f"one-layer streamed layer {i} routes differently"
                d_out = (runs1[i].outs[0].float() - ref_out[i].float()).abs().max().item()
                assert d_out <= 2e-3, f"one-layer streamed layer {i}: {d_out:.2e}"
            ev = [[[hip.event() for _ in range(4)] for _ in range(n_layers)] for _ in range(args.steps)]
            torch.cuda.synchronize()
            for s_ in range(args.steps):
                torch.cuda._sleep(hold)
                for i in range(n_layers):
                    runs1[i].run_profiled(ev[s_][i])
            torch.cuda.synchronize()
            modes["per_layer_streamed_eager"] = pct([hip.elapsed_ms(ev[s_][0][0], ev[s_][-1][3])
                                                     for s_ in range(args.steps)])
            streamed_parts = {name: pct([hip.elapsed_ms(ev[s_][i][k], ev[s_][i][k + 1])
                                         for s_ in range(args.steps) for i in range(n_layers)])
                              for k, name in enumerate(("routes", "streams", "merges"))}
            per_layer_streamed_us = pct([hip.elapsed_ms(ev[s_][i][0], ev[s_][i][3])
                                         for s_ in range(args.steps) for i in range(n_layers)])
            for s_ in ev:
                for e2 in s_:
                    for e in e2:
                        hip.destroy(e)
            log(f"per-layer streamed eager: {modes['per_layer_streamed_eager']['median']:.4f} ms/step; per layer "
                f"{per_layer_streamed_us['median'] * 1e3:.2f} us (routings "
                f"{streamed_parts['routes']['median'] * 1e3:.2f}, streams "
                f"{streamed_parts['streams']['median'] * 1e3:.2f}, merges "
                f"{streamed_parts['merges']['median'] * 1e3:.2f})")
            if not args.no_graph:
                ms, g = graph_steps(torch, np, lambda i, st: step_streamed(st), 1, args.steps, args.warmup)
                del g
                modes["per_layer_streamed_hipgraph"] = pct(ms)
                log(f"per-layer streamed hipGraph: {modes['per_layer_streamed_hipgraph']['median']:.4f} ms/step")
        del runs1

    # ---- every layer's decode step at once (dkv_decode_layers)
    lb_parts = None
    streamed = False
    if args.mode in ("all", "layer-batched"):
        run = lib.Layers(pools, batches, K, wl.scale)
        streamed = bool(run.plan.stream)
        for _ in range(args.warmup):
            run.run()
        torch.cuda.synchronize()
        # the same routing; outputs equal the per-layer ones up to the rounding of
        # another split of the rows into partials
        for i in range(n_layers):
            assert torch.equal(run.idxs[i], idxs[i]), f"layer-batched layer {i} routes differently"
            d_out = (run.outs[i].float() - ref_out[i].float()).abs().max().item()
            d_lse = (run.lses[i] - ref_lse[i]).abs().max().item()
            assert d_out <= 2e-3 and d_lse <= 1e-4, f"layer-batched layer {i}: {d_out:.2e} {d_lse:.2e}"
        lb_ref = [o.clone() for o in run.outs]
        ev = [[hip.event() for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(hold)
        for s in range(args.steps):
            run.run_profiled(ev[s])
        torch.cuda.synchronize()
        steps_ms = [hip.elapsed_ms(ev[s][0], ev[s][3]) for s in range(args.steps)]
        part = [[hip.elapsed_ms(ev[s][k], ev[s][k + 1]) for s in range(args.steps)] for k in range(3)]
        for s in ev:
            for e in s:
                hip.destroy(e)
        modes["layer_batched_eager"] = pct(steps_ms)
        lb_parts = {"routes": pct(part[0]), "streams": pct(part[1]), "merges": pct(part[2])}
        log(f"layer-batched eager: {modes['layer_batched_eager']['median']:.4f} ms/step; routings "
            f"{lb_parts['routes']['median'] * 1e3:.1f} us, streams {lb_parts['streams']['median'] * 1e3:.1f} us "
            f"(p10 {lb_parts['streams']['p10'] * 1e3:.1f}, p90 {lb_parts['streams']['p90'] * 1e3:.1f}), "
            f"merges {lb_parts['merges']['median'] * 1e3:.1f} us")
        assert run.timeout_flag() == 0, "a wait in the layer-batched step timed out"
        for i in range(n_layers):
            assert torch.equal(run.outs[i], lb_ref[i]), "layer-batched steps are not bit-identical"
        if not args.no_graph:
            ms, g = graph_steps(torch, np, lambda i, st: run.run(st), 1, args.steps, args.warmup)
            for i in range(n_layers):
                assert torch.equal(run.outs[i], lb_ref[i]), "layer-batched graph replays differ"
            del g
            modes["layer_batched_hipgraph"] = pct(ms)
            log(f"layer-batched hipGraph: {modes['layer_batched_hipgraph']['median']:.4f} ms/step")
        del run

    mode = min(modes, key=lambda k: modes[k]["median"])
    best_ms = modes[mode]["median"]
    pl = [k for k in modes if k.startswith("per_layer")]
    per_layer_best = min(pl, key=lambda k: modes[k]["median"]) if pl else None
    qps = queries_per_step / (best_ms * 1e-3)
    gbps = by["step"] / (best_ms * 1e-3) / 1e9
    digest = source_digest()
    if mode.startswith("layer_batched") and streamed:
        kernel_name, launch_bytes, kern = "k_blocks", by["streams"], lb_parts["streams"]
    elif mode.startswith("layer_batched"):
        kernel_name, launch_bytes, kern = "k_decode_layers", by["step"], modes["layer_batched_eager"]
    else:
        kernel_name, launch_bytes, kern = "k_decode", by["step"] / n_layers, kernel_ms
    kernel_gbps = launch_bytes / (kern["mean"] * 1e-3) / 1e9
    traffic = measured_traffic(kernel_name, digest)

    res = {
        "metric": METRIC,
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": best_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": synth.CONFIG_NAMES[2] if n_layers == 28 else
                   f"{synth.CONFIG_NAMES[2]}_first{n_layers}layers",
                   "batch": B, "layers": n_layers, "context": 65536, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "window": W, "blocks_per_seq": N, "block_size": 256, "top_k": K,
                   "resid_rows": R, "ranks": "24 (layers 0-8), 48 (9-18), 16 (19-27)",
                   "timed_mode": mode, "accumulate": "f32",
                   "timed_mode_needs": ("all layers' queries at once (independent layers: micro-batches "
                                        "in flight at different layers)") if mode.startswith("layer_batched")
                   else "one layer at a time (one token's decode)"},
        "achieved_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": by["step"],
        "bytes_by_part": {k: by[k] for k in ("route", "blocks", "window", "q", "merge")},
        "queries_per_step": queries_per_step,
        "ms_per_step_by_mode": {k: v["median"] for k, v in modes.items()},
        "ms_per_step_pct_by_mode": modes,
        "per_layer_schedule": None if per_layer_best is None else {
            "mode": per_layer_best,
            "ms_per_step": modes[per_layer_best]["median"],
            "us_per_layer": modes[per_layer_best]["median"] * 1e3 / n_layers,
            "queries_per_s": queries_per_step / (modes[per_layer_best]["median"] * 1e-3),
            "GBps": by["step"] / (modes[per_layer_best]["median"] * 1e-3) / 1e9,
            "k_decode_us_per_layer": kernel_ms["median"] * 1e3 if kernel_ms else None,
            "one_layer_streamed_us_by_launch": None if streamed_parts is None else
            {k: {q: v[q] * 1e3 for q in ("median", "p10", "p90")} for k, v in streamed_parts.items()}},
        "layer_batched_us_by_launch": None if lb_parts is None else
        {k: {q: v[q] * 1e3 for q in ("median", "p10", "p90")} for k, v in lb_parts.items()},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": kernel_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": kernel_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": launch_bytes,
                     "avg_launch_us": kern["mean"] * 1e3, "median_launch_us": kern["median"] * 1e3},
        "read_ceiling": ceiling,
        "resident_cache_GB": resident / 1e9,
        "kernel_source_sha256_16": digest,
    }
    if not args.no_cpu_baseline:
        samples = [((lay.pool(), lay.q, lay.win_k, lay.win_v, w.block_table, w.n_blocks, w.win_len,
                     w.n_kv_heads, w.top_k, w.scale), w.batch * w.n_q_heads)
                   for w in [cpu_sample[k] for k in sorted(cpu_sample)] for lay in [w.layers[0]]] or \
            [((meta.layers[0].pool(), meta.layers[0].q, meta.layers[0].win_k, meta.layers[0].win_v, meta.block_table,
               meta.n_blocks, meta.win_len, meta.n_kv_heads, meta.top_k, meta.scale), meta.batch * meta.n_q_heads)]
        cqps, runs, spent = cpu_decode_rate(samples, args.cpu_seconds, log, "stack")
        res["cpu_baseline"] = {"value": cqps, "unit": "queries/s", "cores": oracle_threads(),
                               "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"{runs} one-layer decode steps of all 4 sequences (48 queries each), "
                                         f"cycling over layers {sorted(cpu_sample)} of the stack: routing over "
                                         f"all 252 blocks, explicit decompression of the 32 routed blocks and "
                                         f"dense fp64 softmax; {spent:.1f} s"}
    del pools, batches, wss, outs, lses, idxs, cpu_sample, meta, wl
    torch.cuda.empty_cache()

    # ---- every configuration
    cfgs = [int(c) for c in args.configs.split(",") if c.strip()]
    entries = []
    for cfg in cfgs:
        if cfg == 2:
            continue
        entries.append(measure_config(cfg, lib, synth, torch, np, args.steps, args.warmup, args.config_cpu_seconds,
                                      log, not args.no_cpu_baseline))
    # the stack itself, from the headline's numbers (its 4.5 GB are far beyond the Infinity Cache)
    stack_entry = {"config": res["config"]["workload"], "queries_per_step": queries_per_step,
                   "algorithmic_bytes_per_step": by["step"], "cache_copies": 1,
                   "streamed": streamed, "best_mode": mode, "queries_per_s": qps, "GBps": gbps,
                   "hbm_frac": gbps / HBM_PEAK_GBPS,
                   "modes": {k: {"ms_per_step": v, "queries_per_s": queries_per_step / (v["median"] * 1e-3),
                                 "GBps": by["step"] / (v["median"] * 1e-3) / 1e9}
                             for k, v in modes.items()}}
    if "cpu_baseline" in res:
        stack_entry["cpu_baseline"] = res["cpu_baseline"]
    entries.insert(min(2, len(entries)), stack_entry)
    res["configs"] = entries

    if args.quantised != "none" and args.mode != "per-layer":
        variants = {"int8": ["Q8"], "int4": ["Q4"], "both": ["Q8", "Q4"]}[args.quantised]
        res["quantised_residuals"] = [measure_variant(lib, synth, torch, np, v, n_layers, args.steps,
                                                      args.warmup, log) for v in variants]
    if not args.no_unrotated and args.mode != "per-layer":
        res["unrotated_pool"] = measure_variant(lib, synth, torch, np, "U", n_layers, args.steps, args.warmup,
                                                log)
        res["shared_basis"] = measure_variant(lib, synth, torch, np, "UC2", n_layers, args.steps, args.warmup,
                                              log)
        res["shared_basis"]["resident_pool_bytes_unshared"] = res["unrotated_pool"]["resident_pool_bytes"]
        res["shared_basis"]["joins"] = measure_joins(lib, synth, torch, np, log)
    if not args.no_sealing and args.mode != "per-layer":
        res["sealing"] = measure_sealing(lib, synth, torch, np, log)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())

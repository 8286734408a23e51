#!/usr/bin/env python3
"""Decode-attention benchmark over a compressed KV cache on one MI355X.

Workload: the Qwen2.5-1.5B-shaped 28-layer stack at 64k context, batch 4
(12 query heads over 2 KV heads, d = 128, 252 compressed blocks of 256 tokens
plus a 1024-token exact window per sequence, 128 residual rows per block, top-K
= 32 routed blocks, layer ranks 24 / 48 / 16).  Synthetic seeded caches of that
shape stand in for model-derived KV (no weights or datasets are used).

One step = one decode query for each of the 4 sequences in each of the 28
layers (112 queries): routing, block and window attention and the log-sum-exp
merge of every layer, with every input resident in HBM.  The step is timed in
three launch modes:
  per_layer_eager         28 dkv_decode calls, hipEvents around every kernel;
  per_layer_hipgraph      the same 28 calls captured once as a hipGraph;
  layer_batched_eager     one dkv_decode_layers launch for all 28 layers;
  layer_batched_hipgraph  that launch captured as a hipGraph.
`value` is the queries/s of the fastest mode (named in config.timed_mode);
every mode is reported in ms_per_step_by_mode.  The layer-batched launch does
the same work, on the same inputs, with the same routing (checked in the run).

Roofline: the kernel of the timed mode (k_decode for the per-layer modes,
k_decode_layers for the layer-batched ones).  Its algorithmic bytes per launch
are, for each (sequence, KV head, layer), the fp32 routing keys of all N blocks
(512 N bytes), K_eff routed blocks of P(r, R) = 2*(2d + 255 r + 2 r d + 2 R d) + R
bytes and 2*2*W*d window bytes, plus the fp16 queries, outputs, lse and routed
indices; divided by that kernel's duration measured with events around it in
the timed eager steps (kernels back to back behind a spin kernel, as in a
replay).  `traffic` is the committed rocprofv3 PMC summary for that kernel
(`--pmc-summary` writes it), null when the kernel source changed since.

Beside the decode (not part of `value`): the same stack with its residual rows
in the 8- and 4-bit formats (`quantised_residuals`), the same stack read as
un-rotated pools whose keys are rotated to their absolute positions at read
(`unrotated_pool`) and with pairs of blocks sharing one basis (`shared_basis`),
and the write side,
dkv_seal_blocks sealing one layer's 1008 blocks x 2 KV heads at each of the
stack's ranks (`sealing`: block-heads per second and the fp32 arithmetic rate
of its main products).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
METRIC = "decode attention queries/sec + achieved HBM GB/s over compressed KV at 64k ctx"
D = 128


RESID_ROW_BYTES = {0: 2 * D, 1: D + 8, 2: D // 2 + 8}   # fp16; 8- / 4-bit codes + fp16 scale, bias per 64


def bytes_per_block(rank: int, n_resid: int, resid_format: int = 0) -> int:
    """Algorithmic bytes of one routed block of one KV head (fp16 low-rank state,
    residual rows in their storage format, u8 positions)."""
    return 2 * (2 * D + 255 * rank + 2 * rank * D) + 2 * n_resid * RESID_ROW_BYTES[resid_format] + n_resid


def layer_bytes(batch, hkv, hq, top_k_eff, rank, n_resid, window, n_blocks, resid_format: int = 0):
    """Per-layer algorithmic bytes by stage: route keys + q (routing), routed
    blocks + window + q (attention), output (merge)."""
    route = batch * hkv * n_blocks * D * 4 + batch * hq * D * 2
    attend = batch * hkv * (top_k_eff * bytes_per_block(rank, n_resid, resid_format) + 2 * 2 * window * D) \
        + batch * hq * D * 2
    merge = batch * hq * (D * 2 + 4) + batch * hkv * top_k_eff * 4
    return route, attend, merge


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


def source_digest() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "compressed_kv_cache_amd", "csrc", "dkv_attn.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, digest: str):
    """HBM bytes per launch of `kernel` (read + written, scaled by the
    copy-kernel calibration) from the committed rocprofv3 PMC summary, or None
    when the kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_traffic_stack64k_b4.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != digest:
        return None
    return t.get("bytes_per_launch")


def step_algorithmic_bytes(n_layers: int, resid_format: int = 0) -> int:
    """Algorithmic bytes of one step over the first n_layers layers of the stack."""
    from compressed_kv_cache_amd import synth
    B, Hq, Hkv, K, R, W, N = 4, 12, 2, 32, 128, 1024, 252
    return sum(sum(layer_bytes(B, Hkv, Hq, min(K, N), synth.STACK_RANKS[i], R, W, N, resid_format))
               for i in range(n_layers))


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


def measure_variant(lib, synth, torch, np, variant: str, n_layers: int, steps: int, warmup: int, log):
    """The same 64k batch-4 stack with its residual rows stored in the 8- or
    4-bit group-quantised format (variant "Q8" / "Q4"), or read as un-rotated
    pools whose keys are rotated to their positions at read (variant "U"): one
    layer-batched launch per step, timed eagerly with events and as a graph
    replay."""
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
    kern = float(np.mean([e0[s].elapsed_time(e1[s]) for s in range(steps)]))
    assert run.timeout_flag() == 0 and all(torch.equal(a, b) for a, b in zip(ref, run.outs))
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        run.run(cs)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run.run(torch.cuda.current_stream())
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    assert all(torch.equal(a, b) for a, b in zip(ref, run.outs))
    fmt = {"Q8": 1, "Q4": 2, "U": 0, "UB": 0}[variant]
    alg = step_algorithmic_bytes(n_layers, fmt)
    log(f"{variant} variant, layer-batched: {ms:.4f} ms/step (graph); kernel {kern * 1e3:.1f} us; "
        f"{alg / 1e6:.1f} MB per step")
    res = {"resid_format": {"Q8": "int8", "Q4": "int4", "U": "fp16", "UB": "fp16"}[variant],
           "keys": "unrotated, rotated at read" if variant in ("U", "UB") else "rotated",
           "shared_basis": "pairs of consecutive blocks" if variant == "UB" else None, "ms_per_step": ms,
           "queries_per_s": 4 * n_layers / (ms * 1e-3), "algorithmic_bytes_per_step": alg,
           "kernel_us_per_launch": kern * 1e3, "achieved_GBps": alg / (kern * 1e-3) / 1e9}
    del run, pools, batches
    torch.cuda.empty_cache()
    return res


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
        kern = [v for d, v in vals.items() if args.pmc_kernel + "<" in names[d] or
                names[d].split("(")[0].endswith(args.pmc_kernel)]
        if not probe or not kern:
            print(f"{path}: no copy-probe or {args.pmc_kernel} dispatches", file=sys.stderr)
            return 2
        probe_kib = max(probe)
        scale = copy_bytes / (probe_kib * 1024.0)
        out[key] = {"counter": counter, "probe_KiB": probe_kib, "scale": scale, "dispatches": len(kern),
                    "bytes_per_launch": sum(kern) / len(kern) * 1024.0 * scale}
    n_layers = max(1, min(28, args.layers))
    alg = step_algorithmic_bytes(n_layers)
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


CPU_SAMPLE_LAYERS = (0, 9, 19, 27)      # one layer of each rank (24, 48, 16) and the last


def cpu_baseline(sample: dict, seconds: float, log):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    decode steps of the sample layers (all 4 sequences each), cycled until about
    `seconds` of CPU time are spent.  sample: {layer index: Workload}."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                                   # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    runs, spent = 0, 0.0
    keys = sorted(sample)
    while spent < seconds:
        li = keys[runs % len(keys)]
        wl = sample[li]
        lay = wl.layers[0]
        t0 = time.perf_counter()
        oracle.decode(lay.pool(), lay.q, lay.win_k, lay.win_v, wl.block_table, wl.n_blocks,
                      wl.win_len, wl.n_kv_heads, wl.top_k, wl.scale)
        spent += time.perf_counter() - t0
        runs += 1
        if runs % len(keys) == 0:
            log(f"cpu baseline: {runs} layer decodes, {spent:.1f} s")
    queries = runs * 4
    return {"value": queries / spent, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} one-layer decode steps (4 sequences each) cycling over layers "
                      f"{list(keys)} of the stack: routing over all 252 blocks, explicit "
                      f"decompression of the 32 routed blocks and dense fp64 softmax; {spent:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=28, help="layers of the stack to use (default all 28)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-unrotated", action="store_true",
                    help="skip the stack read as un-rotated pools (keys rotated at read)")
    ap.add_argument("--no-sealing", action="store_true",
                    help="skip the block-sealing measurement (dkv_seal_blocks, reported beside the decode)")
    ap.add_argument("--quantised", choices=("none", "int8", "int4", "both"), default="both",
                    help="also time the stack with its residual rows in the 8- / 4-bit format "
                         "(layer-batched launch; reported beside the fp16 value)")
    ap.add_argument("--mode", choices=("all", "per-layer", "layer-batched"), default="all",
                    help="which launch modes to time (default: all)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this benchmark "
                         "into profiles/<kernel>_traffic_stack64k_b4.{json,md} and exit")
    ap.add_argument("--pmc-kernel", default="k_decode_layers", help="kernel the PMC summary is for")
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
    ranks = [synth.STACK_RANKS[i] for i in layer_ids]
    per_layer = [layer_bytes(B, Hkv, Hq, min(K, N), r, R, W, N) for r in ranks]
    step_route = sum(x[0] for x in per_layer)
    step_attend = sum(x[1] for x in per_layer)
    step_merge = sum(x[2] for x in per_layer)
    step_bytes = step_route + step_attend + step_merge
    queries_per_step = B * n_layers

    def step_eager():
        for i in range(n_layers):
            lib.decode(pools[i], batches[i], K, wl.scale, workspace=wss[i], out=outs[i],
                       out_lse=lses[i], out_idx=idxs[i])

    per_layer_modes = args.mode in ("all", "per-layer")
    # ---- eager, with hipEvents around every layer's decode kernel, in the timed steps
    for _ in range(args.warmup if per_layer_modes else 1):
        step_eager()
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in outs]
    ref_lse = [x.clone() for x in lses]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    ms_eager = kernel_ms = None
    hold = int(2e-3 * 2.4e9)                              # ~2 ms of shader clock
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
        ms_eager = float(np.mean([s_start[s].elapsed_time(s_end[s]) for s in range(args.steps)]))
        kern = np.array([[hip.elapsed_ms(ev[s][i][0], ev[s][i][1]) for i in range(n_layers)]
                         for s in range(args.steps)])
        kernel_ms = float(kern.mean())
        for s in ev:
            for e2 in s:
                for e in e2:
                    hip.destroy(e)
        log(f"eager: {ms_eager:.4f} ms/step; decode kernel {kernel_ms * 1e3:.2f} us per layer "
            f"(p10 {np.percentile(kern, 10) * 1e3:.2f}, p90 {np.percentile(kern, 90) * 1e3:.2f})")
        for i in range(n_layers):
            assert torch.equal(outs[i], ref_out[i]) and torch.equal(lses[i], ref_lse[i]), \
                "eager steps are not bit-identical"

    # ---- the same step captured once as a hipGraph
    ms_graph = None
    if per_layer_modes and not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step_eager()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step_eager()
        torch.cuda.synchronize()
        for rep in range(3):                              # every replay equals eager
            for o in outs:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            for i in range(n_layers):
                assert torch.equal(outs[i], ref_out[i]) and torch.equal(lses[i], ref_lse[i]), \
                    f"graph replay {rep} differs from eager"
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.steps):
            g.replay()
        t_end.record()
        torch.cuda.synchronize()
        ms_graph = t_start.elapsed_time(t_end) / args.steps
        log(f"hipGraph: {ms_graph:.4f} ms/step")

    # ---- every layer's decode step in ONE layer-batched launch (k_decode_layers)
    ms_lb = ms_lb_graph = lb_kernel_ms = None
    if args.mode in ("all", "layer-batched"):
        run = lib.Layers(pools, batches, K, wl.scale)
        for _ in range(args.warmup):
            run.run()
        torch.cuda.synchronize()
        # the same routing; outputs equal the per-layer ones up to the rounding of
        # another split of the rows (the window has parts of its own here)
        for i in range(n_layers):
            assert torch.equal(run.idxs[i], idxs[i]), f"layer-batched layer {i} routes differently"
            d_out = (run.outs[i].float() - ref_out[i].float()).abs().max().item()
            d_lse = (run.lses[i] - ref_lse[i]).abs().max().item()
            assert d_out <= 2e-3 and d_lse <= 1e-4, f"layer-batched layer {i}: {d_out:.2e} {d_lse:.2e}"
        lb_ref = [o.clone() for o in run.outs]
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(hold)
        for s in range(args.steps):
            e0[s].record()
            run.run()
            e1[s].record()
        torch.cuda.synchronize()
        lb = np.array([e0[s].elapsed_time(e1[s]) for s in range(args.steps)])
        lb_kernel_ms = float(lb.mean())
        ms_lb = float(e0[0].elapsed_time(e1[-1])) / args.steps
        log(f"layer-batched: {ms_lb:.4f} ms/step; k_decode_layers {lb_kernel_ms * 1e3:.2f} us per launch "
            f"(p10 {np.percentile(lb, 10) * 1e3:.2f}, p90 {np.percentile(lb, 90) * 1e3:.2f})")
        assert run.timeout_flag() == 0, "a wait in k_decode_layers timed out"
        for i in range(n_layers):
            assert torch.equal(run.outs[i], lb_ref[i]), "layer-batched steps are not bit-identical"
        if not args.no_graph:
            g2 = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                run.run(cs)
            torch.cuda.current_stream().wait_stream(cs)
            torch.cuda.synchronize()
            with torch.cuda.graph(g2):
                run.run(torch.cuda.current_stream())
            torch.cuda.synchronize()
            for rep in range(3):
                for o in run.outs:
                    o.zero_()
                g2.replay()
                torch.cuda.synchronize()
                for i in range(n_layers):
                    assert torch.equal(run.outs[i], lb_ref[i]), f"layer-batched replay {rep} differs"
            for _ in range(args.warmup):
                g2.replay()
            torch.cuda.synchronize()
            t_start.record()
            for _ in range(args.steps):
                g2.replay()
            t_end.record()
            torch.cuda.synchronize()
            ms_lb_graph = t_start.elapsed_time(t_end) / args.steps
            log(f"layer-batched hipGraph: {ms_lb_graph:.4f} ms/step")

    modes = {"per_layer_eager": ms_eager, "per_layer_hipgraph": ms_graph,
             "layer_batched_eager": ms_lb, "layer_batched_hipgraph": ms_lb_graph}
    mode = min((k for k in modes if modes[k] is not None), key=lambda k: modes[k])
    best_ms = modes[mode]
    qps = queries_per_step / (best_ms * 1e-3)
    gbps = step_bytes / (best_ms * 1e-3) / 1e9
    digest = source_digest()
    if mode.startswith("layer_batched"):
        # one k_decode_layers launch processes the whole step
        kernel_name, launch_bytes, kern_ms = "k_decode_layers", step_bytes, lb_kernel_ms
    else:
        # one k_decode launch per layer; duration from the events around every
        # decode kernel in the timed eager steps (kernels back to back, as in a replay)
        kernel_name, launch_bytes, kern_ms = "k_decode", step_bytes / n_layers, kernel_ms
    kernel_gbps = launch_bytes / (kern_ms * 1e-3) / 1e9
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
                   "timed_mode": mode, "accumulate": "f32"},
        "achieved_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "queries_per_step": queries_per_step,
        "ms_per_step_by_mode": modes,
        "k_decode_us_per_layer": None if kernel_ms is None else kernel_ms * 1e3,
        "k_decode_layers_us_per_launch": None if lb_kernel_ms is None else lb_kernel_ms * 1e3,
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": kernel_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": kernel_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": launch_bytes,
                     "avg_launch_us": kern_ms * 1e3},
        "resident_cache_GB": resident / 1e9,
        "kernel_source_sha256_16": digest,
    }
    if args.quantised != "none" and args.mode != "per-layer":
        # free the fp16 stack first: the quantised stacks are built the same way
        variants = {"int8": ["Q8"], "int4": ["Q4"], "both": ["Q8", "Q4"]}[args.quantised]
        res["quantised_residuals"] = [measure_variant(lib, synth, torch, np, v, n_layers, args.steps,
                                                      args.warmup, log) for v in variants]
    if not args.no_unrotated and args.mode != "per-layer":
        res["unrotated_pool"] = measure_variant(lib, synth, torch, np, "U", n_layers, args.steps, args.warmup,
                                                log)
        res["shared_basis"] = measure_variant(lib, synth, torch, np, "UB", n_layers, args.steps, args.warmup, log)
        res["shared_basis"]["joins"] = measure_joins(lib, synth, torch, np, log)
    if not args.no_sealing and args.mode != "per-layer":
        res["sealing"] = measure_sealing(lib, synth, torch, np, log)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cpu_sample or {layer_ids[0]: meta}, args.cpu_seconds, log)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())

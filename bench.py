#!/usr/bin/env python3
"""Benchmark of the paged-decode hot path on one MI355X.

One step = the whole decode hot path over one batch: slot mapping of the new
tokens and their K/V written into the paged pools (one launch,
pa_write_new_tokens, as pa_decode_step runs it; ``--separate-write`` for the
two launches pa_slot_mapping + pa_reshape_and_cache), paged attention over
every sequence's context (partition kernel + merge kernel).  Default workload: the
Llama-style GQA layer, 256 sequences x 4096 tokens, 32 query / 8 KV heads,
head_dim 128, bf16, block 16 (4 GiB of K/V read per step).

``--workload chunked_prefill_llama_bf16`` (or another varlen batch) times the
prefill form instead: varlen slot mapping, the pool write of every new token
and causal paged attention of all new tokens, with the roofline taken against
the dense matrix-core peak (the attention flops per step / the attention
kernel's time).  ``--workload cow_copy_llama_bf16`` times the copy-on-write
block copy (8192 whole-block copies in both pools of the Llama-style layer),
``--workload swap_llama_bf16`` the swap of 2048 blocks to pinned host memory
and back.

Prints ONE JSON line.  ``value`` = decode tokens/s (one new token per
sequence per step) with every input resident in HBM; ``roofline`` = KV bytes
the partition kernel must read per launch / its average launch time, timed
live with HIP events on the stream the kernels run on; ``cpu_baseline`` = the
float64 CPU oracle on a bounded sample of the same batch.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}  # MI355X dense matrix-core peaks, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_size_amd", "csrc", "pa_kernels.hip")
METRIC = "paged decode attention tokens/s and KV-read GB/s (% of MI355X HBM peak)"
PREFILL_METRIC = "chunked-prefill paged attention new tokens/s and TFLOP/s (% of MI355X dense MFMA peak)"
MULTI_TOKEN_METRIC = "multi-token paged attention new tokens/s and KV-read GB/s (% of MI355X HBM peak)"
COPY_METRIC = "copy-on-write block copies/s and copy GB/s (% of MI355X HBM peak)"
SWAP_METRIC = "block swap-out + swap-in GB/s between HBM and pinned host memory (% of a PCIe Gen5 x16 link)"
HOST_LINK_GBPS = 64.0  # PCIe Gen5 x16, one direction, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama_gqa4k_bf16")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--partition-size", type=int, default=0)
    p.add_argument("--replicas", type=int, default=1,
                   help="rotate over this many copies of the pools (cold caches for small batches)")
    p.add_argument("--block-size", type=int, default=0,
                   help="pool block size for the Llama-layer decode and chunked-prefill workloads (default 16)")
    p.add_argument("--layout", choices=("split", "fused"), default="split",
                   help="pool layout: split K and V pools, or one fused [NB, H_kv, BS, 2D] pool")
    p.add_argument("--shared-prefix", action="store_true",
                   help="decode with shared prompt prefixes read once per group (cascade)")
    p.add_argument("--separate-write", action="store_true",
                   help="slot mapping and pool write as two launches (pa_slot_mapping, pa_reshape_and_cache) "
                        "instead of one (pa_write_new_tokens, as pa_decode_step runs them)")
    p.add_argument("--graph", action="store_true",
                   help="time the step as one captured HIP graph (launch costs gone; per-kernel times stay eager)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=16.0,
                   help="target oracle time (split between the one-thread and all-cores runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration) and exit")
    return p.parse_args()


# the device sources each counted kernel is built from
KERNEL_SOURCES = {
    "decode_partition": ("pa_kernels.hip", "pa_device.h"),
    "prefill_attention": ("pa_prefill.hip", "pa_device.h"),
    "copy_blocks": ("pa_copy.hip",),
}


def kernel_source_hash(prefix="decode_partition"):
    """Hash of the device sources of one kernel family."""
    h = hashlib.sha256()
    csrc = os.path.dirname(KERNEL_SRC)
    for name in KERNEL_SOURCES[prefix]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, prefix="decode_partition"):
    """HBM bytes per launch of the dominant kernel from committed counter
    runs, or None when the kernel source changed since they were taken."""
    path = os.path.join(PROFILES, f"{prefix}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(prefix):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def cpu_pool_size():
    """Worker processes for the all-cores oracle run: the cores this process
    may use, at most 16 (one GPU's share of a host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def start_oracle_pool():
    """Workers for the all-cores oracle run, forked before this process first
    touches the GPU (they never do), each limited to one BLAS thread."""
    import multiprocessing as mp
    return mp.get_context("fork").Pool(cpu_pool_size(), initializer=_oracle_worker_init)


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    global _WORKER_LIMITS
    _WORKER_LIMITS = threadpool_limits(1)


def _oracle_seq(task):
    """Slot mapping, pool write and float64 decode attention (the oracle) of
    one sequence whose compacted inputs sit in a host file mapping; returns
    the seconds spent."""
    import numpy as np

    import oracle as O
    path, fields, table, L, block_size, scale, dtype = task
    mm = np.memmap(path, dtype=np.uint8, mode="r+")
    a = {k: np.ndarray(shape, np.dtype(dt), buffer=mm, offset=off) for k, (off, shape, dt) in fields.items()}
    t0 = time.perf_counter()
    slots = O.slot_mapping([table], [L], block_size)
    O.reshape_and_cache(a["kp"], a["key"], slots)
    O.reshape_and_cache(a["vp"], a["val"], slots)
    O.decode_attention(a["q"], a["kp"], a["vp"], [table], [L], scale, dtype)
    return time.perf_counter() - t0


def cpu_baseline(w, t, seconds, pool):
    """The oracle as it stands, timed on the host on whole sequences of the
    same batch (slot mapping, pool write, float64 decode attention): on one
    thread, and on all cores with one sequence per worker process.  Each
    sequence's blocks are compacted into a host file mapping that the workers
    share; copying them there is not timed."""
    import tempfile

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    from paged_kv_cache_size_amd import workloads as W

    nproc = cpu_pool_size()  # the pool's size (start_oracle_pool)
    bs = w.block_size

    def seq_arrays(b):
        nb = O.num_blocks(int(w.context_lens[b]), bs)
        idx = torch.from_numpy(w.block_tables[b, :nb].astype(np.int64)).to(t["k_pool"].device)
        return {"kp": W.raw_numpy(t["k_pool"][idx]), "vp": W.raw_numpy(t["v_pool"][idx]),
                "q": W.raw_numpy(t["query"][b:b + 1]), "key": W.raw_numpy(t["key"][b:b + 1]),
                "val": W.raw_numpy(t["value"][b:b + 1])}, list(range(nb))

    def run_one(b, arrays, table):
        t0 = time.perf_counter()
        slots = O.slot_mapping([table], [int(w.context_lens[b])], bs)
        O.reshape_and_cache(arrays["kp"], arrays["key"], slots)
        O.reshape_and_cache(arrays["vp"], arrays["val"], slots)
        O.decode_attention(arrays["q"], arrays["kp"], arrays["vp"], [table], [int(w.context_lens[b])], w.scale,
                           w.dtype)
        return time.perf_counter() - t0

    half = seconds / 2
    with threadpool_limits(1):
        a0, tab0 = seq_arrays(0)
        one = run_one(0, a0, tab0)
        n1 = int(max(1, min(w.num_seqs, half / max(one, 1e-6))))
        single = 0.0
        for b in range(n1):
            arrays, table = seq_arrays(b)
            single += run_one(b, arrays, table)
    n2 = int(max(1, min(w.num_seqs, half * nproc / max(one, 1e-6))))

    fd, path = tempfile.mkstemp(prefix="pa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    os.close(fd)
    try:
        tasks, off, chunks = [], 0, []
        for b in range(n2):
            arrays, table = seq_arrays(b)
            fields = {}
            for k, x in arrays.items():
                fields[k] = (off, x.shape, x.dtype.str)
                chunks.append((off, x))
                off += (x.nbytes + 63) // 64 * 64
            tasks.append((path, fields, table, int(w.context_lens[b]), bs, w.scale, w.dtype))
        mm = np.memmap(path, dtype=np.uint8, mode="w+", shape=(max(off, 1),))
        for o, x in chunks:
            mm[o:o + x.nbytes] = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
        mm.flush()
        del mm, chunks
        t0 = time.perf_counter()
        busy = sum(pool.map(_oracle_seq, tasks, chunksize=1))
        wall = time.perf_counter() - t0
    finally:
        os.unlink(path)
    return {"value": n2 / wall, "unit": "tokens/s", "cores": nproc, "kind": "oracle",
            "sample": f"{n2} of {w.num_seqs} sequences (whole contexts) of {w.name}, one per worker process, "
                      f"{nproc} processes of one thread: slot mapping + pool write + float64 attention, "
                      f"{wall:.1f} s wall ({busy:.1f} s busy)",
            "single_thread": {"value": n1 / single, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} sequences, {single:.1f} s"},
            "os_cpu_count": os.cpu_count(), "sched_affinity": len(os.sched_getaffinity(0))}


def prefill_cpu_baseline(pb, t, seconds):
    """The oracle on whole sequences of the batch (every new row of each)."""
    import time as _t
    import numpy as np
    import torch

    import oracle as O
    from paged_kv_cache_size_amd import workloads as W

    w = pb.workload
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    qsl = pb.query_start_loc

    def run(seqs):
        dt = 0.0
        for b in seqs:
            L = int(w.context_lens[b])
            nb = O.num_blocks(L, w.block_size)
            ids = torch.tensor(w.block_tables[b, :nb].astype(np.int64), device="cuda")
            kp, vp = W.raw_numpy(t["k_pool"][ids]), W.raw_numpy(t["v_pool"][ids])
            q = W.raw_numpy(t["query"][int(qsl[b]):int(qsl[b + 1])])
            t0 = _t.perf_counter()
            O.paged_attention(q, kp, vp, [list(range(nb))], [L], [0, q.shape[0]], w.scale, w.dtype)
            dt += _t.perf_counter() - t0
        return dt

    one = run([0])
    n = int(max(1, min(w.num_seqs, seconds / max(one, 1e-6))))
    dt = one + (run(list(range(1, n))) if n > 1 else 0.0)
    rows = int(pb.query_lens[:n].sum())
    return {"value": rows / dt, "unit": "new tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {w.num_seqs} sequences ({rows} new rows, whole contexts) of {pb.name}; "
                      f"float64 causal attention, {dt:.1f} s"}


def main_prefill(args):
    import torch

    from paged_kv_cache_size_amd import binding as PB
    from paged_kv_cache_size_amd import workloads as W

    PB.lib()
    extra = {"block_size": args.block_size} if args.block_size else {}
    pb = W.PREFILL_BUILDERS[args.workload](seed=args.seed, **extra)
    w = pb.workload
    t = W.make_prefill_tensors(pb, seed=args.seed, device="cuda")
    bt = torch.from_numpy(w.block_tables).cuda()
    lens = torch.from_numpy(w.context_lens).cuda()
    T, H, D = t["query"].shape
    ps = args.partition_size
    ws_bytes = PB.pa_prefill_workspace_bytes(T, H, D, w.max_context_len, w.block_size, ps)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["query"])
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    base = None if args.no_cpu_baseline else prefill_cpu_baseline(pb, t, args.cpu_seconds)

    def k_slot():
        PB.pa_slot_mapping(bt, lens, w.block_size, query_start_loc=t["query_start_loc"], num_tokens=T, out=slots)

    def k_write():
        PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)

    def k_attn():
        PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, t["query_start_loc"], w.scale,
                                pb.max_query_len, w.max_context_len, out=out, workspace=ws, partition_size=ps)

    if args.layout == "fused":  # the same rows rearranged on the device into one fused pool
        fused = torch.empty((w.num_blocks, w.num_kv_heads, w.block_size, 2 * D), dtype=t["k_pool"].dtype,
                            device="cuda")
        every = torch.arange(w.num_blocks, dtype=torch.int64, device="cuda")
        PB.pa_convert_blocks(fused, None, PB.PA_KV_FUSED, t["k_pool"], t["v_pool"], PB.PA_KV_SPLIT, every, every)

        def k_write():
            PB.pa_reshape_and_cache(t["key"], t["value"], fused, None, slots, layout=PB.PA_KV_FUSED)

        def k_attn():
            PB.pa_prefill_attention(t["query"], fused, None, bt, lens, t["query_start_loc"], w.scale,
                                    pb.max_query_len, w.max_context_len, out=out, workspace=ws, partition_size=ps,
                                    layout=PB.PA_KV_FUSED)

    stages = [k_slot, k_write, k_attn]
    ms_per_step, per_kernel_ms, wall = time_stages(stages, args.steps, args.warmup)
    flops = pb.attention_flops()
    attn_ms = per_kernel_ms[2]
    if w.dtype == "f32":
        # fp32: the matrix-core column tile, bound by HBM (every context
        # token's K and V read once per step)
        kernel = "columns_f32_mfma_kernel (fp32 column tile)"
        achieved = pb.kv_read_bytes() / (attn_ms * 1e-3) / 1e9
        bound, peak, unit = "hbm", HBM_PEAK_GBPS, "GB/s"
    else:
        # the library runs the cooperative tile once a sequence brings more
        # than 16 (token, query head) columns per KV head
        rep = H // w.num_kv_heads
        repc = max(c for c in range(1, 17) if rep % c == 0)
        kernel = "prefill_wg_kernel" if pb.max_query_len * repc > 16 else "prefill_mfma_kernel"
        achieved = flops / (attn_ms * 1e-3) / 1e12
        bound, peak, unit = "mfma", MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
    rec = {
        "metric": MULTI_TOKEN_METRIC if bound == "hbm" else PREFILL_METRIC, "value": T / (ms_per_step * 1e-3),
        "unit": "new tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "accumulate": "f32", "data": "synthetic",
        "config": {"workload": pb.name, "num_seqs": w.num_seqs, "new_tokens": T, "max_query_len": pb.max_query_len,
                   "context_lens_sum": int(w.context_lens.sum()), "max_context_len": w.max_context_len,
                   "num_heads": H, "num_kv_heads": w.num_kv_heads, "head_dim": D, "block_size": w.block_size,
                   "num_blocks": w.num_blocks, "partition_size": ps, "pool_layout": args.layout,
                   "description": pb.description},
        "attention_flops_per_step": flops,
        "kernel_us": {"slot_mapping": per_kernel_ms[0] * 1e3, "reshape_and_cache": per_kernel_ms[1] * 1e3,
                      "prefill_attention": attn_ms * 1e3},
        "roofline": {"bound": bound, "kernel": kernel, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": (load_traffic(pb.name, "decode_partition" if w.dtype == "f32" else "prefill_attention")
                                 if args.layout == "split" else None)},
        "kv_read_bytes_per_step": pb.kv_read_bytes(),
        "cpu_baseline": base,
        "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


def main_copy(args):
    import numpy as np
    import torch

    import oracle as O
    from paged_kv_cache_size_amd import binding as PB
    from paged_kv_cache_size_amd import workloads as W

    PB.lib()
    cb = W.COPY_BUILDERS[args.workload](seed=args.seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    shape = (cb.num_blocks, cb.block_size, cb.num_kv_heads, cb.head_dim)
    kp = W._randn(shape, cb.dtype, g, "cuda")
    vp = W._randn(shape, cb.dtype, g, "cuda")
    src, dst = torch.from_numpy(cb.src).cuda(), torch.from_numpy(cb.dst).cuda()
    base = None
    if not args.no_cpu_baseline:
        n = min(len(cb.src), 2048)
        pool = W.raw_numpy(kp)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 2:
            O.copy_blocks(pool, cb.src[:n], cb.dst[:n])
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        base = {"value": 2 * n / dt, "unit": "block copies/s", "cores": 1, "kind": "oracle",
                "sample": f"{n} of {len(cb.src)} pairs of {cb.name}, K and V pools, {reps} repetitions"}
        del pool
    stage, kernel = (lambda: PB.pa_copy_blocks(kp, vp, src, dst)), "copy_blocks_kernel"
    if args.layout == "fused":
        # the same pairs copied out of the split pools into a fused pool: the layout conversion
        fused = torch.empty((cb.num_blocks, cb.num_kv_heads, cb.block_size, 2 * cb.head_dim), dtype=kp.dtype,
                            device="cuda")
        stage = lambda: PB.pa_convert_blocks(fused, None, PB.PA_KV_FUSED, kp, vp, PB.PA_KV_SPLIT, src, dst)  # noqa: E731
        kernel = "convert_blocks_kernel"
    ms, per, wall = time_stages([stage], args.steps, args.warmup)
    nbytes = cb.copy_bytes()
    achieved = nbytes / (per[0] * 1e-3) / 1e9
    ceiling = copy_ceiling(nbytes)
    rec = {
        "metric": COPY_METRIC, "value": 2 * len(cb.src) / (ms * 1e-3), "unit": "block copies/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cb.dtype, "data": "synthetic",
        "config": {"workload": cb.name, "num_pairs": int(len(cb.src)), "num_blocks": cb.num_blocks,
                   "block_size": cb.block_size, "num_kv_heads": cb.num_kv_heads, "head_dim": cb.head_dim,
                   "block_bytes": cb.block_bytes, "description": cb.description,
                   "destination_layout": args.layout},
        "copy_bytes_per_step": nbytes,
        "kernel_us": {kernel.replace("_kernel", ""): per[0] * 1e3},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic(cb.name, "copy_blocks") if args.layout == "split" else None,
                     "device_copy_GBps": ceiling, "frac_of_device_copy": achieved / ceiling},
        "cpu_baseline": base, "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


def main_swap(args):
    import torch

    import oracle as O
    from paged_kv_cache_size_amd import binding as PB
    from paged_kv_cache_size_amd import workloads as W

    PB.lib()
    cb = W.SWAP_BUILDERS[args.workload](seed=args.seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    shape = (cb.num_blocks, cb.block_size, cb.num_kv_heads, cb.head_dim)
    kp = W._randn(shape, cb.dtype, g, "cuda")
    vp = W._randn(shape, cb.dtype, g, "cuda")
    n = len(cb.src)
    hshape = (n,) + shape[1:]
    hk = torch.empty(hshape, dtype=kp.dtype, pin_memory=True)
    hv = torch.empty(hshape, dtype=kp.dtype, pin_memory=True)
    dev_ids, host_ids = torch.from_numpy(cb.src).cuda(), torch.from_numpy(cb.dst).cuda()
    base = None
    if not args.no_cpu_baseline:
        pool, host = W.raw_numpy(kp[:1]), None
        sub = min(n, 1024)
        src_np = W.raw_numpy(kp[dev_ids[:sub]])  # the blocks themselves, host side
        host = W.raw_numpy(hk[:sub])
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 2:
            O.swap_blocks(host, src_np, list(range(sub)), list(range(sub)))
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        base = {"value": 2 * sub * cb.block_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{sub} of {n} K blocks, host array to host array, {reps} repetitions"}
        del pool
    out = lambda: PB.pa_swap_blocks(hk, hv, kp, vp, dev_ids, host_ids)  # noqa: E731
    back = lambda: PB.pa_swap_blocks(kp, vp, hk, hv, host_ids, dev_ids)  # noqa: E731
    ms, per, wall = time_stages([out, back], args.steps, args.warmup)
    moved = n * cb.block_bytes * 2  # K and V, one direction
    gbps = [moved / (x * 1e-3) / 1e9 for x in per]
    rec = {
        "metric": SWAP_METRIC, "value": 2 * moved / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cb.dtype, "data": "synthetic",
        "config": {"workload": cb.name, "num_blocks_moved": n, "block_bytes": cb.block_bytes,
                   "description": cb.description},
        "bytes_per_direction": moved,
        "kernel_us": {"swap_out": per[0] * 1e3, "swap_in": per[1] * 1e3},
        "GBps": {"swap_out": gbps[0], "swap_in": gbps[1]},
        "roofline": {"bound": "host-link", "kernel": "copy_blocks_kernel (device <-> pinned host)",
                     "achieved": min(gbps), "peak": HOST_LINK_GBPS, "unit": "GB/s",
                     "frac": min(gbps) / HOST_LINK_GBPS, "traffic": None},
        "cpu_baseline": base, "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


def time_stages(stages, steps, warmup):
    """Whole-step time (events around all launches) and per-stage times
    (events between launches), on torch's current stream where every call
    is enqueued."""
    import torch

    def step():
        for f in stages:
            f()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record()
        for j, f in enumerate(stages):
            f()
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    samples = [[evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)] for j in range(len(stages))]
    per = [sum(x) / steps for x in samples]
    time_stages.samples = samples  # per stage, per step (ms)
    return ms_per_step, per, wall


def time_plain_entry(t, bt, lens, w, steps, warmup, sched_ps):
    """pa_decode_attention called as a C user calls it: no host lengths, so
    the library picks the partition size itself (taking every sequence at
    max_context_len), workspace sized by pa_decode_workspace_bytes.  Time per
    call from events around back-to-back calls on the current stream, beside
    pa_decode_attention_ex at the scheduler's size `sched_ps` timed the same
    way."""
    import ctypes

    import torch

    from paged_kv_cache_size_amd import binding as PB

    lib = PB.lib()
    q = t["query"]
    B, H, D = q.shape
    need = int(lib.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    ptr = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (ptr(out), ptr(q), ptr(t["k_pool"]), ptr(t["v_pool"]), ptr(bt), ptr(lens), B, H, w.num_kv_heads, D,
            w.block_size, w.max_blocks_per_seq, w.max_context_len, w.scale, PB.pa_dtype(q), ptr(ws), need, stream)

    sched_need = PB.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size, sched_ps)
    sched_ws = torch.empty(max(sched_need, 1), dtype=torch.uint8, device=q.device)
    sched_args = args[:15] + (ptr(sched_ws), sched_need, int(sched_ps), stream)

    def plain():
        rc = lib.pa_decode_attention(*args)
        if rc != PB.PA_OK:
            raise PB.PAError(rc, "pa_decode_attention")

    def sched():
        rc = lib.pa_decode_attention_ex(*sched_args)
        if rc != PB.PA_OK:
            raise PB.PAError(rc, "pa_decode_attention_ex")

    def per_call_us(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    us, us_sched = per_call_us(plain), per_call_us(sched)
    ps = PB.pa_decode_partition_size(B, H, w.num_kv_heads, D, w.max_context_len, w.block_size, q.dtype)
    gbps = w.kv_unique_read_bytes() / (us * 1e-6) / 1e9
    return {"partition_size": ps, "us_per_call": us, "kv_GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "scheduler_partition_size": int(sched_ps), "scheduler_us_per_call": us_sched,
            "plain_over_scheduler": us / us_sched}


def time_graph(stages, steps, warmup):
    """The step captured once as a HIP graph and replayed: time per replay
    (events around all replays on the current stream)."""
    import torch

    def step():
        for f in stages:
            f()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture, as torch requires
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def percentiles_us(ms):
    """p10 / p50 / p90 of a list of times in ms, in us."""
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(ms, dtype=np.float64) * 1e3, [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90)}


def stream_ceiling(buffers, reps=20):
    """The device's streaming read rate over the given device tensors (each
    read once per rep with pa_stream_read), default and non-temporal loads."""
    import torch

    from paged_kv_cache_size_amd import binding as PB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = sum(b.numel() * b.element_size() for b in buffers)
    res = {"bytes": nbytes}
    for name, nt in (("default_GBps", False), ("nontemporal_GBps", True)):
        def rep():
            for b in buffers:
                PB.pa_stream_read(b, sink, nontemporal=nt)
        for _ in range(3):
            rep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            rep()
        e1.record()
        torch.cuda.synchronize()
        res[name] = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    res["GBps"] = max(res["default_GBps"], res["nontemporal_GBps"])
    return res


def copy_ceiling(nbytes, reps=20):
    """The device's own contiguous copy rate (the runtime's device-to-device
    copy of nbytes / 2 bytes, so nbytes are read + written per rep), in GB/s
    of bytes read + written."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library runs one GPU per process and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    from paged_kv_cache_size_amd import workloads as W

    if args.workload in W.PREFILL_BUILDERS:
        main_prefill(args)
        return
    if args.workload in W.COPY_BUILDERS:
        main_copy(args)
        return
    if args.workload in W.SWAP_BUILDERS:
        main_swap(args)
        return
    # the oracle's worker processes are forked before anything touches the GPU
    oracle_pool = None if args.no_cpu_baseline else start_oracle_pool()
    try:
        main_decode(args, oracle_pool)
    finally:
        if oracle_pool is not None:
            oracle_pool.terminate()
            oracle_pool.join()


def main_decode(args, oracle_pool):
    import torch

    from paged_kv_cache_size_amd import binding as PB
    from paged_kv_cache_size_amd import workloads as W

    PB.lib()  # fail loudly before any work if the HIP library is missing
    extra = {"block_size": args.block_size} if args.block_size else {}
    w = W.make_workload(args.workload, seed=args.seed, **extra)
    t = W.make_tensors(w, seed=args.seed, device="cuda")
    dev = "cuda"
    # Batches smaller than the 256 MiB MALL stay cache-resident when one pool
    # is re-read every step; --replicas R rotates the steps over R copies.
    pools = [(t["k_pool"], t["v_pool"])] + [(t["k_pool"].clone(), t["v_pool"].clone())
                                            for _ in range(max(1, args.replicas) - 1)]
    turn = [0]

    def pool():
        return pools[turn[0] % len(pools)]
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    B, H, D = t["query"].shape
    # the partition size a scheduler would ask for: it holds the lengths on the host
    ps = args.partition_size or PB.pa_decode_partition_size(B, H, w.num_kv_heads, D, w.max_context_len,
                                                            w.block_size, t["query"].dtype,
                                                            context_lens=w.context_lens)
    ws_bytes = PB.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size, ps)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["query"])
    slots = torch.empty(B, dtype=torch.int64, device=dev)

    base = None
    if oracle_pool is not None:
        base = cpu_baseline(w, t, args.cpu_seconds, oracle_pool)

    def k_slot():
        PB.pa_slot_mapping(bt, lens, w.block_size, out=slots)

    def k_write():
        turn[0] += 1
        PB.pa_reshape_and_cache(t["key"], t["value"], *pool(), slots)

    def k_write_new():  # slots and rows in one launch
        turn[0] += 1
        PB.pa_write_new_tokens(t["key"], t["value"], *pool(), bt, lens, slot_out=slots)

    # the step's first two stages: the slot mapping and the pool write, or
    # both in one launch and an empty second stage
    def write_stages(sep, fused_new):
        return [k_slot, sep] if args.separate_write else [fused_new, lambda: None]

    def k_part():
        PB.pa_decode_partitions(t["query"], *pool(), bt, lens, w.scale, w.max_context_len, ps,
                                workspace=ws, out=out)

    def k_comb():
        PB.pa_decode_combine(out, lens, w.max_context_len, ps, workspace=ws)

    stages = write_stages(k_write, k_write_new) + [k_part, k_comb]
    kernel = "decode_partition_kernel" if w.dtype == "f32" else "decode_mfma_kernel"
    stream_buffers = [t["k_pool"], t["v_pool"]]
    fused = None
    if args.layout == "fused":
        if args.shared_prefix or len(pools) > 1:
            raise SystemExit("--layout fused runs without --shared-prefix and --replicas")
        # the same rows rearranged on the device into one fused pool
        fused = torch.empty((w.num_blocks, w.num_kv_heads, w.block_size, 2 * w.head_dim), dtype=t["k_pool"].dtype,
                            device=dev)
        every = torch.arange(w.num_blocks, dtype=torch.int64, device=dev)
        PB.pa_convert_blocks(fused, None, PB.PA_KV_FUSED, t["k_pool"], t["v_pool"], PB.PA_KV_SPLIT, every, every)

        def k_write():
            PB.pa_reshape_and_cache(t["key"], t["value"], fused, None, slots, layout=PB.PA_KV_FUSED)

        def k_write_new_fused():
            PB.pa_write_new_tokens(t["key"], t["value"], fused, None, bt, lens, slot_out=slots,
                                   layout=PB.PA_KV_FUSED)

        def k_part():  # the merge kernel runs inside when a sequence spans several partitions
            PB.pa_decode_attention(t["query"], fused, None, bt, lens, w.scale, w.max_context_len, out=out,
                                   workspace=ws, partition_size=ps, layout=PB.PA_KV_FUSED)

        stages = write_stages(k_write, k_write_new_fused) + [k_part, lambda: None]
        stream_buffers = [fused]
    if args.shared_prefix:
        # groups found on the host from the tables (scheduler work, untimed)
        groups = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
        dgroups = tuple(torch.from_numpy(x).to(dev)
                        for x in (groups.group_start, groups.prefix_lens, groups.seq_prefix_lens))
        cws = torch.empty(max(1, PB.lib().pa_shared_prefix_workspace_bytes(B, H, D, w.max_context_len,
                                                                            groups.max_prefix_len)),
                          dtype=torch.uint8, device=dev)

        def k_cascade():
            PB.pa_decode_attention_shared_prefix(t["query"], *pool(), bt, lens, groups, w.scale,
                                                 w.max_context_len, out=out, workspace=cws, device_groups=dgroups)

        stages = write_stages(k_write, k_write_new) + [k_cascade, lambda: None]
        kernel = "prefill_mfma_kernel prefix + suffix passes and merge_slots_kernel (one stage)"
        ps = 0
    ms_per_step, per_kernel_ms, wall = time_stages(stages, args.steps, args.warmup)
    stage_samples = time_stages.samples
    staged_ms = ms_per_step
    step_call = "one library call per stage"
    if not args.shared_prefix and not args.separate_write:
        # The step as a caller makes it: one library call, pa_decode_step (the
        # same launches as the stages above, bitwise the same results); the
        # stages above give the per-kernel times.
        layout = PB.PA_KV_FUSED if args.layout == "fused" else PB.PA_KV_SPLIT

        def one_call():
            turn[0] += 1
            k, v = (fused, None) if args.layout == "fused" else pool()
            PB.pa_decode_step(t["query"], t["key"], t["value"], k, v, bt, lens, w.scale, w.max_context_len,
                              out=out, workspace=ws, slot_out=slots, partition_size=ps, layout=layout)

        ms_per_step, _, wall = time_stages([one_call], args.steps, args.warmup)
        step_call = "pa_decode_step (one call)"
    eager_ms = ms_per_step
    if args.graph:
        if len(pools) > 1:
            raise SystemExit("--graph captures one pool; it runs without --replicas")
        ms_per_step = time_graph(stages, args.steps, args.warmup)
    part_pct = percentiles_us(stage_samples[2])
    step_pct = percentiles_us([sum(x) for x in zip(*stage_samples)])
    # the merge stage launches a kernel only when some context spans several partitions
    merged = ps > 0 and args.layout == "split" and not args.shared_prefix and \
        PB.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size, ps) > 0
    plain = None
    if not args.shared_prefix and args.layout == "split" and len(pools) == 1:
        plain = time_plain_entry(t, bt, lens, w, args.steps, args.warmup, ps)
    ceiling = stream_ceiling(stream_buffers)

    kv_bytes = w.kv_read_bytes()
    # a block several sequences share need be read only once: the roofline
    # counts the distinct rows (equal to kv_bytes when nothing is shared)
    kv_unique = w.kv_unique_read_bytes()
    part_ms = per_kernel_ms[2]
    achieved = kv_unique / (part_ms * 1e-3) / 1e9
    tokens_per_s = B / (ms_per_step * 1e-3)
    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": B, "context_lens_sum": int(w.context_lens.sum()),
                   "max_context_len": w.max_context_len, "num_heads": H, "num_kv_heads": w.num_kv_heads,
                   "head_dim": D, "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "partition_size": ps, "shared_prefix_cascade": bool(args.shared_prefix),
                   "pool_layout": args.layout, "hip_graph": bool(args.graph),
                   "new_token_write": "two launches" if args.separate_write else "one launch",
                   "pool_replicas": len(pools),
                   "description": w.description},
        "kv_read_bytes_per_step": kv_bytes,
        "kv_unique_read_bytes_per_step": kv_unique,
        "aux_bytes_per_step": w.aux_bytes(),
        "ms_per_step_eager": eager_ms,
        "step_call": step_call,
        "ms_per_step_separate_calls": staged_ms,
        "kv_GBps_step": kv_bytes / (ms_per_step * 1e-3) / 1e9,
        "context_tokens_per_s": float(w.context_lens.sum()) / (ms_per_step * 1e-3),
        "kernel_us": dict(({"slot_mapping": per_kernel_ms[0] * 1e3, "reshape_and_cache": per_kernel_ms[1] * 1e3}
                           if args.separate_write else {"write_new_tokens": per_kernel_ms[0] * 1e3}),
                          decode_partition=per_kernel_ms[2] * 1e3,
                          combine=per_kernel_ms[3] * 1e3 if merged else None),
        "plain_entry_point": plain,
        "decode_partition_us_percentiles": part_pct,
        "step_us_percentiles": step_pct,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if args.shared_prefix or args.layout != "split" else load_traffic(w.name),
                     "stream_read_GBps": ceiling["GBps"], "frac_of_stream_read": achieved / ceiling["GBps"]},
        "stream_read_ceiling": ceiling,
        "cpu_baseline": base,
        "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

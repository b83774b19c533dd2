#!/usr/bin/env python3
"""Benchmark of one decode step over a paged K/V cache on one MI355X.

A step is the whole path over one batch: page copies for copy-on-write, the
scatter of the new K/V rows, and paged decode attention (split + merge), all
through the C ABI on one stream, with every input resident in HBM.  The
default workload is the batch-64 GQA decode (32 q / 8 kv heads, head_dim 128,
pages of 16 rows, context lengths uniform in [1, 4096], bf16).

By default every timed step starts cold: a 1 GiB read first evicts the K/V
from L2 and from the 256 MB last-level cache, so the attended rows come from
HBM as they would between two layers of a model; step and decode times are then
taken with HIP events on the launch stream.  The same number of back-to-back
steps (where part of one step's K/V is still cached for the next) is reported
beside it.

Prints one JSON line: effective KV GB/s of the step (attended K/V bytes per
step / step time), the decode call's own time and its fraction of HBM peak
from HIP events on the launch stream, and the CPU oracle timed on a bounded
sample of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2)")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--q-len", type=int, default=1,
                   help="query tokens per sequence (a verify step or a prefill chunk): the last "
                        "N rows of each context, through pa_prefill")
    p.add_argument("--sinks", type=int, default=0,
                   help="attention-sink rows kept besides the window (workloads with a window)")
    p.add_argument("--warm-steps", type=int, default=None,
                   help="also time this many back-to-back steps without a flush "
                        "(default: --steps; 0: skip)")
    p.add_argument("--flush", choices=["none", "read", "write"], default="read",
                   help="before each step (outside the events) read (clean eviction) or "
                        "overwrite a 1 GiB buffer, so no K/V row is still in the 256 MB "
                        "last-level cache")
    p.add_argument("--layout", choices=["token", "head"], default="token",
                   help="pool layout: token-major [pages, page_size, kv_heads, head_dim] "
                        "(default) or head-major [pages, kv_heads, page_size, head_dim]")
    p.add_argument("--no-layout-compare", action="store_true",
                   help="skip timing the same calls on head-major copies of the pools after "
                        "the timed steps (a profile then holds one layout only)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="replay the step as a HIP graph (measured slower than launching the "
                        "kernels one by one on this part)")
    p.add_argument("--traffic", type=str,
                   default=os.path.join(ROOT, "profiles", "decode_gqa_b64_hbm_traffic.md"),
                   help="counter summary holding the measured HBM bytes per decode call")
    p.add_argument("--no-copy-ceiling", action="store_true",
                   help="skip the device-to-device copy reference measurement")
    a = p.parse_args()
    if a.warm_steps is None:
        a.warm_steps = a.steps if a.flush != "none" else 0
    return a


def decode_bytes(sc) -> dict:
    """Algorithmic bytes of one decode launch and of the attended K/V alone."""
    import numpy as np
    s = sc.spec
    elt = 4 if s.dtype == "f32" else 2
    n = sc.lens - sc.lo
    kv = int((2 * n * s.kv_heads * s.head_dim * elt).sum())
    tps = sc.table_page_size
    if s.sinks:
        # table entries of the sink rows' pages and of the window's (the hole is skipped)
        W, S = s.window, s.sinks
        table = 0
        for L in sc.lens.tolist():
            if L > W:
                table += 4 * (-(-S // tps) + (L - 1) // tps - max(-(-S // tps), (L - W + S) // tps) + 1)
            elif L > 0:
                table += 4 * ((L - 1) // tps + 1)
    else:
        first = sc.lo // tps
        last = np.where(sc.lens > 0, (sc.lens - 1) // tps, first - 1)
        table = int((4 * (last - first + 1)).clip(min=0).sum())
    nq = len(sc.q)
    q = nq * s.q_heads * s.head_dim * elt
    out = nq * s.q_heads * s.head_dim * 4
    extra = 4 * s.num_seqs + (4 * (s.num_seqs + 1) if sc.q_start is not None else 0)
    return {"kv": kv, "total": kv + table + q + out + extra, "unique_kv": None}


def attention_flops(sc) -> int:
    """Multiply-adds x 2 of scores and P.V: 4 head_dim flops per (query head, attended row)."""
    s = sc.spec
    W = s.window
    if sc.q_start is None:
        keys = (sc.lens - sc.lo).sum()
    else:
        keys = 0
        for L, n in zip(sc.lens.tolist(), sc.nq.tolist()):
            for i in range(n):
                p = L - n + i
                keys += min(p + 1, W) if W > 0 else p + 1
    return int(4 * s.head_dim * s.q_heads * keys)


def unique_kv_bytes(sc) -> int:
    """K/V bytes of distinct physical rows attended (differs from kv when pages are shared)."""
    import numpy as np
    s = sc.spec
    elt = 4 if s.dtype == "f32" else 2
    bt = sc.block_tables.cpu().numpy()
    seen = set()
    P = sc.table_page_size
    for i in range(s.num_seqs):
        for r in range(int(sc.lo[i]), int(sc.lens[i]), P):
            seen.add(int(bt[i, r // P]))
    rows_per = P if P > 1 else 1
    # rows of each distinct page that some sequence attends (approximate at page grain)
    return len(seen) * rows_per * 2 * s.kv_heads * s.head_dim * elt


# The files the decode call's kernel is compiled from, the host code that sizes its
# launch, and the build flags.
DECODE_SOURCES = ("paged_kv_cache_41_amd/csrc/pa_decode_stream.hpp",
                  "paged_kv_cache_41_amd/csrc/pa_common.hpp",
                  "paged_kv_cache_41_amd/csrc/pa_decode_mfma.hpp",
                  "paged_kv_cache_41_amd/csrc/pa_kernels.hip",
                  "include/pa.h", "paged_kv_cache_41_amd/build.py")


def kernel_sources_sha256() -> str:
    """Hash of the decode kernel's sources (names and contents)."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        h.update(os.path.basename(f).encode())
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def measured_traffic(path: str, workload: str, layout: str = "token"):
    """HBM bytes per decode call from a committed counter summary, if it covers this
    workload and pool layout and was taken on the current kernel sources; else None."""
    if not path or not os.path.exists(path) or workload != "gqa_b64":
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "|", "#")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    if vals.get("pool_layout", "token") != layout:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_TIMING = ("launch_us: mean of the cold steps (copy, store, attention) less the mean "
                 "of as many cold steps without the attention call, HIP events on the launch "
                 "stream; decode.avg_us brackets the call alone, which adds the ~5 us an event "
                 "record between two kernels holds the next one back")


def head_major_timing(sc, attend_on, step_on, do_flush, stream, steps, nb, flops,
                      mfma_bound):
    """The timed attention calls again, cold, on head-major copies of the pools
    (PA_HEAD_MAJOR, [pages, kv_heads, page_size, head_dim]) holding the same rows: the
    result is bit-identical, only where each row sits in its page differs."""
    import numpy as np
    import torch
    hk = sc.k_pool.transpose(1, 2).contiguous()
    hv = sc.v_pool.transpose(1, 2).contiguous()
    attend_on(hk, hv, "head")

    def pairs():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)]
    ev, sev, pev = pairs(), pairs(), pairs()
    torch.cuda.synchronize()
    for i in range(steps):
        do_flush()
        step_on(hk, hv, "head")
        ev[i][0].record(stream)
        attend_on(hk, hv, "head")
        ev[i][1].record(stream)
    for i in range(steps):
        do_flush()
        sev[i][0].record(stream)
        step_on(hk, hv, "head")
        attend_on(hk, hv, "head")
        sev[i][1].record(stream)
    for i in range(steps):
        do_flush()
        pev[i][0].record(stream)
        step_on(hk, hv, "head")
        pev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    avg = float(ms.mean())
    kern = float(np.mean([a.elapsed_time(b) for a, b in sev]) -
                 np.mean([a.elapsed_time(b) for a, b in pev]))
    kern = kern if 0 < kern < avg else avg
    del hk, hv
    # priced as the headline's roofline: bytes over HBM peak, or flops over matrix peak
    if mfma_bound:
        ach = flops / (kern * 1e-3) / 1e12
        rate = {"achieved_tflops": round(ach, 2), "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = nb["total"] / (kern * 1e-3) / 1e9
        rate = {"achieved_gbps": round(ach, 1), "frac": round(ach / HBM_PEAK_GBPS, 4)}
    return {"pool_layout": "head-major [pages, kv_heads, page_size, head_dim]",
            "decode_avg_us": round(avg * 1e3, 2),
            "decode_median_us": round(float(np.median(ms)) * 1e3, 2),
            "kernel_us": round(kern * 1e3, 2),
            "kv_gbps": round(nb["kv"] / (kern * 1e-3) / 1e9, 1),
            **rate,
            "note": "the same cold steps as the headline, after them, on head-major copies "
                    "of the pools (rates over kernel_us, taken as for roofline.launch_us); "
                    "the headline uses the token-major layout"}


def allocator_unshared(sc) -> bool:
    """The allocator's answer to "is any page held twice?": the batch's tables are
    registered in a ``PagedKVCache`` (each page named takes a reference) and it reports
    whether every page has a single holder.  A raw slot table is read as the pages behind
    it: logical page j of a sequence is the page of its slot at position j * page_size."""
    from paged_kv_cache_41_amd.alloc import PagedKVCache
    s = sc.spec
    P = s.page_size
    cache = PagedKVCache(sc.pool_pages, P)
    bt = sc.block_tables.cpu().numpy()
    for b, L in enumerate(sc.lens.tolist()):
        row = bt[b] if sc.table_page_size == P else bt[b, 0:max(int(L), 1):P] // P
        cache.adopt(b, row, int(L), sinks=s.sinks)
    return cache.unshared(range(len(sc.lens)))


def copy_ceiling(dev, nbytes: int = 2 << 30, reps: int = 10) -> dict:
    """Bandwidth of a plain device-to-device copy (torch's copy kernel) of known size:
    a measured reference next to the nominal peak, and the calibration kernel for the
    HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / reps * 1e-3
    return {"bytes_read": nbytes, "bytes_written": nbytes,
            "gbps_read_plus_write": round(2 * nbytes / sec / 1e9, 1)}


def memory_report(sc) -> dict:
    """Pages the batch holds and their fragmentation: unused slots of each sequence's
    final page over the slots of its live pages (host arithmetic on the tables)."""
    import numpy as np
    s = sc.spec
    P = s.page_size
    bt = sc.block_tables.cpu().numpy()
    live = unused = 0
    for i in range(s.num_seqs):
        L = int(sc.lens[i])
        if L == 0:
            continue
        if sc.table_page_size == 1:
            n = len({int(x) // P for x in bt[i, :L]} & set(range(sc.pool_pages)))
        else:
            n = int((bt[i] >= 0).sum())
        live += n * P
        unused += (-L) % P
    row_bytes = 2 * s.kv_heads * s.head_dim * (4 if s.dtype == "f32" else 2)
    return {"live_page_slots": live, "unused_last_page_slots": unused,
            "fragmentation": round(unused / live, 5) if live else 0.0,
            "unused_bytes": unused * row_bytes, "pool_pages": sc.pool_pages}


def table_update_timing(sc, dev, reps: int = 50) -> dict:
    """pa_update_tables for one step of this batch: every sequence maps one new page
    (the page its new row opens), scattered into a copy of the batch's table."""
    import numpy as np
    import torch

    from paged_kv_cache_41_amd import ops
    s = sc.spec
    B = s.num_seqs
    tps = sc.table_page_size
    table = sc.block_tables.clone()
    lens = np.maximum(sc.lens, 1)
    if tps == 1:
        # slot table: the page's positions get its slots
        rows = torch.arange(B, dtype=torch.int32, device=dev)
        js = torch.as_tensor(((lens - 1) // s.page_size).astype(np.int32), device=dev)
        pages = torch.as_tensor(np.arange(B, dtype=np.int32), device=dev)
        kw = dict(page_size=s.page_size, slot_table=table, dummy_slot=0)
    else:
        rows = torch.arange(B, dtype=torch.int32, device=dev)
        js = torch.as_tensor(((lens - 1) // tps).astype(np.int32), device=dev)
        pages = torch.as_tensor(np.arange(B, dtype=np.int32), device=dev)
        kw = dict(page_size=tps, block_tables=table)
    f = lambda: ops.update_tables(rows, js, pages, **kw)
    for _ in range(5):
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        f()
    b.record()
    torch.cuda.synchronize()
    return {"updates": B, "avg_us": round(a.elapsed_time(b) / reps * 1e3, 2),
            "table": "slot" if tps == 1 else "block",
            "note": "calls back to back through the Python binding, HIP events on the "
                    "current stream: the rate the host issues them, an upper bound on the "
                    "kernel's own time"}


# ---- CPU baseline: the oracle on a pool of worker processes ------------------------------
# The pool is forked before this process touches the GPU, and the inputs reach the
# workers through named shared memory once the GPU run has made them, so no worker is a
# copy of a process holding a GPU context.  One BLAS thread per worker, one task per
# sequence (or per sequence's query rows).
_WORK = {}


def _worker_init():
    # one BLAS thread per worker, whether or not the parent had loaded BLAS before the fork
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401  (loads BLAS, so the limit below finds it)
    from threadpoolctl import threadpool_limits
    _WORK["limit"] = threadpool_limits(limits=1)


def _worker_attach(desc):
    """Map the shared arrays named in ``desc`` (once per worker and workload)."""
    import numpy as np
    from multiprocessing import resource_tracker, shared_memory
    if _WORK.get("key") != desc["key"]:
        arrays, handles = {}, []
        for name, (shm_name, shape, dtype) in desc["arrays"].items():
            h = shared_memory.SharedMemory(name=shm_name)
            # the creating process owns (and unlinks) the segment: keep the tracker this
            # attach registered it with from claiming it too
            resource_tracker.unregister(h._name, "shared_memory")
            handles.append(h)
            arrays[name] = np.ndarray(shape, dtype=dtype, buffer=h.buf)
        _WORK.update(key=desc["key"], arrays=arrays, handles=handles)
    return _WORK["arrays"]


def _worker_task(job):
    desc, i = job
    import oracle
    a = _worker_attach(desc)
    kw = desc["scalars"]
    if "q_start" in a:
        qs = a["q_start"]
        oracle.attention.prefill(a["q"], a["k"], a["v"], a["bt"], a["ctx"], qs, kw["tps"],
                                 kw["window"], kw["scale"], kw["dtype"],
                                 rows=range(int(qs[i]), int(qs[i + 1])))
    else:
        oracle.attention.decode(a["q"], a["k"], a["v"], a["bt"], a["ctx"], kw["tps"],
                                kw["window"], kw["scale"], kw["dtype"], seqs=[i],
                                sinks=kw["sinks"])
    return i


def cpu_workers() -> int:
    """Workers of the oracle pool: the cores this process may run on, at most 16 (the
    host share of one GPU on the boxes this runs on)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def start_cpu_pool():
    """Fork the worker pool; call before anything initialises the GPU."""
    import multiprocessing as mp
    return mp.get_context("fork").Pool(cpu_workers(), initializer=_worker_init)


def cpu_baseline(sc, pool, budget_s: float = 3.0) -> dict:
    """The oracle over the same batch on the pool: one warm-up pass, then three timed
    runs, each as many whole passes over the batch as fit in ``budget_s`` seconds of
    wall time; the median run's rate is reported."""
    import numpy as np
    import torch
    from multiprocessing import shared_memory

    def bits(t):
        t = t.detach().cpu()
        return (t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16
                else t.view(torch.int32).numpy().view(np.uint32))

    s = sc.spec
    tps = sc.table_page_size
    kp, vp = bits(sc.k_pool), bits(sc.v_pool)
    n_, P = kp.shape[:2]
    host = {"k": kp.reshape(n_ * P // tps, tps, *kp.shape[2:]),
            "v": vp.reshape(n_ * P // tps, tps, *vp.shape[2:]),
            "q": bits(sc.q), "bt": sc.block_tables.cpu().numpy().astype(np.int64),
            "ctx": sc.context_lens.cpu().numpy().astype(np.int64)}
    if sc.q_start is not None:
        host["q_start"] = sc.q_start.cpu().numpy().astype(np.int64)
    handles = []
    try:
        arrays = {}
        for name, arr in host.items():
            h = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            handles.append(h)
            np.ndarray(arr.shape, dtype=arr.dtype, buffer=h.buf)[...] = arr
            arrays[name] = (h.name, arr.shape, arr.dtype.str)
        desc = {"key": f"{s.name}-{sc.seed}", "arrays": arrays,
                "scalars": {"tps": tps, "window": s.window, "scale": sc.scale,
                            "dtype": s.dtype, "sinks": s.sinks}}
        B = s.num_seqs
        jobs = [(desc, i) for i in range(B)]
        elt = 4 if s.dtype == "f32" else 2
        pass_bytes = int((2 * (sc.lens - sc.lo) * s.kv_heads * s.head_dim * elt).sum())
        pool.map(_worker_task, jobs, chunksize=1)          # warm-up: attach, page in
        rates = []
        for _ in range(3):
            passes, t0 = 0, time.perf_counter()
            while True:
                pool.map(_worker_task, jobs, chunksize=1)
                passes += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            rates.append((passes * pass_bytes / dt, passes * B / dt, passes, dt))
        rates.sort()
        gbps, seqs, passes, dt = rates[1]
    finally:
        for h in handles:
            h.close()
            h.unlink()
    n = cpu_workers()
    return {"value": round(gbps / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "seqs_per_s": round(seqs, 3),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"the whole batch ({B} sequences), {passes} passes in {dt:.1f} s (median "
                      f"of 3 runs after a warm-up pass): fp64 gather + dense attention, one "
                      f"task per sequence on {n} worker processes with one BLAS thread each"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or kv head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads
    from paged_kv_cache_41_amd import ops

    pool = None if args.no_cpu_baseline else start_cpu_pool()
    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    over = {}
    if args.sinks:
        base = workloads.config_spec(args.config)
        if base.window <= args.sinks:
            print(f"--sinks {args.sinks} needs a workload whose window is wider "
                  f"(workload {args.config} has window {base.window})", file=sys.stderr)
            sys.exit(2)
        over = dict(sinks=args.sinks, name=f"{base.name}_sinks{args.sinks}")
    if args.q_len > 1:
        base = workloads.config_spec(args.config)
        over.update(q_lo=args.q_len, q_hi=args.q_len,
                    name=f"{over.get('name', base.name)}_q{args.q_len}")
    sc = workloads.make_config(args.config, seed=args.seed, device="cuda:0", **over)
    s = sc.spec
    hkv, d = s.kv_heads, s.head_dim
    kv_view = (sc.k_pool, sc.v_pool) if sc.table_page_size == s.page_size else (
        sc.k_pool.view(-1, 1, hkv, d), sc.v_pool.view(-1, 1, hkv, d))
    layout = args.layout
    pools = (sc.k_pool, sc.v_pool)
    if layout == "head":
        if sc.table_page_size != s.page_size:
            print("a raw slot table addresses pools viewed as pages of one row, which needs "
                  "the token-major layout", file=sys.stderr)
            sys.exit(2)
        # the same rows, head-major; the oracle baseline keeps reading the token-major pools
        pools = (sc.k_pool.transpose(1, 2).contiguous(), sc.v_pool.transpose(1, 2).contiguous())
        kv_view = pools
    out = torch.empty(len(sc.q), s.q_heads, d, dtype=torch.float32, device=dev)
    multi = sc.q_start is not None
    max_q = max(int(sc.nq.max()), 1) if multi else 1
    if multi:
        need = ops.prefill_workspace_bytes(sc.q, sc.q_start, kv_view[0], kv_view[1],
                                           sc.block_tables, sc.context_lens, max_q_len=max_q,
                                           window=s.window, scale=sc.scale,
                                           max_context_len=sc.max_context_len, layout=layout)
    else:
        need = ops.decode_workspace_bytes(sc.q, kv_view[0], kv_view[1], sc.block_tables,
                                          sc.context_lens, window=s.window, sinks=s.sinks,
                                          max_context_len=sc.max_context_len, layout=layout)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    flush = None
    if args.flush != "none":
        flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device=dev)

    def do_flush():
        if args.flush == "write":
            flush.fill_(1)
        else:
            flush.sum(dtype=torch.int64)
    stream = torch.cuda.current_stream(dev)
    nb = decode_bytes(sc)
    kv_bytes_step = nb["kv"]

    # the cache hint is passed only when the allocator holding the batch's tables finds
    # no page with two holders
    unshared = allocator_unshared(sc)

    def step_on(kp, vp, lay):
        ops.copy_pages(kp, vp, sc.copy_src, sc.copy_dst, layout=lay)
        ops.store_kv(kp, vp, sc.k_new, sc.v_new, sc.slot_mapping, layout=lay)

    def step():
        step_on(pools[0], pools[1], layout)

    def attend_on(kp, vp, lay):
        if multi:
            ops.prefill(sc.q, sc.q_start, kp, vp, sc.block_tables, sc.context_lens,
                        max_q_len=max_q, window=s.window, scale=sc.scale,
                        max_context_len=sc.max_context_len, out=out, workspace=ws, layout=lay,
                        unshared_pages=unshared)
        else:
            ops.decode(sc.q, kp, vp, sc.block_tables, sc.context_lens, window=s.window,
                       sinks=s.sinks, scale=sc.scale, max_context_len=sc.max_context_len,
                       out=out, workspace=ws, unshared_pages=unshared, layout=lay)

    def attend():
        attend_on(kv_view[0], kv_view[1], layout)

    # warm-up steps start cold as the timed ones do, so that a profile of a run with
    # --warm-steps 0 holds cold calls only
    for _ in range(args.warmup):
        if flush is not None:
            do_flush()
        step()
        attend()
    torch.cuda.synchronize()

    # With --graph the step is a HIP graph replay (copy, store and the attention call
    # recorded once).  The workspace was zeroed before capture and every call leaves it
    # zeroed, so replays need no memset.  The cache flush stays outside the graphs.
    if args.graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        graphs = {}
        for name, fn in (("both", lambda: (step(), attend())), ("step", step),
                         ("attend", attend)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn()
            graphs[name] = g
        stream.wait_stream(side)
        torch.cuda.synchronize()
        eager_step, eager_attend = step, attend
        step = graphs["step"].replay
        attend = graphs["attend"].replay
        both = graphs["both"].replay
        for _ in range(3):
            both()
        torch.cuda.synchronize()
    else:
        both = lambda: (step(), attend())

    def ev_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # warm: K steps back to back (the K/V of one step partly survives in the 256 MB
    # last-level cache for the next)
    warm = None
    if args.warm_steps > 0:
        wev = [ev_pair() for _ in range(args.warm_steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warm_steps):
            step()
            wev[i][0].record(stream)
            attend()
            wev[i][1].record(stream)
        torch.cuda.synchronize()
        wwall = time.perf_counter() - t0
        wdec = float(np.mean([a.elapsed_time(b) for a, b in wev]))
        warm = {"steps": args.warm_steps, "ms_per_step": round(wwall / args.warm_steps * 1e3, 5),
                "decode_avg_us": round(wdec * 1e3, 2),
                "kv_gbps": round(kv_bytes_step / (wwall / args.warm_steps) / 1e9, 1),
                "decode_kv_gbps": round(kv_bytes_step / (wdec * 1e-3) / 1e9, 1)}

    # timed: K steps; with a flush, each step starts with the K/V evicted from every
    # cache and is timed on the stream with events.  The steps (copy, store, decode) are
    # timed with one event pair each; the decode calls alone in a second pass of K steps
    # (events between the store and the decode would add their own gap to the step).
    # A third pass times the steps without the attention call: an event recorded between
    # two kernels holds the next one back by ~5 us, so the call's own duration is taken
    # as the difference of the step passes with and without it (the attention kernel
    # follows the store with no gap), which the kernel trace's duration matches.
    ev = [ev_pair() for _ in range(args.steps)]
    sev = [ev_pair() for _ in range(args.steps)]
    pev = [ev_pair() for _ in range(args.steps)]
    wall = 0.0
    if flush is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            sev[i][0].record(stream)
            both()
            sev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = wall / args.steps * 1e3
        for i in range(args.steps):
            step()
            ev[i][0].record(stream)
            attend()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
    else:
        torch.cuda.synchronize()
        for i in range(args.steps):
            do_flush()
            sev[i][0].record(stream)
            both()
            sev[i][1].record(stream)
        for i in range(args.steps):
            do_flush()
            step()
            ev[i][0].record(stream)
            attend()
            ev[i][1].record(stream)
        for i in range(args.steps):
            do_flush()
            pev[i][0].record(stream)
            step()
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        ms_step = float(np.mean([a.elapsed_time(b) for a, b in sev]))
    step_ms = np.array([a.elapsed_time(b) for a, b in sev])
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec_avg = float(dec_ms.mean())
    # the attention call's own duration: cold steps with it less cold steps without it
    # (the events' gap can only add time, so a difference above the bracketed time is noise)
    kern_ms = dec_avg
    if flush is not None:
        prep_ms = np.array([a.elapsed_time(b) for a, b in pev])
        diff = float(step_ms.mean() - prep_ms.mean())
        if 0 < diff < dec_avg:
            kern_ms = diff
    achieved = nb["total"] / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.traffic, s.name, layout)
    flops = attention_flops(sc)
    G = s.q_heads // s.kv_heads
    streaming = (s.dtype == "bf16" and s.head_dim == 128 and G <= 16 and
                 (sc.table_page_size & (sc.table_page_size - 1)) == 0 and s.num_seqs <= 2048)
    if multi:
        streaming = streaming and (G & (G - 1)) == 0 and s.num_seqs * -(-max_q // (16 // G)) <= 2048
    call = "pa_prefill" if multi else "pa_decode"
    kernel = (f"{call} call: decode_stream_kernel (one launch)" if streaming else
              f"{call} call: per-row kernels and merge")
    if multi:
        # the tile kernel: 128 score columns per workgroup, two workgroups per compute unit
        tiles = s.num_seqs * s.kv_heads * -(-max_q // (128 // G)) if (G & (G - 1)) == 0 else 0
        if (s.dtype == "bf16" and s.head_dim == 128 and G <= 16 and (G & (G - 1)) == 0 and
                (sc.table_page_size & (sc.table_page_size - 1)) == 0 and max_q * G >= 48 and
                tiles >= 512):
            kernel = "pa_prefill call: prefill_tile_kernel (one launch)"
    # the bound: matrix cores when the call does more flops per byte than the ridge point
    if flops / nb["total"] > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        tflops = flops / (kern_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(tflops, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "flops_per_launch": flops, "bytes_per_launch": nb["total"],
                    "launch_us": round(kern_ms * 1e3, 2), "timing": KERNEL_TIMING}
    else:
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                    "bytes_per_launch": nb["total"], "flops_per_launch": flops,
                    "launch_us": round(kern_ms * 1e3, 2), "timing": KERNEL_TIMING}
    result = {
        "metric": "paged decode attention effective KV GB/s (% HBM peak) + seqs/s",
        "value": round(nb["kv"] / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "num_seqs": s.num_seqs, "q_heads": s.q_heads,
                   "kv_heads": s.kv_heads, "head_dim": s.head_dim, "page_size": s.page_size,
                   "window": s.window, "sinks": s.sinks, "seed": sc.seed, "context_sum": int(sc.lens.sum()),
                   "kv_bytes_per_step": nb["kv"], "copies": int(len(sc.copy_src)),
                   "stored_rows": int((sc.slot_mapping >= 0).sum()),
                   "cache": ("cold: every timed step starts after a 1 GiB read that evicts "
                             "the K/V from L2 and the 256 MB last-level cache; step and decode "
                             "times from HIP events on the launch stream")
                            if args.flush == "read" else
                            ("back-to-back steps" if args.flush == "none" else
                             "every step starts after a 1 GiB write"),
                   "pool_layout": ("head-major [pages, kv_heads, page_size, head_dim]"
                                   if layout == "head" else
                                   "token-major [pages, page_size, kv_heads, head_dim]"),
                   "launch": ("each step one HIP graph replay (copy, store, attention)"
                              if args.graph else "kernels launched one by one"),
                   "cache_hint": ("unshared pages (the allocator's reference counts): V rows read "
                                  "with the non-temporal hint on the streaming path"
                                  if unshared else "none")},
        "seqs_per_s": round(s.num_seqs / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * nb["kv"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "step": {"avg_us": round(float(step_ms.mean()) * 1e3, 2),
                 "median_us": round(float(np.median(step_ms)) * 1e3, 2),
                 "p10_us": round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                 "p90_us": round(float(np.percentile(step_ms, 90)) * 1e3, 2)},
        "decode": {"avg_us": round(dec_avg * 1e3, 2),
                   "median_us": round(float(np.median(dec_ms)) * 1e3, 2),
                   "p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                   "p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                   "kv_gbps": round(nb["kv"] / (dec_avg * 1e-3) / 1e9, 1),
                   "seqs_per_s": round(s.num_seqs / (dec_avg * 1e-3), 1),
                   "kernel_us": round(kern_ms * 1e3, 2)},
        "roofline": roofline,
    }
    if multi:
        result["config"]["q_len"] = max_q
        result["config"]["num_q"] = int(len(sc.q))
        result["decode"]["tflops"] = round(flops / (dec_avg * 1e-3) / 1e12, 2)
    if warm is not None:
        result["warm_back_to_back"] = warm
    if (layout == "token" and not args.no_layout_compare and flush is not None and
            sc.table_page_size == s.page_size):
        result["head_major_layout"] = head_major_timing(
            sc, attend_on, step_on, do_flush, stream, args.steps, nb, flops,
            roofline["bound"] == "mfma")
    if s.prefix_len:
        result["config"]["unique_kv_bytes"] = unique_kv_bytes(sc)
    result["table_update"] = table_update_timing(sc, dev)
    result["memory"] = memory_report(sc)
    if not args.no_copy_ceiling:
        result["hbm_copy_reference"] = copy_ceiling(dev)
    if pool is not None:
        result["cpu_baseline"] = cpu_baseline(sc, pool)
        pool.close()
        pool.join()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of gist-compressed KV attention on one MI355X.

A step is one full pass of the hot path over one batch: for every layer, one
gist_attn_forward call (gather of each pair's gist K/V from that layer's
100k-item pool, RoPE on Q and K_new, masked GQA softmax attention, output
store).  The default workload is 24 layers, Hq=14, H=2 KV heads, head_dim 64,
k=8 gist positions, ell=64 query tokens, 500 (item, query) pairs = 10 queries
x 50 candidates, bf16, each layer with its own pool and its own Q/K/V/O.

Prints one JSON line.  `value` is pairs/s for the whole pass with all inputs
resident in HBM; `roofline` prices the dominant kernel's algorithmic bytes per
launch against its average launch duration (HIP events on the launch stream);
`cpu_baseline` times the fp64 oracle on a bounded sample on the host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "pairs/s + % of HBM peak, gist-KV attention (24L, GQA 14:2, k=8, ℓ=64)"
CSRC = os.path.join(ROOT, "gist_compressed_kv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated) per
# workload, and the kernel source they were taken on
COUNTER_FILES = {
    "24L_b500": ("gist_fwd_mfma_d64_24L_b500_counters.json", "gist_forward.hip"),
    "24L_b500_grouped": ("gist_fwd_mfma_grouped_d64_24L_b500_counters.json", "gist_forward.hip"),
    "24L_b2000": ("gist_fwd_mfma_d64_24L_b2000_counters.json", "gist_forward.hip"),
    "wide_ell64": ("gist_fwd_mfma_d128_wide_ell64_counters.json", "gist_forward.hip"),
    "wide_eos": ("gist_fwd_eos_d128_wide_eos_counters.json", "gist_forward.hip"),
    "wide_eos_grouped": ("gist_fwd_eos_grouped_d128_wide_eos_counters.json", "gist_forward.hip"),
    "wide_eos_fp8": ("gist_fwd_eos_fp8_d128_wide_eos_counters.json", "gist_forward.hip"),
    "paged": ("paged_decode_32x4096_counters.json", "paged_decode.hip"),
    "paged_fp8": ("paged_decode_fp8_32x4096_counters.json", "paged_decode.hip"),
    "prefill": ("prefill_attn_d64_256items_counters.json", "prefill.hip"),
}


def gist_bytes_per_pair_layer(wl, last_only: bool = False) -> int:
    """Algorithmic HBM bytes one (pair, layer) must move: the item's gist K/V
    (and query gist, if any), Q in, K_new/V_new in, O out, the 4-byte id.
    An fp8 gist record is one byte per element plus a 4-byte scale per (K or
    V, head).  last_only: Q and O of the last token only."""
    b = wl.dtype.itemsize

    def record(rows):
        if wl.fp8:
            return 2 * rows * wl.h * wl.d + 2 * wl.h * 4
        return 2 * rows * wl.h * wl.d * b

    gist = record(wl.k)
    # a query's gist rows are shared by its candidates: counted once per query
    qgist = record(wl.kq) * wl.queries / wl.pairs if wl.kq else 0
    rows = 1 if last_only else wl.ell
    q = rows * wl.hq * wl.d * b
    kv_new = 2 * wl.ell * wl.h * wl.d * b
    o = rows * wl.hq * wl.d * b
    ids = 4 * (2 if wl.kq else 1)
    return int(round(gist + qgist + q + kv_new + o + ids))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed passes (default 200; 4800 for the one-launch single-layer workloads)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed passes first (default 20; 480 for the single-layer workloads)")
    ap.add_argument("--workload", default="24L_b500",
                    choices=["24L_b500", "24L_b500_last", "24L_b500_grouped", "wide_eos_grouped",
                             "wide_eos_fp8_grouped", "24L_b2000", "1L_b500",
                             "1L_b500_paged",
                             "wide_ell64",
                             "wide_ell64_fp8", "wide_eos", "wide_eos_fp8", "paged", "paged_fp8",
                             "prefill", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    # A single-layer pass is one launch of about 30 us: 200 of them time 6 ms,
    # too short a region (the launch time read 31-34 us in runs of 200
    # passes and 28.6 us in runs of 4800).  Those workloads time as many
    # launches as the 24-layer pass does by default.
    one_launch = args.workload in ("1L_b500", "1L_b500_paged")
    if args.steps is None:
        args.steps = 4800 if one_launch else 200
    if args.warmup is None:
        args.warmup = 480 if one_launch else 20
    return args


def kernel_source_hash(source: str) -> str:
    with open(os.path.join(CSRC, source), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload_name: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, only if they
    were taken on the current kernel source."""
    if workload_name not in COUNTER_FILES:
        return None
    fname, source = COUNTER_FILES[workload_name]
    try:
        with open(os.path.join(PROFILES, fname)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash(source) or c.get("workload") != workload_name:
        return None
    return c.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# The fp64 oracle timed on the host (a baseline, not the target).  A seeded
# sample of each workload is cut into tasks (one layer and a slice of its
# pairs or requests), timed once on one thread and once on every core this
# process may use: worker processes for the gist oracle (its Python loops hold
# the interpreter), threads for decode and prefill (large numpy products).
# BLAS runs one thread per task either way.
# ---------------------------------------------------------------------------


def _bits(t):
    """A host copy of a tensor as numpy: bf16 as its uint16 bits (exact and
    half the bytes of fp32), other dtypes as they are."""
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def _f64(a):
    """bf16 bits (uint16) or fp32 values as fp64 (exactly)."""
    import numpy as np
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float64)


def _oracle_task(task):
    """Run one oracle task (BLAS on one thread); returns its units of work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gist_oracle as O

    with threadpool_limits(1):
        if task["kind"] == "gist":
            if task["fp8"]:
                pool = O.dequantize_gist(*task["pool"])[None]
                qpool = O.dequantize_gist(*task["qpool"])[None] if task["qpool"] is not None else None
            else:
                pool = _f64(task["pool"])[None]
                qpool = _f64(task["qpool"])[None] if task["qpool"] is not None else None
            n = pool.shape[1]
            O.gist_attn_forward(pool, 0, np.arange(n), _f64(task["q"]), _f64(task["kn"]),
                                _f64(task["vn"]), task["pos0"], 10000.0, task["scale"],
                                qpool=qpool, q_ids=np.arange(n) if qpool is not None else None)
            return n
        if task["kind"] == "decode":
            if task["fp8"]:
                kc = O.dequantize_blocks(*task["kc"])
                vc = O.dequantize_blocks(*task["vc"])
            else:
                kc, vc = _f64(task["kc"]), _f64(task["vc"])
            O.paged_decode(kc, vc, task["table"], task["lens"], _f64(task["q"]), _f64(task["kn"]),
                           _f64(task["vn"]), task["positions"], 10000.0, task["scale"])
            return len(task["lens"])
        if task["kind"] == "prefill":
            O.prefill_attention(_f64(task["q"]), _f64(task["k"]), _f64(task["v"]), task["seq_start"],
                                10000.0, task["scale"])
            return int(task["seq_start"][-1])
    raise ValueError(task["kind"])


def _warm_worker(_):
    # lowest priority: the workers must not slow the GPU launch loop
    os.nice(19)
    import numpy  # noqa: F401
    import threadpoolctl  # noqa: F401

    from oracle import gist_oracle  # noqa: F401
    return 0


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


_ORACLE_POOL = None  # (pool, workers, warm-up result): started before the GPU is touched


def start_oracle_pool():
    """Start the oracle's worker processes (at most 16: a one-GPU share of a
    box) from a process that has not touched the GPU yet; their interpreter
    start-up and imports run while the GPU work goes on."""
    global _ORACLE_POOL
    import multiprocessing
    n = max(1, min(len(os.sched_getaffinity(0)), 16))
    # the workers inherit this environment: BLAS and OpenMP on one thread each
    # (no idle thread pools spinning in sixteen processes)
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({k: "1" for k in keys})
    try:
        pool = multiprocessing.get_context("spawn").Pool(n)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    _ORACLE_POOL = (pool, n, pool.map_async(_warm_worker, range(n)))


def stop_oracle_pool():
    global _ORACLE_POOL
    if _ORACLE_POOL is not None:
        _ORACLE_POOL[0].close()
        _ORACLE_POOL[0].join()
        _ORACLE_POOL = None


def time_oracle(tasks, processes: bool):
    """Seconds for all tasks on one thread, and on every core this process
    may use (at most 16); returns (t1, tn, n).  processes: the worker pool
    started by start_oracle_pool, else threads."""
    from concurrent.futures import ThreadPoolExecutor

    t0 = time.perf_counter()
    for task in tasks:
        _oracle_task(task)
    t1 = time.perf_counter() - t0
    if processes:
        pool, n, warm = _ORACLE_POOL
        warm.get()
        t0 = time.perf_counter()
        pool.map(_oracle_task, tasks, chunksize=1)
        tn = time.perf_counter() - t0
    else:
        n = max(1, min(len(os.sched_getaffinity(0)), 16))
        with ThreadPoolExecutor(n) as ex:
            t0 = time.perf_counter()
            list(ex.map(_oracle_task, tasks))
            tn = time.perf_counter() - t0
    return t1, tn, n


def baseline_record(unit, pass_units, pass_work, sample_work, t1, tn, n, sample, how):
    """The oracle's throughput for whole passes: a pass yields pass_units
    units (pairs, requests, tokens) from pass_work units of work (those per
    layer, summed over the layers); sample_work of them took t1 s on one thread
    and tn s on n cores."""
    def rate(t):
        return sample_work / t / pass_work * pass_units
    return {"value": rate(tn), "unit": unit, "cores": n, "kind": "oracle",
            "sample": f"{sample}; fp64 numpy, BLAS one thread per task; {how}; "
                      f"{t1:.1f} s on one thread, {tn:.1f} s on {n}",
            "one_thread": {"value": rate(t1), "unit": unit, "cores": 1},
            "host": host_info()}


def gist_baseline(wl, pool, ids, qs, kns, vns, n_sets, qpool=None, q_ids=None):
    """cpu_baseline of a gist workload: a seeded sample of pairs in a sample
    of layers (all layers where that stays near 10 s of one-thread work)."""
    import numpy as np
    import torch

    if wl.d == 64:
        layers = list(range(wl.layers))
        npairs = wl.pairs if wl.layers == 1 else min(256, wl.pairs)
    elif wl.ell > 1:
        layers = sorted({0, wl.layers // 3, 2 * wl.layers // 3, wl.layers - 1})
        npairs = 128
    else:
        layers = list(range(0, wl.layers, 4))
        npairs = 128
    g = torch.Generator().manual_seed(wl.seed * 7919 + 17)
    sample = torch.randperm(wl.pairs, generator=g)[:npairs].sort().values
    idx = sample.to(ids.device)
    item = ids[idx].long()
    qrow = q_ids[idx].long() if q_ids is not None else None
    tasks = []
    for li in layers:
        si = li % n_sets
        for c0 in range(0, npairs, 16):
            sl = slice(c0, min(npairs, c0 + 16))
            if pool.fp8:
                prec = (_bits(pool.codes[li][item[sl]]), _bits(pool.scales[li][item[sl]]))
                qrec = (_bits(qpool.codes[li][qrow[sl]]), _bits(qpool.scales[li][qrow[sl]])) if qpool else None
            else:
                prec = _bits(pool.storage[li][item[sl]])
                qrec = _bits(qpool.storage[li][qrow[sl]]) if qpool else None
            tasks.append({"kind": "gist", "fp8": pool.fp8, "pool": prec, "qpool": qrec,
                          "q": _bits(qs[si][idx[sl]]), "kn": _bits(kns[si][idx[sl]]),
                          "vn": _bits(vns[si][idx[sl]]), "pos0": wl.pos0,
                          "scale": 1.0 / math.sqrt(wl.d)})
    t1, tn, n = time_oracle(tasks, processes=True)
    return baseline_record("pairs/s", wl.pairs, wl.pairs * wl.layers, npairs * len(layers), t1, tn, n,
                           f"{npairs} of {wl.pairs} pairs (seeded) in layers "
                           f"{layers if len(layers) < wl.layers else 'all ' + str(wl.layers)}, "
                           f"every head and token", f"{len(tasks)} tasks of <= 16 pairs, worker processes")


def copy_probe(args):
    """A plain device-to-device copy of 1 GiB: the reference whose HBM counter
    readings (FETCH_SIZE, WRITE_SIZE) calibrate the counter runs."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"metric": "device copy", "value": 2 * n / dt / 1e9, "unit": "GB/s",
                      "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "ms_per_step": dt * 1e3}), flush=True)


def decode_bytes_per_request_layer(wl, fp8: bool = False) -> int:
    """Algorithmic bytes of one decode step of one request in one layer: the
    cached K and V it attends over (1 byte per element plus one fp32 scale per
    block and head for each of K and V when the cache is fp8), q, k_new, v_new,
    the output, and its block-table row, context length and position."""
    b = wl.dtype.itemsize
    if fp8:
        cache = 2 * wl.context * wl.h * wl.d + 2 * 4 * wl.blocks_per_request * wl.h
    else:
        cache = 2 * wl.context * wl.h * wl.d * b
    return (cache + wl.hq * wl.d * b + 2 * wl.h * wl.d * b + wl.hq * wl.d * b
            + 4 * wl.blocks_per_request + 8)


def paged_bench(args, fp8: bool = False):
    """One decode step of 32 requests over 4096 cached tokens in every one of
    32 layers (each layer its own paged cache and its own inputs); with fp8
    the cache holds E4M3 codes with per-(block, head) scales."""
    import torch

    import gist_compressed_kv_amd as G
    from gist_compressed_kv_amd import synth

    wl = synth.PAGED_FP8 if fp8 else synth.PAGED
    dev = "cuda"
    nblk = wl.requests * wl.blocks_per_request
    print(f"[bench] generating inputs: {wl.name}", file=sys.stderr, flush=True)
    table = synth.block_table(wl.requests, wl.blocks_per_request, nblk, wl.seed, dev)
    lens = torch.full((wl.requests,), wl.context, dtype=torch.int32, device=dev)
    pos = lens + 1
    layers = []
    for li in range(wl.layers):
        shape = (nblk, wl.h, wl.block_size, wl.d)
        if fp8:
            kc = synth.randn_fp8_blocks(shape, synth.tensor_seed(wl.seed, 11, li), dev)
            vc = synth.randn_fp8_blocks(shape, synth.tensor_seed(wl.seed, 12, li), dev)
        else:
            kc = synth.randn(shape, synth.tensor_seed(wl.seed, 11, li), wl.dtype, dev)
            vc = synth.randn(shape, synth.tensor_seed(wl.seed, 12, li), wl.dtype, dev)
        q = synth.randn((wl.requests, wl.hq, wl.d), synth.tensor_seed(wl.seed, 13, li), wl.dtype, dev)
        kn = synth.randn((wl.requests, wl.h, wl.d), synth.tensor_seed(wl.seed, 14, li), wl.dtype, dev)
        vn = synth.randn((wl.requests, wl.h, wl.d), synth.tensor_seed(wl.seed, 15, li), wl.dtype, dev)
        layers.append((kc, vc, q, kn, vn, torch.empty_like(q)))
    ws = torch.empty(G.paged_decode_workspace_bytes(wl.requests, wl.hq, wl.blocks_per_request,
                                                    wl.block_size, wl.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        for kc, vc, q, kn, vn, out in layers:
            if fp8:
                G.paged_decode_attn_fp8(kc[0], vc[0], kc[1], vc[1], table, lens, q, kn, vn, pos,
                                        10000.0, None, out=out, workspace=ws, stream=stream)
            else:
                G.paged_decode_attn(kc, vc, table, lens, q, kn, vn, pos, 10000.0, None, out=out,
                                    workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # one call = the split kernel then the combine kernel
    avg_s = ev0.elapsed_time(ev1) / 1e3 / (args.steps * wl.layers)
    bytes_unit = decode_bytes_per_request_layer(wl, fp8)
    achieved = bytes_unit * wl.requests / avg_s / 1e9
    res = {
        "metric": "paged decode tokens/s (32 requests x 4096 cached tokens, 32 layers"
                  + (", fp8 E4M3 cache)" if fp8 else ")"),
        "value": wl.requests / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 cache, bf16 activations" if fp8 else "bf16",
        "data": "synthetic N(0,1) caches" + (" quantized per (block, head)" if fp8 else "")
                + ", seeded block tables",
        "config": {"workload": wl.name},
        "roofline": {"bound": "hbm",
                     "kernel": "decode_split<fp8> + decode_combine" if fp8 else "decode_split + decode_combine",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("paged_fp8" if fp8 else "paged"),
                     "bytes_per_unit": bytes_unit, "units_per_launch": wl.requests,
                     "avg_launch_us": avg_s * 1e6}}
    if not args.no_cpu_baseline:
        import numpy as np
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        # every request in two layers, one task per (layer, request) holding
        # the request's own blocks
        layers_s = [0, wl.layers - 1]
        tab = table.cpu().numpy()
        tasks = []
        for li in layers_s:
            kc, vc, q, kn, vn, _ = layers[li]
            for r in range(wl.requests):
                blk = torch.as_tensor(tab[r], device=dev).long()
                if fp8:
                    kcr = (_bits(kc[0][blk]), _bits(kc[1][blk]))
                    vcr = (_bits(vc[0][blk]), _bits(vc[1][blk]))
                else:
                    kcr, vcr = _bits(kc[blk]), _bits(vc[blk])
                tasks.append({"kind": "decode", "fp8": fp8, "kc": kcr, "vc": vcr,
                              "table": np.arange(wl.blocks_per_request)[None],
                              "lens": np.array([wl.context]), "q": _bits(q[r:r + 1]),
                              "kn": _bits(kn[r:r + 1]), "vn": _bits(vn[r:r + 1]),
                              "positions": np.array([wl.context + 1]),
                              "scale": 1.0 / math.sqrt(wl.d)})
        t1, tn, n = time_oracle(tasks, processes=False)
        res["cpu_baseline"] = baseline_record(
            "tokens/s", wl.requests, wl.requests * wl.layers, wl.requests * len(layers_s), t1,
            tn, n,
            f"all {wl.requests} requests in layers {layers_s}, every head",
            f"{len(tasks)} tasks (one per layer and request), threads")
    print(json.dumps(res), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def prefill_flops(lens, hq: int, d: int) -> int:
    """Algorithmic FLOPs of causal attention over sequences of these lengths:
    token t of a sequence takes t+1 keys, 2*d FLOPs per key for q·k and 2*d
    for the weighted V sum, for every query head."""
    return sum(2 * n * (n + 1) * d for n in lens) * hq


def prefill_bench(args):
    """Offline gist extraction: one step is every layer's causal prefill over
    a batch of items [item ; gist], with the gist rows stored into that
    layer's pool."""
    import torch

    import gist_compressed_kv_amd as G
    from gist_compressed_kv_amd import synth

    wl = synth.PREFILL
    dev = "cuda"
    print(f"[bench] generating inputs: {wl.name}", file=sys.stderr, flush=True)
    lens = synth.prefill_lengths(wl, "cpu")
    T = int(lens.sum())
    st = torch.zeros(wl.items + 1, dtype=torch.int32)
    st[1:] = torch.cumsum(lens, 0)
    st = st.to(dev)
    max_len = int(lens.max())
    pool_t = torch.zeros((wl.layers, wl.items, 2, wl.h, wl.k, wl.d), dtype=torch.bfloat16, device=dev)
    pool = G.GistPool(pool_t)
    ids = torch.arange(wl.items, dtype=torch.int32, device=dev)
    # two activation sets, used by alternate layers (one set is 0.6 GB)
    sets = []
    for si in range(2):
        sets.append((synth.randn((T, wl.hq, wl.d), synth.tensor_seed(wl.seed, 21, si), torch.bfloat16, dev),
                     synth.randn((T, wl.h, wl.d), synth.tensor_seed(wl.seed, 22, si), torch.bfloat16, dev),
                     synth.randn((T, wl.h, wl.d), synth.tensor_seed(wl.seed, 23, si), torch.bfloat16, dev)))
    out = torch.empty_like(sets[0][0])
    ws = torch.empty(G.gist_prefill_workspace_bytes(T, wl.h, wl.d), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(wl.d)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step():
        for li in range(wl.layers):
            q, k, v = sets[li % 2]
            G.gist_prefill_attn(q, k, v, st, max_len, 10000.0, scale, out=out, workspace=ws,
                                pool=pool, layer=li, item_ids=ids, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # one call = the K rotation / gist store kernel, then the attention kernel
    avg_s = ev0.elapsed_time(ev1) / 1e3 / (args.steps * wl.layers)
    flops = prefill_flops(lens.tolist(), wl.hq, wl.d)
    achieved = flops / avg_s / 1e12
    res = {
        "metric": "offline gist extraction tokens/s (causal prefill over items + gist, 24 layers)",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V; seeded item lengths",
        "config": {"workload": wl.name, "items": wl.items, "tokens": T, "max_len": max_len},
        "items_per_s": wl.items / (ms / 1e3),
        "roofline": {"bound": "mfma", "kernel": "prefill_prep + prefill_attn (per call)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic("prefill"),
                     "flops_per_launch": flops, "avg_launch_us": avg_s * 1e6},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        # eight seeded items in four layers (each layer uses activation set
        # layer % 2), one task per (layer, item)
        g = torch.Generator().manual_seed(wl.seed * 7919 + 23)
        items = torch.randperm(wl.items, generator=g)[:8].sort().values.tolist()
        layers = [0, 7, 14, 23]
        st_h = st.cpu().numpy()
        tasks = []
        for li in layers:
            q, k, v = sets[li % 2]
            for b in items:
                s0, s1 = int(st_h[b]), int(st_h[b + 1])
                tasks.append({"kind": "prefill", "q": _bits(q[s0:s1]), "k": _bits(k[s0:s1]),
                              "v": _bits(v[s0:s1]), "seq_start": np.array([0, s1 - s0]),
                              "scale": scale})
        sample_tokens = sum(int(st_h[b + 1] - st_h[b]) for b in items) * len(layers)
        t1, tn, n = time_oracle(tasks, processes=False)
        res["cpu_baseline"] = baseline_record(
            "tokens/s", T, T * wl.layers, sample_tokens, t1, tn, n,
            f"items {items} ({sample_tokens // len(layers)} tokens) in layers {layers}, every head",
            f"{len(tasks)} tasks (one per layer and item), threads")
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the gist path has no "
              "cross-GPU step.", file=sys.stderr)
        sys.exit(2)
    if not args.no_cpu_baseline and args.workload not in ("copy", "paged", "paged_fp8", "prefill"):
        start_oracle_pool()  # before anything touches the GPU
    try:
        run(args)
    finally:
        stop_oracle_pool()


def run(args):
    import torch

    if args.workload == "copy":
        copy_probe(args)
        return
    if args.workload in ("paged", "paged_fp8"):
        paged_bench(args, fp8=args.workload == "paged_fp8")
        return
    if args.workload == "prefill":
        prefill_bench(args)
        return

    import gist_compressed_kv_amd as G
    from gist_compressed_kv_amd import synth

    # 24L_b500_last: the same pass with the final layer producing only the last
    # token's rows (what the score head reads)
    last_layer_eos = args.workload == "24L_b500_last"
    wl = {"24L_b500": synth.L24_B500, "24L_b500_last": synth.L24_B500,
          "24L_b500_grouped": synth.L24_B500, "wide_eos_grouped": synth.WIDE_EOS,
          "wide_eos_fp8_grouped": synth.WIDE_EOS_FP8, "24L_b2000": synth.L24_B2000,
          "1L_b500": synth.SINGLE_LAYER, "1L_b500_paged": synth.SINGLE_LAYER,
          "wide_ell64": synth.WIDE_ELL64, "wide_ell64_fp8": synth.WIDE_ELL64_FP8,
          "wide_eos": synth.WIDE_EOS, "wide_eos_fp8": synth.WIDE_EOS_FP8}[args.workload]
    dev = "cuda"
    torch.cuda.init()

    # ---- inputs, all resident in HBM ------------------------------------
    print(f"[bench] generating inputs: {wl.name}", file=sys.stderr, flush=True)
    if wl.fp8:
        pool_t = synth.randn_fp8_gist_pool(wl.layers, wl.n_items, wl.k, wl.h, wl.d,
                                           synth.tensor_seed(wl.seed, 1), dev)
        pool = G.GistPool(pool_t, shape=(wl.layers, wl.n_items, wl.k, wl.h, wl.d))
    else:
        pool_t = synth.randn((wl.layers, wl.n_items, 2, wl.h, wl.k, wl.d),
                             synth.tensor_seed(wl.seed, 1), wl.dtype, dev)
        pool = G.GistPool(pool_t)
    ids = synth.item_ids_per_query(wl.queries, wl.pairs // wl.queries, wl.n_items, wl.seed, dev)
    qpool = q_ids = None
    if wl.kq:
        if wl.fp8:
            qpool_t = synth.randn_fp8_gist_pool(wl.layers, wl.queries, wl.kq, wl.h, wl.d,
                                                synth.tensor_seed(wl.seed, 2), dev)
            qpool = G.GistPool(qpool_t, shape=(wl.layers, wl.queries, wl.kq, wl.h, wl.d))
        else:
            qpool_t = synth.randn((wl.layers, wl.queries, 2, wl.h, wl.kq, wl.d),
                                  synth.tensor_seed(wl.seed, 2), wl.dtype, dev)
            qpool = G.GistPool(qpool_t)
        q_ids = (torch.arange(wl.pairs, device=dev) // (wl.pairs // wl.queries)).to(torch.int32)
    # one distinct activation set per layer, and at least four for the
    # single-layer workload (one 133 MB set would stay in the 256 MB
    # Infinity Cache); consecutive passes walk through the sets.  The wide
    # l = 64 workloads reuse one set: 4.8 GB per layer already dwarfs every
    # cache.  The wide EOS workloads walk through eight sets (a layer's
    # 72 MB of Q, K/V_new and O would otherwise stay cached between layers).
    n_sets = max(wl.layers, 4) if wl.d == 64 else (8 if wl.ell == 1 else 1)
    qs, kns, vns, outs = [], [], [], []
    for li in range(n_sets):
        qs.append(synth.randn((wl.pairs, wl.ell, wl.hq, wl.d), synth.tensor_seed(wl.seed, 3, li), wl.dtype, dev))
        kns.append(synth.randn((wl.pairs, wl.ell, wl.h, wl.d), synth.tensor_seed(wl.seed, 4, li), wl.dtype, dev))
        vns.append(synth.randn((wl.pairs, wl.ell, wl.h, wl.d), synth.tensor_seed(wl.seed, 5, li), wl.dtype, dev))
        outs.append(torch.empty_like(qs[-1]))
    # 1L_b500_paged: the same gists read from a paged cache of 16-row blocks,
    # item i's gist in rows 0..k-1 of block i (the rest of each block unused)
    paged = args.workload == "1L_b500_paged"
    if paged:
        kc = torch.zeros((wl.n_items, wl.h, 16, wl.d), dtype=wl.dtype, device=dev)
        vc = torch.zeros_like(kc)
        kc[:, :, :wl.k], vc[:, :, :wl.k] = pool_t[0, :, 0], pool_t[0, :, 1]
    # *_grouped: the pass's layer calls as one grouped launch (each layer a
    # group with the activation set the per-layer pass gives it, and an
    # output of its own)
    grouped = None
    if args.workload.endswith("_grouped"):
        specs = []
        for li in range(wl.layers):
            sp = {"layer": li, "item_ids": ids, "q": qs[li % n_sets], "k_new": kns[li % n_sets],
                  "v_new": vns[li % n_sets], "out": torch.empty_like(qs[li % n_sets])}
            if qpool is not None:
                sp["q_ids"] = q_ids
            specs.append(sp)
        grouped = G.GroupedForward(pool, specs, pos0=wl.pos0, rope_base=10000.0,
                                   scale=1.0 / math.sqrt(wl.d), qpool=qpool)
    q_lasts = [q[:, -1].contiguous() for q in qs] if last_layer_eos else None
    out_last = torch.empty_like(q_lasts[0]) if last_layer_eos else None
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(wl.d)
    stream = torch.cuda.current_stream()

    passes = [0]

    def step():
        if grouped is not None:
            grouped(stream)
            passes[0] += 1
            return
        base = passes[0] * wl.layers
        for li in range(wl.layers):
            si = (base + li) % n_sets
            if last_layer_eos and li == wl.layers - 1:
                G.gist_attn_forward_last(pool, li, ids, q_lasts[si], kns[si], vns[si], wl.pos0,
                                         10000.0, scale, qpool=qpool, q_ids=q_ids, out=out_last,
                                         stream=stream)
            elif paged:
                G.gist_attn_forward_paged(kc, vc, ids, wl.k, qs[si], kns[si], vns[si], pos0=wl.pos0,
                                          scale=scale, out=outs[si], stream=stream)
            else:
                G.gist_attn_forward(pool, li, ids, qs[si], kns[si], vns[si], wl.pos0, 10000.0, scale,
                                    qpool=qpool, q_ids=q_ids, out=outs[si], stream=stream)
        passes[0] += 1

    # the oracle baseline runs here, on the inputs just generated, and its
    # worker processes are gone before the timed region: with them alive the
    # host-side launch loop of the short-launch workloads ran up to 1.5x
    # slower
    cpu_base = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu_base = gist_baseline(wl, pool, ids, qs, kns, vns, n_sets, qpool, q_ids)
        stop_oracle_pool()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole passes -------------------------------------
    # HIP events on the launch stream bracket the region; every launch in it
    # runs the one kernel, back to back, so region time / launches is that
    # kernel's average launch duration
    # (an event after every pass as well, for the median pass)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # a grouped workload runs the whole pass as one launch
    launches = 1 if grouped is not None else wl.layers
    avg_launch_s = evs[0].elapsed_time(evs[-1]) / 1e3 / (args.steps * launches)
    pass_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    median_pass_ms = pass_ms[len(pass_ms) // 2]

    bytes_unit = gist_bytes_per_pair_layer(wl)
    bytes_launch = bytes_unit * wl.pairs * (wl.layers // launches)
    if last_layer_eos:
        # the pass moves L-1 full layers and one last-token layer; price the
        # pass's bytes over the pass's launches
        last_bytes = gist_bytes_per_pair_layer(wl, last_only=True) * wl.pairs
        bytes_launch = (bytes_launch * (wl.layers - 1) + last_bytes) / wl.layers
    achieved_gbps = bytes_launch / avg_launch_s / 1e9
    pairs_per_s = wl.pairs / (ms_per_step / 1e3)
    traffic = measured_traffic(args.workload)

    res = {
        "metric": METRIC if args.workload == "24L_b500" else
                  "pairs/s + % of HBM peak, gist-KV attention (24L, GQA 14:2, k=8, ℓ=64; final "
                  "layer for the last token only)" if last_layer_eos else
                  f"pairs/s + % of HBM peak, gist-KV attention ({args.workload})",
        "value": pairs_per_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic: N(0,1) pools" + (" (E4M3 codes, scale amax/448 per block)" if wl.fp8 else "")
                + ", Q/K/V; seeded item ids (50 distinct candidates per query)"
                + ("; gists read from a paged cache of 16-row blocks" if paged else "")
                + (f"; the {wl.layers} layer calls of a pass as one grouped launch" if grouped is not None else ""),
        "config": {"workload": wl.name + (", gists in a paged cache" if paged else ""), "layers": wl.layers, "pairs": wl.pairs, "hq": wl.hq,
                   "h": wl.h, "head_dim": wl.d, "k": wl.k, "k_query_gist": wl.kq, "ell": wl.ell,
                   "pool_items": wl.n_items, "parallelism": "single GPU"},
        "tokens_per_s": pairs_per_s * wl.ell,
        "pass_hbm_gbps_algorithmic": bytes_launch * launches / (ms_per_step / 1e3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "kernel": "gist_fwd_mfma<64> (23 full layers + 1 last-token layer; pass bytes / "
                      "launches)" if last_layer_eos else
                      (f"gist_fwd_{'mfma' if wl.ell > 1 else 'eos'}_grouped<{wl.d}{', fp8 gist' if wl.fp8 else ''}>"
                       f" ({wl.layers} layer groups in one launch)") if grouped is not None else
                      "gist_fwd_mfma<64>" if wl.ell > 1 and wl.d == 64 else
                      (("gist_fwd_mfma<128, fp8 gist>" if wl.fp8 else "gist_fwd_mfma<128>") if wl.ell > 1 else
                       ("gist_fwd_eos<128, fp8 gist>" if wl.fp8 else "gist_fwd_eos<128>")),
            "achieved": achieved_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "bytes_per_unit": bytes_unit,
            "units_per_launch": wl.pairs * (wl.layers // launches),
            "avg_launch_us": avg_launch_s * 1e6,
            "median_launch_us": median_pass_ms * 1e3 / launches,
        },
        "median_pass_ms": median_pass_ms,
    }
    if cpu_base is not None:
        res["cpu_baseline"] = cpu_base
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

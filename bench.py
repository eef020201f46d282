#!/usr/bin/env python3
"""Benchmark: one paged-decode serving step on one MI355X.

A step is the whole hot path over one batch: the copy-on-write block copies
and the write of every sequence's new token into the pool (one
kv_cache_append launch; --two-launch-edits: copy_blocks then kv_cache_write),
and paged decode attention (with its split-K merge).  The default workload is the GQA
prefix-sharing batch: 256 sequences, lognormal context lengths (median 1024,
cap 8192), 32 query / 8 KV heads, head_dim 128, 16-token blocks, bf16, each
group of 16 sequences sharing the physical blocks of a 1024-token prefix.
Inputs are seeded synthetic data resident in HBM before timing starts.

Prints one JSON line.  `value` is the step's unique HBM bytes (each distinct
KV slot read once -- the least HBM must deliver -- plus q, out, tables,
partials and the edits) per second of step time (the timed steps run with no
event between their launches).  `roofline` prices the decode call (the
dispatch sort of large launches, the decode kernel and the partition merge;
the mean of as many calls back to back, timed with HIP events on the stream
they run on) against the MI355X HBM
peak with the same unique algorithmic bytes: `frac` is the one "% of peak"
figure of the line.  Beside it: `effective_gbps`, the same call priced with
attended bytes (K and V once per sequence and KV head through its block
table, which counts a shared prefix once per sequence that reads it: more
than HBM has to deliver), and `traffic`, the bytes the rocprofv3
FETCH_SIZE/WRITE_SIZE counters saw per decode call, scaled by what the same
counters read for a copy of known size (`--copy-calibration`), when the
committed counter summary was taken on the current decode sources, with
`reread_ratio` = traffic / unique bytes (1.0 = every byte fetched once).

Other modes:
  --copy-calibration      also run one copy_blocks call over a 1 GiB pool first
                          (512 MiB read + 512 MiB written): the reference
                          dispatch for the counter scale factors
  --summarize-counters F W
                          read the rocprofv3 counter CSVs of a FETCH_SIZE run
                          (directory F) and a WRITE_SIZE run (directory W) of
                          this script with --copy-calibration, and print the
                          JSON record kept in profiles/decode_counters.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode achieved HBM GB/s (% of peak) and attended KV tokens/s, 1 GPU"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
CSRC = os.path.join(ROOT, "paged_kv_cache_386_amd", "csrc")
# what decides the decode kernels' memory traffic: their sources (with the
# dispatch-order sort) and the partition policy (the text of
# resolve_partitions in api.hip)
DECODE_SOURCES = ["decode.hip", "decode_mfma.hip", "schedule.hip"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_counters.json")
SCHEDULE_MIN_WORKGROUPS = 1024  # launches above this sort their items first

# calibration copy: CAL_PAIRS blocks of CAL_BLOCK_BYTES in each of two caches
CAL_BLOCKS = 16384
CAL_PAIRS = 8192
CAL_SHAPE = (CAL_BLOCKS, 8, 16, 128)  # [blocks][kv_heads][block_size][head_dim], bf16: 32 KiB
CAL_BLOCK_BYTES = 8 * 16 * 128 * 2
CAL_READ_BYTES = 2 * CAL_PAIRS * CAL_BLOCK_BYTES
CAL_WRITE_BYTES = CAL_READ_BYTES


# ---------------------------------------------------------------- byte model

def kv_row_bytes(case) -> int:
    """Bytes of one token's K (or V) row over all KV heads, as stored in the
    pool (one byte per element for an FP8 pool)."""
    el = getattr(case, "kv_elem_bytes", None) or (4 if case.dtype == "f32" else 2)
    return case.num_kv_heads * case.head_dim * el


def unique_slots(case) -> int:
    """Distinct (physical block, offset) pairs decode reads: a slot shared by
    several sequences (a prefix block) counts once."""
    import numpy as np
    B = case.block_size
    ids = []
    for s, L in enumerate(case.context_lens.tolist()):
        pos = np.arange(L, dtype=np.int64)
        ids.append(case.block_tables[s, pos // B].astype(np.int64) * B + pos % B)
    return int(np.unique(np.concatenate(ids)).size) if ids else 0


def decode_bytes(case, num_partitions: int, partition_size: int, unique: bool) -> int:
    """Algorithmic bytes of one decode call: K and V rows (each distinct slot
    once when ``unique``, else once per attending sequence), q, out, the used
    block-table entries, context lengths, for split sequences the partition
    partials written by decode and read by the merge, and for large launches
    the dispatch list (int32 per (sequence, partition), written and read)."""
    import numpy as np
    L = case.context_lens.astype(np.int64)
    S, Hq, D, B = case.num_seqs, case.num_q_heads, case.head_dim, case.block_size
    el = 4 if case.dtype == "f32" else 2
    slots = unique_slots(case) if unique else int(L.sum())
    kv = 2 * slots * kv_row_bytes(case)
    qo = S * Hq * D * (el + 4)
    tables = int(((L + B - 1) // B).sum()) * 4 + S * 4
    partials = 0
    if num_partitions > 1:
        n = np.minimum((L + partition_size - 1) // partition_size, num_partitions)
        split = n[n > 1].sum()
        partials = 2 * int(split) * Hq * (D + 2) * 4
    order = 0
    if S * case.num_kv_heads * num_partitions > SCHEDULE_MIN_WORKGROUPS:
        order = 2 * 4 * S * num_partitions + 4 * S  # the list, and the lengths it sorts by
    return kv + qo + tables + partials + order


def edit_bytes(case) -> int:
    """Algorithmic bytes of the step's cache edits: each copied block read and
    written in K and V; each new token's K and V rows read and written."""
    if not case.has_step:
        return 0
    blk = case.block_size * kv_row_bytes(case)
    copies = 2 * 2 * blk * len(case.copy_pairs)
    T = len(case.slot_mapping)
    src_row = case.num_kv_heads * case.head_dim * (4 if case.dtype == "f32" else 2)
    writes = 2 * (src_row + kv_row_bytes(case)) * T + 4 * T + 8 * len(case.copy_pairs)
    return copies + writes


# ---------------------------------------------------------------- counters

def decode_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(CSRC, "api.hip"), "rb") as f:
        api = f.read()
    start = api.index(b"int32_t resolve_partitions(")
    h.update(api[start:api.index(b"\n}\n", start)])
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """Measured HBM bytes per decode call from the committed counter summary,
    or None when absent or taken on different decode sources."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("decode_src_sha256_16") != decode_source_hash():
        return None
    return entry.get("bytes_per_call")


def _counter_rows(directory: str, counter: str):
    """(dispatch id, kernel name, grid size, value in KiB) of every dispatch."""
    paths = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                                 float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_counters(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """Scale factors from the calibration copy (the first copy_blocks dispatch,
    whose grid covers CAL_PAIRS pairs) and measured bytes per decode call
    (dispatch sort, decode kernel and merge, averaged over the calls after
    the first)."""
    out = {}
    for counter, directory, true_bytes in (("FETCH_SIZE", fetch_dir, CAL_READ_BYTES),
                                           ("WRITE_SIZE", write_dir, CAL_WRITE_BYTES)):
        rows = _counter_rows(directory, counter)
        cal = [r for r in rows if "copy_blocks_kernel" in r[1]]
        if not cal:
            raise SystemExit("no calibration copy_blocks dispatch: run bench.py --copy-calibration")
        factor = true_bytes / (cal[0][3] * 1024.0)
        # one decode call = the dispatch sort (large launches), one
        # decode-kernel dispatch and the merge that follows it
        calls = []
        pending = 0.0
        for did, name, grid, kib in rows:
            if "decode_schedule_kernel" in name:
                pending += kib
            elif "paged_decode_mfma_kernel" in name or "paged_decode_kernel" in name:
                calls.append(kib + pending)
                pending = 0.0
            elif "paged_decode_merge_kernel" in name and calls:
                calls[-1] += kib
        if len(calls) < 2:
            raise SystemExit(f"{counter}: fewer than two decode calls in {directory}")
        per_call = sum(calls[1:]) / len(calls[1:]) * 1024.0 * factor
        out[counter] = {"factor": round(factor, 4), "raw_kib_calibration": cal[0][3],
                        "bytes_per_call": int(per_call), "calls": len(calls)}
    return {
        workload: {
            "bytes_per_call": out["FETCH_SIZE"]["bytes_per_call"] + out["WRITE_SIZE"]["bytes_per_call"],
            "fetch": out["FETCH_SIZE"],
            "write": out["WRITE_SIZE"],
            "decode_src_sha256_16": decode_source_hash(),
        }
    }


# ---------------------------------------------------------------- helpers

def to_dev(a, dev):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def copy_calibration(dev) -> None:
    """One copy_blocks call of known size: CAL_PAIRS blocks copied in each of
    two bf16 caches of CAL_BLOCKS 32 KiB blocks (1 GiB in all)."""
    import torch

    import paged_kv_cache_386_amd as pa
    kc = torch.ones(CAL_SHAPE, dtype=torch.bfloat16, device=dev)
    vc = torch.ones(CAL_SHAPE, dtype=torch.bfloat16, device=dev)
    src = torch.arange(CAL_PAIRS, dtype=torch.int32)
    pairs = torch.stack([src, src + CAL_PAIRS], dim=1).contiguous().to(dev)
    torch.cuda.synchronize()
    pa.copy_blocks(pairs, kc, vc)
    torch.cuda.synchronize()
    del kc, vc, pairs
    torch.cuda.empty_cache()


def cpu_baseline(case, budget_s: float):
    """Time the oracle (single thread) on the same workload: the step's edits
    and decode for as many sequences as fit the time budget (all of them for
    the default workload)."""
    from threadpoolctl import threadpool_limits

    from oracle import oracle as O

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kc, vc = case.k_cache, case.v_cache
        if case.has_step:
            kc, vc = O.copy_blocks(case.copy_pairs, kc, vc)
            kc, vc = O.kv_cache_write(case.k_new, case.v_new, case.slot_mapping, kc, vc,
                                      case.block_size)
        t_edit = time.perf_counter() - t0
        done = 0
        t_dec = 0.0
        for s in range(case.num_seqs):
            t1 = time.perf_counter()
            O.paged_attention_decode(case.q[s:s + 1], kc, vc, case.block_tables[s:s + 1],
                                     case.context_lens[s:s + 1], case.scale, case.block_size,
                                     case.dtype)
            t_dec += time.perf_counter() - t1
            done += 1
            if t_edit + t_dec > budget_s:
                break
    frac = done / case.num_seqs
    tokens = int(case.context_lens[:done].sum())
    # scale the oracle's time to the whole step (edits once, decode pro rata)
    est_step = t_edit + t_dec / max(frac, 1e-9)
    res = {
        "seconds": t_edit + t_dec,
        "est_step_seconds": est_step,
        "edit_seconds": t_edit,
        "seqs": done,
        "tokens": tokens,
        "tokens_per_s": tokens / t_dec if t_dec > 0 else None,
    }
    res["all_cores"] = _cpu_baseline_pool(case, kc, vc, done)
    return res


_POOL = {}
CPU_WORKER_CAP = 16  # worker processes one GPU's job may run on a shared host


def _pool_decode(seq_ids):
    """Worker: the oracle's decode of some sequences, one thread."""
    from threadpoolctl import threadpool_limits

    from oracle import oracle as O

    c, kc, vc = _POOL["case"], _POOL["kc"], _POOL["vc"]
    with threadpool_limits(limits=1):
        for s in seq_ids:
            O.paged_attention_decode(c.q[s:s + 1], kc, vc, c.block_tables[s:s + 1],
                                     c.context_lens[s:s + 1], c.scale, c.block_size, c.dtype)
    return len(seq_ids)


def _cpu_baseline_pool(case, kc, vc, num_seqs):
    """The same oracle decode over the same sequences, spread over the host's
    cores by a fork-started process pool, one single-threaded worker per core
    of the affinity set, capped at 16 worker processes: the host CPU share
    one GPU's job is allowed on a shared multi-GPU host (the record states
    both counts).  Must run before the process touches the GPU: the workers
    are forked from it."""
    import multiprocessing as mp

    available = len(os.sched_getaffinity(0))
    cores = max(1, min(CPU_WORKER_CAP, available))
    _POOL.update(case=case, kc=kc, vc=vc)
    # longest first, dealt round-robin, so that the workers finish together
    order = sorted(range(num_seqs), key=lambda s: -int(case.context_lens[s]))
    chunks = [order[i::cores * 4] for i in range(cores * 4)]
    chunks = [c for c in chunks if c]
    try:
        with mp.get_context("fork").Pool(cores) as pool:
            pool.map(len, [[0]] * cores)  # start every worker before timing
            t0 = time.perf_counter()
            pool.map(_pool_decode, chunks, chunksize=1)
            t = time.perf_counter() - t0
    finally:
        _POOL.clear()
    return {"cores": cores, "cores_available": available, "decode_seconds": t,
            "seqs": num_seqs, "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- serving

SERVING_METRIC = "continuous-batching decode: generated tokens/s and per-step latency, 1 GPU"
SERVING = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=40960,
               max_batch=512, max_context_len=2048, max_prompt_rows=16384,
               prompt=(16, 1536), new_tokens=(16, 512), fork_every=8, samples=4,
               requests=8192, seed=4)


def serving_bench(args) -> int:
    """The native engine (include/pagedattn_engine.h) over a stream of
    requests shaped like the continuous-batching step: 32 q / 8 KV heads,
    head_dim 128, 16-token blocks, bf16, prompts U[16, 1536], outputs
    U[16, 512] tokens, every 8th request with 4 parallel samples, all queued
    at the start, at most 512 sequences per step.  Warm-up steps fill the
    batch; the timed steps run at steady state (finishes, admissions, forks
    and copy-on-write as they come).  Token data are synthetic and fixed
    (the engine's bookkeeping, not the values, sets the work)."""
    import numpy as np
    import torch

    import paged_kv_cache_386_amd as pa

    c = SERVING
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()
    g = torch.Generator(device=dev)
    g.manual_seed(c["seed"])
    NB, Hkv, B, D, Hq = c["num_blocks"], c["num_kv_heads"], c["block_size"], c["head_dim"], \
        c["num_q_heads"]
    mb, R = c["max_batch"], c["max_prompt_rows"]

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    # the pool: bfloat16, or 8-bit codes (one byte per element, one scale per
    # cache) written by the engine's quantising writes from bfloat16 rows
    pool_dtype = torch.uint8 if args.kv_fp8 else torch.int8 if args.kv_int8 else torch.bfloat16
    k_scale, v_scale = (0.25, 0.5) if args.kv_fp8 else (0.02, 0.03) if args.kv_int8 else (1., 1.)
    kc = torch.zeros((NB, Hkv, B, D), dtype=pool_dtype, device=dev)
    vc = torch.zeros_like(kc)
    q, kn, vn = randn(mb, Hq, D), randn(mb, Hkv, D), randn(mb, Hkv, D)
    pk, pv = randn(R, Hkv, D), randn(R, Hkv, D)
    out = torch.empty((mb, Hq, D), dtype=torch.float32, device=dev)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    eng = pa.Engine(kc, vc, num_q_heads=Hq, max_batch=mb, max_context_len=c["max_context_len"],
                    max_prompt_rows=R, k_scale=k_scale, v_scale=v_scale,
                    host_plan=not args.no_host_plan)
    rng = np.random.default_rng(c["seed"])
    for r in range(c["requests"]):
        samples = c["samples"] if r % c["fork_every"] == c["fork_every"] - 1 else 1
        eng.submit(r, int(rng.integers(c["prompt"][0], c["prompt"][1] + 1)),
                   int(rng.integers(c["new_tokens"][0], c["new_tokens"][1] + 1)), samples)
    stream = torch.cuda.current_stream()

    def step():
        return eng.step(q, kn, vn, pk, pv, scale, out, stream=stream, arrays=False)

    t0 = time.perf_counter()
    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] serving warm-up: {args.warmup} steps in {time.perf_counter() - t0:.2f}s, "
          f"{eng.num_running()} running, {eng.num_waiting()} waiting", file=sys.stderr, flush=True)

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    infos = []
    host = np.zeros(K)
    # the Python loop around the engine is the harness, not the engine: keep
    # the collector's pauses (milliseconds, leaving the GPU idle) out of it
    import gc
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        h0 = time.perf_counter()
        infos.append(step())
        host[i] = time.perf_counter() - h0
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    gpu_ms = np.array([a.elapsed_time(b) for a, b in ev])
    tokens = sum(x.batch for x in infos)
    ctx = sum(x.context_tokens for x in infos)
    uniq = sum(x.unique_tokens for x in infos)
    kv_token_bytes = 2 * Hkv * D * kc.element_size()
    # unique bytes (each shared prefix slot once, as the decode benchmark
    # counts them) per second of GPU step time; attended beside it
    unique_gbps = uniq * kv_token_bytes / (gpu_ms.sum() * 1e-3) / 1e9
    attended_gbps = ctx * kv_token_bytes / (gpu_ms.sum() * 1e-3) / 1e9
    host_us = np.array([x.host_us for x in infos])
    wait_us = np.array([x.wait_us for x in infos])
    rec = {
        "metric": SERVING_METRIC,
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if pool_dtype == torch.bfloat16 else
                 ("fp8-e4m3 pool (bf16 q and rows)" if args.kv_fp8 else
                  "int8 pool (bf16 q and rows)"),
        "data": "synthetic (fixed N(0,1) token rows; seeded request lengths and samples)",
        "config": {
            "workload": ("serving: engine over 8192 queued requests, prompts U[16,1536], "
                         "outputs U[16,512], every 8th with 4 samples, <=512 seqs/step, "
                         "32q/8kv, d128, B16, 40960-block pool"
                         + (", FP8 pool" if args.kv_fp8 else ", INT8 pool" if args.kv_int8
                            else "")),
            **{k: v for k, v in c.items() if k not in ("seed",)},
            "host_plan": not args.no_host_plan,
        },
        "step_latency_ms": {
            "gpu_mean": round(float(gpu_ms.mean()), 4),
            "gpu_p50": round(float(np.percentile(gpu_ms, 50)), 4),
            "gpu_p99": round(float(np.percentile(gpu_ms, 99)), 4),
            # the host's time in pa_engine_step, and of it the wait for a
            # staging buffer the device still reads (the host runs ahead)
            "host_call_mean": round(float(host.mean() * 1e3), 4),
            "host_wait_mean": round(float(wait_us.mean() / 1e3), 4),
            "host_work_mean": round(float((host_us - wait_us).mean() / 1e3), 4),
            "wall_mean": round(wall / K * 1e3, 4),
        },
        "batch_mean": round(tokens / K, 1),
        "context_tokens_per_step": round(ctx / K, 1),
        "unique_tokens_per_step": round(uniq / K, 1),
        "attended_kv_tokens_per_s": round(ctx / wall, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "one engine step (index copy, prompt writes, copies, token writes, decode)",
            "achieved": round(unique_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(unique_gbps / PEAK_HBM_GBPS, 4),
            "traffic": None,
            "frac_definition": ("unique KV bytes per step (attended tokens with each shared "
                                "prefix slot once, 2 * kv_heads * head_dim * element bytes "
                                "each) / mean GPU step time / 8 TB/s"),
            "algorithmic_bytes_per_step": int(uniq * kv_token_bytes / K),
            "attended_bytes_per_step": int(ctx * kv_token_bytes / K),
            "effective_gbps": round(attended_gbps, 1),
        },
        "admitted": sum(x.admitted for x in infos),
        "finished": sum(x.finished for x in infos),
        "preempted": sum(x.preempted for x in infos),
        "copies": sum(x.num_copies for x in infos),
        "prompt_rows": sum(x.prompt_rows for x in infos),
        "free_blocks_min": min(x.free_blocks for x in infos),
    }
    eng.close()
    print(json.dumps(rec))
    return 0


# ---------------------------------------------------------------- multi-query

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def multi_query_bench(args) -> int:
    """Causal multi-query paged attention on one of its two workloads:
    chunked prefill (16 sequences, contexts U[1024, 8192], a 512-token chunk
    each) is bound by the matrix cores and priced in bf16 TFLOP/s (4 * D
    flops per query head and attended position: q.K and p.V); speculative
    verification (256 sequences, 5 tokens each, prefix-shared lognormal
    contexts) is bound by HBM and priced in GB/s of K/V read once per
    (sequence, KV head)."""
    import numpy as np
    import torch

    import paged_kv_cache_386_amd as pa
    from workloads import make_multi_query_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()
    c = make_multi_query_workload(args.multi_query, poison=False)
    b = c.base
    if args.multi_query == "spec-verify" and args.verify_tokens != 5:
        from workloads import make_multi_query_case
        c = make_multi_query_case(b, np.minimum(b.context_lens, args.verify_tokens), 7,
                                  c.name, c.description)
    q = to_dev(c.q, dev)
    c8 = None
    if args.kv_fp8 or args.kv_int8:
        from workloads.generate import make_fp8_case, make_int8_case
        c8 = make_fp8_case(b, 71) if args.kv_fp8 else make_int8_case(b, 71)
        kc = torch.from_numpy(c8.k8).to(dev)
        vc = torch.from_numpy(c8.v8).to(dev)
    else:
        kc, vc = to_dev(b.k_cache, dev), to_dev(b.v_cache, dev)
    tables = torch.from_numpy(b.block_tables).to(dev)
    lens = torch.from_numpy(b.context_lens).to(dev)
    qs = torch.from_numpy(c.query_start).to(dev)
    out = torch.empty((c.num_tokens, b.num_q_heads, b.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    max_ctx = int(b.context_lens.max())
    P = pa.multi_query_partitions(b.num_seqs, b.num_q_heads, b.num_kv_heads, c.max_query_len,
                                  max_ctx, args.partition_size)
    # shared prefixes (speculative verification: the groups' prompts): found
    # by the host in the tables it built, at most 16 members per group
    groups_np = np.zeros((0, 2), np.int32)
    shared_np = np.zeros(b.num_seqs, np.int32)
    if not args.no_prefix and args.multi_query == "spec-verify":
        groups_np, shared_np = pa.prefix_groups(b.block_tables, b.context_lens, b.block_size,
                                                b.num_q_heads, b.num_kv_heads, 16)
        keep = []
        for f, m in groups_np.tolist():
            keep += [[s, min(16, f + m - s)] for s in range(f, f + m, 16)]
        groups_np = np.array(keep, np.int32).reshape(-1, 2)
    use_prefix = len(groups_np) > 0
    # the library takes prefix items over bf16 pools with at most 8 (token,
    # head) rows per sequence and KV head; otherwise the call is the plain one
    prefix_items = (use_prefix and c8 is None and
                    c.max_query_len * (b.num_q_heads // b.num_kv_heads) <= 8)
    kv_code = (pa.PA_BF16 if c8 is None else pa.PA_FP8_E4M3 if args.kv_fp8 else pa.PA_INT8)
    if use_prefix:
        groups_d = torch.from_numpy(groups_np).to(dev)
        shared_d = torch.from_numpy(shared_np).to(dev)
        ws_bytes = pa.multi_query_prefix_workspace_size(
            b.num_seqs, c.num_tokens, b.num_q_heads, b.num_kv_heads, b.head_dim,
            c.max_query_len, max_ctx, args.partition_size, len(groups_np), kv_code)
    else:
        ws_bytes = pa.multi_query_workspace_size(
            b.num_seqs, c.num_tokens, b.num_q_heads, b.num_kv_heads, b.head_dim,
            c.max_query_len, max_ctx, args.partition_size)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # the dispatch list planned on the host, once (the lengths and groups are
    # the host's); --device-sort sorts on the device in every call instead
    plan_d = None
    if not args.device_sort:
        plan = pa.multi_query_plan(
            b.context_lens, groups_np if use_prefix else None, shared_np if use_prefix else None,
            num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
            block_size=b.block_size, max_blocks_per_seq=b.block_tables.shape[1],
            max_query_len=c.max_query_len, max_context_len=max_ctx, kv_dtype=kv_code,
            partition_size=args.partition_size)
        plan_d = torch.from_numpy(plan).to(dev)

    def call():
        if use_prefix or plan_d is not None:
            pa.paged_attention_multi_query_prefix(
                q, kc, vc, tables, lens, qs, groups_d if use_prefix else None,
                shared_d if use_prefix else None, float(b.scale), out,
                max_query_len=c.max_query_len, max_context_len=max_ctx,
                k_scale=1.0 if c8 is None else float(c8.k_scale),
                v_scale=1.0 if c8 is None else float(c8.v_scale),
                partition_size=args.partition_size, workspace=ws, dispatch=plan_d,
                stream=stream)
        elif c8 is not None:
            mq8 = (pa.paged_attention_multi_query_fp8 if args.kv_fp8 else
                   pa.paged_attention_multi_query_int8)
            mq8(
                q, kc, vc, tables, lens, qs, float(b.scale), float(c8.k_scale),
                float(c8.v_scale), out, max_query_len=c.max_query_len, max_context_len=max_ctx,
                partition_size=args.partition_size, workspace=ws, stream=stream)
        else:
            pa.paged_attention_multi_query(q, kc, vc, tables, lens, qs, float(b.scale), out,
                                           max_query_len=c.max_query_len,
                                           max_context_len=max_ctx,
                                           partition_size=args.partition_size, workspace=ws,
                                           stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    Hq, Hkv, D = b.num_q_heads, b.num_kv_heads, b.head_dim
    attended = 0  # (query token, position) pairs
    kv_tokens = 0  # positions read per (sequence, KV head) group
    for s in range(b.num_seqs):
        n = int(c.query_start[s + 1] - c.query_start[s])
        L = int(b.context_lens[s])
        attended += sum(L - n + i + 1 for i in range(n))
        kv_tokens += L if n else 0
    flops = attended * Hq * 4 * D
    el = 1 if c8 is not None else 2
    # K/V priced with each distinct slot once (a shared prefix block counts
    # once, as for decode); attended (once per sequence and KV head) beside it
    kv_bytes = unique_slots(b) * Hkv * D * 2 * el
    kv_attended = kv_tokens * Hkv * D * 2 * el
    io_bytes = c.num_tokens * Hq * D * (2 + 4) + b.block_tables.nbytes + 8 * b.num_seqs
    tflops = flops / (us * 1e-6) / 1e12
    gbps = (kv_bytes + io_bytes) / (us * 1e-6) / 1e9
    mfma_bound = args.multi_query == "chunked-prefill"
    from workloads import MULTI_QUERY_NAMES
    rec = {
        "metric": ("multi-query paged attention: achieved bf16 TFLOP/s" if mfma_bound else
                   "multi-query paged attention: achieved HBM GB/s"),
        "value": round(tflops if mfma_bound else gbps, 2),
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c8 is None else
                 ("fp8-e4m3 (bf16 q)" if args.kv_fp8 else "int8 (bf16 q)"),
        "data": "synthetic (seeded N(0,1) q/K/V; lengths as described)" + (
            "" if c8 is None else
            f"; K/V as random {'E4M3' if args.kv_fp8 else 'INT8'} codes, k_scale "
            f"{float(c8.k_scale)}, v_scale {float(c8.v_scale)}"),
        "config": {"workload": f"{args.multi_query}: " + MULTI_QUERY_NAMES[args.multi_query].replace(
                       "5 tokens", f"{args.verify_tokens} tokens")
                               + ("" if c8 is None else
                                  " over an FP8 pool" if args.kv_fp8 else " over an INT8 pool"),
                   "num_seqs": b.num_seqs, "num_tokens": c.num_tokens,
                   "max_query_len": c.max_query_len, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": b.block_size,
                   "total_context_tokens": int(b.context_lens.sum()), "num_partitions": P,
                   "prefix_groups": int(len(groups_np)),
                   "call": ("paged_attention_multi_query_prefix (shared prefixes read once "
                            "per group; + merge)" if prefix_items else
                            "paged_attention_multi_query_prefix (the plain call, groups "
                            "ignored: prefix items take bf16 pools with at most 8 rows per "
                            "sequence and KV head)"
                            if use_prefix else
                            "paged_attention_multi_query_prefix with no groups (the plain "
                            "call)" if plan_d is not None else
                            "paged_attention_multi_query" + ("" if c8 is None else
                                                             "_fp8" if args.kv_fp8 else
                                                             "_int8"))
                           + ("; dispatch list planned on the host" if plan_d is not None else
                              "; dispatch list sorted on the device")},
        "attended_pairs_per_s": round(attended * Hq / (us * 1e-6), 1),
        "query_tokens_per_s": round(c.num_tokens / (us * 1e-6), 1),
        "kernel_us": round(us, 2),
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": "paged_multi_query_kernel",
            "achieved": round(tflops if mfma_bound else gbps, 2),
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round((tflops / PEAK_BF16_TFLOPS) if mfma_bound else (gbps / PEAK_HBM_GBPS), 4),
            "traffic": None,
            "frac_definition": (
                "4 * head_dim flops per (query head, attended position) per call / mean call "
                "time / 2.5 PFLOP/s dense bf16" if mfma_bound else
                "unique algorithmic bytes per call (each distinct KV slot once, plus q, out, "
                "tables, lengths) / mean call time / 8 TB/s"),
            "algorithmic_flops_per_call": flops,
            "algorithmic_bytes_per_call": kv_bytes + io_bytes,
            "attended_bytes_per_call": kv_attended + io_bytes,
            "effective_gbps": round((kv_attended + io_bytes) / (us * 1e-6) / 1e9, 1),
            "other": {"tflops": round(tflops, 2), "gbps": round(gbps, 1)},
        },
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(rec))
    return 0


# ---------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 300 with --serving)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 10; 200 with --serving)")
    ap.add_argument("--serving", action="store_true",
                    help="time the continuously batched engine over a request stream instead")
    ap.add_argument("--multi-query", choices=["chunked-prefill", "spec-verify"], default=None,
                    help="time causal multi-query attention on one of its workloads instead")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4],
                    help="workload (default 2: the GQA prefix-sharing batch)")
    ap.add_argument("--block-size", type=int, default=None, help="config 3 only: 512 or 16")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="split-K partition in tokens (0 = library policy, -1 = never)")
    ap.add_argument("--cpu-budget", type=float, default=25.0,
                    help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="the workload over an FP8 (E4M3) pool: quantising write and FP8 decode")
    ap.add_argument("--kv-int8", action="store_true",
                    help="the workload over an INT8 pool: quantising write and INT8 decode")
    ap.add_argument("--no-host-plan", action="store_true",
                    help="--serving: plain decode with the device sort instead of the "
                         "engine's host-planned prefix groups and dispatch list")
    ap.add_argument("--two-launch-edits", action="store_true",
                    help="the step's cache edits as copy_blocks then kv_cache_write (or "
                         "kv_cache_write_fp8 / _int8) instead of one kv_cache_append launch")
    ap.add_argument("--device-sort", action="store_true",
                    help="sort the work on the device in every call instead of passing the "
                         "dispatch list planned on the host (paged_attention_decode_plan, "
                         "paged_attention_multi_query_plan for --multi-query)")
    ap.add_argument("--verify-tokens", type=int, default=5,
                    help="--multi-query spec-verify: tokens to verify per sequence")
    ap.add_argument("--no-prefix", action="store_true",
                    help="plain paged_attention_decode (or, with --multi-query spec-verify, "
                         "paged_attention_multi_query) even where sequences share prefixes "
                         "(default: the _prefix call with the groups pa_prefix_groups finds "
                         "in the host tables)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()

    if args.serving:
        args.steps = 300 if args.steps is None else args.steps
        args.warmup = 200 if args.warmup is None else args.warmup
    else:
        args.steps = 50 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
    workload = f"cfg{args.config}" + (f"-B{args.block_size or 512}" if args.config == 3 else "")
    if args.kv_fp8 or args.kv_int8:
        if args.kv_fp8 and args.kv_int8:
            print("one of --kv-fp8 / --kv-int8", file=sys.stderr)
            return 2
        workload += "-fp8" if args.kv_fp8 else "-int8"
        args.no_cpu_baseline = True
    if args.no_prefix:
        workload += "-noprefix"
    if args.serving:
        workload = "serving"
    if args.multi_query:
        workload = args.multi_query
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters, workload), indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the paged-decode "
              "library has no cross-GPU exchange (each GPU would run its own share of the "
              "sequences and KV heads)", file=sys.stderr)
        return 2
    rank = int(os.environ.get("RANK", "0"))

    import numpy as np
    import torch

    import paged_kv_cache_386_amd as pa
    from workloads import make_case

    if torch.cuda.device_count() == 0:  # counts devices without initialising them
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.serving:
        return serving_bench(args)
    if args.multi_query:
        return multi_query_bench(args)

    t_gen = time.perf_counter()
    case = make_case(args.config, poison=False, block_size=args.block_size)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] workload {case.name}: {case.description}; generated in {t_gen:.1f}s",
          file=sys.stderr, flush=True)

    # the oracle baseline runs first: its worker pool is forked from this
    # process, which must not have touched the GPU yet
    cb = None
    if not args.no_cpu_baseline and rank == 0:
        t_cb = time.perf_counter()
        cb = cpu_baseline(case, args.cpu_budget)
        print(f"[bench] oracle baseline done in {time.perf_counter() - t_cb:.1f}s",
              file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)

    c8 = None
    if args.kv_fp8:
        from workloads import make_fp8_case
        c8 = make_fp8_case(case, args.config)
        case.kv_elem_bytes = 1
    elif args.kv_int8:
        from workloads import make_int8_case
        c8 = make_int8_case(case, args.config)
        case.kv_elem_bytes = 1
    q = to_dev(case.q, dev)
    kc = to_dev(case.k_cache if c8 is None else c8.k8, dev)
    vc = to_dev(case.v_cache if c8 is None else c8.v8, dev)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty(case.q.shape, dtype=torch.float32, device=dev)
    has_step = case.has_step
    if has_step:
        pairs = torch.from_numpy(case.copy_pairs).to(dev)
        slots = torch.from_numpy(case.slot_mapping).to(dev)
        k_new = to_dev(case.k_new, dev)
        v_new = to_dev(case.v_new, dev)
    max_ctx = case.max_context_len
    S, Hq, Hkv, D = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim
    P = pa.num_partitions(S, Hkv, max_ctx, args.partition_size)
    ps = pa.partition_tokens(S, Hkv, max_ctx, args.partition_size) if P > 1 else 0
    # shared prefixes: the host finds them in the tables it built (the block
    # manager's knowledge; not part of the timed step)
    groups_np = np.zeros((0, 2), np.int32)
    shared_np = np.zeros(S, np.int32)
    if not args.no_prefix:
        groups_np, shared_np = pa.prefix_groups(case.block_tables, case.context_lens,
                                                case.block_size, Hq, Hkv, 16)
    kv_code = pa.PA_BF16 if c8 is None else (pa.PA_FP8_E4M3 if args.kv_fp8 else pa.PA_INT8)
    if case.dtype == "f32":
        kv_code = pa.PA_F32
    # the dispatch list, planned on the host from the lengths it knows (as
    # the tables and groups are); --device-sort sorts in every call instead
    dispatch_np = None
    if not args.device_sort:
        dispatch_np = pa.decode_plan(case.context_lens, groups_np, shared_np, num_q_heads=Hq,
                                     num_kv_heads=Hkv, head_dim=D, block_size=case.block_size,
                                     max_blocks_per_seq=case.max_blocks_per_seq,
                                     max_context_len=max_ctx, kv_dtype=kv_code,
                                     partition_size=args.partition_size)
    use_prefix = len(groups_np) > 0 or dispatch_np is not None
    dispatch_d = None if dispatch_np is None else torch.from_numpy(dispatch_np).to(dev)
    if use_prefix:
        groups_d = torch.from_numpy(groups_np.reshape(-1, 2)).to(dev)
        shared_d = torch.from_numpy(shared_np).to(dev)
        ws_bytes = pa.prefix_workspace_size(S, Hq, Hkv, D, max_ctx, args.partition_size,
                                            len(groups_np), kv_code)
    else:
        ws_bytes = pa.workspace_size(S, Hq, Hkv, D, max_ctx, args.partition_size)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def edits():
        if not args.two_launch_edits:
            pa.kv_cache_append(pairs, k_new, v_new, slots, kc, vc,
                               k_scale=1.0 if c8 is None else float(c8.k_scale),
                               v_scale=1.0 if c8 is None else float(c8.v_scale), stream=stream)
            return
        pa.copy_blocks(pairs, kc, vc, stream=stream)
        if c8 is None:
            pa.kv_cache_write(k_new, v_new, slots, kc, vc, stream=stream)
        else:
            write = pa.kv_cache_write_fp8 if args.kv_fp8 else pa.kv_cache_write_int8
            write(k_new, v_new, slots, kc, vc, float(c8.k_scale), float(c8.v_scale),
                  stream=stream)

    def decode():
        if use_prefix:
            pa.paged_attention_decode_prefix(
                q, kc, vc, tables, lens, groups_d, shared_d, float(case.scale), out,
                max_context_len=max_ctx, k_scale=1.0 if c8 is None else float(c8.k_scale),
                v_scale=1.0 if c8 is None else float(c8.v_scale),
                partition_size=args.partition_size, workspace=ws, dispatch=dispatch_d,
                stream=stream)
        elif c8 is None:
            pa.paged_attention_decode(q, kc, vc, tables, lens, float(case.scale), out,
                                      max_context_len=max_ctx,
                                      partition_size=args.partition_size, workspace=ws,
                                      stream=stream)
        else:
            dec = pa.paged_attention_decode_fp8 if args.kv_fp8 else pa.paged_attention_decode_int8
            dec(q, kc, vc, tables, lens, float(case.scale), float(c8.k_scale),
                float(c8.v_scale), out, max_context_len=max_ctx,
                partition_size=args.partition_size, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        if has_step:
            edits()
        decode()
    torch.cuda.synchronize()

    # 1. the timed steps: nothing but the step's own launches between the two
    # events (an event recorded between two kernels holds the queue for
    # about 5 us on these GPUs, so per-call events would lengthen the step)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if has_step:
            edits()
        decode()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps
    # 2. the decode call's mean duration: the same number of calls back to
    # back between two events on the launch stream
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(args.steps):
        decode()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_us = d0.elapsed_time(d1) * 1e3 / args.steps
    # 3. the spread of single calls, each between its own pair of events
    # (which adds the events' own time to every sample)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        if has_step:
            edits()
        ev[i][0].record(stream)
        decode()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])

    dec_unique = decode_bytes(case, P, ps, unique=True)
    dec_attended = decode_bytes(case, P, ps, unique=False)
    step_bytes = dec_unique + edit_bytes(case)
    tokens = int(case.context_lens.astype(np.int64).sum())
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # roofline: the unique algorithmic bytes of one decode call (each
    # distinct KV slot once: what HBM must deliver at least) over the call's
    # mean duration; attended bytes (a shared block once per sequence that
    # reads it) give the "effective" rate beside it, and the committed
    # counter traffic the measured bytes
    achieved = dec_unique / (dec_us * 1e-6) / 1e9
    traffic = load_traffic(workload)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype if c8 is None else
                 ("fp8-e4m3 (bf16 q)" if args.kv_fp8 else "int8 (bf16 q)"),
        "data": "synthetic (seeded N(0,1) q/K/V; lengths, prefix groups and forks as described)"
                + ("" if c8 is None else
                   f"; K/V as random {'E4M3' if args.kv_fp8 else 'INT8'} codes, k_scale "
                   f"{float(c8.k_scale)}, v_scale {float(c8.v_scale)}"),
        "config": {
            "workload": f"{workload}: {case.description}",
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": case.block_size, "max_context_len": max_ctx,
            "total_context_tokens": tokens, "unique_kv_slots": unique_slots(case),
            "copy_pairs": int(len(case.copy_pairs)), "new_tokens": int(len(case.slot_mapping)),
            "partition_size": ps if P > 1 else None, "num_partitions": P,
            "prefix_groups": int(len(groups_np)),
            "shared_tokens": int(shared_np.sum()),
            "dispatch": "device sort" if dispatch_np is None else "planned on the host",
            "step": (("copy_blocks + kv_cache_write + " if args.two_launch_edits else
                      "kv_cache_append (copies + new-token writes, one launch) + ")
                     if has_step else "") +
                    ("paged_attention_decode_prefix (" +
                     ("shared prefixes read once per group, " if len(groups_np) else
                      "no shared prefixes found, ") +
                     ("dispatch list planned on the host; " if dispatch_np is not None else
                      "dispatch sorted on the device; ") + "+ merge)" if use_prefix else
                     "paged_attention_decode (+ split-K merge)"),
        },
        "attended_kv_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        # mean decode-call time: `steps` calls back to back between two HIP
        # events on the launch stream
        "decode_us": round(dec_us, 2),
        # spread of single calls, each between its own pair of events (their
        # own time included, a few us per call)
        "decode_us_pct": {k: round(float(np.percentile(dec_ms, q)) * 1e3, 2)
                          for k, q in (("p10", 10), ("p50", 50), ("p90", 90))},
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_attention_decode_prefix (decode kernel with the prefix items, "
                       "merge; one call)" if use_prefix else
                       "paged_attention_decode (dispatch sort, decode kernel, partition merge; "
                       "one call)"),
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "frac_definition": ("unique algorithmic bytes per decode call (each distinct KV "
                                "slot once, plus q, out, used table entries, lengths, split "
                                "partials and the dispatch list) / mean decode-call time "
                                "(calls back to back between two HIP events) / 8 TB/s"),
            "algorithmic_bytes_per_call": dec_unique,
            "attended_bytes_per_call": dec_attended,
            # a shared block counted once per sequence that reads it: above
            # what HBM has to deliver when blocks are shared
            "effective_gbps": round(dec_attended / (dec_us * 1e-6) / 1e9, 1),
            # measured bytes (committed counters on these decode sources)
            # over the same duration, and their ratio to the unique bytes
            "traffic_gbps": None if traffic is None else round(traffic / (dec_us * 1e-6) / 1e9, 1),
            "reread_ratio": None if traffic is None else round(traffic / dec_unique, 3),
        },
        "wall_s_timed": round(wall, 3),
    }
    if cb is not None:
        cpu_value = step_bytes / cb["est_step_seconds"] / 1e9
        ac = cb["all_cores"]
        frac = cb["seqs"] / S
        ac_step = cb["edit_seconds"] + ac["decode_seconds"] / max(frac, 1e-9)
        rec["cpu_baseline"] = {
            "value": round(cpu_value, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle, one thread: the step's edits plus decode of "
                       f"{cb['seqs']}/{S} sequences ({cb['tokens']} context tokens) in "
                       f"{cb['seconds']:.1f}s; value scales the decode time to all {S} "
                       f"sequences and uses the same byte count as `value`"),
            "tokens_per_s": round(cb["tokens_per_s"], 1) if cb["tokens_per_s"] else None,
            "all_cores": {
                "value": round(step_bytes / ac_step / 1e9, 4),
                "unit": "GB/s",
                "cores": ac["cores"],
                "cores_available": ac["cores_available"],
                "cpu": ac["cpu"],
                "sample": (f"the same oracle decode of the same {ac['seqs']} sequences over "
                           f"{ac['cores']} single-threaded worker processes "
                           f"({ac['cores_available']} cores in the affinity set; at most "
                           f"{CPU_WORKER_CAP} worker processes per GPU job on this host) in "
                           f"{ac['decode_seconds']:.2f}s, plus the single-threaded edits"),
                "gpu_speedup": round(ac_step / (ms_step * 1e-3), 1),
            },
            "gpu_speedup": round(cb["est_step_seconds"] / (ms_step * 1e-3), 1),
        }
    if rank == 0:
        print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Benchmark: one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: pa_reshape_and_cache writes this
step's new token of every sequence through slot_mapping, then pa_decode
attends each sequence's query over its paged context (single pass or split
pass + log-sum-exp reduce, as the library plans it).

Workload (default): Llama-3-8B-shaped single-layer decode -- 64 sequences with
lengths uniform in [512, 4096], 32 query / 8 KV heads, head_dim 128,
block_size 16, fp16 KV in a 20,000-block pool filled from a seeded shuffled
free list; 64 new tokens written per step.  Inputs are seeded synthetic data.

Consecutive steps use different layers' pools (--layers copies, 1.3 GB each),
as a model's consecutive attention calls do, so no step finds its KV in the
256 MB Infinity Cache left behind by the previous one.

Prints ONE JSON line.  `value` is achieved algorithmic GB/s of the whole step
(K/V context, q, out, tables, lengths, and the new tokens' write), from wall
time over exactly --steps steps, with no timing event between them.
`roofline` covers the dominant kernel (pa_decode): its average launch
duration is the GPU time between two HIP events on its stream around the same
number of calls, back to back over the same rotated pools, right after the
timed steps.  (A timing event recorded between calls is not free: each record
adds about 4 us of queue time, which per-call event pairs would add to a
100 us call; the per-call distribution is reported separately, from calls
each between its own pair of events.)  `cpu_baseline` times the fp64 CPU
oracle on the host cores over the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode achieved HBM GB/s (% of MI355X peak) + KV tokens/s"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def _code_only(text: str) -> str:
    """C++ source without comments, trailing blanks or empty lines."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash() -> str:
    """Hash of the library's device sources (.hip and .h; the host-only C++
    of the block pool is left out), comments excluded: a stored counter
    measurement stays valid across documentation edits but not across any
    change of kernel code."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "paged_kv_cache_72_amd", "csrc"))):
        if not f.endswith((".hip", ".h")):
            continue
        with open(os.path.join(ROOT, "paged_kv_cache_72_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode() + b"\0")
    return h.hexdigest()[:16]


def unique_kv_tokens(w) -> int:
    """Token rows the batch reads when every physical block is counted once:
    a block listed by several sequences contributes the most slots any of them
    uses."""
    bs = w.block_size
    used = {}
    for s in range(w.num_seqs):
        n = int(w.seq_lens[s])
        w0 = max(0, n - w.window) if w.window else 0       # sliding window: read from w0
        for j in range(w0 // bs, (n + bs - 1) // bs):
            b = int(w.block_tables[s, j])
            lo, hi = max(j * bs, w0), min((j + 1) * bs, n)
            used[b] = max(used.get(b, 0), hi - lo)
    return sum(used.values())


def alg_bytes(w) -> dict:
    """Bytes the method itself must move (no partials, no masked slots).  With
    blocks shared between sequences the K/V term counts each block once (the
    logical figure, every sequence reading its whole context, is kept too)."""
    e = w.kv_elem_bytes
    lens = w.seq_lens.astype(np.int64)
    row = w.num_kv_heads * w.head_dim * e * 2
    seen = np.minimum(lens, w.window) if w.window else lens      # positions each query reads
    kv_logical = int(seen.sum()) * row
    kv = unique_kv_tokens(w) * row if w.has_shared_blocks else kv_logical
    qo = w.num_seqs * w.num_q_heads * w.head_dim * 2 * 2
    tables = int(((lens + w.block_size - 1) // w.block_size).sum()) * 4 + w.num_seqs * 4
    T = int(w.new_idx.size)
    write = T * w.num_kv_heads * w.head_dim * (2 * 2 + 2 * e) + T * 8
    return {"kv": kv, "kv_logical": kv_logical, "decode": kv + qo + tables,
            "decode_logical": kv_logical + qo + tables, "write": write}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Every core this process may run on, but no more than OMP_NUM_THREADS
    when that is set (the share of the host's cores a one-GPU job gets)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def _time_oracle_decode(w, pool, nthreads: int, budget_s: float):
    import oracle as O
    reps, t0 = 0, time.perf_counter()
    while True:
        O.decode(pool, w.q, w.block_tables, w.seq_lens, w.scale, nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return el / reps, reps, el


def cpu_baseline(w, budget_s: float, single_thread_configs=()) -> dict:
    """The fp64 oracle, as it stands, on the host: the full decode of w on
    every allowed core, then (single_thread_configs) one thread on each listed
    workload for about a second each."""
    import oracle as O
    from paged_kv_cache_72_amd import workloads as W
    nthreads = oracle_threads()
    pool = O.pool_for_workload(w, nthreads=nthreads)
    per, reps, el = _time_oracle_decode(w, pool, nthreads, budget_s)
    del pool
    b = alg_bytes(w)
    res = {"value": round(b["decode"] / per / 1e9, 4), "unit": "GB/s", "cores": nthreads,
           "kind": "oracle", "ms_per_step": round(per * 1e3, 2),
           "kv_tokens_per_s": round(float(w.seq_lens.sum()) / per, 1),
           "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
           "sample": f"full decode of the {w.name} step (all {w.num_seqs} sequences, "
                     f"{w.num_q_heads} query heads), repeated {reps}x over {el:.1f} s; "
                     "fp64 C oracle, OpenMP"}
    single = {}
    for name in single_thread_configs:
        ws = W.CONFIGS[name]()
        p1 = O.pool_for_workload(ws, nthreads=nthreads)
        per1, reps1, _ = _time_oracle_decode(ws, p1, 1, 1.0)
        del p1
        single[name] = {"ms_per_step": round(per1 * 1e3, 2),
                        "GB_per_s": round(alg_bytes(ws)["decode"] / per1 / 1e9, 4), "reps": reps1}
    if single:
        res["single_thread"] = single
    return res


def probe_ceiling(nbytes: int) -> dict:
    """The plain-read ceiling at the decode call's size: the wave-contiguous
    read probe (libpa_probe.so) over nbytes, rotating three buffers so no read
    finds its data in the Infinity Cache; 30 launches back to back between one
    pair of events."""
    import torch
    lib_path = os.path.join(ROOT, "paged_kv_cache_72_amd", "libpa_probe.so")
    if not os.path.exists(lib_path):
        return {}
    P = C.CDLL(lib_path)
    P.pa_probe_wave_chunk.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_void_p,
                                      C.c_void_p]
    waves, unroll = 2048, 16
    steps = max(unroll, (nbytes // (waves * 1024)) // unroll * unroll)
    n = waves * steps * 1024
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(3)]
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(5):
        P.pa_probe_wave_chunk(bufs[i % 3].data_ptr(), waves, steps, unroll, sink.data_ptr(), st)
    ms = span_avg_ms(lambda i: P.pa_probe_wave_chunk(bufs[i % 3].data_ptr(), waves, steps,
                                                     unroll, sink.data_ptr(), st),
                     30, torch.cuda.current_stream())
    del bufs
    return {"bytes": n, "avg_ms": round(ms, 5), "GB_per_s": round(n / (ms * 1e-3) / 1e9, 1),
            "probe": f"wave-contiguous 16-byte loads, {waves} waves, {unroll} KiB in flight per "
                     "wave"}


def percentiles_ms(ms) -> dict:
    a = np.asarray(ms, np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5), "p50": round(float(np.median(a)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5)}


def span_avg_ms(fn, reps: int, stream) -> float:
    """Average GPU time per call of fn(0) .. fn(reps - 1) run back to back:
    one pair of HIP events on `stream` around all of them."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def traffic_entry(config: str):
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = d.get(config)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


DECODE_KERNELS = ("decode_flat_group_kernel", "flat_group_merge_kernel", "decode_flat_kernel",
                  "flat_merge_heads_kernel", "decode_group_kernel", "decode_kernel",
                  "lse_reduce_kernel")
PREFILL_KERNELS = ("prefill_f16_kernel", "prefill_kernel")


def ingest_counters(fetch_csv: str, write_csv: str, calib_gib: float, config: str,
                    commands: list) -> dict:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --calib-copy-gib) into HBM bytes per pa_decode (or,
    for a prefill workload, pa_prefill) call.  Each counter is scaled by what it
    reads for the plain device copies of calib_gib GiB that the script runs
    last (torch's copy kernel)."""
    import csv
    from paged_kv_cache_72_amd import workloads as W
    kernels = PREFILL_KERNELS if config in W.PREFILL_CONFIGS else DECODE_KERNELS
    # the kernel that runs once per call of the measured path, and the kernels
    # that follow it within the call; the first listed one present is the
    # path (a grouped workload's run also times the plain pa_decode, whose
    # decode_kernel is then left out)
    paths = (("prefill_f16_kernel", ()), ("prefill_kernel", ()),
             ("decode_flat_group_kernel", ("flat_group_merge_kernel",)),
             ("decode_flat_kernel", ("flat_merge_heads_kernel",)),
             ("decode_group_kernel", ()), ("decode_kernel", ("lse_reduce_kernel",)))

    def load(path):
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows

    def kernel_of(r):
        return next((k for k in kernels if k in r["Kernel_Name"]), None)

    out = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = load(path)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]][-3:]
        kib_copy = sum(float(r["Counter_Value"]) for r in copies) / len(copies)
        factor = calib_gib * (1 << 30) / (kib_copy * 1024)
        present = {kernel_of(r) for r in rows}
        primary, followers = next((p, f) for p, f in paths if p in present)
        dec = [r for r in rows if kernel_of(r) in (primary,) + followers]
        calls = sum(1 for r in dec if kernel_of(r) == primary)
        per_kernel = {}
        for r in dec:
            per_kernel.setdefault(kernel_of(r), []).append(float(r["Counter_Value"]))
        kib_per_call = sum(sum(v) for v in per_kernel.values()) / calls
        out[key] = {"counter": rows[0]["Counter_Name"], "kib_per_call_raw": round(kib_per_call, 2),
                    "copy_kib_raw": round(kib_copy, 2), "factor": round(factor, 5),
                    "bytes_per_call": int(kib_per_call * 1024 * factor),
                    "kib_raw_by_kernel": {k: round(sum(v) / len(v), 2)
                                          for k, v in per_kernel.items()}}
    entry = {"kernel_source_hash": kernel_source_hash(),
             "bytes_per_launch": out["fetch"]["bytes_per_call"] + out["write"]["bytes_per_call"],
             "fetch": out["fetch"], "write": out["write"], "commands": commands}
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        d = {}
    d[config] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return entry


PREFILL_METRIC = "paged-attn prefill achieved TFLOP/s (% of MI355X fp16 MFMA peak)"
MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_flops(w, rows=None) -> int:
    """Algorithmic flops of causal prefill: every (query row, head) scores and
    weights pos + 1 positions, 2 flops per multiply-add in q.k and in p.v."""
    ql = w.q_lens.astype(np.int64)
    ctx = w.seq_lens.astype(np.int64) - ql
    if rows is None:
        keys = int((ql * ctx + ql * (ql + 1) // 2).sum())
        return 4 * w.head_dim * w.num_q_heads * keys
    keys = sum(int(ctx[s]) + i + 1 for s, _, i in rows)
    return 4 * w.head_dim * w.gqa * keys


def prefill_bytes(w) -> int:
    """K/V read once (shared blocks once), q read and out written once."""
    e = w.kv_elem_bytes
    row = w.num_kv_heads * w.head_dim * e * 2
    kv = unique_kv_tokens(w) * row
    return kv + int(w.q.shape[0]) * w.num_q_heads * w.head_dim * 2 * 2


def cpu_baseline_prefill(w, budget_s: float) -> dict:
    """The oracle's prefill on seeded query rows for about budget_s seconds."""
    import oracle as O
    nthreads = oracle_threads()
    pool = O.pool_for_workload(w, nthreads=nthreads)
    rng = np.random.default_rng(0)
    qs = w.q_start
    done_rows, done_flops, el = 0, 0, 0.0
    t0 = time.perf_counter()
    while el < budget_s:
        rows = []
        for _ in range(4 * nthreads):
            s = int(rng.integers(w.num_seqs))
            if w.q_lens[s]:
                rows.append((s, int(rng.integers(w.num_kv_heads)),
                             int(rng.integers(int(w.q_lens[s])))))
        O.prefill(pool, w.q, qs, w.block_tables, w.seq_lens, w.scale, rows=rows,
                  nthreads=nthreads)
        done_rows += len(rows)
        done_flops += prefill_flops(w, rows)
        el = time.perf_counter() - t0
    rate = done_flops / el
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle", "ms_per_step": round(prefill_flops(w) / rate * 1e3, 1),
            "cpu_model": cpu_model(),
            "sample": f"{done_rows} seeded (sequence, KV head, new token) rows of the "
                      f"{w.name} step, each for its {w.gqa} query heads, over {el:.1f} s; "
                      "fp64 C oracle, OpenMP; ms_per_step extrapolates to the whole step"}


def run_prefill(args, w) -> int:
    import torch
    from paged_kv_cache_72_amd import lib as L

    dev = "cuda"
    stream = torch.cuda.current_stream()
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    qs = torch.from_numpy(w.q_start).to(dev)
    out = torch.empty_like(q)
    k_all = torch.from_numpy(w.tok_k).to(dev)
    v_all = torch.from_numpy(w.tok_v).to(dev)
    slots = torch.from_numpy(w.tok_slot).to(dev)
    shared = w.has_shared_blocks
    base = L.KVPool.allocate(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                             w.kv_dtype, w.k_scale, w.v_scale, dev, fill_bits=0,
                             shared_blocks=shared)
    L.pa_reshape_and_cache(base, k_all, v_all, slots)
    idx = torch.from_numpy(w.new_idx).to(dev)
    k_new = k_all.index_select(0, idx).contiguous()
    v_new = v_all.index_select(0, idx).contiguous()
    slot_new = slots.index_select(0, idx).contiguous()
    del k_all, v_all, slots
    pools = [base]
    for _ in range(args.layers - 1):
        pools.append(L.KVPool(base.k.clone(), base.v.clone(), w.block_size, w.num_kv_heads,
                              w.head_dim, w.kv_dtype, w.k_scale, w.v_scale,
                              shared_blocks=shared))
    torch.cuda.synchronize()

    def prefill(p):
        L.pa_prefill(p, out, q, qs, bt, lens, w.max_q_len, w.scale, stream)

    def step(i):
        p = pools[i % len(pools)]
        L.pa_reshape_and_cache(p, k_new, v_new, slot_new, stream)
        prefill(p)

    warmup = warm_up(step, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the same calls over the same rotated pools, back to back between one
    # pair of events
    pf_avg = span_avg_ms(lambda i: prefill(pools[(warmup + i) % len(pools)]), args.steps, stream)
    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    flops = prefill_flops(w)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (pf_avg * 1e-3) / 1e12
    nbytes = prefill_bytes(w)
    res = {
        "metric": PREFILL_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and free-list block ids)",
        "config": {"workload": f"{w.name}: {w.num_seqs} seqs, new tokens "
                               f"{int(w.q_lens.min())}-{int(w.q_lens.max())} "
                               f"(sum {int(w.q_lens.sum())}), context "
                               f"{int(w.seq_lens.min())}-{int(w.seq_lens.max())}, "
                               f"{w.num_q_heads} q / {w.num_kv_heads} kv heads, head_dim "
                               f"{w.head_dim}, block_size {w.block_size}, {w.kv_dtype} KV; "
                               f"step = reshape_and_cache of {w.new_idx.size} tokens + prefill",
                   "global_batch": w.num_seqs, "seq_len": w.max_seq_len, "parallelism": "none",
                   "layers_rotated": args.layers, "shared_blocks": shared},
        "pct_of_peak": round(100 * value / MFMA_F16_PEAK_TFLOPS, 2),
        "prefill_tokens_per_s": round(float(w.q_lens.sum()) / (ms_step * 1e-3), 1),
        "rows_per_workgroup": L.pa_prefill_plan(base, w.num_seqs, w.num_q_heads, w.max_q_len),
        "alg_flops_per_launch": flops,
        "alg_bytes_per_launch": nbytes,
        "hbm_GB_per_s": round(nbytes / (pf_avg * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": "pa_prefill", "achieved": round(achieved, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic_entry(w.name), "avg_launch_ms": round(pf_avg, 5),
                     "alg_flops_per_launch": flops,
                     "kernel_source_hash": kernel_source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def run_block_pool(args) -> int:
    """Host block pool on the pages' prefix-cache scenario, driven the way a
    scheduler drives it: 64 requests are live; every step grows each live
    request by one generated token (one batched call); a request that has
    generated 300 tokens is freed and a new one admitted, whose 2,000-token
    system prompt (125 full blocks of 16) hits the prefix cache while its own
    50 tokens get new blocks, registered once written."""
    from paged_kv_cache_72_amd import lib as L
    bs, live, prompt, own, gen = 16, 64, 2000, 50, 300
    rng = np.random.default_rng(7220)
    sys_prompt = [int(x) for x in rng.integers(0, 128000, size=prompt)]
    pool = L.BlockPool(8192, bs)
    first = sys_prompt + [int(x) for x in rng.integers(0, 128000, size=own)]
    pool.allocate_request(-1, first)
    pool.cache_request(-1, first)
    pool.free_request(-1)
    # token arrays built once (int32, passed to the library in place)
    prompts = [np.asarray(sys_prompt + [int(x) for x in rng.integers(0, 128000, size=own)],
                          np.int32) for _ in range(256)]
    n_req = max(256, args.steps * 4)
    lib = L.load()
    LP, IP = C.POINTER(C.c_int64), C.POINTER(C.c_int32)
    # the live set as arrays the batched call reads in place; slot i starts
    # i * gen / live tokens into its generation so that completions spread
    # evenly over the steps
    rids = np.zeros(live, np.int64)
    lens = np.zeros(live, np.int32)
    made = np.zeros(live, np.int32)
    t0 = time.perf_counter()
    hits, admitted, done, steps = 0, 0, 0, 0

    def admit(i, start):
        nonlocal admitted, hits
        toks = prompts[admitted % len(prompts)]
        hits += pool.allocate_request(admitted, toks)
        pool.cache_request(admitted, toks)
        if start:
            pool.append_slots(admitted, len(toks) + start)
        rids[i], lens[i], made[i] = admitted, len(toks) + start, start
        admitted += 1

    for i in range(live):
        admit(i, i * gen // live)
    rp, lp = rids.ctypes.data_as(LP), lens.ctypes.data_as(IP)
    while done < n_req:
        lens += 1
        made += 1
        st = lib.pa_bp_append_slots_batch(pool._p, rp, lp, live)
        if st:
            raise L.PaError(st, lib.pa_bp_last_error().decode())
        steps += 1
        for i in np.nonzero(made == gen)[0]:
            pool.free_request(int(rids[i]))
            done += 1
            admit(int(i), 0)
    el = time.perf_counter() - t0
    # native hash rate: the chained hashes of whole prompts, one call each,
    # with the token arrays built beforehand
    arrs = [t.ctypes.data_as(IP) for t in prompts[:64]]
    nblk = (prompt + own) // bs
    out = (L.pa_block_hash * nblk)()
    reps = 2000
    t1 = time.perf_counter()
    for i in range(reps):
        lib.pa_hash_blocks(arrs[i % 64], prompt + own, bs, None, 0, out, nblk)
    hash_us = (time.perf_counter() - t1) / (reps * nblk) * 1e6
    res = {"metric": "host block pool: requests per second (prefix-hit admission, one batched "
                     "append per scheduler step for 64 live requests, 300 generated tokens, "
                     "free)",
           "value": round(n_req / el, 1), "unit": "requests/s", "n_gpus": 0,
           "steps": n_req, "warmup": 1, "ms_per_step": round(el / n_req * 1e3, 4),
           "higher_is_better": True, "scaling": "none", "vs_baseline": None, "dtype": "int32",
           "data": "synthetic token ids (seeded)",
           "config": {"workload": "2,000-token shared system prompt + 50 own tokens, block_size "
                                  "16, 8,192-block pool, 64 live requests"},
           "scheduler_steps_per_s": round(steps / el, 1),
           "us_per_scheduler_step": round(el / steps * 1e6, 2),
           "cached_tokens_per_request": hits / admitted,
           "hash_us_per_block": round(hash_us, 3),
           "hash_note": "chained SHA-256 of a whole 2,050-token prompt (128 full blocks of 16) "
                        "in one native call, per block, for the pages' remark that SHA-256 "
                        "costs a few microseconds per block"}
    print(json.dumps(res), flush=True)
    return 0


def warm_up(step, requested) -> int:
    """Run the untimed steps and return how many ran: exactly `requested` if
    given, else at least 20 and as many more as take about 250 ms of wall time
    (a GPU idle during set-up starts the timed steps at low clocks; a 0.5 ms
    prefill step measured 5-18% slower after 5 warm-up steps than after 500)."""
    import torch
    if requested is not None:
        for i in range(requested):
            step(i)
        return requested
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < 20 or time.perf_counter() - t0 < 0.25:
        step(n)
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    return n


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 20, and "
                         "more until about 250 ms of steps have run, so that the GPU's "
                         "clocks have ramped up; the count run is reported)")
    ap.add_argument("--config", default="llama3_8b_b64")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--decode", choices=("auto", "plain", "grouped"), default="auto",
                    help="auto: pa_decode_grouped when blocks are shared between sequences "
                         "(planned on the host once), else pa_decode")
    ap.add_argument("--grouped-schedule", type=int, default=0,
                    help="pa_decode_grouped schedule: 0 library choice, 1 flat, 2 per group")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the plain-read ceiling probe (pct_of_probe)")
    ap.add_argument("--cpu-single-thread", type=int, default=1,
                    help="1: also time the oracle on one thread on the tiny, Llama, Qwen and "
                         "prefix-sharing workloads (about a second each)")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write the HBM traffic of --config's pa_decode call into "
                         "profiles/hbm_traffic.json from two rocprofv3 --pmc runs")
    ap.add_argument("--command", action="append", default=[],
                    help="with --ingest-counters: the profiler commands, recorded verbatim")
    args = ap.parse_args()

    if args.ingest_counters:
        e = ingest_counters(*args.ingest_counters, args.calib_copy_gib or 1.0, args.config,
                            args.command)
        print(json.dumps(e, indent=1))
        return 0

    if args.config == "block_pool":
        return run_block_pool(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path shards by sequence or KV head "
              "with no exchange, so a single-GPU figure is the per-GPU figure. Run with "
              "--gpus 1.", file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_72_amd import lib as L
    from paged_kv_cache_72_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.load()
    if args.config in W.PREFILL_CONFIGS:
        return run_prefill(args, W.PREFILL_CONFIGS[args.config]())
    w = W.CONFIGS[args.config]()
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ---- inputs resident in HBM: per-layer pools holding the context
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty_like(q)
    k_all = torch.from_numpy(w.tok_k).to(dev)
    v_all = torch.from_numpy(w.tok_v).to(dev)
    slots = torch.from_numpy(w.tok_slot).to(dev)
    shared = w.has_shared_blocks      # cacheable K/V reads when blocks have several readers
    base = L.KVPool.allocate(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                             w.kv_dtype, w.k_scale, w.v_scale, dev, fill_bits=0,
                             shared_blocks=shared, k_head_scales=w.k_head_scales,
                             v_head_scales=w.v_head_scales, sliding_window=w.window,
                             block_scales=w.block_scales)
    L.pa_reshape_and_cache(base, k_all, v_all, slots)
    if w.cow_pairs is not None:
        L.pa_copy_blocks(base, torch.from_numpy(w.cow_pairs).to(dev))
    idx = torch.from_numpy(w.new_idx).to(dev)
    k_new = k_all.index_select(0, idx).contiguous()
    v_new = v_all.index_select(0, idx).contiguous()
    slot_new = slots.index_select(0, idx).contiguous()
    del k_all, v_all, slots
    pools = [base]
    for _ in range(args.layers - 1):
        bs_copy = (lambda t: None if t is None else t.clone())
        pools.append(L.KVPool(base.k.clone(), base.v.clone(), w.block_size, w.num_kv_heads,
                              w.head_dim, w.kv_dtype, w.k_scale, w.v_scale,
                              shared_blocks=shared, k_head_scales=base.k_head_scales,
                              v_head_scales=base.v_head_scales, sliding_window=w.window,
                              k_block_scales=bs_copy(base.k_block_scales),
                              v_block_scales=bs_copy(base.v_block_scales)))
    part = L.pa_decode_plan(base, w.num_seqs, w.num_q_heads, w.max_seq_len, args.partition)
    ws = L.alloc_workspace(base, w.num_seqs, w.num_q_heads, w.max_seq_len, args.partition)
    grouped = args.decode == "grouped" or (args.decode == "auto" and shared and not w.window)
    groups, plan_us = None, None
    if grouped:   # the host planner, as a scheduler would run it each step (timed on its own)
        t_p = time.perf_counter()
        for _ in range(20):
            groups = L.pa_decode_group_plan(w.block_tables, w.seq_lens, w.block_size,
                                            w.num_q_heads, w.num_kv_heads)
        plan_us = (time.perf_counter() - t_p) / 20 * 1e6
        gsched = L.pa_decode_grouped_plan(base, w.num_seqs, w.num_q_heads, w.max_seq_len,
                                          groups.num_groups, args.grouped_schedule)
        gws = L.alloc_grouped_workspace(base, w.num_seqs, w.num_q_heads, w.max_seq_len,
                                        groups.num_groups, gsched)
    torch.cuda.synchronize()

    def decode(p):
        if grouped:
            L.pa_decode_grouped(p, out, q, bt, lens, w.max_seq_len, w.scale, groups,
                                schedule=gsched, workspace=gws, stream=stream)
        else:
            L.pa_decode(p, out, q, bt, lens, w.max_seq_len, w.scale, args.partition, ws, stream)

    def step(i, ev=None):
        p = pools[i % len(pools)]
        L.pa_reshape_and_cache(p, k_new, v_new, slot_new, stream)
        if ev is not None:
            ev[0].record(stream)
        decode(p)
        if ev is not None:
            ev[1].record(stream)

    warmup = warm_up(step, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # the call's average duration: the same calls over the same rotated pools,
    # back to back between one pair of events
    dec_avg = span_avg_ms(lambda i: decode(pools[(warmup + i) % len(pools)]), args.steps, stream)
    # the per-call distribution: as many steps again, each call between its
    # own pair of events (whose records the figures include)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        step(warmup + args.steps + i, events[i])
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in events]

    # ---- the two write paths, timed on their own (after the decode timing)
    def back_to_back_ms(fn, reps=50):
        for i in range(5):
            fn(i)
        return span_avg_ms(fn, reps, stream)

    # warm: back-to-back calls on one pool (K/V partly served from the
    # Infinity Cache), labelled as such
    warm_ms = back_to_back_ms(lambda i: decode(pools[0]))
    plain_ms = None
    if grouped:   # the same step through pa_decode, for comparison
        plain_ms = back_to_back_ms(lambda i: L.pa_decode(pools[i % len(pools)], out, q, bt, lens,
                                                         w.max_seq_len, w.scale, args.partition,
                                                         ws, stream), reps=100)
    rc_ms = back_to_back_ms(lambda i: L.pa_reshape_and_cache(pools[i % len(pools)], k_new, v_new,
                                                              slot_new, stream))
    pairs = w.cow_pairs
    if pairs is None:   # copy 256 context blocks into blocks no table lists
        nb_used = (w.seq_lens.astype(np.int64) + w.block_size - 1) // w.block_size
        used = np.unique(np.concatenate([w.block_tables[s_, :nb_used[s_]]
                                         for s_ in range(w.num_seqs)]))
        free = np.setdiff1d(np.arange(w.num_blocks), used)
        n_p = int(min(256, used.size, free.size))
        pairs = np.stack([used[:n_p], free[:n_p]], axis=1).astype(np.int64)
    pairs_d = torch.from_numpy(np.ascontiguousarray(pairs)).to(dev)
    cb_ms = back_to_back_ms(lambda i: L.pa_copy_blocks(pools[i % len(pools)], pairs_d, stream))
    blk_bytes = w.block_size * w.num_kv_heads * w.head_dim * w.kv_elem_bytes
    cb_bytes = int(pairs.shape[0]) * 2 * blk_bytes * 2

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    b = alg_bytes(w)
    step_bytes = b["decode"] + b["write"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = b["decode"] / (dec_avg * 1e-3) / 1e9
    del pools
    probe = probe_ceiling(b["decode"]) if not args.no_probe else {}
    pct = percentiles_ms(dec_ms)
    call = {"back_to_back_ms": round(dec_avg, 5),
            "events_ms": pct,
            "events_note": "each call between its own pair of events, whose records add "
                           "their queue time",
            "GB_per_s_at_p50": round(b["decode"] / (pct["p50"] * 1e-3) / 1e9, 1),
            "pct_of_peak_at_p50": round(100 * b["decode"] / (pct["p50"] * 1e-3) / 1e9
                                        / HBM_PEAK_GBS, 2),
            "warm_back_to_back_ms": round(warm_ms, 5),
            "warm_GB_per_s": round(b["decode"] / (warm_ms * 1e-3) / 1e9, 1)}
    if grouped:
        call["entry_point"] = "pa_decode_grouped"
        call["grouped_schedule"] = {1: "flat ranges over the groups", 2: "workgroup per group"}[gsched]
        call["groups"] = groups.num_groups
        call["host_group_plan_us"] = round(plan_us, 1)
        call["pa_decode_ms_same_step"] = round(plain_ms, 5)
    if probe:
        call["probe_ceiling"] = probe
        call["pct_of_probe"] = round(100 * achieved / probe["GB_per_s"], 2)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and free-list block ids)",
        "config": {"workload": f"{w.name}: {w.num_seqs} seqs, seq_lens "
                               f"{int(w.seq_lens.min())}-{int(w.seq_lens.max())} "
                               f"(sum {int(w.seq_lens.sum())}), {w.num_q_heads} q / "
                               f"{w.num_kv_heads} kv heads, head_dim {w.head_dim}, block_size "
                               f"{w.block_size}, {w.kv_dtype} KV, {w.num_blocks}-block pool; "
                               f"step = reshape_and_cache of {w.new_idx.size} tokens + decode",
                   "global_batch": w.num_seqs, "seq_len": w.max_seq_len, "parallelism": "none",
                   "layers_rotated": args.layers,
                   "partition_tokens": "grouped" if grouped else part,
                   "shared_blocks": shared},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(float((np.minimum(w.seq_lens, w.window) if w.window
                                        else w.seq_lens).sum()) / (ms_step * 1e-3), 1),
        "decode_tokens_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "alg_bytes_per_step": step_bytes,
        "reshape_and_cache": {"tokens": int(w.new_idx.size), "avg_ms": round(rc_ms, 5),
                              "alg_bytes": b["write"],
                              "GB_per_s": round(b["write"] / (rc_ms * 1e-3) / 1e9, 1)},
        "copy_blocks": {"pairs": int(pairs.shape[0]), "avg_ms": round(cb_ms, 5),
                        "alg_bytes": cb_bytes,
                        "GB_per_s": round(cb_bytes / (cb_ms * 1e-3) / 1e9, 1)},
        "logical_decode_bytes": b["decode_logical"],
        "pa_decode_call": call,
        "roofline": {"bound": "hbm", "kernel": "pa_decode_grouped" if grouped else "pa_decode",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_entry(w.name), "avg_launch_ms": round(dec_avg, 5),
                     "alg_bytes_per_launch": b["decode"],
                     "kernel_source_hash": kernel_source_hash()},
    }
    if not args.no_cpu_baseline:
        singles = ("tiny", "llama3_8b_b64", "qwen25_7b_8k", "prefix_share_bs16") \
            if args.cpu_single_thread else ()
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, singles)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache hot path on one MI355X.

One step = the GPU calls of a decode step over one synthetic batch with every
input already resident in HBM: copy_blocks (copy-on-write pairs),
reshape_and_cache (the new tokens) and paged_attn_decode_plan (the batch's work
list), issued as one decode_step_prologue launch (decode_step_prologue_fp8
over an fp8 cache), then paged_attn_decode_run (the attention; segments of
long rows merged by the
log-sum-exp reduce).  The roofline figure is for the attention run
alone, timed with HIP events on the stream it runs on.
Default workload: the LLaMA-13B-shaped batch (128 sequences, 40 MHA heads,
head 128, block 16, fp16, lognormal contexts with median 600 capped at 2048,
13 groups of 3 parallel samples sharing prompt blocks).

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-seconds S]
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(wl, step):
    """Algorithmic bytes of one step.  K/V: every unique live (block, slot) once,
    2 * Hkv * 128 * cb bytes each, cb = 2 (fp16/bf16 cache) or 1 (fp8 cache)
    (parallel samples that share a prompt block count it once); plus q and out
    (2 bytes per element), one 4-byte block-table entry per logical block and
    one context length per sequence; plus the copy-on-write pages (read +
    write) and the new tokens' rows (2-byte rows read, cache elements written)
    and slots."""
    import numpy as np

    eb = 2  # q, out and the new rows
    cb = 1 if wl.kv_dtype == "fp8e4m3" else 2  # one cache element
    hkv, hq, D = wl.num_kv_heads, wl.num_heads, 128
    S = wl.num_seqs
    lens = wl.context_lens.astype(np.int64)
    per_token = 2 * hkv * D * cb  # K and V rows of one token, all KV heads
    tables = step.block_tables_host
    live = set()
    for s in range(S):
        L = int(lens[s])
        for j in range(-(-L // 16)):
            b = int(tables[s, j])
            for t in range(min(16, L - 16 * j)):
                live.add(b * 16 + t)
    kv_seq = int(lens.sum()) * per_token
    kv_unique = len(live) * per_token
    nblk = int(sum(-(-int(L) // 16) for L in lens))
    qo = 2 * S * hq * D * eb
    meta = nblk * 4 + S * 4
    decode = kv_unique + qo + meta
    n_pairs = int(step.block_pairs_host.shape[0])
    copy = n_pairs * 2 * hkv * 2048 * cb * 2  # K and V pages of every head, read + write
    T = int(step.slot_mapping_host.shape[0])
    write = T * hkv * D * 2 * (eb + cb) + T * 4  # K and V rows read, cache elements written, slots read
    return dict(kv_per_sequence=kv_seq, kv_unique=kv_unique, decode=decode, copy=copy, write=write,
                step=decode + copy + write, q_out=qo, meta=meta)


DECODE_SOURCES = ("paged_kv_cache_345_amd/csrc/decode.hip", "paged_kv_cache_345_amd/csrc/pkv_device.h",
                  "paged_kv_cache_345_amd/csrc/pkv_launch.h", "paged_kv_cache_345_amd/csrc/api.hip",
                  "paged_kv_cache_345_amd/csrc/plan.hip", "paged_kv_cache_345_amd/csrc/plan_body.h",
                  "paged_kv_cache_345_amd/csrc/decode_common.h")


PREFILL_SOURCES = ("paged_kv_cache_345_amd/csrc/prefill.hip", "paged_kv_cache_345_amd/csrc/decode_common.h",
                   "paged_kv_cache_345_amd/csrc/pkv_device.h", "paged_kv_cache_345_amd/csrc/pkv_launch.h",
                   "paged_kv_cache_345_amd/csrc/api.hip")


def measured_traffic(stem: str, sources=DECODE_SOURCES):
    """HBM bytes per call from the committed rocprofv3 counter summary
    profiles/<stem>_hbm_traffic.md (FETCH_SIZE + WRITE_SIZE, calibrated against
    a plain copy), or None when there is no summary for this workload or the
    kernel sources changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{stem}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_call", "sources_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("sources_sha256") != h.hexdigest() or "traffic_bytes_per_call" not in fields:
        return None
    return int(fields["traffic_bytes_per_call"])


def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (the machine type if absent)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


# --- cpu baseline: the oracle, in a child process that never touches the GPU ---

_CB = {}  # the child's oracle state, inherited by its forked workers


def _cb_eval(s):
    """One sequence through the oracle's paged decode (a worker task):
    (sequence, per-sequence KV bytes, max-abs error against the GPU output or
    -1, CPU seconds)."""
    import numpy as np

    import oracle

    wl, ref, got = _CB["wl"], _CB["ref"], _CB["got"]
    c0 = time.process_time()
    if wl.kv_dtype == "fp8e4m3":
        o = oracle.fp8.paged_decode_fp8_ref(wl.q, ref.k_cache, ref.v_cache, ref.block_tables, ref.context_lens,
                                            wl.scale, wl.num_kv_heads, wl.dtype, wl.k_scale, wl.v_scale, seqs=[s])
    else:
        o = oracle.paged_decode_ref(wl.q, ref.k_cache, ref.v_cache, ref.block_tables, ref.context_lens,
                                    wl.scale, wl.num_kv_heads, wl.dtype, seqs=[s])
    err = -1.0 if got is None else float(np.abs(got[s] - o[0]).max())
    per_token = 2 * wl.num_kv_heads * 128 * (1 if wl.kv_dtype == "fp8e4m3" else 2)
    return s, int(wl.context_lens[s]) * per_token, err, time.process_time() - c0


def cpu_baseline_child(workload: str, seconds: float, decode_bytes: int, got_path: str) -> dict:
    """The fp64 oracle's paged decode on the host cores, run in a process that
    has not initialised the GPU, so its worker processes can be forked.  Setup
    and data generation are untimed.  A third of the budget runs it on one
    core (whole sequences, cycling through the batch); the rest runs the same
    per-sequence calls on a pool of one worker process per host CPU (BLAS held
    to one thread per worker), in three equal windows whose median rate is
    reported.  Rates count the step's algorithmic decode bytes (every unique
    live slot once, as for the GPU figure) per pass over the batch; the
    per-sequence count is reported beside it.  Every row the baseline
    evaluates is also compared with the GPU's timed output: max_abs_err."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    wl = synth.make_workload(workload)
    log("cpu baseline: building the oracle's cache (untimed)")
    _CB["wl"] = wl
    _CB["ref"] = oracle.run_decode_step(wl, compute_out=False)
    _CB["got"] = np.load(got_path) if got_path else None
    S = wl.num_seqs
    worst = [0.0, -1]
    seen = set()

    def note(r):
        s, _b, e, _c = r
        seen.add(s)
        if e > worst[0]:
            worst[0], worst[1] = e, s

    threadpool_limits(limits=1, user_api="blas")  # also inherited by the forked workers
    budget1 = seconds / 3
    n1, b1, wall1 = 0, 0, 0.0
    while wall1 < budget1:
        t0 = time.perf_counter()
        r = _cb_eval(n1 % S)
        wall1 += time.perf_counter() - t0
        note(r)
        b1 += r[1]
        n1 += 1
    workers = len(os.sched_getaffinity(0))
    window = (seconds - budget1) / 3
    rates, nxt, evals, cpu = [], n1, 0, 0.0
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(_cb_eval, range(min(S, workers)))  # start-up of the workers, untimed
        t_all = time.perf_counter()
        for _ in range(3):
            # keep two tasks per worker in flight until the window ends, then drain
            n0, b0, t0 = 0, 0, time.perf_counter()
            pending = []
            while pending or time.perf_counter() - t0 < window:
                while len(pending) < 2 * workers and time.perf_counter() - t0 < window:
                    pending.append(pool.apply_async(_cb_eval, ((nxt % S),)))
                    nxt += 1
                r = pending.pop(0).get()
                note(r)
                b0 += r[1]
                cpu += r[3]
                n0 += 1
            rates.append((n0, b0, time.perf_counter() - t0))
            evals += n0
    wall = time.perf_counter() - t_all
    med = sorted(rates, key=lambda r: r[0] / r[2])[1]
    gbs = lambda n, t: n / S * decode_bytes / t / 1e9  # noqa: E731
    return {
        "value": round(gbs(med[0], med[2]), 4),
        "unit": "GB/s",
        "cores": max(1, int(round(cpu / wall))),
        "kind": "oracle",
        "sample": (f"fp64 numpy paged decode (the oracle's paged decode reference) on whole sequences of the "
                   f"batch, all {wl.num_heads} heads: {evals} sequence evaluations = {evals / S:.2f} passes over the "
                   f"{S}-sequence batch on {workers} worker processes in 3 windows of {window:.1f} s "
                   f"({wall:.1f} s wall, {cpu:.1f} s CPU in the workers; cores = CPU / wall time); value = the "
                   f"median window's passes x the step's algorithmic decode bytes (unique live slots, as for the "
                   f"GPU) / wall time"),
        "per_sequence_bytes_value": round(med[1] / med[2] / 1e9, 4),
        "window_rates_gbs": [round(gbs(r[0], r[2]), 4) for r in rates],
        "single_thread": {"value": round(gbs(n1, wall1), 4), "unit": "GB/s",
                          "per_sequence_bytes_value": round(b1 / wall1 / 1e9, 4),
                          "sample": f"{n1} sequence evaluations on one core, {wall1:.1f} s"},
        "workers": workers,
        "host_cpus": workers,
        "host_cpu_model": host_cpu_model(),
        "max_abs_err": None if _CB["got"] is None else round(worst[0], 7),
        "max_abs_err_sequence": None if _CB["got"] is None else worst[1],
        "max_abs_err_rows": (None if _CB["got"] is None else
                             f"every head of the {len(seen)} distinct sequences the baseline evaluated"),
    }


def cpu_baseline(wl, seconds: float, nb, gpu_out=None):
    """Runs ``cpu_baseline_child`` in a child Python process (this process has
    initialised the GPU, and forking it is not safe); the GPU output goes to
    the child through a temporary .npy file."""
    import subprocess
    import tempfile

    import numpy as np

    with tempfile.TemporaryDirectory() as tmp:
        path = ""
        if gpu_out is not None:
            path = os.path.join(tmp, "gpu_out.npy")
            np.save(path, gpu_out)
        cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", wl.spec.name,
               str(seconds), str(nb["decode"]), path]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed with status {r.returncode}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def copy_probe(mib: int, reps: int = 3):
    """A plain device-to-device copy of known size, for calibrating the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) against a kernel whose traffic is
    exactly known."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {mib} MiB")


def prefill_flops(context_lens, chunk_lens, num_heads: int) -> int:
    """Algorithmic flops of a chunked-prefill call: chunk query j of sequence s
    sits at position p = L_s - C_s + j and sees the p + 1 keys 0..p; each
    (query, visible key, head) costs 2 * 128 flops for its score and 2 * 128
    for its share of P V."""
    visible = sum((2 * int(L) - int(C) + 1) * int(C) // 2 for L, C in zip(context_lens, chunk_lens))  # sum of p + 1
    return visible * 4 * 128 * int(num_heads)


def prefill_bench(args, name: str) -> int:
    """Chunked-prefill leg: one paged_attn_prefill call over a batch whose
    chunks attend causally to their paged prefixes.  Roofline: the matrix
    cores (4 * 128 flops per (query, visible key, head): QK and PV)."""
    import numpy as np
    import torch

    import harness
    import paged_kv_cache_345_amd as pkv
    import synth

    wl = synth.make_prefill(name)
    log(f"workload {name}: {wl.description}")
    pre = harness.build_prefill(wl, partition_tokens=args.partition_tokens or 0)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        pre.run()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for a, b in ev:
        a.record()
        pre.run()
        b.record()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    calls = np.array([a.elapsed_time(b) for a, b in ev])
    call_ms = float(np.median(calls))
    log(f"prefill call median {call_ms * 1e3:.1f} us, min {calls.min() * 1e3:.1f} us, mean {calls.mean() * 1e3:.1f} us")
    L = wl.context_lens.astype(np.int64)
    C = wl.chunk_lens.astype(np.int64)
    flops = prefill_flops(L, C, wl.num_heads)
    kv_bytes = int(L.sum()) * 2 * wl.num_kv_heads * 128 * (1 if wl.kv_dtype == "fp8e4m3" else 2)
    qo_bytes = 2 * int(C.sum()) * wl.num_heads * 128 * 2
    tflops = flops / (call_ms * 1e-3) / 1e12
    peak = 2500.0  # MI355X dense fp16 / bf16 matrix-core TFLOP/s
    result = {
        "metric": "chunked-prefill paged attention TFLOP/s (% of MI355X dense matrix-core peak) at 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype if wl.kv_dtype is None else f"{wl.dtype} ({wl.kv_dtype} cache)", "data": "synthetic",
        "config": {"workload": wl.description, "name": name, "num_seqs": wl.num_seqs, "num_heads": wl.num_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_size": 128, "block_size": 16,
                   "context_tokens": int(L.sum()), "query_tokens": int(C.sum()),
                   "step": "paged_attn_prefill", "parallelism": "single GPU"},
        "flops": flops,
        "bytes": {"kv": kv_bytes, "q_out": qo_bytes},
        "prefill_call_us": round(call_ms * 1e3, 2),
        "timing": {"flushed": False, "prefill_call_us": {"median": round(call_ms * 1e3, 2),
                                                          "min": round(float(calls.min()) * 1e3, 2),
                                                          "mean": round(float(calls.mean()) * 1e3, 2)}},
        "query_tokens_per_s": round(int(C.sum()) / (call_ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "paged_attn_prefill: prefill_kernel", "achieved": round(tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": measured_traffic(name, PREFILL_SOURCES),
                     "hbm_gbs": round((kv_bytes + qo_bytes) / (call_ms * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    print(json.dumps(result), flush=True)
    return 0


def swap_bench(args, name: str) -> int:
    """Block-swap leg: every used block of the batch swapped out to a pinned
    host pool (shuffled host slots), then back in to shuffled device blocks,
    one swap_blocks call each.  Roofline: the host link (PCIe Gen5 x16, 64 GB/s
    per direction); a contiguous device<->pinned copy of the same bytes by the
    DMA engines is reported beside it."""
    import numpy as np
    import torch

    import harness
    import paged_kv_cache_345_amd as pkv
    import synth

    wl = synth.make_workload(name[len("swap_"):])
    log(f"workload {name}: block swap of every used block of {wl.spec.name}")
    step = harness.build_step(wl)
    torch.cuda.synchronize()
    tables = step.block_tables_host
    used = np.unique(tables[tables >= 0]).astype(np.int32)
    n = len(used)
    rng = np.random.default_rng(0)
    host_ids = rng.permutation(n).astype(np.int32)
    dev_ids = rng.permutation(wl.pool_blocks)[:n].astype(np.int32)
    shape = (n,) + tuple(step.k_cache.shape[1:])
    hk = torch.empty(shape, dtype=step.k_cache.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=step.k_cache.dtype, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([used, host_ids], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([host_ids, dev_ids], 1)).cuda()
    k2, v2 = torch.empty_like(step.k_cache), torch.empty_like(step.v_cache)
    nbytes = 2 * n * int(np.prod(shape[1:])) * step.k_cache.element_size()
    flat_dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    flat_host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    K = max(1, args.steps // 10)
    t_out = timed(lambda: pkv.swap_blocks(hk, hv, step.k_cache, step.v_cache, out_pairs), K)
    t_in = timed(lambda: pkv.swap_blocks(k2, v2, hk, hv, in_pairs), K)
    t_d2h = timed(lambda: flat_host.copy_(flat_dev, non_blocking=True), K)
    t_h2d = timed(lambda: flat_dev.copy_(flat_host, non_blocking=True), K)
    gbs = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    log(f"{n} blocks, {nbytes / 1e9:.3f} GB: swap out {t_out:.3f} ms ({gbs(t_out)} GB/s), in {t_in:.3f} ms "
        f"({gbs(t_in)} GB/s); contiguous DMA copy d2h {gbs(t_d2h)} GB/s, h2d {gbs(t_h2d)} GB/s")
    peak = 64.0
    result = {
        "metric": "paged KV block swap GB/s (device <-> pinned host) at 1 GPU",
        "value": gbs((t_out + t_in) / 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": 2,
        "ms_per_step": round(t_out + t_in, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.kv_dtype, "data": "synthetic",
        "config": {"workload": f"block swap of the {n} used blocks of: {wl.spec.description}", "name": name,
                   "blocks": n, "bytes_per_direction": nbytes, "step": "swap_blocks out + swap_blocks in",
                   "parallelism": "single GPU"},
        "swap_out_gbs": gbs(t_out), "swap_in_gbs": gbs(t_in),
        "dma_copy_gbs": {"d2h": gbs(t_d2h), "h2d": gbs(t_h2d)},
        "roofline": {"bound": "host-link", "kernel": "swap_blocks_kernel", "achieved": gbs((t_out + t_in) / 2),
                     "peak": peak, "unit": "GB/s", "frac": round(gbs((t_out + t_in) / 2) / peak, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def prefix_bench(args, name: str) -> int:
    """Prefix-cache leg: admission of a batch of new prompts that share a
    system prompt already in the cache.  With prefix caching the block manager
    (add_cached) hands back the shared blocks, only the own tokens are written
    (reshape_and_cache) and only they are evaluated (paged_attn_prefill,
    attending to the cached prefix); without it every prompt token is written
    and evaluated.  Both GPU paths are timed with HIP events, and the host
    manager's calls with the wall clock.  Roofline: the prefill kernel of the
    cached path on the matrix cores (4 * 128 flops per (query, visible key,
    head))."""
    import numpy as np
    import torch

    import harness
    import paged_kv_cache_345_amd as pkv
    import synth

    wl, desc = synth.make_prefix(name)
    log(f"workload {name}: {desc}")
    dev = "cuda"
    reqs = list(range(wl.phase1, wl.num_requests))
    prompts = {r: wl.prompt(r) for r in range(wl.num_requests)}

    def admit(cached: bool):
        bm = pkv.BlockManager(wl.pool_blocks, 16, wl.free_order)
        for r in range(wl.phase1):  # the earlier requests that registered the system prompt
            bm.add_cached(r, prompts[r][0]) if cached else bm.add(r, prompts[r][0].shape[0])
        t0 = time.perf_counter()
        res = {r: (bm.add_cached(r, prompts[r][0]) if cached else (bm.add(r, prompts[r][0].shape[0]), 0))
               for r in reqs}
        return bm, res, time.perf_counter() - t0

    host = {}
    for cached in (True, False):
        times = [admit(cached)[2] for _ in range(5)]
        host[cached] = min(times) / len(reqs) * 1e6
    log(f"host admission: add_cached {host[True]:.1f} us/request, add {host[False]:.1f} us/request")

    def build(cached: bool):
        bm, res, _ = admit(cached)
        k_cache, v_cache = pkv.allocate_cache(wl.pool_blocks, wl.num_kv_heads, harness.torch_dtype(wl.dtype), dev)
        for r in range(wl.phase1):  # earlier requests' rows: written once, outside the timed step
            bm_slots = bm.block_table([r], bm.num_seq_blocks(r))[0]
            ids, k, v = prompts[r]
            slots = np.array([bm_slots[t // 16] * 16 + t % 16 for t in range(ids.shape[0])], dtype=np.int32)
            pkv.reshape_and_cache(harness.to_device(k, wl.dtype, dev), harness.to_device(v, wl.dtype, dev),
                                  k_cache, v_cache, torch.from_numpy(slots).to(dev))
        slots, ks, vs, qs_rows, ctx, first = [], [], [], [], [], []
        for r in reqs:
            sl, c = res[r]
            ids, k, v = prompts[r]
            L = ids.shape[0]
            fp = min(c, L - 1)
            slots.append(np.asarray(sl[c:], dtype=np.int32))
            ks.append(k[c:])
            vs.append(v[c:])
            qs_rows.append(wl.q_rows(r)[fp:L])
            ctx.append(L)
            first.append(fp)
        ctx = np.array(ctx, dtype=np.int64)
        chunks = ctx - np.array(first, dtype=np.int64)
        qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        mb = max(bm.num_seq_blocks(r) for r in reqs)
        d = dict(k=harness.to_device(np.concatenate(ks), wl.dtype, dev),
                 v=harness.to_device(np.concatenate(vs), wl.dtype, dev),
                 slots=torch.from_numpy(np.concatenate(slots)).to(dev),
                 q=harness.to_device(np.concatenate(qs_rows), wl.dtype, dev),
                 tables=torch.from_numpy(bm.block_table(reqs, mb)).to(dev),
                 ctx=torch.from_numpy(ctx.astype(np.int32)).to(dev), qs=torch.from_numpy(qs).to(dev),
                 max_q=int(chunks.max()), k_cache=k_cache, v_cache=v_cache, chunks=chunks, ctx_np=ctx,
                 written=int(sum(x.shape[0] for x in slots)), hit=int(sum(res[r][1] for r in reqs)))
        d["out"] = torch.empty_like(d["q"])
        desc_ = pkv.cache_desc(wl.pool_blocks, wl.num_kv_heads, k_cache.dtype)
        ws = pkv.prefill_workspace_size(len(reqs), wl.num_heads, mb, int(qs[-1]), d["max_q"], desc_)
        d["ws"] = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
        return d

    def step_fns(d):
        w = lambda: pkv.reshape_and_cache(d["k"], d["v"], d["k_cache"], d["v_cache"], d["slots"])  # noqa: E731
        a = lambda: pkv.paged_attn_prefill(d["out"], d["q"], d["k_cache"], d["v_cache"], d["tables"],  # noqa: E731
                                           d["ctx"], d["qs"], wl.scale, wl.num_kv_heads, max_query_len=d["max_q"],
                                           workspace=d["ws"])
        return w, a

    def timed(d):
        w, a = step_fns(d)
        for _ in range(max(1, args.warmup)):
            w()
            a()
        torch.cuda.synchronize()
        K = args.steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        for e0, e1, e2 in ev:
            e0.record()
            w()
            e1.record()
            a()
            e2.record()
        torch.cuda.synchronize()
        wr = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
        at = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))
        return wr, at

    res = {}
    for cached in (True, False):
        d = build(cached)
        torch.cuda.synchronize()
        wr, at = timed(d)
        res[cached] = (d, wr, at)
        log(f"{'cached' if cached else 'plain '}: {d['written']} rows written ({d['hit']} cached), "
            f"write {wr * 1e3:.1f} us, prefill {at * 1e3:.1f} us")
    d, wr, at = res[True]
    _, pwr, pat = res[False]
    prompt_tokens = int(d["ctx_np"].sum())
    C, L = d["chunks"], d["ctx_np"]
    visible = int(sum(int(((L[i] - C[i] + 1) + L[i]) * C[i] // 2) for i in range(len(C))))
    flops = visible * 4 * 128 * wl.num_heads
    tflops = flops / (at * 1e-3) / 1e12
    peak = 2500.0
    step_ms = wr + at
    result = {
        "metric": "prefix-cached prompt admission: prompt tokens/s (write + chunked prefill) at 1 GPU",
        "value": round(prompt_tokens / (step_ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": desc, "name": name, "requests": len(reqs), "num_heads": wl.num_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_size": 128, "block_size": 16,
                   "prompt_tokens": prompt_tokens, "cached_tokens": d["hit"], "written_tokens": d["written"],
                   "step": "reshape_and_cache (uncached rows) + paged_attn_prefill (uncached queries)",
                   "parallelism": "single GPU"},
        "without_prefix_cache": {"tokens_per_s": round(prompt_tokens / ((pwr + pat) * 1e-3), 1),
                                 "write_us": round(pwr * 1e3, 2), "prefill_us": round(pat * 1e3, 2)},
        "speedup": round((pwr + pat) / step_ms, 3),
        "write_us": round(wr * 1e3, 2), "prefill_us": round(at * 1e3, 2),
        "host_us_per_request": {"add_cached": round(host[True], 2), "add": round(host[False], 2)},
        "roofline": {"bound": "mfma", "kernel": "paged_attn_prefill: prefill_kernel", "achieved": round(tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-flush", dest="flush", action="store_false",
                    help="decode workloads: run the timed steps back to back, without the cache flush")
    ap.add_argument("--separate-prologue", action="store_true",
                    help="decode workloads: issue copy_blocks, the write and the plan as three calls instead of "
                         "one decode_step_prologue launch")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: also time the step captured in a HIP graph and replayed")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the bench, run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--cpu-baseline-child", nargs=4, metavar=("WORKLOAD", "SECONDS", "DECODE_BYTES", "GPU_OUT"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_baseline_child:  # the cpu_baseline leg's child process: no GPU, no torch
        w, sec, nbytes, path = args.cpu_baseline_child
        print(json.dumps(cpu_baseline_child(w, float(sec), int(nbytes), path)), flush=True)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("this build runs on one GPU only: the decode hot path is measured on a single MI355X "
               "(no multi-GPU sharding is implemented); run with --gpus 1")
        if int(os.environ.get("RANK", "0")) == 0:
            print(msg, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import harness
    import paged_kv_cache_345_amd as pkv
    import synth

    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_cache_345_amd.build import build
        build()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)

    if args.workload in synth.PREFILL_CONFIGS:
        return prefill_bench(args, args.workload)
    if args.workload.startswith("swap_"):
        return swap_bench(args, args.workload)
    if args.workload.startswith("prefix_"):
        return prefix_bench(args, args.workload)
    wl = synth.make_workload(args.workload)
    log(f"workload {wl.spec.name}: {wl.spec.description}")
    t0 = time.perf_counter()
    step = harness.build_step(wl, partition_tokens=args.partition_tokens)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t0:.1f} s (partition {pkv.partition_tokens_for(wl.num_seqs, wl.num_heads, step.max_blocks, step.desc, step.partition_tokens)} tokens)")
    nb = step_bytes(wl, step)

    # Cache flush between timed steps, outside the timed events: write a 1 GiB
    # scratch buffer, then read it back, so the 256 MB memory-side cache and
    # the L2s hold only clean scratch lines when a step starts.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if args.flush else None
    sink = torch.empty(1, dtype=torch.int64, device="cuda")

    def flush(i):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
            torch.sum(scratch.view(torch.int64), dim=0, keepdim=True, out=sink)

    def one_step():
        if args.separate_prologue:
            step.copy()
            step.write()
            step.plan()
        else:  # the same three operations in one launch
            step.prologue()

    for i in range(args.warmup):
        flush(i)
        one_step()
        step.run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(K):
        flush(i)
        e0, e1, e2 = ev[i]
        e0.record()
        one_step()
        e1.record()
        step.run()
        e2.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    step_ms = np.array([a.elapsed_time(c) for a, _b, c in ev])
    dec_ms = np.array([b.elapsed_time(c) for _a, b, c in ev])
    ms_per_step = float(step_ms.mean())
    dec_med, dec_min, dec_avg = float(np.median(dec_ms)), float(dec_ms.min()), float(dec_ms.mean())
    log(f"step mean {ms_per_step * 1e3:.1f} us, median {np.median(step_ms) * 1e3:.1f} us "
        f"({'flushed' if args.flush else 'not flushed'}; wall {wall_s / K * 1e6:.1f} us per step with the flush); "
        f"decode median {dec_med * 1e3:.1f} us, min {dec_min * 1e3:.1f} us, mean {dec_avg * 1e3:.1f} us")

    # The page-read ceiling: the attention call's page reads alone (same work
    # list, wave ranges and loads, no arithmetic), timed the same way.
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    step.plan()
    rp_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        flush(i)
        rp_ev[i][0].record()
        pkv.paged_attn_decode_read_pages(step.k_cache, step.v_cache, step.block_tables, step.context_lens,
                                         wl.num_heads, sink, workspace=step.workspace,
                                         partition_tokens=step.partition_tokens)
        rp_ev[i][1].record()
    torch.cuda.synchronize()
    rp_ms = np.array([a.elapsed_time(b) for a, b in rp_ev])
    rp_med = float(np.median(rp_ms))
    log(f"page reads alone: median {rp_med * 1e3:.1f} us, min {rp_ms.min() * 1e3:.1f} us "
        f"({nb['decode'] / (rp_med * 1e-3) / 1e9:.0f} GB/s of the call's algorithmic bytes)")

    graph_us = None
    if args.graph:
        # the same step captured once in a HIP graph and replayed: no host
        # launch work between the kernels
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
            step.run()
        for _ in range(args.warmup):
            graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record()
        for _ in range(K):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) / K * 1e3
        log(f"graph replay: step {graph_us:.1f} us")

    seg_tokens = pkv.partition_tokens_for(wl.num_seqs, wl.num_heads, step.max_blocks, step.desc,
                                          step.partition_tokens)
    step_gbs = nb["step"] / (ms_per_step * 1e-3) / 1e9
    dec_gbs = nb["decode"] / (dec_med * 1e-3) / 1e9
    S = wl.num_seqs
    result = {
        "metric": "paged decode-attention KV GB/s (% of MI355X HBM peak) and tokens/s at 1 GPU",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype if wl.kv_dtype == wl.dtype else f"{wl.dtype} (fp8e4m3 cache)",
        "data": "synthetic",
        "config": {
            "workload": wl.spec.description,
            "name": wl.spec.name,
            "num_seqs": S,
            "num_heads": wl.num_heads,
            "num_kv_heads": wl.num_kv_heads,
            "head_size": 128,
            "block_size": 16,
            "context_tokens": wl.total_context,
            "partition_tokens": pkv.partition_tokens_for(S, wl.num_heads, step.max_blocks, step.desc,
                                                         step.partition_tokens),
            "copy_pairs": int(step.block_pairs_host.shape[0]),
            "kv_cache_dtype": wl.kv_dtype,
            "step": (("copy_blocks + reshape_and_cache{0} + paged_attn_decode_plan + paged_attn_decode_run{0}"
                      if args.separate_prologue else
                      "decode_step_prologue{0} (copy_blocks + reshape_and_cache{0} + paged_attn_decode_plan in one "
                      "launch) + paged_attn_decode_run{0}").format("_fp8" if step.fp8 else "")),
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "context_tokens_per_s": round(wl.total_context / (ms_per_step * 1e-3), 1),
        "bytes": nb,
        "decode_call_us": round(dec_med * 1e3, 2),
        "timing": {"flushed": bool(args.flush),
                   "flush": ("1 GiB scratch written then read between timed steps, outside the events"
                             if args.flush else None),
                   "step_us": {"mean": round(ms_per_step * 1e3, 2), "median": round(float(np.median(step_ms)) * 1e3, 2),
                               "min": round(float(step_ms.min()) * 1e3, 2)},
                   "decode_call_us": {"median": round(dec_med * 1e3, 2), "min": round(dec_min * 1e3, 2),
                                      "mean": round(dec_avg * 1e3, 2)},
                   "decode_gbs_at_min": round(nb["decode"] / (dec_min * 1e-3) / 1e9, 2),
                   "events": "HIP events on the stream the kernels run on, around each step and each "
                             "paged_attn_decode_run call"},
        "graph_step_us": None if graph_us is None else round(graph_us, 2),
        "page_read_ceiling": {
            "what": ("paged_attn_decode_read_pages: the attention call's work list, wave ranges and page loads "
                     "with no arithmetic, flushed and timed like the call"),
            "us": {"median": round(rp_med * 1e3, 2), "min": round(float(rp_ms.min()) * 1e3, 2)},
            "gbs": round(nb["decode"] / (rp_med * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(nb["decode"] / (rp_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_call_over_ceiling": round(dec_med / rp_med, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_attn_decode_run: " + ("decode_mha_kernel" if wl.num_heads == wl.num_kv_heads
                                                    else "decode_gqa_kernel")
                       + (" + decode_reduce_kernel" if step.max_blocks * 16 > seg_tokens else "")),
            "achieved": round(dec_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(f"decode_{wl.spec.name}"),
        },
        "cpu_baseline": None,
    }
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    if not args.no_cpu_baseline:
        bits = harness.to_host_bits(step.out)  # the output of the last timed step, widened exactly
        if wl.dtype == "fp16":
            got = bits.view(np.float16).astype(np.float64)
        else:
            got = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        cb = cpu_baseline(wl, args.cpu_seconds, nb, gpu_out=got)
        tol = 2e-3 if wl.dtype == "fp16" else 1e-2
        cb["tolerance"] = tol
        cb["within_tolerance"] = bool(cb["max_abs_err"] <= tol)
        result["cpu_baseline"] = cb
        result["max_abs_err"] = cb["max_abs_err"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

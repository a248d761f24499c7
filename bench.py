"""Decode-step benchmark on one MI355X: slot-mapping append + paged attention.

A step is one pass of the whole path over one batch: each sequence's newest
token's K/V goes into its cache slot, then one query per sequence attends over
its paged K/V.  By default the step is the library's fused call,
paged_attention_decode_step (append and attention in one launch); with
--two-call-step it is paged_kv_write + paged_attention_decode (both forms are
timed and reported).  The default workload is the LLaMA-2-13B-shaped
single-layer batch (64 sequences, 40 heads, head_dim 128, block 16, bf16,
contexts uniform in [128, 2048], pool 1.25x the needed blocks in a shuffled
free list).  Inputs are resident in HBM before timing starts; consecutive steps
rotate over independent copies of the inputs (each larger than the 256 MB
Infinity Cache) so no step reads data the previous one left in the caches.

Prints one JSON line:
  value          algorithmic GB/s of the whole step (append + decode bytes / step time)
  roofline       the decode call (the partition kernel, plus the LSE reduce when the
                 context is split), algorithmic bytes per launch / its mean duration from
                 HIP events on the launch stream, vs the 8 TB/s HBM peak
  cpu_baseline   the float64 CPU oracle on a bounded sample of the same workload
Timing: the K steps run back to back with no event between them (wall clock and one HIP event
pair bracket them); then the other form of the step, the decode call alone and the write alone
run K times back to back, each bracketed by a HIP event pair, for the per-launch averages.
Other workloads (--workload): parallel_sampling, continuous_batching, prefill, split_sweep.
Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--config 2]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "paged-attn decode achieved HBM GB/s (% of MI355X peak); tokens·heads/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def elem_bytes(dtype):
    return 4 if dtype == "f32" else 2


def algorithmic_bytes(meta):
    """Bytes the method must move per call (no workspace, no re-reads)."""
    import numpy as np
    cfg = meta.cfg
    es = elem_bytes(cfg.dtype)
    L = meta.context_lens.astype(np.int64)
    B, H, D, bs = len(L), cfg.num_heads, cfg.head_dim, cfg.block_size
    kv = int(L.sum()) * H * D * 2 * es
    qo = B * H * D * 2 * es
    meta_b = 4 * int(((L + bs - 1) // bs).sum()) + 4 * B
    decode = kv + qo + meta_b
    T = B                                          # one new token per sequence
    write = 2 * T * H * D * es * 2 + 8 * T         # read k, v; write both into the caches; slot ids
    return {"decode": decode, "write": write, "step": decode + write, "kv": kv}


CPU_MAX_WORKERS = 16           # one GPU's share of the host's cores


def cpu_workers():
    """Threads for the CPU oracle: the cores this process may run on, at most CPU_MAX_WORKERS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, CPU_MAX_WORKERS))


def cpu_host_info():
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"host_cpus": os.cpu_count(), "affinity_cpus": affinity}


def cpu_baseline(meta, w, budget_s=12.0, single_s=4.0):
    """The oracle, untouched, on the same workload and the host's cores.  Whole steps: the oracle's write of
    the batch's new tokens (a copy of the whole pool), then oracle.decode of every sequence, the sequences
    shared out to a pool of threads (one per core of this process's CPU share, at most 16; NumPy releases the
    GIL inside the oracle's array operations), until about budget_s.  Then, for comparison, sequence after
    sequence on one thread for about single_s."""
    import resource
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import workloads as W
    cfg = meta.cfg
    q = W.storage_numpy(w.q)
    k0, v0 = W.storage_numpy(w.k_cache), W.storage_numpy(w.v_cache)
    kn, vn = W.storage_numpy(w.k_new), W.storage_numpy(w.v_new)
    B = len(meta.context_lens)
    es = elem_bytes(cfg.dtype)
    H, D, bs = cfg.num_heads, cfg.head_dim, cfg.block_size
    L = meta.context_lens.astype(np.int64)
    per_seq = L * H * D * 2 * es + H * D * 2 * es + 4 * ((L + bs - 1) // bs) + 4 + 2 * H * D * es * 2 + 8
    order = np.argsort(-L, kind="stable").tolist()          # longest first: the pool's tail stays short
    nw = cpu_workers()

    def one(args):
        kc, vc, i = args
        oracle.decode(q, kc, vc, meta.block_tables, meta.context_lens, cfg.scale, bs, cfg.dtype, seqs=[i])
        return i

    nbytes, tokens, steps = 0, 0, 0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nw) as ex:
        while steps == 0 or time.perf_counter() - t0 < budget_s:
            kc, vc = oracle.kv_write(kn, vn, meta.slot_mapping, k0, v0, cfg.block_size)
            for i in ex.map(one, [(kc, vc, i) for i in order]):
                nbytes += int(per_seq[i])
                tokens += int(L[i]) * H
            steps += 1
    wall = time.perf_counter() - t0
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    # one thread, for comparison: the decode of sequence after sequence (the write excluded)
    sb, st, sn = 0, 0, 0
    t1 = time.perf_counter()
    del k0, v0
    for i in order:
        one((kc, vc, i))
        sb += int(per_seq[i])
        st += int(L[i]) * H
        sn += 1
        if time.perf_counter() - t1 >= single_s:
            break
    single_wall = time.perf_counter() - t1
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": nw, "kind": "oracle",
            "sample": f"{steps} whole step(s) of the {B}-sequence batch, each the oracle's write of the {B} new "
                      f"tokens (a whole-pool copy) and then every sequence's decode on {nw} threads; "
                      f"{wall:.1f} s wall, {cpu:.1f} s CPU ({cpu / wall:.1f} cores busy on average)",
            "tokens_heads_per_s": round(tokens / wall, 1),
            "single_thread": {"value": round(sb / single_wall / 1e9, 4), "unit": "GB/s",
                              "tokens_heads_per_s": round(st / single_wall, 1),
                              "sample": f"decode of the {sn} longest sequences one after another, "
                                        f"{single_wall:.1f} s (no write)"},
            **cpu_host_info()}


def cpu_oracle_steps(q, k0, v0, kn, vn, tables, lens, slots, scale, bs, dtype, step_bytes, copies=None,
                     budget_s=12.0, what="one step"):
    """Whole steps of a decode workload by the oracle, untouched, on the host's cores: the oracle's block copies
    (when ``copies`` is given), its write of the new tokens (a copy of the whole pool) and oracle.decode of every
    row, the rows shared out to a pool of threads as in cpu_baseline, until about budget_s.  ``step_bytes`` is
    the GPU step's algorithmic byte count, so the rate is in the workload's own unit."""
    import resource
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from oracle import block_manager
    L = np.asarray(lens).astype(np.int64)
    H = q.shape[1]
    order = np.argsort(-L, kind="stable").tolist()
    order = [i for i in order if L[i] > 0]
    nw = cpu_workers()

    def one(args):
        kc, vc, i = args
        oracle.decode(q, kc, vc, tables, lens, scale, bs, dtype, seqs=[i])

    steps = 0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nw) as ex:
        while steps == 0 or time.perf_counter() - t0 < budget_s:
            kc, vc = (block_manager.copy_blocks(k0, v0, copies) if copies is not None and len(copies)
                      else (k0, v0))
            kc, vc = oracle.kv_write(kn, vn, slots, kc, vc, bs)
            list(ex.map(one, [(kc, vc, i) for i in order]))
            steps += 1
    wall = time.perf_counter() - t0
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    return {"value": round(steps * step_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": nw, "kind": "oracle",
            "sample": f"{steps} x ({what}), {len(order)} rows each, on {nw} threads; {wall:.1f} s wall, "
                      f"{cpu:.1f} s CPU ({cpu / wall:.1f} cores busy on average)",
            "tokens_heads_per_s": round(steps * int(L.sum()) * H / wall, 1), **cpu_host_info()}


def cpu_baseline_prefill(q, kc, vc, tables, lens, scale, bs, dtype, budget_s=12.0):
    """The oracle's prefill, untouched, on the same prompts and the host's cores: each prompt's queries over its
    own cache blocks, prompts shared out to a pool of threads (as for the decode baseline), new prompts
    started until about budget_s; the prompts still running then finish and count."""
    import resource
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

    import numpy as np

    import oracle
    import workloads as W
    qh, kh, vh = W.storage_numpy(q), W.storage_numpy(kc), W.storage_numpy(vc)
    H, D = qh.shape[1], qh.shape[2]
    starts = np.concatenate([[0], np.cumsum(lens)])
    nw = cpu_workers()

    def one(i):
        P = int(lens[i])
        oracle.prefill(qh[starts[i]:starts[i] + P], kh, vh, tables[i:i + 1], np.array([0, P]), np.array([P]),
                       scale, bs, dtype)
        return i

    tokens, pairs, done = 0, 0, 0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nw) as ex:
        pending, nxt = set(), 0
        while nxt < len(lens) or pending:
            while nxt < len(lens) and len(pending) < nw and time.perf_counter() - t0 < budget_s:
                pending.add(ex.submit(one, nxt))
                nxt += 1
            if not pending:
                break
            finished, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in finished:
                P = int(lens[f.result()])
                tokens += P
                pairs += P * (P + 1) // 2
                done += 1
    wall = time.perf_counter() - t0
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    return {"value": round(tokens / wall, 1), "unit": "prompt tokens/s", "cores": nw, "kind": "oracle",
            "sample": f"{done} of the {len(lens)} prompts ({tokens} tokens), shortest first, each prefilled alone, "
                      f"on {nw} threads; {wall:.1f} s wall, {cpu:.1f} s CPU ({cpu / wall:.1f} cores busy on average)",
            "tflops": round(pairs * H * 4 * D / wall / 1e12, 6), **cpu_host_info()}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partition_llama13b_b64_hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_383_amd", "csrc", f) for f in ("decode.hip", "pkv_internal.h")]


def kernel_fingerprint():
    """sha256 over the decode kernel's sources and compile flags: counters taken on another
    version of the kernel no longer describe this one."""
    import hashlib
    from paged_kv_cache_383_amd import build as b
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(b.compile_flags()).replace(ROOT, "").encode())
    return h.hexdigest()


def measured_traffic(workload, partition):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or
    None when that summary was taken on a different kernel, workload or partition size."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("traffic-json:"):
                t = json.loads(line.split(":", 1)[1])
                if (t.get("kernel_sha256") == kernel_fingerprint() and t.get("workload") == workload
                        and t.get("partition_size") == partition):
                    return t
    return None


def copy_calibration(mib):
    """A plain elementwise copy of known size (read N bytes, write N bytes) whose FETCH_SIZE / WRITE_SIZE
    counters calibrate the decode kernel's: run under rocprofv3 --pmc beside the bench."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": "torch.neg fp32", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 5}), flush=True)


def torch_stream_reference(reps=20):
    """Plain PyTorch streaming on the same GPU, timed the same way, to read the decode's roofline fraction
    against: a 1 GiB fp32 elementwise copy (torch.neg: reads 1 GiB, writes 1 GiB) and a read-only sum over
    2 GiB. Both buffers are far larger than the caches. A diagnostic only: not the library's path."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    big = torch.ones(2 * n, dtype=torch.float32, device="cuda:0")
    for _ in range(3):
        torch.neg(src, out=dst)
        big.sum()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / reps
    e0.record()
    for _ in range(reps):
        big.sum()
    e1.record()
    torch.cuda.synchronize()
    sum_s = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst, big
    torch.cuda.empty_cache()
    return {"torch_copy_1GiB_GBps": round(2 * n * 4 / copy_s / 1e9, 1),
            "torch_sum_2GiB_read_GBps": round(2 * n * 4 / sum_s / 1e9, 1),
            "note": "plain PyTorch streaming on the same GPU (torch.neg copy, torch.sum read), events"}


def read_ceiling(meta, sets, partition, reps=20):
    """HBM read ceilings on this GPU from the library's read probe (pkv_read_probe: the decode kernel's loads
    and wave layout, with no arithmetic), over the benchmark's own rotating K/V pools:
      decode_pattern   the decode's tiles in the decode's order: one work-group per (sequence, partition, head)
                       with the head fastest, entries block_tables[s, j] * H + h of the partition's blocks (each
                       group stopping at its row's block count), a ring of 2 stages (the decode kernel's own
                       depth): the decode's gather without arithmetic;
      random_tiles     every (block, head) tile of both pools once, in a random order, 128 per work-group;
      sequential       both pools streamed from start to end, 128 tiles per work-group;
      sequential_one_pool  the K pool alone, streamed, 4-stage ring;
    random and sequential at ring depths 2 and 3.  Each figure is bytes read per launch / mean launch time
    (HIP events on the launch stream, launches back to back, alternating input sets); "best" is the highest."""
    import torch

    import paged_kv_cache_383_amd as pkv
    cfg = meta.cfg
    H, D, bs = cfg.num_heads, cfg.head_dim, cfg.block_size
    tile = bs * D * elem_bytes(cfg.dtype)
    dev = sets[0].k_cache.device
    pool_tiles = meta.num_blocks * H
    tab = sets[0].block_tables.long()
    B, M = tab.shape
    pb = partition // bs if partition else M
    P = -(-M // pb)
    padded = torch.full((B, P * pb), -1, dtype=torch.int64, device=dev)
    padded[:, :M] = tab
    padded = padded.view(B, P, 1, pb)
    h = torch.arange(H, device=dev, dtype=torch.int64).view(1, 1, H, 1)
    order_dec = torch.where(padded >= 0, padded * H + h, torch.full_like(padded * H + h, -1))
    order_dec = order_dec.reshape(B * P * H, pb).to(torch.int32).contiguous()
    nblk = (tab >= 0).sum(dim=1)                                  # each row's block count
    p_first = torch.arange(P, device=dev, dtype=torch.int64).view(1, P, 1) * pb
    len_dec = (nblk.view(B, 1, 1) - p_first).clamp(0, pb).expand(B, P, H).reshape(-1).to(torch.int32).contiguous()
    n_dec = int(nblk.sum().item()) * H
    g = torch.Generator(device=dev)
    g.manual_seed(383383)
    group = 128
    n_groups = -(-pool_tiles // group)
    order_rand = torch.full((n_groups * group,), -1, dtype=torch.int32, device=dev)
    order_rand[:pool_tiles] = torch.randperm(pool_tiles, generator=g, device=dev).to(torch.int32)
    sink = torch.empty(8 * max(B * P * H, n_groups), dtype=torch.int32, device=dev)
    R = len(sets)

    def timed(order, group_tiles, depth, two=True, group_len=None):
        run = lambda i: pkv.read_probe(sets[i % R].k_cache, sets[i % R].v_cache if two else None, tile, order,
                                       group_tiles, sink, depth=depth, group_len=group_len)
        for i in range(3):
            run(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    both = 2 * pool_tiles * tile
    runs = {"decode_pattern": (timed(order_dec, pb, 2, group_len=len_dec), 2 * n_dec * tile)}
    for d in (2, 3):
        runs[f"random_tiles_depth{d}"] = (timed(order_rand, group, d), both)
        runs[f"sequential_depth{d}"] = (timed(None, group, d), both)
    runs["sequential_one_pool_depth4"] = (timed(None, group, 4, two=False), pool_tiles * tile)
    out = {k: {"GB_per_s": round(b / us / 1e3, 1), "mean_launch_us": round(us, 2), "bytes_per_launch": b}
           for k, (us, b) in runs.items()}
    best = max(out, key=lambda k: out[k]["GB_per_s"])
    out["best"] = {"pattern": best, "GB_per_s": out[best]["GB_per_s"]}
    out["tile_bytes"] = tile
    out["kernel"] = "read_probe_kernel (pkv_read_probe)"
    return out


def parallel_sampling(args):
    """Decode step of parallel sampling over shared prompts: the block pool reserves each sample's new
    slot (copying the shared, partly filled last block of a prompt for all but its last writer), then
    copy_blocks + paged_kv_write + paged_attention_decode run on the GPU."""
    import numpy as np
    import torch

    import paged_kv_cache_383_amd as pkv
    import workloads as W
    cfg = W.SamplingConfig()
    dev = torch.device("cuda:0")
    es = elem_bytes(cfg.dtype)
    H, D, bs = cfg.num_heads, cfg.head_dim, cfg.block_size
    block_bytes = H * bs * D * es
    dt = W.torch_dtype(cfg.dtype)
    sets = []
    for r in range(2):                                   # two independent pools, > 256 MB each
        lens, nb, order = W.sampling_prompts(cfg, cfg.seed + r)
        pool = pkv.BlockPool(nb, bs, order)
        gen = torch.Generator(device=dev)
        gen.manual_seed(cfg.seed + r)
        kc, vc = W.kv_pool(nb, H, bs, D, dt, dev)
        W._randn_into(kc, gen, 1.0, 1024)
        W._randn_into(vc, gen, 1.0, 1024)
        seqs, slots, copies = [], [], []
        for p, L in enumerate(lens.tolist()):
            pool.allocate(p * cfg.samples, L)            # prompt K/V: the random pool contents
            for s in range(1, cfg.samples):
                pool.fork(p * cfg.samples, p * cfg.samples + s)
            for s in range(cfg.samples):
                sl, cp = pool.append_slots(p * cfg.samples + s, 1)
                seqs.append(p * cfg.samples + s)
                slots += sl.tolist()
                copies += cp.tolist()
        width = (cfg.max_len + 1 + bs - 1) // bs
        tables, ctx = pool.build_tables(seqs, width)
        B = len(seqs)
        q = torch.randn((B, H, D), generator=gen, device=dev).to(dt)
        kn = torch.randn((B, H, D), generator=gen, device=dev).to(dt)
        vn = torch.randn((B, H, D), generator=gen, device=dev).to(dt)
        sets.append(dict(kc=kc, vc=vc, q=q, kn=kn, vn=vn, out=torch.empty_like(q),
                         slots=torch.tensor(slots, dtype=torch.int64, device=dev),
                         copies=torch.tensor(copies, dtype=torch.int64, device=dev).reshape(-1, 2),
                         tables=torch.from_numpy(tables).to(dev), lens=torch.from_numpy(ctx).to(dev),
                         ctx=ctx, pool=pool))
    ws = torch.zeros(1, dtype=torch.uint8, device=dev)
    B = len(sets[0]["ctx"])
    n_copy = sets[0]["copies"].shape[0]
    ctx = sets[0]["ctx"].astype(np.int64)
    decode_b = int(ctx.sum()) * H * D * 2 * es + B * H * D * 2 * es + 4 * int(((ctx + bs - 1) // bs).sum()) + 4 * B
    write_b = 2 * B * H * D * es * 2 + 8 * B
    copy_b = n_copy * 2 * 2 * block_bytes + 16 * n_copy
    tab0 = sets[0]["tables"].cpu().numpy()
    unique_b = int(np.unique(tab0[tab0 >= 0]).size) * 2 * block_bytes      # each shared block once
    log(f"{cfg.name}: {cfg.prompts} prompts x {cfg.samples} samples, {n_copy} block copies per step, "
        f"sum(L) = {int(ctx.sum())}")

    def copy(i):
        st = sets[i % 2]
        pkv.paged_kv_copy_blocks(st["kc"], st["vc"], st["copies"])

    def write(i):
        st = sets[i % 2]
        pkv.paged_kv_write(st["kn"], st["vn"], st["slots"], st["kc"], st["vc"])

    def decode(i):
        st = sets[i % 2]
        pkv.paged_attention_decode(st["q"], st["kc"], st["vc"], st["tables"], st["lens"], cfg.scale,
                                   out=st["out"], workspace=ws)

    for i in range(args.warmup):
        copy(i)
        write(i)
        decode(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        copy(i)
        write(i)
        decode(i)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    decode_us, copy_us = timed(decode, args.steps), timed(copy, args.steps)
    # the copy kernel at scale: every block of the first 1.3 GB of the pool copied to the rest
    big = sets[0]
    nb = big["kc"].shape[0]
    n_big = min(nb // 2, 4096)
    pairs = torch.stack([torch.arange(n_big), torch.arange(n_big) + nb - n_big], 1).to(dev)
    big_us = timed(lambda i: pkv.paged_kv_copy_blocks(big["kc"], big["vc"], pairs), 10)
    big_b = n_big * 2 * 2 * block_bytes + 16 * n_big
    achieved = decode_b / (decode_us * 1e-6) / 1e9
    step_b = decode_b + write_b + copy_b
    log(f"step {step_s * 1e6:.1f} us; decode {decode_us:.1f} us = {achieved:.0f} GB/s; copies {copy_us:.1f} us; "
        f"copy kernel at scale {n_big} pairs {big_us:.1f} us = {big_b / big_us / 1e3:.0f} GB/s")
    rec = {
        "metric": METRIC, "value": round(step_b / step_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "num_seqs": B, "prompts": cfg.prompts, "samples": cfg.samples,
                   "num_heads": H, "head_dim": D, "block_size": bs, "sum_context_tokens": int(ctx.sum()),
                   "block_copies_per_step": n_copy,
                   "step": "paged_kv_copy_blocks + paged_kv_write + paged_attention_decode",
                   "step_algorithmic_bytes": step_b},
        "tokens_heads_per_s": round(int(ctx.sum()) * H / step_s, 1),
        "kernels_us": {"paged_kv_copy_blocks": round(copy_us, 2), "paged_attention_decode": round(decode_us, 2)},
        "copy_kernel_at_scale": {"pairs": n_big, "bytes": big_b, "us": round(big_us, 2),
                                 "GB_per_s": round(big_b / big_us / 1e3, 1),
                                 "frac": round(big_b / big_us / 1e3 / PEAK_HBM_GBS, 4)},
        "roofline": {"kernel": "paged_attention_decode (decode_partition_kernel)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": decode_b, "mean_launch_us": round(decode_us, 2),
                     "note": "algorithmic bytes count every sample's read of a shared prompt block; the blocks "
                             "themselves hold unique_kv_bytes, so caches may serve repeat reads"},
        "unique_kv_bytes": unique_b,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        st = sets[0]
        rec["cpu_baseline"] = cpu_oracle_steps(
            W.storage_numpy(st["q"]), W.storage_numpy(st["kc"]), W.storage_numpy(st["vc"]),
            W.storage_numpy(st["kn"]), W.storage_numpy(st["vn"]), tab0, st["ctx"], st["slots"].cpu().numpy(),
            cfg.scale, bs, cfg.dtype, step_b, copies=st["copies"].cpu().numpy().tolist(),
            what="the step's block copies, its write of the new tokens and its decode")
        log(f"cpu oracle: {rec['cpu_baseline']}")
    print(json.dumps(rec), flush=True)


def continuous_batching(args):
    """A multi-step decode loop: rows run requests from a seeded stream; each step the C++ block pool and
    batch planner reserve every running row's slot, and the prompt writes of new requests,
    paged_kv_prepare_step, block copies, paged_kv_write and paged_attention_decode run on the GPU; a
    request that reaches its length releases its blocks and its row takes the next request."""
    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_383_amd.decode_loop import DecodeLoop
    cfg = W.BatchingConfig()
    dev = torch.device("cuda:0")
    H, D, bs, R = cfg.num_heads, cfg.head_dim, cfg.block_size, cfg.rows
    es = elem_bytes(cfg.dtype)
    dt = W.torch_dtype(cfg.dtype)
    NB = R * cfg.width                         # every row can reach its longest request: no preemption
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    kc, vc = W.kv_pool(NB, H, bs, D, dt, dev)
    W._randn_into(kc, gen, 1.0, 512)
    W._randn_into(vc, gen, 1.0, 512)
    src_k = torch.randn((cfg.prompt_max, H, D), generator=gen, device=dev).to(dt)
    src_v = torch.randn((cfg.prompt_max, H, D), generator=gen, device=dev).to(dt)
    q = torch.randn((R, H, D), generator=gen, device=dev).to(dt)
    kn = torch.randn((R, H, D), generator=gen, device=dev).to(dt)
    vn = torch.randn((R, H, D), generator=gen, device=dev).to(dt)
    out = torch.empty_like(q)
    n_req = 20000
    prompts, gens = W.batching_requests(cfg, n_req)
    loop = DecodeLoop(kc, vc, R, cfg.width, free_order=np.random.default_rng(cfg.seed).permutation(NB))
    state = {"next": 0, "row_req": [-1] * R, "left": [0] * R}

    def fill():
        for r in range(R):
            if state["row_req"][r] < 0 and state["next"] < n_req:
                i = state["next"]
                P = int(prompts[i])
                loop.admit(r, i, src_k[:P], src_v[:P])
                state["row_req"][r], state["left"][r] = i, int(gens[i])
                state["next"] += 1

    def end_of_step():
        for r in range(R):
            if state["row_req"][r] >= 0:
                state["left"][r] -= 1
                if state["left"][r] == 0:
                    loop.release(r)
                    state["row_req"][r] = -1

    totals = {"kv": 0, "tokens": 0, "prompt": 0, "copies": 0, "rows": 0}

    def one_step(count):
        fill()
        loop.step(q, kn, vn, out=out)
        if count:
            lens = loop.last_lens.astype(np.int64)
            totals["kv"] += int(lens.sum())
            totals["rows"] += int((lens > 0).sum())
            totals["prompt"] += loop.last_prompt_tokens
            totals["copies"] += len(loop.last_copies)
        end_of_step()

    log(f"{cfg.name}: pool {NB} blocks ({2 * NB * H * bs * D * es / 1e9:.1f} GB K+V), {R} rows")
    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        one_step(True)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = a.elapsed_time(b) * 1e-3
    row_b = H * D * es
    nbytes = (totals["kv"] * 2 * row_b + totals["rows"] * 2 * row_b       # decode: K/V reads, q + out
              + totals["rows"] * 4 * row_b + totals["prompt"] * 4 * row_b  # new-token and prompt writes
              + totals["copies"] * 4 * bs * row_b)                         # copy-on-write
    # the decode kernel alone at the loop's final state, back to back
    lens_now = loop.last_lens.astype(np.int64)
    ctx = lens_now[lens_now > 0]
    decode_b = int(ctx.sum()) * 2 * row_b + len(ctx) * 2 * row_b + 4 * int(((ctx + bs - 1) // bs).sum()) + 4 * R
    from paged_kv_cache_383_amd import paged_attention_decode
    for _ in range(3):
        paged_attention_decode(q, kc, vc, loop.tables, loop.lens, loop.scale, out=out, workspace=loop.workspace)
    a.record()
    for _ in range(20):
        paged_attention_decode(q, kc, vc, loop.tables, loop.lens, loop.scale, out=out, workspace=loop.workspace)
    b.record()
    torch.cuda.synchronize()
    decode_us = a.elapsed_time(b) * 1e3 / 20
    achieved = decode_b / decode_us / 1e3
    step_s = wall / args.steps
    log(f"{args.steps} steps in {wall * 1e3:.1f} ms (GPU {gpu_s * 1e3:.1f} ms): {step_s * 1e6:.1f} us/step, "
        f"{totals['rows'] / wall:.0f} generated tokens/s, {nbytes / wall / 1e9:.0f} GB/s; "
        f"{state['next']} requests admitted; decode alone {decode_us:.1f} us = {achieved:.0f} GB/s")
    rec = {
        "metric": METRIC, "value": round(nbytes / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "rows": R, "num_heads": H, "head_dim": D, "block_size": bs,
                   "pool_blocks": NB, "requests_admitted": state["next"],
                   "step": "plan (host) + prompt writes + paged_kv_prepare_step + paged_kv_copy_blocks + "
                           "paged_kv_write + paged_attention_decode",
                   "algorithmic_bytes": nbytes},
        "tokens_heads_per_s": round(totals["kv"] * H / wall, 1),
        "generated_tokens_per_s": round(totals["rows"] / wall, 1),
        "mean_running_rows": round(totals["rows"] / args.steps, 1),
        "gpu_time_fraction": round(gpu_s / wall, 4),
        "roofline": {"kernel": "paged_attention_decode (decode_partition_kernel), loop's final batch",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": decode_b, "mean_launch_us": round(decode_us, 2)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # the oracle on the loop's final batch: whole steps of its write of the running rows' new tokens and
        # its decode of every running row, over a pool of just the blocks the batch holds (ids renumbered)
        import oracle
        tab = loop.tables.cpu().numpy().astype(np.int64)
        lens_h = loop.lens.cpu().numpy()
        used = np.unique(tab[tab >= 0])
        renum = np.full(NB, -1, dtype=np.int64)
        renum[used] = np.arange(len(used))
        tab_c = np.where(tab >= 0, renum[np.maximum(tab, 0)], -1).astype(np.int32)
        idx = torch.from_numpy(used).to(dev)
        active = int((lens_h > 0).sum())
        rec["cpu_baseline"] = cpu_oracle_steps(
            W.storage_numpy(q), W.storage_numpy(kc.index_select(0, idx)), W.storage_numpy(vc.index_select(0, idx)),
            W.storage_numpy(kn), W.storage_numpy(vn), tab_c, lens_h, oracle.newest_token_slots(tab_c, lens_h, bs),
            loop.scale, bs, cfg.dtype, decode_b + active * 4 * row_b + 8 * active,
            what="the loop's final batch: its write of the running rows' new tokens and its decode")
        log(f"cpu oracle: {rec['cpu_baseline']}")
    print(json.dumps(rec), flush=True)


PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks, published


def mfma_ceiling(dtype_name, reps=4):
    """Matrix-core ceilings on this GPU from the library's probe (pkv_mfma_probe: the prefill kernel's product
    instruction, v_mfma_f32_32x32x16, with nothing else to do), at 1, 2 and 3 waves per SIMD (the prefill kernel
    runs 3), and at 3 waves with 4 vector additions per product.  Each: TFLOP/s over the launch (events, the last
    of ``reps`` launches of about 1-3 ms) and the shader clock the waves recorded.  A diagnostic only."""
    import torch

    import paged_kv_cache_383_amd as pkv
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype_name]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = pkv.MFMA_PROBE_MAX_ITERS
    out = {}
    for waves, valu in ((1, 0), (2, 0), (3, 0), (3, 4)):
        groups = cus * waves
        sink = torch.empty(groups * 256, dtype=torch.float32, device="cuda:0")
        clocks = torch.zeros(groups * 8, dtype=torch.int64, device="cuda:0")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(reps):
            a.record()
            pkv.mfma_probe(dt, groups, iters, sink, clocks, valu=valu)
            b.record()
            torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3
        flops = groups * 4 * iters * 8 * 32 * 32 * 16 * 2
        c = clocks.view(-1, 2).double()
        ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
        ok = bool((sink == float(2048 * iters + 8 * valu * iters)).all())
        out[f"waves{waves}_valu{valu}"] = {"us": round(us, 1), "tflops": round(flops / us / 1e6, 1),
                                            "clock_ghz": round(ghz, 3), "sums_exact": ok}
    out["best_tflops"] = max(v["tflops"] for k, v in out.items() if k.endswith("valu0"))
    return out


def prefill(args):
    """Prefill of a batch of prompts: the prompts' K/V are written into the paged cache (paged_kv_write),
    then every prompt token attends causally over its sequence (paged_attention_prefill, MFMA)."""
    import numpy as np
    import torch

    import paged_kv_cache_383_amd as pkv
    import workloads as W
    import dataclasses
    cfg = W.PrefillConfig()
    if args.prefill_dtype != cfg.dtype:
        cfg = dataclasses.replace(cfg, dtype=args.prefill_dtype, name=cfg.name.rsplit("_", 1)[0] + "_" + args.prefill_dtype)
    dev = torch.device("cuda:0")
    H, D, bs = cfg.num_heads, cfg.head_dim, cfg.block_size
    es = elem_bytes(cfg.dtype)
    dt = W.torch_dtype(cfg.dtype)
    lens, nb, order = W.prefill_prompts(cfg)
    pool = pkv.BlockPool(nb, bs, order)
    for i, L in enumerate(lens.tolist()):
        pool.allocate(i, L)
    width = (cfg.max_len + bs - 1) // bs
    tables, ctx = pool.build_tables(list(range(len(lens))), width)
    T = int(lens.sum())
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.concatenate([pool.slots(i, 0, L) for i, L in enumerate(lens.tolist())])
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    kc, vc = W.kv_pool(nb, H, bs, D, dt, dev, zero=True)
    kp = torch.randn((T, H, D), generator=gen, device=dev).to(dt)
    vp = torch.randn((T, H, D), generator=gen, device=dev).to(dt)
    q = torch.randn((T, H, D), generator=gen, device=dev).to(dt)
    out = torch.empty_like(q)
    t_tables, t_ctx = torch.from_numpy(tables).to(dev), torch.from_numpy(ctx).to(dev)
    t_qs, t_slots = torch.from_numpy(qs).to(dev), torch.from_numpy(slots).to(dev)
    maxq = int(lens.max())
    # useful flops: each (query, key <= its position, head) pair costs 2 D for q.k and 2 D for p.v
    pairs = int((lens * (lens + 1) // 2).sum())
    flops = pairs * H * 4 * D
    write_b = 2 * T * H * D * es * 2 + 8 * T

    def step():
        pkv.paged_kv_write(kp, vp, t_slots, kc, vc)
        pkv.paged_attention_prefill(q, kc, vc, t_tables, t_qs, t_ctx, cfg.scale, maxq, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        pkv.paged_attention_prefill(q, kc, vc, t_tables, t_qs, t_ctx, cfg.scale, maxq, out=out)
    b.record()
    torch.cuda.synchronize()
    pre_us = a.elapsed_time(b) * 1e3 / args.steps
    # isolated launches: each bracketed by its own event pair with the GPU idle before it (no overlap with a
    # neighbouring launch), the start-to-end duration a kernel trace records
    iso = []
    for _ in range(min(args.steps, 20)):
        torch.cuda.synchronize()
        a.record()
        pkv.paged_attention_prefill(q, kc, vc, t_tables, t_qs, t_ctx, cfg.scale, maxq, out=out)
        b.record()
        torch.cuda.synchronize()
        iso.append(a.elapsed_time(b) * 1e3)
    iso_us = sum(iso) / len(iso)
    tflops = flops / pre_us / 1e6
    peak = PEAK_MFMA_TFLOPS[cfg.dtype]
    log(f"{cfg.name}: {T} tokens, {pairs} causal pairs; step {step_s * 1e6:.1f} us; prefill kernel {pre_us:.1f} us "
        f"= {tflops:.1f} TFLOP/s ({tflops / peak:.1%} of {peak:.0f}); isolated launches {iso_us:.1f} us "
        f"({flops / iso_us / 1e6 / peak:.1%})")
    rec = {
        "metric": METRIC, "value": round(T / step_s, 1), "unit": "prompt tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "prompts": len(lens), "prompt_tokens": T, "num_heads": H, "head_dim": D,
                   "block_size": bs, "step": "paged_kv_write(prompt K/V) + paged_attention_prefill",
                   "flops_per_step": flops, "write_bytes_per_step": write_b},
        "tokens_heads_per_s": round(T * H / step_s, 1),
        "kernels_us": {"paged_attention_prefill": round(pre_us, 2), "paged_attention_prefill_isolated": round(iso_us, 2)},
        "roofline": {"kernel": ("paged_attention_prefill (prefill_kernel: 16x16x4 fp32 MFMA tiles)" if cfg.dtype == "f32"
                               else "paged_attention_prefill (prefill32_kernel: 32x32x16 MFMA tiles)"), "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "mean_launch_us": round(pre_us, 2)},
        "cpu_baseline": None,
    }
    if not args.no_diagnostic and cfg.dtype in ("bf16", "f16"):
        ceiling = mfma_ceiling(cfg.dtype)
        ceiling["prefill_frac_of_best"] = round(tflops / ceiling["best_tflops"], 4)
        rec["diagnostic"] = {"mfma_probe": ceiling}
        log("mfma probe: " + "; ".join(f"{k} {v['tflops']} TFLOP/s at {v['clock_ghz']} GHz" for k, v in ceiling.items()
                                       if isinstance(v, dict))
            + f" -> prefill {tflops:.0f} TFLOP/s = {ceiling['prefill_frac_of_best']:.1%} of the best")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle's prefill on a sample of the same prompts ...")
        order_short = np.argsort(lens, kind="stable")           # shortest prompts first: more of them fit
        sub = [int(x) for x in order_short]
        qs_sub = np.concatenate([[0], np.cumsum(lens[sub])])
        q_sub = torch.cat([q[int(qs[i]):int(qs[i + 1])] for i in sub])
        rec["cpu_baseline"] = cpu_baseline_prefill(q_sub, kc, vc, tables[sub], lens[sub], cfg.scale, bs, cfg.dtype)
        log(f"cpu oracle: {rec['cpu_baseline']}")
    print(json.dumps(rec), flush=True)


SPLIT_SWEEP_SHAPES = [(1, 40, 32768), (2, 40, 16384), (1, 32, 8192), (4, 40, 32768)]   # (sequences, heads, context)


def split_sweep(args):
    """The decode call at few (sequence, head) rows, where the library splits contexts into partitions: the
    library's automatic choice beside fixed partition sizes, at the LLaMA-2-13B head shape (D 128, 16-token
    blocks, bf16, every sequence at the full context, blocks in a shuffled pool).  One JSON line."""
    import torch

    import paged_kv_cache_383_amd as pkv
    import workloads as W
    dev = torch.device("cuda:0")
    bs, D = 16, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(383500)
    rows = []
    for B, H, L in SPLIT_SWEEP_SHAPES:
        nb_seq = L // bs
        NB = B * nb_seq
        k, v = W.kv_pool(NB, H, bs, D, torch.bfloat16, dev)
        W._randn_into(k, gen, 1.0, 1024)
        W._randn_into(v, gen, 1.0, 1024)
        tables = torch.randperm(NB, generator=gen, device=dev).to(torch.int32).view(B, nb_seq).contiguous()
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        q = torch.randn((B, H, D), generator=gen, device=dev).to(torch.bfloat16)
        out = torch.empty_like(q)
        nbytes = B * L * H * D * 2 * 2 + B * H * D * 2 * 2 + 4 * B * nb_seq + 4 * B
        res = {}
        # two rounds over the partition sizes; the first only warms the new pools, the second is reported
        for part in [pkv.PARTITION_AUTO, 512, 1024, 2048, 4096] * 2:
            ws = torch.empty(max(pkv.paged_attention_workspace_bytes(B, H, D, nb_seq, bs, part), 1), dtype=torch.uint8,
                             device=dev)
            run = lambda: pkv.paged_attention_decode(q, k, v, tables, lens, 1.0 / math.sqrt(D), out=out, workspace=ws,
                                                     partition_size=part)
            for _ in range(args.warmup):
                run()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                run()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / args.steps
            res["auto" if part == pkv.PARTITION_AUTO else str(part)] = {"us": round(us, 2),
                                                                       "GB_per_s": round(nbytes / us / 1e3, 1)}
        auto = pkv.paged_attention_partition_size(B, H, nb_seq, bs, pkv.PARTITION_AUTO)
        log(f"B={B} H={H} L={L}: automatic partition {auto} tokens; " +
            " ".join(f"{k_}: {v_['us']} us" for k_, v_ in res.items()))
        rows.append({"num_seqs": B, "num_heads": H, "context": L, "auto_partition": auto, "bytes": nbytes,
                     "decode": res})
        del k, v
        torch.cuda.empty_cache()
    first = rows[0]["decode"]["auto"]          # the line's value: the first shape at the automatic split
    rec = {"metric": METRIC, "value": first["GB_per_s"], "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(first["us"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "split_sweep_few_rows_h40_d128_bs16_bf16", "shapes": rows},
           "cpu_baseline": None}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--workload", choices=["decode", "parallel_sampling", "continuous_batching", "prefill",
                                           "split_sweep"],
                    default="decode",
                    help="decode: one decode step of --config; parallel_sampling: a decode step over "
                         "prompts shared by parallel samples (copy-on-write copies + write + decode); "
                         "continuous_batching: a many-step decode loop with admissions and releases; "
                         "prefill: prompt K/V writes + causal paged prefill attention (MFMA); "
                         "split_sweep: the decode call at few rows, automatic split beside fixed partitions")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-context partition in tokens (0 = one pass); default: the library's choice")
    ap.add_argument("--rotate", type=int, default=None, help="independent input copies cycled over")
    ap.add_argument("--block-size", type=int, choices=[16, 32], default=None,
                    help="decode: store the configuration's context lengths in blocks of this many tokens "
                         "instead of its own block size (same lengths and bytes)")
    ap.add_argument("--placement", choices=["shuffled", "consecutive"], default="shuffled",
                    help="decode: block ids from the shuffled free list (default) or one consecutive run per "
                         "sequence (same lengths and bytes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-diagnostic", action="store_true",
                    help="skip the read-probe and matrix-core-probe ceilings and the PyTorch streaming figures (counter runs)")
    ap.add_argument("--two-call-step", action="store_true",
                    help="time the decode step as paged_kv_write + paged_attention_decode instead of the fused "
                         "paged_attention_decode_step")
    ap.add_argument("--prefill-dtype", choices=["bf16", "f16", "f32"], default="bf16",
                    help="element type of --workload prefill (the fp32 kernel is measured against the fp32 MFMA peak)")
    ap.add_argument("--copy-calibration", type=int, default=None, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU variant in this library "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import paged_kv_cache_383_amd as pkv
    import workloads as W
    from paged_kv_cache_383_amd import build as b
    b.ensure_built()
    pkv.lib()
    if args.workload == "parallel_sampling":
        parallel_sampling(args)
        return
    if args.workload == "continuous_batching":
        continuous_batching(args)
        return
    if args.workload == "prefill":
        prefill(args)
        return
    if args.workload == "split_sweep":
        split_sweep(args)
        return

    dev = torch.device("cuda:0")
    base_cfg = W.CONFIGS[args.config]
    if args.block_size and args.block_size != base_cfg.block_size:
        import dataclasses
        name = base_cfg.name.replace(f"_bs{base_cfg.block_size}", "") + f"_bs{args.block_size}"
        base_cfg = dataclasses.replace(base_cfg, block_size=args.block_size, name=name)
    meta = W.make_metadata(base_cfg, placement=args.placement)
    cfg = meta.cfg
    part = pkv.PARTITION_AUTO if args.partition_size is None else args.partition_size
    resolved = pkv.paged_attention_partition_size(len(meta.context_lens), cfg.num_heads, cfg.max_blocks,
                                                  cfg.block_size, part)
    nbytes = algorithmic_bytes(meta)
    per_set = 2 * meta.num_blocks * cfg.num_heads * cfg.block_size * cfg.head_dim * elem_bytes(cfg.dtype)
    rotate = args.rotate or max(2, math.ceil(1.0e9 / per_set))
    log(f"config {cfg.cfg_id} {cfg.name}: B={len(meta.context_lens)} sum(L)={meta.total_tokens} "
        f"pool={meta.num_blocks} blocks ({per_set / 1e9:.2f} GB K+V), {rotate} rotating input sets, "
        f"partition {part} -> {resolved} tokens")
    sets = [W.make_workload(meta, dev, seed=meta.seed + 1000 * r) for r in range(rotate)]
    outs = [torch.empty_like(s.q) for s in sets]
    wsb = pkv.paged_attention_workspace_bytes(len(meta.context_lens), cfg.num_heads, cfg.head_dim,
                                              cfg.max_blocks, cfg.block_size, part)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def write(i):
        s = sets[i % rotate]
        pkv.paged_kv_write(s.k_new, s.v_new, s.slot_mapping, s.k_cache, s.v_cache)

    def decode(i):
        s = sets[i % rotate]
        pkv.paged_attention_decode(s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens, cfg.scale,
                                   out=outs[i % rotate], workspace=ws, partition_size=part)

    def fused_step(i):
        s = sets[i % rotate]
        pkv.paged_attention_decode_step(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.block_tables,
                                        s.context_lens, cfg.scale, out=outs[i % rotate], workspace=ws,
                                        partition_size=part)

    def two_call_step(i):
        write(i)
        decode(i)

    step = two_call_step if args.two_call_step else fused_step
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: whole steps, no per-step events (an event record between kernels adds several
    # microseconds of queue work); wall clock and a HIP event pair around it.  A step is the library's
    # decode step (paged_attention_decode_step: the newest tokens' append and the attention in one
    # launch), or with --two-call-step paged_kv_write + paged_attention_decode.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    step_ev_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    # the other form of the step, for comparison
    other = fused_step if args.two_call_step else two_call_step
    ev0.record()
    for i in range(args.steps):
        other(i)
    ev1.record()
    torch.cuda.synchronize()
    other_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

    # Timed region 2: the dominant kernel alone, launched back to back over the rotating inputs on the
    # stream the library launches on (torch's current stream); average launch duration from a HIP
    # event pair, the same quantity a rocprofv3 kernel trace averages.
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record()
    for i in range(args.steps):
        decode(i)
    ev3.record()
    torch.cuda.synchronize()
    decode_us = ev2.elapsed_time(ev3) * 1e3 / args.steps
    # Timed region 3: the write alone, likewise.
    ev2.record()
    for i in range(args.steps):
        write(i)
    ev3.record()
    torch.cuda.synchronize()
    write_us = ev2.elapsed_time(ev3) * 1e3 / args.steps
    # Timed region 4: the fused steps recorded once into a HIP graph (one step per input set, in rotation
    # order) and replayed: the step without the host's per-call work, which bounds the small configurations.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fused_step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(rotate):
            fused_step(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // rotate)
    ev2.record()
    for _ in range(reps):
        g.replay()
    ev3.record()
    torch.cuda.synchronize()
    graph_us = ev2.elapsed_time(ev3) * 1e3 / (reps * rotate)
    del g
    achieved = nbytes["decode"] / (decode_us * 1e-6) / 1e9
    log(f"step {step_s * 1e6:.1f} us (wall; {step_ev_us:.1f} us by events; "
        f"{'fused' if args.two_call_step else 'two-call'} step {other_us:.1f} us; fused step from a HIP graph "
        f"{graph_us:.1f} us), decode {decode_us:.1f} us, "
        f"write {write_us:.1f} us -> decode {achieved:.0f} GB/s = {achieved / PEAK_HBM_GBS:.1%} of peak")

    stream_ref = probe = None
    if not args.no_diagnostic:
        stream_ref = torch_stream_reference()
        log(f"plain PyTorch streaming on this GPU: {stream_ref}")
        probe = read_ceiling(meta, sets, resolved)
        probe["decode_call_frac_of_best"] = round(achieved / probe["best"]["GB_per_s"], 4)
        log(f"read probe on this GPU: {probe}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same workload ...")
        cpu = cpu_baseline(meta, sets[0])
        log(f"cpu oracle: {cpu}")

    traffic = measured_traffic(cfg.name, resolved) if args.placement == "shuffled" else None
    th = meta.total_tokens * cfg.num_heads
    rec = {
        "metric": METRIC,
        "value": round(nbytes["step"] / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "num_seqs": len(meta.context_lens),
            "num_heads": cfg.num_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "sum_context_tokens": meta.total_tokens,
            "pool_blocks": meta.num_blocks,
            "block_placement": args.placement,
            "partition_size": resolved,
            "partition_choice": "library (PKV_PARTITION_AUTO)" if part == pkv.PARTITION_AUTO else "caller",
            "step": ("paged_kv_write(one new token per sequence) + paged_attention_decode" if args.two_call_step
                     else "paged_attention_decode_step (append of one new token per sequence + attention, "
                          "one launch)"),
            "step_algorithmic_bytes": nbytes["step"],
        },
        "tokens_heads_per_s": round(th / step_s, 1),
        "fraction_of_peak": round(nbytes["step"] / step_s / 1e9 / PEAK_HBM_GBS, 4),
        "kernels_us": {"paged_kv_write": round(write_us, 2), "paged_attention_decode": round(decode_us, 2),
                       "step_by_events": round(step_ev_us, 2),
                       ("paged_attention_decode_step" if args.two_call_step else "two_call_step"): round(other_us, 2),
                       "fused_step_graph_replay": round(graph_us, 2)},
        "roofline": {
            "kernel": ("paged_attention_decode (decode_partition_kernel"
                       + (" + lse_reduce_kernel)" if resolved else ")")),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes_per_launch": nbytes["decode"],
            "mean_launch_us": round(decode_us, 2),
        },
        "diagnostic": None if args.no_diagnostic else {"read_probe": probe, "torch_streaming": stream_ref},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

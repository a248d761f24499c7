"""Decode-step benchmark on one MI355X: slot-mapping write + paged attention.

A step is one pass of the whole path over one batch: paged_kv_write of each
sequence's newest token into its cache slot, then paged_attention_decode of
one query per sequence over its paged K/V.  The default workload is the
LLaMA-2-13B-shaped single-layer batch (64 sequences, 40 heads, head_dim 128,
block 16, bf16, contexts uniform in [128, 2048], pool 1.25x the needed blocks
in a shuffled free list).  Inputs are resident in HBM before timing starts;
consecutive steps rotate over independent copies of the inputs (each larger
than the 256 MB Infinity Cache) so no step reads data the previous one left
in the caches.

Prints one JSON line:
  value          algorithmic GB/s of the whole step (write + decode bytes / step time)
  roofline       the decode call (the partition kernel, plus the LSE reduce when the
                 context is split), algorithmic bytes per launch / its mean duration from
                 HIP events on the launch stream, vs the 8 TB/s HBM peak
  cpu_baseline   the float64 CPU oracle on a bounded sample of the same workload
Timing: the K steps run back to back with no event between them (wall clock and one HIP event
pair bracket them); then the decode call alone and the write alone run K times back to back, each
bracketed by a HIP event pair, for the per-launch averages.
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


def cpu_baseline(meta, w, budget_s=10.0):
    """The oracle, untouched, on the same workload: whole steps (write, then decode of sequence after
    sequence) until about budget_s of CPU work; a step cut short counts only its finished sequences."""
    import numpy as np
    import resource

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
    nbytes, tokens, steps, seqs = 0, 0, 0, 0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        kc, vc = oracle.kv_write(kn, vn, meta.slot_mapping, k0, v0, cfg.block_size)
        for i in range(B):
            oracle.decode(q, kc, vc, meta.block_tables, meta.context_lens, cfg.scale, bs, cfg.dtype, seqs=[i])
            nbytes += int(per_seq[i])
            tokens += int(L[i]) * H
            seqs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        steps += 1
    wall = time.perf_counter() - t0
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"{seqs} sequence decodes over {steps} step(s) of the same {B}-sequence batch, each step "
                      f"starting with the oracle's write of the {B} new tokens (a whole-pool copy); "
                      f"{wall:.1f} s wall, {cpu:.1f} s CPU",
            "tokens_heads_per_s": round(tokens / wall, 1)}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-context partition in tokens (0 = one pass); default: the library's choice")
    ap.add_argument("--rotate", type=int, default=None, help="independent input copies cycled over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    if not os.path.exists(b.LIB_PATH):
        b.build()
    pkv.lib()

    dev = torch.device("cuda:0")
    meta = W.make_metadata(args.config)
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

    for i in range(args.warmup):
        write(i)
        decode(i)
    torch.cuda.synchronize()

    # Timed region 1: whole steps (write + decode), no per-step events (an event record between
    # kernels adds several microseconds of queue work); wall clock and a HIP event pair around it.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        write(i)
        decode(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    step_ev_us = ev0.elapsed_time(ev1) * 1e3 / args.steps

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
    achieved = nbytes["decode"] / (decode_us * 1e-6) / 1e9
    log(f"step {step_s * 1e6:.1f} us (wall; {step_ev_us:.1f} us by events), decode {decode_us:.1f} us, "
        f"write {write_us:.1f} us -> decode {achieved:.0f} GB/s = {achieved / PEAK_HBM_GBS:.1%} of peak")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same workload ...")
        cpu = cpu_baseline(meta, sets[0])
        log(f"cpu oracle: {cpu}")

    traffic = measured_traffic(cfg.name, resolved)
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
            "partition_size": resolved,
            "partition_choice": "library (PKV_PARTITION_AUTO)" if part == pkv.PARTITION_AUTO else "caller",
            "step": "paged_kv_write(one new token per sequence) + paged_attention_decode",
            "step_algorithmic_bytes": nbytes["step"],
        },
        "tokens_heads_per_s": round(th / step_s, 1),
        "fraction_of_peak": round(nbytes["step"] / step_s / 1e9 / PEAK_HBM_GBS, 4),
        "kernels_us": {"paged_kv_write": round(write_us, 2), "paged_attention_decode": round(decode_us, 2),
                       "step_by_events": round(step_ev_us, 2)},
        "roofline": {
            "kernel": "paged_attention_decode (decode_partition_kernel" + (" + lse_reduce_kernel)" if resolved else ")"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes_per_launch": nbytes["decode"],
            "mean_launch_us": round(decode_us, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""The oracle over a whole batch, its sequences shared out to a pool of threads.

Each worker calls the oracle unchanged (oracle.decode or oracle.decode_split)
on its own list of sequences; NumPy releases the GIL inside the oracle's array
operations, so the workers run on separate cores.  Only how many sequences run
at once changes, never what is computed for each.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

MAX_WORKERS = 16          # one GPU's share of the host's cores


def workers() -> int:
    """Threads to use: the cores this process may run on, at most MAX_WORKERS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


def chunks_by_length(lens, n_chunks):
    """Sequence indices dealt round-robin, longest first, into n_chunks lists of similar total length."""
    order = np.argsort(-np.asarray(lens, dtype=np.int64), kind="stable")
    out = [order[i::n_chunks].tolist() for i in range(n_chunks)]
    return [c for c in out if c]


def decode_all(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype, partition_size=None,
               n_workers=None):
    """float64 [B, H, D]: oracle.decode (or oracle.decode_split with partition_size) for every sequence."""
    nw = n_workers or workers()
    B = len(context_lens)
    parts = chunks_by_length(context_lens, min(B, 4 * nw))

    def run(seqs):
        if partition_size:
            return seqs, oracle.decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                                             dtype, partition_size, seqs=seqs)
        return seqs, oracle.decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype,
                                   seqs=seqs)

    out = None
    with ThreadPoolExecutor(nw) as ex:
        for seqs, r in ex.map(run, parts):
            if out is None:
                out = np.zeros_like(r)
            out[seqs] = r[seqs]
    return out

"""Plain float64 CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py import this module.  The GPU library never imports, links or
calls it, and it shares no code, header, table or helper with the GPU path.

Sources (web pages on vLLM's PagedAttention):
  [card]    "PagedAttention", llm-engineer.pages.dev (sections "OS paging과 같은
            발상", "Kernel은 무엇이 달라지는가", "vLLM에서의 위치")
  [explain] "vLLM KV cache and PagedAttention explained", hrletsgo.me (Steps 5-9,
            "Why Waste Stays Below 4%", Appendix: The Attention Score Formula)
  [velog]   "vLLM의 PagedAttention 아키텍처와 GPU 메모리 최적화 원리", velog.io
            (section 4, the 4-D tensor layout)

What is computed.  PagedAttention changes where the KV cache lives, not the
attention formula ([card], opening paragraph; [explain], Appendix).  So each
function below is the plain definition written out:
  * the cache is a pool of fixed-size blocks laid out [Block, Head, Block_Size,
    Head_D] ([velog] section 4); K and V are two such pools;
  * a sequence's block table maps logical block j (tokens j*bs .. j*bs+bs-1) to
    a physical block id ([card] "OS paging과 같은 발상"; [explain] Step 5);
  * a sequence of L tokens holds ceil(L / bs) blocks ([explain] Step 6, the
    block-allocation line; "Why Waste Stays Below 4%");
  * a flat slot id is block * bs + offset ("slot 6 of block 42", [explain]
    Steps 6 and 7; the flat encoding is this library's reading);
  * Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V ([explain] Appendix), with
    the scale passed explicitly;
  * the split-context variant evaluates the same softmax per partition and
    merges partitions by their log-sum-exp, which is exact algebra (the pages
    only name FlashDecoding, [card] "헷갈리기 쉬운 구분").

All floating-point work is float64 on values upcast exactly from storage
(bf16 arrives as uint16 bit patterns).  Every function here is pinned by
tests/test_oracle_pins.py against brute force, closed forms, invariants and the
pages' worked examples.
"""
from __future__ import annotations

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


def to_float64(storage, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements.

    bf16 is the upper 16 bits of an IEEE binary32, so its value is the binary32
    whose bits are (pattern << 16); fp16 and fp32 upcast exactly by definition.
    """
    a = np.asarray(storage)
    if dtype == F32:
        return a.astype(np.float32, copy=False).astype(np.float64)
    if dtype == F16:
        return a.view(np.float16).astype(np.float64)
    if dtype == BF16:
        bits = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks held by a sequence of ``num_tokens`` tokens: ceil(n / bs).

    [explain] Step 6 (6 tokens -> 1 block) and "Why Waste Stays Below 4%"
    (32 tokens -> 2 full blocks, 17 tokens -> 2 blocks).
    """
    return -(-int(num_tokens) // int(block_size))


def slot_to_block_offset(slot: int, block_size: int):
    """Flat slot id -> (physical block, offset in block); slot = block * bs + offset."""
    return slot // block_size, slot % block_size


def kv_write(k, v, slot_mapping, k_cache, v_cache, block_size: int):
    """Store token t's K/V rows at its slot; returns new cache arrays.

    k, v: [T, H, D] storage; caches: [NB, H, bs, D] storage; slot_mapping: [T]
    int.  A negative slot means "no write" (padding).  The copy is bitwise:
    it moves stored elements, never values.  ([card] "vLLM에서의 위치": the
    worker hands the slot mapping to the kernel; [explain] Step 6: the new
    token's K/V goes to its slot of the sequence's block.)
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = slot_to_block_offset(int(slot), block_size)
        k_out[b, :, o, :] = k[t]
        v_out[b, :, o, :] = v[t]
    return k_out, v_out


def newest_token_slots(block_tables, context_lens, block_size: int) -> np.ndarray:
    """Flat slot of each sequence's newest token (position L - 1), or -1 for an empty row.

    This is where a decode step writes the token it adds ([explain] Step 6:
    the decode token's K/V goes to the next slot of the sequence's block, a
    new block once the previous one is full): logical block (L - 1) // bs,
    offset (L - 1) % bs, through the block table.
    """
    out = np.full(len(context_lens), -1, dtype=np.int64)
    for i, L in enumerate(np.asarray(context_lens).tolist()):
        if L > 0:
            b = int(block_tables[i][(L - 1) // block_size])
            out[i] = b * block_size + (L - 1) % block_size
    return out


def gather_sequence(cache, table_row, num_tokens: int, block_size: int, dtype: str) -> np.ndarray:
    """Logical float64 [H, L, D] K (or V) of one sequence, read through its table.

    Logical token t lives in physical block table_row[t // bs] at offset
    t % bs ([card] "OS paging과 같은 발상"; [velog] section 4 layout).  Only the
    first ceil(L / bs) table entries are read.
    """
    nb = blocks_needed(num_tokens, block_size)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = to_float64(np.asarray(cache)[ids], dtype)          # [nb, H, bs, D]
    H, D = blocks.shape[1], blocks.shape[3]
    logical = blocks.transpose(1, 0, 2, 3).reshape(H, nb * block_size, D)
    return logical[:, :num_tokens, :]


def attend(q, K, V, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for every head: q [H, D], K, V [H, L, D] -> [H, D].

    [explain] Appendix: scores are the query's dot products with every cached
    key, divided by sqrt(d) (here: times ``scale``), normalised by softmax, and
    used to weight the values.  The max is subtracted before exp (same value in
    exact arithmetic, no overflow in float64).
    """
    s = np.einsum("hd,htd->ht", q, K) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return np.einsum("ht,htd->hd", p, V) / p.sum(axis=1)[:, None]


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, block_size: int,
           dtype: str, seqs=None) -> np.ndarray:
    """One decode step: every sequence's query attends over its first L cached tokens.

    q: [B, H, D] storage; caches [NB, H, bs, D] storage; block_tables [B, M] int;
    context_lens [B] int.  Returns float64 [B, H, D]; rows with L == 0 are zero
    and rows not listed in ``seqs`` (when given) are left zero.
    """
    q64 = to_float64(q, dtype)
    B, H, D = q64.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    for i in (range(B) if seqs is None else seqs):
        L = int(context_lens[i])
        if L == 0:
            continue
        K = gather_sequence(k_cache, block_tables[i], L, block_size, dtype)
        V = gather_sequence(v_cache, block_tables[i], L, block_size, dtype)
        out[i] = attend(q64[i], K, V, scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, query_start, context_lens, scale: float, block_size: int,
            dtype: str) -> np.ndarray:
    """Causal attention of a batch of new tokens over their sequences' paged caches.

    Sequence i brings the queries q[query_start[i] : query_start[i+1]] (P_i of
    them) and holds L_i = context_lens[i] cached tokens, the last P_i of which
    are these new tokens' own K/V (written before the call), so query j sits
    at position p = L_i - P_i + j.  It attends to cached tokens 0 .. p and
    never to a later one: the prefill phase processes all prompt tokens in
    parallel ([explain] Step 6) with causal attention, each token seeing only
    the tokens before it and itself ([explain] Summary: causal attention).  A
    non-empty prefix L_i - P_i > 0 is a cached (e.g. shared) prompt prefix
    ([explain] Step 9) or an earlier chunk.  Returns float64 [T, H, D].
    """
    q64 = to_float64(q, dtype)
    T, H, D = q64.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    qs = np.asarray(query_start).tolist()
    for i in range(len(qs) - 1):
        a, b = qs[i], qs[i + 1]
        L = int(context_lens[i])
        if b == a:
            continue
        K = gather_sequence(k_cache, block_tables[i], L, block_size, dtype)        # [H, L, D]
        V = gather_sequence(v_cache, block_tables[i], L, block_size, dtype)
        first = L - (b - a)                                                         # position of query 0
        for j in range(b - a):
            p = first + j
            out[a + j] = attend(q64[a + j], K[:, :p + 1], V[:, :p + 1], scale)
    return out


def partition_state(q, K, V, scale: float):
    """(m, l, acc) of one context partition, per head.

    m = max score, l = sum exp(s - m), acc = sum exp(s - m) * V.  Then
    softmax(s) V over the union of partitions p equals
    sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p with M = max_p m_p.
    """
    s = np.einsum("hd,htd->ht", q, K) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), np.einsum("ht,htd->hd", p, V)


def lse_merge(states) -> np.ndarray:
    """Merge partition states (m_p, l_p, acc_p) by their log-sum-exp weights."""
    M = np.max(np.stack([m for m, _, _ in states]), axis=0)                   # [H]
    num = sum(np.exp(m - M)[:, None] * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den[:, None]


def decode_split(q, k_cache, v_cache, block_tables, context_lens, scale: float, block_size: int,
                 dtype: str, partition_size: int, seqs=None) -> np.ndarray:
    """The decode step evaluated per partition of ``partition_size`` tokens, then merged.

    Partition p of a sequence covers tokens [p * P, min((p + 1) * P, L)), so a
    sequence has ceil(L / P) non-empty partitions.
    """
    q64 = to_float64(q, dtype)
    B, H, D = q64.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    for i in (range(B) if seqs is None else seqs):
        L = int(context_lens[i])
        if L == 0:
            continue
        K = gather_sequence(k_cache, block_tables[i], L, block_size, dtype)
        V = gather_sequence(v_cache, block_tables[i], L, block_size, dtype)
        states = [partition_state(q64[i], K[:, a:a + partition_size], V[:, a:a + partition_size], scale)
                  for a in range(0, L, partition_size)]
        out[i] = lse_merge(states)
    return out

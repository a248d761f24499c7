"""The CPU oracle against its pins, and the pins against planted mistakes.

Every pin in oracle_pins.PINS must pass on the oracle as committed.  Then each
plausible mistake below is planted in a copy of one oracle function (on the
CPU, by monkeypatching the oracle module) and at least one pin must fail.
"""
import numpy as np
import pytest

import oracle.oracle as O
import oracle_pins as P


@pytest.mark.parametrize("pin", P.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


# ------------------------------------------------------------- planted mistakes

def _floor_blocks(n, bs):
    return int(n) // int(bs)


def _gather_no_transpose(cache, table_row, num_tokens, block_size, dtype):
    nb = O.blocks_needed(num_tokens, block_size)
    blocks = O.to_float64(np.asarray(cache)[np.asarray(table_row[:nb])], dtype)
    H, D = blocks.shape[1], blocks.shape[3]
    return blocks.reshape(H, nb * block_size, D)[:, :num_tokens, :]


def _gather_shifted_table(cache, table_row, num_tokens, block_size, dtype):
    nb = O.blocks_needed(num_tokens, block_size)
    row = np.asarray(table_row)
    ids = np.concatenate([row[1:nb + 1], row[:1]])[:nb]
    blocks = O.to_float64(np.asarray(cache)[ids], dtype)
    H, D = blocks.shape[1], blocks.shape[3]
    return blocks.transpose(1, 0, 2, 3).reshape(H, nb * block_size, D)[:, :num_tokens, :]


def _attend_no_scale(q, K, V, scale):
    s = np.einsum("hd,htd->ht", q, K)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return np.einsum("ht,htd->hd", p, V) / p.sum(axis=1)[:, None]


def _attend_neg_exp(q, K, V, scale):
    s = np.einsum("hd,htd->ht", q, K) * scale
    p = np.exp(-(s - s.max(axis=1, keepdims=True)))
    return np.einsum("ht,htd->hd", p, V) / p.sum(axis=1)[:, None]


def _attend_unnormalised(q, K, V, scale):
    s = np.einsum("hd,htd->ht", q, K) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return np.einsum("ht,htd->hd", p, V)


def _attend_swapped_kv(q, K, V, scale):
    return O.__dict__["_orig_attend"](q, V, K, scale)


def _upcast_wrong_shift(storage, dtype):
    if dtype == "bf16":
        bits = np.asarray(storage).view(np.uint16).astype(np.uint32) << np.uint32(8)
        return bits.view(np.float32).astype(np.float64)
    return O.__dict__["_orig_to_float64"](storage, dtype)


def _slot_swapped(slot, bs):
    return slot % bs, slot // bs


def _merge_unweighted(states):
    num = sum(acc for _, _, acc in states)
    den = sum(l for _, l, _ in states)
    return num / den[:, None]


def _merge_wrong_sign(states):
    M = np.max(np.stack([m for m, _, _ in states]), axis=0)
    num = sum(np.exp(M - m)[:, None] * acc for m, _, acc in states)
    den = sum(np.exp(M - m) * l for m, l, _ in states)
    return num / den[:, None]


def _state_no_scale(q, K, V, scale):
    return O.__dict__["_orig_partition_state"](q, K, V, 1.0)


def _decode_skip_last(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype, seqs=None):
    B = np.asarray(q).shape[0]
    return O.__dict__["_orig_decode"](q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                                      dtype, seqs=range(B - 1) if seqs is None else seqs)


def _decode_short_context(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype, seqs=None):
    lens = np.maximum(np.asarray(context_lens) - 1, 1)
    return O.__dict__["_orig_decode"](q, k_cache, v_cache, block_tables, lens, scale, block_size, dtype,
                                      seqs=seqs)


def _write_skips_token0(k, v, slot_mapping, k_cache, v_cache, block_size):
    sm = np.array(slot_mapping, copy=True)
    sm[0] = -1
    return O.__dict__["_orig_kv_write"](k, v, sm, k_cache, v_cache, block_size)


def _write_swaps_kv(k, v, slot_mapping, k_cache, v_cache, block_size):
    return O.__dict__["_orig_kv_write"](v, k, slot_mapping, k_cache, v_cache, block_size)


def _write_ignores_padding(k, v, slot_mapping, k_cache, v_cache, block_size):
    # forgets that a negative slot means "no write" (Python's negative indexing then hits the last block)
    k_out, v_out = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        b, o = slot // block_size, slot % block_size
        k_out[b, :, o, :] = k[t]
        v_out[b, :, o, :] = v[t]
    return k_out, v_out


def _slots_oldest_token(block_tables, context_lens, block_size):
    lens = np.where(np.asarray(context_lens) > 0, np.minimum(np.asarray(context_lens), 2), 0)
    return O.__dict__["_orig_newest_token_slots"](block_tables, lens, block_size)


def _slots_position_l(block_tables, context_lens, block_size):
    out = np.full(len(context_lens), -1, dtype=np.int64)
    for i, L in enumerate(np.asarray(context_lens).tolist()):
        if L > 0:
            out[i] = int(block_tables[i][L // block_size]) * block_size + L % block_size
    return out


def _prefill_core(q, k_cache, v_cache, block_tables, query_start, context_lens, scale, block_size, dtype, keys):
    q64 = O.to_float64(q, dtype)
    out = np.zeros(q64.shape, dtype=np.float64)
    qs = np.asarray(query_start).tolist()
    for i in range(len(qs) - 1):
        a, b = qs[i], qs[i + 1]
        L = int(context_lens[i])
        if b == a:
            continue
        K = O.gather_sequence(k_cache, block_tables[i], L, block_size, dtype)
        V = O.gather_sequence(v_cache, block_tables[i], L, block_size, dtype)
        for j in range(b - a):
            n = keys(L, b - a, j)
            out[a + j] = O.attend(q64[a + j], K[:, :n], V[:, :n], scale)
    return out


def _prefill_not_causal(*a):
    return _prefill_core(*a, keys=lambda L, n, j: L)


def _prefill_excludes_self(*a):
    return _prefill_core(*a, keys=lambda L, n, j: max(L - n + j, 1))


def _prefill_ignores_prefix(*a):
    return _prefill_core(*a, keys=lambda L, n, j: j + 1)


MUTANTS = {
    "prefill attends to later tokens": ("prefill", _prefill_not_causal),
    "prefill query does not see itself": ("prefill", _prefill_excludes_self),
    "prefill ignores the cached prefix": ("prefill", _prefill_ignores_prefix),
    "newest slot taken at position 1": ("newest_token_slots", _slots_oldest_token),
    "newest slot taken at position L": ("newest_token_slots", _slots_position_l),
    "blocks_needed floors": ("blocks_needed", _floor_blocks),
    "gather drops the head transpose": ("gather_sequence", _gather_no_transpose),
    "gather reads the next table entry": ("gather_sequence", _gather_shifted_table),
    "attend drops the scale": ("attend", _attend_no_scale),
    "attend negates the exponent": ("attend", _attend_neg_exp),
    "attend skips the normalisation": ("attend", _attend_unnormalised),
    "attend swaps K and V": ("attend", _attend_swapped_kv),
    "bf16 upcast shifts by 8": ("to_float64", _upcast_wrong_shift),
    "slot decoding swaps block and offset": ("slot_to_block_offset", _slot_swapped),
    "merge forgets the LSE weights": ("lse_merge", _merge_unweighted),
    "merge weights with the wrong sign": ("lse_merge", _merge_wrong_sign),
    "partition state drops the scale": ("partition_state", _state_no_scale),
    "decode skips the last sequence": ("decode", _decode_skip_last),
    "decode reads one token too few": ("decode", _decode_short_context),
    "write drops a token": ("kv_write", _write_skips_token0),
    "write swaps K and V": ("kv_write", _write_swaps_kv),
    "write ignores negative-slot padding": ("kv_write", _write_ignores_padding),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setitem(O.__dict__, "_orig_" + attr, getattr(O, attr))
    monkeypatch.setattr(O, attr, bad)
    failed = []
    for pin in P.PINS:
        try:
            pin(O)
        except Exception:          # an assertion, or the mistake breaking the computation outright
            failed.append(pin.__name__)
    assert failed, f"no pin catches: {name}"


# ------------------------------------------------------------- block pool: pins and planted mistakes

import oracle.block_manager as BM


@pytest.mark.parametrize("pin", P.POOL_PINS, ids=lambda f: f.__name__)
def test_pool_pin(pin):
    pin(BM, O)


def _orig(name):
    return BM.__dict__["_orig_" + name]


def _append_no_cow(self, seq, n):
    bs, table = self.block_size, self.tables[seq]
    slots = []
    for t in range(self.tokens[seq], self.tokens[seq] + int(n)):
        j, off = divmod(t, bs)
        if j == len(table):
            table.append(self._take())
        slots.append(table[j] * bs + off)
    self.tokens[seq] += int(n)
    return slots, []


def _append_cow_keeps_count(self, seq, n):
    rc = self.refcount
    before = list(rc)
    slots, copies = _orig("append_slots")(self, seq, n)
    for s, _ in copies:
        rc[s] = before[s]                 # forgets that the writer no longer references the source
    return slots, copies


def _append_reversed_copies(self, seq, n):
    slots, copies = _orig("append_slots")(self, seq, n)
    return slots, [(d, s) for s, d in copies]


def _append_late_block(self, seq, n):
    bs, table = self.block_size, self.tables[seq]
    slots, copies = [], []
    for t in range(self.tokens[seq], self.tokens[seq] + int(n)):
        j, off = divmod(t, bs)
        if j == len(table) and off > 0:   # waits one token too long before adding a block
            table.append(self._take())
        jj = min(j, len(table) - 1)
        slots.append(table[jj] * bs + off)
    self.tokens[seq] += int(n)
    return slots, copies


def _append_offset_off_by_one(self, seq, n):
    slots, copies = _orig("append_slots")(self, seq, n)
    return [s + 1 for s in slots], copies


def _free_keeps_blocks(self, seq):
    for b in self.tables.pop(seq):
        self.refcount[b] -= 1
    del self.tokens[seq]
    return []


def _free_to_back(self, seq):
    released = []
    for b in self.tables.pop(seq):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            released.append(b)
    del self.tokens[seq]
    self.free.extend(released)
    return released


def _free_ignores_sharing(self, seq):
    released = list(self.tables.pop(seq))
    for b in released:
        self.refcount[b] = 0
    del self.tokens[seq]
    self.free[:0] = released
    return released


def _fork_no_refcount(self, parent, child):
    self.tables[child] = list(self.tables[parent])
    self.tokens[child] = self.tokens[parent]


def _allocate_floor(self, seq, num_tokens):
    need = max(1, int(num_tokens) // self.block_size)
    if need > len(self.free):
        raise BM.OutOfBlocks("")
    self.tables[seq] = [self._take() for _ in range(need)]
    self.tokens[seq] = int(num_tokens)
    return list(self.tables[seq])


def _copy_k_only(k_cache, v_cache, copies):
    k2, _ = _orig("copy_blocks")(k_cache, v_cache, copies)
    return k2, np.array(v_cache, copy=True)


def _copy_backwards(k_cache, v_cache, copies):
    return _orig("copy_blocks")(k_cache, v_cache, [(d, s) for s, d in copies]) if copies else \
        (np.array(k_cache, copy=True), np.array(v_cache, copy=True))


def _usage_counts_holders(pool):
    u = _orig("usage")(pool)
    bs = pool.block_size
    u["stored_tokens"] = sum(min(bs, pool.tokens[s] - j * bs) for s, t in pool.tables.items() for j in range(len(t)))
    return u


def _usage_counts_free_blocks(pool):
    u = _orig("usage")(pool)
    u["allocated_slots"] = pool.num_blocks * pool.block_size
    return u


def _waste_from_logical(u):
    return 1.0 - u["logical_tokens"] / u["allocated_slots"] if u["allocated_slots"] else 0.0


POOL_MUTANTS = {
    "usage counts a shared block once per holder": ("usage", _usage_counts_holders),
    "usage counts free blocks as allocated": ("usage", _usage_counts_free_blocks),
    "paged waste from logical tokens": ("paged_waste", _waste_from_logical),
    "append never copies a shared block": ("BlockPool.append_slots", _append_no_cow),
    "copy-on-write keeps the source's count": ("BlockPool.append_slots", _append_cow_keeps_count),
    "copy pairs reversed": ("BlockPool.append_slots", _append_reversed_copies),
    "new block one token late": ("BlockPool.append_slots", _append_late_block),
    "slot offset off by one": ("BlockPool.append_slots", _append_offset_off_by_one),
    "free never returns blocks": ("BlockPool.free_sequence", _free_keeps_blocks),
    "free returns blocks to the back": ("BlockPool.free_sequence", _free_to_back),
    "free ignores other holders": ("BlockPool.free_sequence", _free_ignores_sharing),
    "fork does not count references": ("BlockPool.fork", _fork_no_refcount),
    "allocate floors the block count": ("BlockPool.allocate", _allocate_floor),
    "copy_blocks copies K only": ("copy_blocks", _copy_k_only),
    "copy_blocks copies backwards": ("copy_blocks", _copy_backwards),
}


@pytest.mark.parametrize("name", sorted(POOL_MUTANTS))
def test_pool_planted_mistake_is_caught(name, monkeypatch):
    where, bad = POOL_MUTANTS[name]
    if where.startswith("BlockPool."):
        attr = where.split(".")[1]
        monkeypatch.setitem(BM.__dict__, "_orig_" + attr, getattr(BM.BlockPool, attr))
        monkeypatch.setattr(BM.BlockPool, attr, bad)
    else:
        monkeypatch.setitem(BM.__dict__, "_orig_" + where, getattr(BM, where))
        monkeypatch.setattr(BM, where, bad)
    failed = []
    for pin in P.POOL_PINS:
        try:
            pin(BM, O)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches: {name}"

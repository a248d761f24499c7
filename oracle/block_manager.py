"""Plain CPU model of the block pool: on-demand allocation, reference counts,
copy-on-write, freeing, and the block copy that copy-on-write asks for.

TEST INFRASTRUCTURE, like the rest of oracle/: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg use it.  It shares no
code with the library's C++ block manager or its HIP copy kernel.

Sources (web pages on vLLM's PagedAttention):
  [card]    "PagedAttention", llm-engineer.pages.dev ("OS paging과 같은 발상":
            a new block is appended to the block table when the cache grows;
            "무엇이 좋아지는가": allocation on demand, waste limited to the last
            block's empty slots)
  [explain] "vLLM KV cache and PagedAttention explained", hrletsgo.me (Step 5:
            any free block can be assigned; Step 6: ceil(n / 16) blocks at
            prefill, a new block when the cache crosses a block boundary;
            Step 7: a finished request's blocks go back to the pool and are
            immediately reusable; Step 8: a finished request's space is given
            to the next request; Step 9: shared prefix blocks carry a reference
            count, and a write into a shared block first copies it into a new
            block that only the writer's table points to)

Readings where the pages leave a step open:
  * Sharing is per block.  A sequence's token t lives in logical block
    t // block_size, so a sequence that shares a partially filled block and
    appends a token writes into that shared block, which triggers the copy.
  * A block is copied only while another table still points to it (reference
    count > 1); the last holder writes in place.
  * The free list is an ordered list.  Allocation takes blocks from its front;
    a block whose count drops to zero goes back to the front, and blocks freed
    together keep their table order, so the next request is handed exactly the
    blocks just released ([explain] Steps 7 and 8: the freed space is the
    space the next request gets).
"""
from __future__ import annotations

import numpy as np


class OutOfBlocks(Exception):
    """The pool has too few free blocks for the request."""


class BlockPool:
    """Block tables of live sequences over a pool of ``num_blocks`` physical blocks."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(self.num_blocks)), "free_order must list every block once"
        self.free = order                      # front of the list = next block handed out
        self.refcount = [0] * self.num_blocks
        self.tables = {}                       # sequence id -> list of physical block ids
        self.tokens = {}                       # sequence id -> number of tokens held

    # -- helpers
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.pop(0)
        self.refcount[b] = 1
        return b

    def _blocks_for(self, n: int) -> int:
        return -(-int(n) // self.block_size)

    # -- operations
    def allocate(self, seq, num_tokens: int):
        """A new sequence holding ``num_tokens`` tokens in ceil(n / bs) fresh blocks."""
        assert seq not in self.tables
        need = self._blocks_for(num_tokens)
        if need > len(self.free):
            raise OutOfBlocks(f"{need} blocks needed, {len(self.free)} free")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.tokens[seq] = int(num_tokens)
        return list(self.tables[seq])

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent``'s table; every shared block gains a reference."""
        assert child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = self.tokens[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def append_slots(self, seq, n: int):
        """Reserve slots for ``n`` new tokens of ``seq``.

        Returns (slots, copies): the flat slot (block * bs + offset) of each
        new token, and the (source, destination) block copies that must run
        before anything is written to those slots.  Raises OutOfBlocks, with
        nothing changed, when the free list cannot supply the new blocks.
        """
        bs = self.block_size
        table = self.tables[seq]
        have = self.tokens[seq]
        need = self._blocks_for(have + int(n)) - len(table)
        if have % bs and self.refcount[table[-1]] > 1 and n > 0:
            need += 1                                # the partly filled last block is shared
        if need > len(self.free):                    # all or nothing: nothing changes on failure
            raise OutOfBlocks(f"{need} blocks needed, {len(self.free)} free")
        slots, copies = [], []
        for t in range(have, have + int(n)):
            j, off = divmod(t, bs)
            if j == len(table):                      # the cache crossed a block boundary
                table.append(self._take())
            elif self.refcount[table[j]] > 1:        # a write into a shared block: copy it first
                src = table[j]
                dst = self._take()
                self.refcount[src] -= 1
                table[j] = dst
                copies.append((src, dst))
            slots.append(table[j] * bs + off)
        self.tokens[seq] += int(n)
        return slots, copies

    def free_sequence(self, seq):
        """Drop ``seq``; blocks no other table references return to the front of the free list."""
        released = []
        for b in self.tables.pop(seq):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                released.append(b)
        del self.tokens[seq]
        self.free[:0] = released
        return released

    # -- views
    def table(self, seq):
        return list(self.tables[seq])

    def num_free(self) -> int:
        return len(self.free)

    def padded_tables(self, seqs, width: int):
        """int32 [len(seqs), width] block tables (padding -1) and int32 context lengths."""
        t = np.full((len(seqs), width), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            row = self.tables[s]
            t[i, :len(row)] = row
            lens[i] = self.tokens[s]
        return t, lens


def usage(pool: BlockPool) -> dict:
    """Slot accounting of a pool (the pages' waste comparison, [explain] "Why Waste Stays Below 4%"
    and the Korean step-6 calculation).

    used_blocks      blocks held by at least one table
    allocated_slots  used_blocks * block_size
    stored_tokens    slots that hold a token: each used block counts the
                     filled slots of its fullest holder, once however many
                     tables share it
    logical_tokens   sum of the sequences' lengths (a shared token counts once
                     per sequence that reads it)
    """
    bs = pool.block_size
    fill = {}
    for seq, table in pool.tables.items():
        n = pool.tokens[seq]
        for j, b in enumerate(table):
            fill[b] = max(fill.get(b, 0), min(bs, n - j * bs))
    return {"num_blocks": pool.num_blocks, "free_blocks": len(pool.free), "used_blocks": len(fill),
            "sequences": len(pool.tables), "logical_tokens": sum(pool.tokens.values()),
            "stored_tokens": sum(fill.values()), "allocated_slots": len(fill) * bs,
            "shared_blocks": sum(1 for b in fill if pool.refcount[b] > 1)}


def paged_waste(u: dict) -> float:
    """Fraction of the allocated slots that hold no token (empty tail slots)."""
    return 1.0 - u["stored_tokens"] / u["allocated_slots"] if u["allocated_slots"] else 0.0


def static_waste(u: dict, max_model_len: int) -> float:
    """Fraction wasted if every sequence had reserved max_model_len contiguous slots instead."""
    reserved = u["sequences"] * int(max_model_len)
    return 1.0 - u["logical_tokens"] / reserved if reserved else 0.0


def copy_blocks(k_cache, v_cache, copies):
    """New cache arrays with block ``dst`` holding what block ``src`` held, for each (src, dst).

    Every head and slot of the block is copied, K and V alike (a physical
    block is the unit of sharing).  Destinations are distinct and none is a
    source, so the order of the copies does not matter.
    """
    dsts = [d for _, d in copies]
    assert len(set(dsts)) == len(dsts) and not set(dsts) & {s for s, _ in copies}
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for s, d in copies:
        k_out[d] = k_cache[s]
        v_out[d] = v_cache[s]
    return k_out, v_out

"""A continuous-batching decode loop over the library's C ABI.

"vLLM KV cache and PagedAttention explained" (hrletsgo.me), Steps 6-8: a
request's prompt K/V fills ceil(n / 16) blocks at prefill; each decode step
adds one token per running request, opening a new block at each block
boundary; a request that ends returns its blocks, and its place in the batch
goes to the next request at once.  Step 9: requests that share a prompt share
its blocks, and a write into a shared block copies it first.

Per step the host side is the library's C++ block pool and batch planner
(pkv_batch_plan_step): it reserves each running row's new slot, copying a
shared last block when needed, and lists the device block-table entries that
changed.  The plan goes to the GPU in one asynchronous copy from pinned memory,
then the kernels run in stream order: the prompt writes of newly admitted
requests (paged_kv_write), paged_kv_prepare_step (table updates, context
lengths and the slot mapping, on the device), paged_kv_copy_blocks, and
paged_attention_decode_step (the new tokens' append and the attention, one
launch).  Nothing waits
for the GPU unless the host runs two steps ahead of it.  This module only
marshals: which request comes next is the caller's choice.
"""
from __future__ import annotations

import numpy as np

from . import (BlockPool, Batch, paged_attention_decode_step, paged_kv_copy_blocks, paged_kv_prepare_step,
               paged_kv_write)


class DecodeLoop:
    """Rows of a decode batch over one K/V cache pair.

    k_cache, v_cache: device [num_blocks, num_heads, block_size, head_dim].
    rows: batch rows; width: block-table width (blocks a sequence may hold).
    """

    def __init__(self, k_cache, v_cache, rows: int, width: int, free_order=None, scale=None):
        import torch
        from . import paged_attention_workspace_bytes
        self.k_cache, self.v_cache = k_cache, v_cache
        NB, H, bs, D = k_cache.shape
        self.num_blocks, self.block_size = NB, bs
        self.scale = 1.0 / float(np.sqrt(D)) if scale is None else float(scale)
        self.rows, self.width = int(rows), int(width)
        self.pool = BlockPool(NB, bs, free_order)
        self.batch = Batch(self.pool, self.rows, self.width)
        dev = k_cache.device
        self.device = dev
        self.tables = torch.full((self.rows, self.width), -1, dtype=torch.int32, device=dev)
        self.lens = torch.zeros(self.rows, dtype=torch.int32, device=dev)
        self.slots = torch.full((self.rows,), -1, dtype=torch.int64, device=dev)
        self.row_seq = [-1] * self.rows
        self._pending = []                 # (host slots, k, v) prompt writes for the next step
        self._stage_host = [None, None]
        self._stage_dev = [None, None]
        self._stage_done = [None, None]
        self._step = 0
        self.last_copies = np.zeros((0, 2), dtype=np.int64)
        ws = paged_attention_workspace_bytes(self.rows, H, D, self.width, bs)
        self.workspace = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)

    # -- requests
    def admit(self, row: int, seq: int, k_prompt, v_prompt):
        """Start request ``seq`` in idle ``row`` with a prompt whose K/V are k_prompt, v_prompt
        (device [P, H, D]); the prompt is written at the next step, before its decode."""
        assert self.row_seq[row] < 0, "row is busy"
        P = int(k_prompt.shape[0])
        self.pool.allocate(seq, P)
        self._pending.append((self.pool.slots(seq, 0, P), k_prompt, v_prompt))
        self.batch.set_row(row, seq)
        self.row_seq[row] = seq

    def fork(self, row: int, parent: int, seq: int):
        """Start ``seq`` in idle ``row`` sharing every block of running sequence ``parent``."""
        assert self.row_seq[row] < 0, "row is busy"
        self.pool.fork(parent, seq)
        self.batch.set_row(row, seq)
        self.row_seq[row] = seq

    def release(self, row: int):
        """The request in ``row`` ended: the row goes idle and its blocks return to the pool."""
        seq = self.row_seq[row]
        self.batch.set_row(row, -1)
        self.pool.free_sequence(seq)
        self.row_seq[row] = -1

    # -- the step
    def _stage(self, n_words: int):
        import torch
        i = self._step % 2
        if self._stage_done[i] is not None:
            self._stage_done[i].synchronize()          # the copy that last used this buffer has run
        if self._stage_host[i] is None or self._stage_host[i].numel() < n_words:
            n = max(n_words, 2 * (self._stage_host[i].numel() if self._stage_host[i] is not None else 4096))
            self._stage_host[i] = torch.empty(n, dtype=torch.int32).pin_memory()
            self._stage_dev[i] = torch.empty(n, dtype=torch.int32, device=self.device)
        return i

    def step(self, q, k_new, v_new, out=None):
        """One decode step: every running row appends one token (K/V rows k_new[r], v_new[r]) and its
        query q[r] attends over the row's cache.  q, k_new, v_new: device [rows, H, D]; idle rows'
        inputs are ignored and their outputs are zero.  Returns out [rows, H, D]."""
        import torch
        updates, lens, copies = self.batch.plan_step(1)
        prompt = [p[0] for p in self._pending]
        n_prompt = sum(len(s) for s in prompt)
        # staging layout (int32 words): lens | updates | copies (int64) | prompt slots (int64)
        o_upd = self.rows
        o_cp = o_upd + 3 * len(updates)
        o_cp += o_cp % 2
        o_pr = o_cp + 4 * len(copies)
        total = o_pr + 2 * n_prompt
        i = self._stage(total)
        h = self._stage_host[i].numpy()
        h[:self.rows] = lens
        h[o_upd:o_upd + 3 * len(updates)] = updates.ravel()
        h[o_cp:o_pr].view(np.int64)[:] = copies.ravel()
        if n_prompt:
            h[o_pr:total].view(np.int64)[:] = np.concatenate(prompt)
        d = self._stage_dev[i]
        d[:total].copy_(self._stage_host[i][:total], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._stage_done[i] = ev
        pos = o_pr
        for slots, k, v in self._pending:
            n = len(slots)
            paged_kv_write(k, v, d[pos:pos + 2 * n].view(torch.int64), self.k_cache, self.v_cache)
            pos += 2 * n
        self._pending = []
        paged_kv_prepare_step(self.tables, self.lens, d[o_upd:o_upd + 3 * len(updates)].view(-1, 3),
                              d[:self.rows], self.slots, self.block_size, self.num_blocks)
        if len(copies):
            paged_kv_copy_blocks(self.k_cache, self.v_cache, d[o_cp:o_pr].view(torch.int64).view(-1, 2))
        out = paged_attention_decode_step(q, k_new, v_new, self.k_cache, self.v_cache, self.tables, self.lens,
                                          self.scale, out=out, workspace=self.workspace)
        self.last_copies = copies.copy()
        self.last_lens = lens.copy()
        self.last_prompt_tokens = n_prompt
        self._step += 1
        return out

"""Seeded synthetic inputs for the paged KV-cache decode path.

This module builds inputs and nothing else: context lengths, a physical block
pool with a shuffled free list, per-sequence block tables, the slot id of each
sequence's newest token, and random q / K / V values.  It stands in for the
scheduler and GPU worker of the pages' serving stack ("PagedAttention" card,
section on vLLM's layers: the scheduler decides which blocks a request gets,
the worker prepares block tables and the slot mapping as device tensors).

It performs no attention arithmetic and no cache write: the K/V of the newest
token of every sequence is returned separately (``k_new``/``v_new``) and its
cache slot is left poisoned, so a decode over ``context_lens`` is only right
after a ``paged_kv_write`` of those tokens.  Both the CPU oracle and the GPU
library consume what this module returns; neither is imported here.

Reading of a decode step used throughout: ``context_lens[i]`` is the length
*after* this step's write, so the step writes token ``L_i - 1`` and then the
new query attends over tokens ``0 .. L_i - 1`` (itself included).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"
SEED_BASE = 383000


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    num_seqs: int
    num_heads: int
    head_dim: int
    block_size: int
    dtype: str              # storage and arithmetic-input type of q, K, V, out
    value_std: float        # q, K, V ~ N(0, value_std^2)
    max_context: int        # table capacity in tokens (max_blocks_per_seq * block_size)
    partition_size: int     # split-context partition, tokens

    @property
    def max_blocks(self) -> int:
        return self.max_context // self.block_size

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    1: Config(1, "tiny_4seq_ctx6-100_h4_d64_f32", 4, 4, 64, 16, F32, 1.0, 112, 512),
    2: Config(2, "llama2_13b_layer_b64_h40_d128_ctx128-2048_bf16", 64, 40, 128, 16, BF16, 1.0, 2048, 512),
    3: Config(3, "long_ctx_b8_ctx32768_h40_d128_bf16", 8, 40, 128, 16, BF16, 1.0, 32768, 512),
    4: Config(4, "cont_batch_b256_lognormal_h32_d128_bf16", 256, 32, 128, 16, BF16, 1.0, 8192, 512),
    5: Config(5, "large_batch_b512_ctx16-4096_h16_d128_bs32_f16", 512, 16, 128, 32, F16, 0.5, 4096, 512),
}

# owner codes in Metadata.owner
FREE = -1
FOREIGN = -2    # pre-occupied by requests outside this batch (config 4)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Metadata:
    cfg: Config
    context_lens: np.ndarray     # int32 [B]
    block_tables: np.ndarray     # int32 [B, max_blocks], unused entries -1
    num_blocks: int
    slot_mapping: np.ndarray     # int64 [B]: flat slot (block * block_size + offset) of token L_i - 1
    owner: np.ndarray            # int32 [num_blocks]: sequence index, FREE or FOREIGN
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    @property
    def blocks_in_tables(self) -> int:
        return int((self.block_tables >= 0).sum())


def _draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.cfg_id == 1:
        return np.array([6, 50, 8, 100], dtype=np.int64)
    if cfg.cfg_id == 2:
        return rng.integers(128, 2048 + 1, cfg.num_seqs)
    if cfg.cfg_id == 3:
        return np.full(cfg.num_seqs, 32768, dtype=np.int64)
    if cfg.cfg_id == 4:
        x = np.exp(rng.normal(math.log(512.0), 1.0, cfg.num_seqs))
        return np.clip(np.rint(x), 8, 8192).astype(np.int64)
    if cfg.cfg_id == 5:
        return rng.integers(16, 4096 + 1, cfg.num_seqs)
    raise ValueError(cfg.cfg_id)


def _pool_and_free_list(cfg: Config, needed: int, rng: np.random.Generator):
    """Pool size, shuffled free list and the set of blocks held by other requests."""
    foreign = np.zeros(0, dtype=np.int64)
    if cfg.cfg_id == 1:
        nb = 64
        free = rng.permutation(nb)
    elif cfg.cfg_id == 2:
        nb = ceil_div(5 * needed, 4)
        free = rng.permutation(nb)
    elif cfg.cfg_id == 3:
        nb = needed
        free = rng.permutation(nb)
    elif cfg.cfg_id == 4:
        nb = ceil_div(125 * needed, 70)          # 1.25x headroom after 30 % is taken
        foreign = rng.choice(nb, size=int(round(0.3 * nb)), replace=False)
        mask = np.ones(nb, dtype=bool)
        mask[foreign] = False
        free = rng.permutation(np.nonzero(mask)[0])
    elif cfg.cfg_id == 5:
        nb = ceil_div(11 * needed, 10)
        free = rng.permutation(nb)
    else:
        raise ValueError(cfg.cfg_id)
    return nb, free, foreign


PLACEMENTS = ("shuffled", "consecutive")


def make_metadata(cfg: Config | int, lens: np.ndarray | None = None, seed: int | None = None,
                  placement: str = "shuffled") -> Metadata:
    """Context lengths, pool, tables and newest-token slots for one decode step.

    Tables take block ids from the shuffled free list in batch order, one id per
    ``block_size`` tokens (the pages' on-demand allocation: a sequence holds
    exactly ceil(L / block_size) blocks).  ``lens`` overrides the drawn lengths
    (the pool is then sized by the same per-config rule).  ``placement =
    "consecutive"`` sorts the free list instead, so each sequence holds a run of
    consecutive block ids (same lengths, pool and bytes; the random draws are
    the same, so only the placement differs).
    """
    if placement not in PLACEMENTS:
        raise ValueError(f"placement must be one of {PLACEMENTS}")
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    seed = SEED_BASE + cfg.cfg_id if seed is None else seed
    rng = np.random.default_rng(seed)
    drawn = _draw_lengths(cfg, rng)
    L = drawn if lens is None else np.asarray(lens, dtype=np.int64)
    if (L < 1).any() or (L > cfg.max_context).any():
        raise ValueError("context lengths must lie in [1, max_context]")
    bs = cfg.block_size
    nblk = (L + bs - 1) // bs
    needed = int(nblk.sum())
    nb, free, foreign = _pool_and_free_list(cfg, needed, rng)
    if placement == "consecutive":
        free = np.sort(free)
    if len(free) < needed:
        raise ValueError("pool too small for the requested lengths")
    B = len(L)
    tables = np.full((B, cfg.max_blocks), -1, dtype=np.int32)
    owner = np.full(nb, FREE, dtype=np.int32)
    owner[foreign] = FOREIGN
    pos = 0
    for i in range(B):
        ids = free[pos:pos + nblk[i]]
        pos += nblk[i]
        tables[i, :nblk[i]] = ids
        owner[ids] = i
    last = L - 1
    slots = tables[np.arange(B), last // bs].astype(np.int64) * bs + last % bs
    return Metadata(cfg, L.astype(np.int32), tables, nb, slots, owner, seed)


@dataclass
class Workload:
    meta: Metadata
    q: "object"            # torch tensors below, on the requested device
    k_cache: "object"
    v_cache: "object"
    k_new: "object"
    v_new: "object"
    block_tables: "object"
    context_lens: "object"
    slot_mapping: "object"
    extras: dict = field(default_factory=dict)


def torch_dtype(dtype: str):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]


def _randn_into(dst, gen, std: float, chunk_rows: int):
    import torch
    n = dst.shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        x = torch.randn((e - s,) + tuple(dst.shape[1:]), generator=gen, device=dst.device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        dst[s:e].copy_(x)          # round-to-nearest-even into the storage dtype


def kv_pool(num_blocks: int, num_heads: int, block_size: int, head_dim: int, dtype, device, zero: bool = False):
    """The K and V caches of one layer as the two halves of a single tensor [2, NB, H, bs, D], the way a serving
    engine allocates a layer's cache; each half is a contiguous [NB, H, bs, D] cache.  On MI355X the decode
    reads the K and V tiles of a block at the same time, and with V right after K in one allocation it measured
    0.6-3 % faster than with two separate allocations at every configuration here (their relative placement
    decides which HBM channels the two streams share)."""
    import torch
    make = torch.zeros if zero else torch.empty
    pool = make((2, num_blocks, num_heads, block_size, head_dim), dtype=dtype, device=device)
    return pool[0], pool[1]


def make_workload(meta: Metadata, device="cpu", poison: bool = True, seed: int | None = None) -> Workload:
    """Random q, caches and newest-token K/V for ``meta`` (torch, on ``device``).

    Values are N(0, value_std^2) drawn in fp32 by torch's generator on
    ``device`` and rounded to the storage dtype.  With ``poison``, every slot
    that no decode may read holds NaN: blocks owned by nobody, and in each
    sequence's last block the newest token's slot and the empty slots after it.
    Blocks held by other requests (config 4) keep random data.
    """
    import torch
    cfg = meta.cfg
    dev = torch.device(device)
    dt = torch_dtype(cfg.dtype)
    B, H, D, bs, NB = len(meta.context_lens), cfg.num_heads, cfg.head_dim, cfg.block_size, meta.num_blocks
    gen = torch.Generator(device=dev)
    gen.manual_seed(meta.seed if seed is None else seed)
    q = torch.empty((B, H, D), dtype=dt, device=dev)
    k_cache, v_cache = kv_pool(NB, H, bs, D, dt, dev)
    k_new = torch.empty((B, H, D), dtype=dt, device=dev)
    v_new = torch.empty_like(k_new)
    rows = max(1, (1 << 26) // (H * bs * D))
    _randn_into(q, gen, cfg.value_std, B)
    _randn_into(k_cache, gen, cfg.value_std, rows)
    _randn_into(v_cache, gen, cfg.value_std, rows)
    _randn_into(k_new, gen, cfg.value_std, B)
    _randn_into(v_new, gen, cfg.value_std, B)
    if poison:
        poison_unreadable(meta, k_cache, v_cache)
    tables = torch.from_numpy(meta.block_tables).to(dev)
    lens = torch.from_numpy(meta.context_lens).to(dev)
    slots = torch.from_numpy(meta.slot_mapping).to(dev)
    return Workload(meta, q, k_cache, v_cache, k_new, v_new, tables, lens, slots)


def unreadable_slots(meta: Metadata):
    """(block ids, offsets) of the newest-token slot and the empty slots after it."""
    bs = meta.cfg.block_size
    L = meta.context_lens.astype(np.int64)
    B = len(L)
    last_blk = meta.block_tables[np.arange(B), (L - 1) // bs].astype(np.int64)
    first = (L - 1) % bs
    blocks, offs = [], []
    for i in range(B):
        o = np.arange(first[i], bs)
        blocks.append(np.full(len(o), last_blk[i]))
        offs.append(o)
    return np.concatenate(blocks), np.concatenate(offs)


def poison_unreadable(meta: Metadata, k_cache, v_cache):
    import torch
    dev = k_cache.device
    free_ids = torch.from_numpy(np.nonzero(meta.owner == FREE)[0]).to(dev)
    b, o = unreadable_slots(meta)
    b = torch.from_numpy(b).to(dev)
    o = torch.from_numpy(o).to(dev)
    for c in (k_cache, v_cache):
        if free_ids.numel():
            c.index_fill_(0, free_ids, float("nan"))
        c[b, :, o, :] = float("nan")


def storage_numpy(t):
    """Host NumPy copy of a torch tensor's stored bits (bf16 as uint16 patterns)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---------------------------------------------------------------- parallel sampling over shared prompts

@dataclass(frozen=True)
class SamplingConfig:
    """Parallel sampling ("vLLM KV cache and PagedAttention explained", Step 9): each prompt's
    blocks are shared by ``samples`` sequences, at the LLaMA-2-13B layer shape."""
    name: str = "parallel_sampling_16x4_llama2_13b_layer_ctx128-2048_bf16"
    prompts: int = 16
    samples: int = 4
    num_heads: int = 40
    head_dim: int = 128
    block_size: int = 16
    dtype: str = BF16
    min_len: int = 128
    max_len: int = 2048
    seed: int = SEED_BASE + 100

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def sampling_prompts(cfg: SamplingConfig, seed: int | None = None):
    """Prompt lengths, pool size (1.25x the prompts' blocks plus one block per sample for copies and
    growth) and a shuffled free order."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = rng.integers(cfg.min_len, cfg.max_len + 1, cfg.prompts)
    needed = int(((lens + cfg.block_size - 1) // cfg.block_size).sum())
    nb = ceil_div(5 * needed, 4) + cfg.prompts * cfg.samples
    return lens.astype(np.int64), nb, rng.permutation(nb).astype(np.int32)


# ---------------------------------------------------------------- continuous batching request stream

@dataclass(frozen=True)
class BatchingConfig:
    """A continuous-batching decode loop ("vLLM KV cache and PagedAttention explained", Step 8) over
    256 batch rows at the continuous-batching configuration's shape (32 heads, head_dim 128, 16-token
    blocks, bf16): prompts lognormal around 512 tokens (clipped to [8, 4096]), each request generating
    a uniform [16, 512] number of tokens; a finished request's row takes the next request at once."""
    name: str = "continuous_batching_256rows_h32_d128_bf16_prompt_lognormal512_gen16-512"
    rows: int = 256
    num_heads: int = 32
    head_dim: int = 128
    block_size: int = 16
    dtype: str = BF16
    prompt_median: float = 512.0
    prompt_sigma: float = 1.0
    prompt_min: int = 8
    prompt_max: int = 4096
    gen_min: int = 16
    gen_max: int = 512
    seed: int = SEED_BASE + 200

    @property
    def width(self) -> int:
        return ceil_div(self.prompt_max + self.gen_max, self.block_size)


def batching_requests(cfg: BatchingConfig, n: int, seed: int | None = None):
    """Prompt and generation lengths of ``n`` requests, in arrival order."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    prompts = np.clip(np.rint(np.exp(rng.normal(math.log(cfg.prompt_median), cfg.prompt_sigma, n))),
                      cfg.prompt_min, cfg.prompt_max).astype(np.int64)
    gens = rng.integers(cfg.gen_min, cfg.gen_max + 1, n).astype(np.int64)
    return prompts, gens


# ---------------------------------------------------------------- prefill

@dataclass(frozen=True)
class PrefillConfig:
    """Prefill ("vLLM KV cache and PagedAttention explained", Step 6) of 16 prompts of U[128, 2048]
    tokens at the LLaMA-2-13B layer shape: 40 heads, head_dim 128, 16-token blocks, bf16."""
    name: str = "prefill_16_prompts_llama2_13b_layer_len128-2048_bf16"
    prompts: int = 16
    num_heads: int = 40
    head_dim: int = 128
    block_size: int = 16
    dtype: str = BF16
    min_len: int = 128
    max_len: int = 2048
    seed: int = SEED_BASE + 300

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def prefill_prompts(cfg: PrefillConfig, seed: int | None = None):
    """Prompt lengths, pool size (1.25x the blocks needed), a shuffled free order."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = rng.integers(cfg.min_len, cfg.max_len + 1, cfg.prompts).astype(np.int64)
    needed = int(((lens + cfg.block_size - 1) // cfg.block_size).sum())
    nb = ceil_div(5 * needed, 4)
    return lens, nb, rng.permutation(nb).astype(np.int32)

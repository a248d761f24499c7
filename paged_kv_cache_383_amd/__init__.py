"""Paged KV-cache decode for AMD MI355X (gfx950): Python binding of the C ABI.

The functions below only marshal arguments: they check torch tensors'
device, dtype, shape and contiguity, then pass raw device pointers, sizes and
torch's current HIP stream to libpagedkv.so (include/pagedkv.h).  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is not built, every call raises.

    paged_kv_write(k, v, slot_mapping, k_cache, v_cache)
    paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                           out=None, workspace=None, partition_size=PARTITION_AUTO)
    paged_attention_workspace_bytes(num_seqs, num_heads, head_dim,
                                    max_blocks_per_seq, block_size, partition_size)
    paged_attention_partition_size(num_seqs, num_heads, max_blocks_per_seq, block_size,
                                   partition_size)

partition_size: tokens per split-context partition, 0 for one pass per
sequence, or PARTITION_AUTO (the default) to let the library choose.
"""
from __future__ import annotations

import ctypes
import os

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EWORKSPACE", 4: "PKV_EHIP"}
PARTITION_AUTO = -1            # let the library choose the split-context partition
DEFAULT_PARTITION = PARTITION_AUTO

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpagedkv.so")
_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python paged_kv_cache_383_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.paged_kv_write.argtypes = [vp, vp, vp, i64, vp, vp, i64, i32, i32, i32, i32, vp]
        L.paged_kv_write.restype = ctypes.c_int
        L.paged_attention_partition_size.argtypes = [i32, i32, i32, i32, i32]
        L.paged_attention_partition_size.restype = i32
        L.paged_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.paged_attention_workspace_bytes.restype = sz
        L.paged_attention_decode.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i64,
                                             ctypes.c_float, i32, vp, vp, sz, i32, vp]
        L.paged_attention_decode.restype = ctypes.c_int
        L.pkv_last_error.argtypes = []
        L.pkv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pkv_last_error().decode()


def _check(status: int):
    if status != PKV_OK:
        raise PagedKVError(status, last_error())


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _device_tensor(name, t, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def paged_kv_write(k, v, slot_mapping, k_cache, v_cache):
    """k_cache[s // bs, :, s % bs] = k[t] (and v) for every t with s = slot_mapping[t] >= 0."""
    import torch
    for n, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        _device_tensor(n, t, k_cache.dtype)
    _device_tensor("slot_mapping", slot_mapping, torch.int64, 1)
    if k.dim() != 3 or k.shape != v.shape or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k, v must be [T, H, D] and caches [NB, H, bs, D]")
    NB, H, bs, D = k_cache.shape
    if k.shape[1:] != (H, D) or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("k/v/slot_mapping shapes do not match the cache")
    with torch.cuda.device(k_cache.device):
        _check(lib().paged_kv_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k.shape[0],
                                    k_cache.data_ptr(), v_cache.data_ptr(), NB, H, D, bs,
                                    _dtype_code(k_cache), _stream(k_cache.device)))


def paged_attention_partition_size(num_seqs, num_heads, max_blocks_per_seq, block_size,
                                   partition_size=DEFAULT_PARTITION) -> int:
    """The partition size (tokens; 0 = no split) the decode call uses for these sizes."""
    return int(lib().paged_attention_partition_size(num_seqs, num_heads, max_blocks_per_seq, block_size,
                                                    partition_size))


def paged_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                                    partition_size=DEFAULT_PARTITION) -> int:
    return int(lib().paged_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                                     block_size, partition_size))


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
                           workspace=None, partition_size=DEFAULT_PARTITION):
    """softmax(scale * q K^T) V per (sequence, head), K/V read through block_tables."""
    import torch
    _device_tensor("q", q, k_cache.dtype, 3)
    _device_tensor("k_cache", k_cache, None, 4)
    _device_tensor("v_cache", v_cache, k_cache.dtype, 4)
    _device_tensor("block_tables", block_tables, torch.int32, 2)
    _device_tensor("context_lens", context_lens, torch.int32, 1)
    NB, H, bs, D = k_cache.shape
    B = q.shape[0]
    if v_cache.shape != k_cache.shape or q.shape[1:] != (H, D):
        raise ValueError("q [B, H, D] and caches [NB, H, bs, D] do not match")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor("out", out, q.dtype, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    M = block_tables.shape[1]
    need = paged_attention_workspace_bytes(B, H, D, M, bs, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _device_tensor("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _check(lib().paged_attention_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                            block_tables.data_ptr(), M, context_lens.data_ptr(), B, H, D,
                                            bs, NB, float(scale), _dtype_code(q), out.data_ptr(),
                                            workspace.data_ptr(), ws_bytes, partition_size,
                                            _stream(q.device)))
    return out

"""Paged attention over a block-structured KV cache on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libpa.so`` (C ABI in ``include/pa.h``).  The functions carry the
C names; they only marshal torch tensors (device memory) and the current HIP stream into
the C calls, and raise ``PaError`` on a non-OK status.  ``validate=True`` (every call) first
checks the contents of the index arrays on host copies (``validate.py``: slots, block-table
entries, lengths), raising ``ValueError`` before any launch; it synchronises with the device.  Every step of the computation runs
in the library's HIP kernels; there is no fallback path: if ``libpa.so`` has not been built
or cannot be loaded, every call raises.

Cache tensor: ``kv_cache[2, num_blocks, block_size, num_kv_heads, head_size]`` (bf16 or
float32, contiguous); plane 0 keys, plane 1 values.  Index tensors are int32.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

from . import validate as _v

__all__ = [
    "PaError", "lib_path", "load", "pa_store_kv", "pa_copy_blocks", "pa_prefill_varlen",
    "pa_decode", "pa_decode_workspace_size", "pa_prefill_varlen_with_store", "pa_decode_with_store",
    "pa_cascade_decode", "pa_cascade_decode_workspace_size", "pa_decode_no_alloc",
    "pa_cascade_prefill_varlen", "pa_cascade_prefill_varlen_workspace_size",
    "DECODE_NO_ALLOC_SCRATCH_BYTES",
]

# pa_decode_no_alloc's per-GPU scratch (PA_DECODE_NO_ALLOC_SCRATCH_BYTES in pa.h)
DECODE_NO_ALLOC_SCRATCH_BYTES = 32 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpa.so"
_lib = None

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
# an FP8 cache holds float8_e4m3fn codes of value / kv_scale; its queries, keys, values and
# outputs are bfloat16
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3}


class PaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({_status_text(status)}): {detail}")


class _CacheDesc(ctypes.Structure):
    _fields_ = [
        ("kv_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("kv_scale", ctypes.c_float),
    ]


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load ``libpa.so`` (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_attention_block_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(_CacheDesc)
    lib.pa_store_kv.argtypes = [D, P, P, P, I32, P]
    lib.pa_copy_blocks.argtypes = [D, P, I32, P]
    lib.pa_prefill_varlen.argtypes = [D, P, P, P, I32, P, P, I32, I32, I32, I32, F32, I32, P, P]
    lib.pa_decode_workspace_size.argtypes = [D, I32, I32, I32, I32, I32]
    lib.pa_decode_workspace_size.restype = SZ
    lib.pa_decode.argtypes = [D, P, P, P, I32, P, I32, I32, I32, F32, I32, P, I32, P, SZ, P]
    lib.pa_prefill_varlen_with_store.argtypes = [D, P, P, P, P, P, I32, P, I32, P, P, I32, I32, I32, I32,
                                                 F32, I32, P, P]
    lib.pa_decode_with_store.argtypes = [D, P, P, P, P, P, P, I32, P, I32, I32, I32, F32, I32, P, I32, P, SZ, P]
    lib.pa_cascade_decode_workspace_size.argtypes = [D, I32, I32, I32, I32, I32]
    lib.pa_cascade_decode_workspace_size.restype = SZ
    lib.pa_cascade_decode.argtypes = [D, P, P, P, I32, P, I32, I32, I32, F32, I32, I32, P, SZ, P]
    lib.pa_decode_no_alloc.argtypes = [D, P, P, P, I32, P, I32, I32, I32, F32, I32, P, I32, P]
    lib.pa_cascade_prefill_varlen_workspace_size.argtypes = [D, I32, I32, I32]
    lib.pa_cascade_prefill_varlen_workspace_size.restype = SZ
    lib.pa_cascade_prefill_varlen.argtypes = [D, P, P, P, I32, P, P, I32, I32, I32, I32, F32, I32, I32, P, SZ, P]
    for name in ("pa_store_kv", "pa_copy_blocks", "pa_prefill_varlen", "pa_decode",
                 "pa_prefill_varlen_with_store", "pa_decode_with_store", "pa_cascade_decode",
                 "pa_decode_no_alloc", "pa_cascade_prefill_varlen"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load().pa_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library itself is unavailable
        return "?"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where, load().pa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> Optional[int]:
    return torch.cuda.current_stream(t.device).cuda_stream


def _alibi(slopes: Optional[torch.Tensor], query: torch.Tensor, dev) -> Optional[int]:
    """Device pointer of optional ALiBi slopes (float32 [num_heads], contiguous)."""
    if slopes is None:
        return None
    _need(slopes, "alibi_slopes", torch.float32, dev, 1)
    if slopes.shape[0] != query.shape[1]:
        raise ValueError(f"alibi_slopes must be [{query.shape[1]}]")
    return _ptr(slopes)


def _act(kv_cache: torch.Tensor) -> torch.dtype:
    """dtype of the queries, keys, values and outputs that go with this cache."""
    return torch.bfloat16 if kv_cache.dtype == torch.float8_e4m3fn else kv_cache.dtype


def _desc(kv_cache: torch.Tensor, kv_scale: float = 1.0) -> _CacheDesc:
    if kv_cache.dim() != 5 or kv_cache.shape[0] != 2:
        raise ValueError(f"kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_size], got {tuple(kv_cache.shape)}")
    if kv_cache.dtype not in _DTYPES:
        raise ValueError(f"kv_cache dtype {kv_cache.dtype} not supported")
    if not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be contiguous")
    _, nb, bs, hkv, d = kv_cache.shape
    return _CacheDesc(kv_cache.data_ptr(), nb, bs, hkv, d, _DTYPES[kv_cache.dtype], float(kv_scale))


def _need(t: torch.Tensor, name: str, dtype, device, dims: Optional[int] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {t.dim()}")


def pa_store_kv(key: torch.Tensor, value: torch.Tensor, kv_cache: torch.Tensor,
                slot_mapping: torch.Tensor, kv_scale: float = 1.0, validate: bool = False) -> None:
    """Scatter ``key``/``value`` ``[T, Hkv, D]`` into ``kv_cache`` at ``slot_mapping`` (-1 skips);
    an FP8 cache stores e4m3(x / kv_scale)."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    _need(key, "key", _act(kv_cache), dev, 3)
    _need(value, "value", _act(kv_cache), dev, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, dev, 1)
    if key.shape != value.shape or key.shape[1:] != kv_cache.shape[3:] or key.shape[0] != slot_mapping.shape[0]:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_size] matching slot_mapping and the cache")
    if validate:
        _v.check_store(slot_mapping, kv_cache.shape[1], kv_cache.shape[2])
    _check(lib.pa_store_kv(ctypes.byref(desc), _ptr(key), _ptr(value), _ptr(slot_mapping),
                           key.shape[0], _stream(kv_cache)), "pa_store_kv")


def pa_copy_blocks(kv_cache: torch.Tensor, block_pairs: torch.Tensor, validate: bool = False) -> None:
    """``kv_cache[:, dst] = kv_cache[:, src]`` for each row ``(src, dst)`` of ``block_pairs``."""
    lib = load()
    desc = _desc(kv_cache)
    _need(block_pairs, "block_pairs", torch.int32, kv_cache.device, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    if validate:
        _v.check_copy_blocks(block_pairs, kv_cache.shape[1])
    _check(lib.pa_copy_blocks(ctypes.byref(desc), _ptr(block_pairs), block_pairs.shape[0],
                              _stream(kv_cache)), "pa_copy_blocks")


def pa_prefill_varlen(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                      cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                      max_seqlen_k: int, scale: float, num_kv_heads: int, sliding_window: int = 0,
                      out: Optional[torch.Tensor] = None,
                      alibi_slopes: Optional[torch.Tensor] = None, kv_scale: float = 1.0,
                      validate: bool = False) -> torch.Tensor:
    """Varlen causal attention of packed ``query [Tq, H, D]`` over the cached keys
    (``alibi_slopes``: optional float32 ``[H]`` ALiBi slopes on the cache's device;
    ``kv_scale``: the scale of an FP8 cache)."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev, 1)
    num_seqs = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != num_seqs + 1 or block_table.shape[0] < num_seqs:
        raise ValueError("cu_seqlens_q/k must be [num_seqs + 1] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    if validate:
        _v.check_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q, max_seqlen_k, sliding_window,
                         kv_cache.shape[1], kv_cache.shape[2], query.shape[0])
    _check(lib.pa_prefill_varlen(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(block_table),
                                 block_table.shape[1], _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                 num_seqs, int(max_seqlen_q), int(max_seqlen_k), query.shape[1],
                                 float(scale), int(sliding_window), _alibi(alibi_slopes, query, dev),
                                 _stream(kv_cache)),
           "pa_prefill_varlen")
    return out


def pa_decode_workspace_size(kv_cache: torch.Tensor, num_seqs: int, num_heads: int, max_seq_len: int,
                             sliding_window: int = 0, partition_size: int = 0) -> int:
    """Workspace bytes ``pa_decode`` needs; asked on the cache's device (the automatic
    split depends on how many workgroups that device holds at once)."""
    lib = load()
    desc = _desc(kv_cache)
    if kv_cache.is_cuda:
        with torch.cuda.device(kv_cache.device):
            return int(lib.pa_decode_workspace_size(ctypes.byref(desc), num_seqs, num_heads,
                                                    max_seq_len, sliding_window, partition_size))
    return int(lib.pa_decode_workspace_size(ctypes.byref(desc), num_seqs, num_heads, max_seq_len,
                                            sliding_window, partition_size))


def pa_decode(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
              seq_lens: torch.Tensor, max_seq_len: int, scale: float, num_kv_heads: int,
              sliding_window: int = 0, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
              alibi_slopes: Optional[torch.Tensor] = None, kv_scale: float = 1.0,
              validate: bool = False) -> torch.Tensor:
    """One query per sequence (``query [B, H, D]``) over its ``seq_lens[s]`` cached keys.

    ``workspace`` is a device byte buffer of at least ``pa_decode_workspace_size(...)``
    bytes; when None one is allocated through torch for this call.  ``kv_scale``: the scale
    of an FP8 cache (ignored otherwise).
    """
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    num_seqs = query.shape[0]
    if seq_lens.shape[0] != num_seqs or block_table.shape[0] < num_seqs:
        raise ValueError("seq_lens must be [num_seqs] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    need = pa_decode_workspace_size(kv_cache, num_seqs, query.shape[1], int(max_seq_len),
                                    int(sliding_window), int(partition_size))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.device != dev:
        raise ValueError("workspace must be on the cache's device")
    with (torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()):
        if validate:
            _v.check_decode(seq_lens, block_table, int(max_seq_len), int(sliding_window), kv_cache.shape[1],
                            kv_cache.shape[2])
        _check(lib.pa_decode(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(block_table),
                             block_table.shape[1], _ptr(seq_lens), num_seqs, int(max_seq_len),
                             query.shape[1], float(scale), int(sliding_window),
                             _alibi(alibi_slopes, query, dev), int(partition_size),
                             _ptr(workspace), ws_bytes, _stream(kv_cache)), "pa_decode")
    return out


def pa_decode_no_alloc(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                       seq_lens: torch.Tensor, max_seq_len: int, scale: float, num_kv_heads: int,
                       sliding_window: int = 0, out: Optional[torch.Tensor] = None, partition_size: int = 0,
                       alibi_slopes: Optional[torch.Tensor] = None, kv_scale: float = 1.0,
                       validate: bool = False) -> torch.Tensor:
    """``pa_decode`` without a workspace: the library's per-GPU scratch holds the split's
    partial states, so the call allocates nothing when ``out`` is given (calls on one GPU
    must not overlap).  Raises ``PaError`` (workspace status) when the split needs more
    than ``DECODE_NO_ALLOC_SCRATCH_BYTES``."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    num_seqs = query.shape[0]
    if seq_lens.shape[0] != num_seqs or block_table.shape[0] < num_seqs:
        raise ValueError("seq_lens must be [num_seqs] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    with (torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()):
        if validate:
            _v.check_decode(seq_lens, block_table, int(max_seq_len), int(sliding_window), kv_cache.shape[1],
                            kv_cache.shape[2])
        _check(lib.pa_decode_no_alloc(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(block_table),
                                      block_table.shape[1], _ptr(seq_lens), num_seqs, int(max_seq_len),
                                      query.shape[1], float(scale), int(sliding_window),
                                      _alibi(alibi_slopes, query, dev), int(partition_size), _stream(kv_cache)),
               "pa_decode_no_alloc")
    return out


def pa_cascade_decode_workspace_size(kv_cache: torch.Tensor, num_seqs: int, num_heads: int,
                                     max_seq_len: int, common_prefix_len: int,
                                     partition_size: int = 0) -> int:
    """Workspace bytes ``pa_cascade_decode`` needs, asked on the cache's device."""
    lib = load()
    desc = _desc(kv_cache)
    with (torch.cuda.device(kv_cache.device) if kv_cache.is_cuda else contextlib.nullcontext()):
        return int(lib.pa_cascade_decode_workspace_size(ctypes.byref(desc), num_seqs, num_heads, max_seq_len,
                                                        common_prefix_len, partition_size))


def pa_cascade_decode(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, scale: float, num_kv_heads: int,
                      common_prefix_len: int, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                      kv_scale: float = 1.0, validate: bool = False) -> torch.Tensor:
    """Decode of a batch whose block-table rows all start with the same
    ``common_prefix_len / block_size`` physical blocks: the shared prefix is attended once
    for every query, then each sequence's own keys (arguments otherwise as ``pa_decode``)."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    num_seqs = query.shape[0]
    if seq_lens.shape[0] != num_seqs or block_table.shape[0] < num_seqs:
        raise ValueError("seq_lens must be [num_seqs] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    need = pa_cascade_decode_workspace_size(kv_cache, num_seqs, query.shape[1], int(max_seq_len),
                                            int(common_prefix_len), int(partition_size))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.device != dev:
        raise ValueError("workspace must be on the cache's device")
    with (torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()):
        if validate:
            _v.check_cascade(seq_lens, block_table, int(max_seq_len), int(common_prefix_len), kv_cache.shape[1],
                             kv_cache.shape[2])
        _check(lib.pa_cascade_decode(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(block_table),
                                     block_table.shape[1], _ptr(seq_lens), num_seqs, int(max_seq_len),
                                     query.shape[1], float(scale), int(common_prefix_len),
                                     int(partition_size), _ptr(workspace), ws_bytes, _stream(kv_cache)),
               "pa_cascade_decode")
    return out


def pa_cascade_prefill_varlen_workspace_size(kv_cache: torch.Tensor, num_tokens: int, num_heads: int,
                                             common_prefix_len: int) -> int:
    """Workspace bytes ``pa_cascade_prefill_varlen`` needs for ``num_tokens`` packed query rows."""
    lib = load()
    desc = _desc(kv_cache)
    return int(lib.pa_cascade_prefill_varlen_workspace_size(ctypes.byref(desc), int(num_tokens), int(num_heads),
                                                            int(common_prefix_len)))


def pa_cascade_prefill_varlen(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                              cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                              max_seqlen_k: int, scale: float, num_kv_heads: int, common_prefix_len: int,
                              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              kv_scale: float = 1.0, validate: bool = False) -> torch.Tensor:
    """Varlen causal attention of packed ``query [Tq, H, D]`` whose sequences share their first
    ``common_prefix_len`` keys (block-table rows starting with the same blocks): the shared
    prefix is attended once for every query row, then each sequence's own keys (arguments
    otherwise as ``pa_prefill_varlen``; no window, no ALiBi)."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev, 1)
    num_seqs = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != num_seqs + 1 or block_table.shape[0] < num_seqs:
        raise ValueError("cu_seqlens_q/k must be [num_seqs + 1] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    num_tokens = query.shape[0]
    need = pa_cascade_prefill_varlen_workspace_size(kv_cache, num_tokens, query.shape[1], int(common_prefix_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.device != dev:
        raise ValueError("workspace must be on the cache's device")
    with (torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()):
        if validate:
            _v.check_cascade_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q, max_seqlen_k,
                                     int(common_prefix_len), kv_cache.shape[1], kv_cache.shape[2], num_tokens)
        _check(lib.pa_cascade_prefill_varlen(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(block_table),
                                             block_table.shape[1], _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                             num_seqs, int(max_seqlen_q), int(max_seqlen_k), query.shape[1],
                                             float(scale), int(common_prefix_len), num_tokens, _ptr(workspace),
                                             ws_bytes, _stream(kv_cache)),
               "pa_cascade_prefill_varlen")
    return out


def _new_rows(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
              rows: int) -> None:
    dev = kv_cache.device
    _need(key, "key", _act(kv_cache), dev, 3)
    _need(value, "value", _act(kv_cache), dev, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, dev, 1)
    want = (rows, kv_cache.shape[3], kv_cache.shape[4])
    if tuple(key.shape) != want or tuple(value.shape) != want or slot_mapping.shape[0] != rows:
        raise ValueError(f"key/value must be {want} and slot_mapping [{rows}]")


def pa_prefill_varlen_with_store(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                 slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                                 block_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                 cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                                 scale: float, num_kv_heads: int, sliding_window: int = 0,
                                 out: Optional[torch.Tensor] = None,
                                 alibi_slopes: Optional[torch.Tensor] = None,
                                 kv_scale: float = 1.0, validate: bool = False) -> torch.Tensor:
    """Store the batch's new tokens (``key``/``value [Tq, Hkv, D]`` at ``slot_mapping``) and run
    the varlen causal attention of ``query [Tq, H, D]`` in one call (one kernel for bf16)."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev, 1)
    _new_rows(key, value, slot_mapping, kv_cache, query.shape[0])
    num_seqs = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != num_seqs + 1 or block_table.shape[0] < num_seqs:
        raise ValueError("cu_seqlens_q/k must be [num_seqs + 1] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    if validate:
        _v.check_prefill_with_store(slot_mapping, cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q,
                                    max_seqlen_k, sliding_window, kv_cache.shape[1], kv_cache.shape[2],
                                    query.shape[0])
    _check(lib.pa_prefill_varlen_with_store(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(key), _ptr(value),
                                            _ptr(slot_mapping), query.shape[0], _ptr(block_table),
                                            block_table.shape[1], _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                            num_seqs, int(max_seqlen_q), int(max_seqlen_k), query.shape[1],
                                            float(scale), int(sliding_window), _alibi(alibi_slopes, query, dev),
                                            _stream(kv_cache)),
           "pa_prefill_varlen_with_store")
    return out


def pa_decode_with_store(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         slot_mapping: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, scale: float, num_kv_heads: int,
                         sliding_window: int = 0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                         alibi_slopes: Optional[torch.Tensor] = None, kv_scale: float = 1.0,
                         validate: bool = False) -> torch.Tensor:
    """Store each sequence's new token (``key``/``value [B, Hkv, D]`` at ``slot_mapping``) and
    decode ``query [B, H, D]`` over the ``seq_lens[s]`` keys that include it, in one call."""
    lib = load()
    desc = _desc(kv_cache, kv_scale)
    dev = kv_cache.device
    if num_kv_heads != kv_cache.shape[3]:
        raise ValueError(f"num_kv_heads {num_kv_heads} != cache's {kv_cache.shape[3]}")
    _need(query, "query", _act(kv_cache), dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    num_seqs = query.shape[0]
    _new_rows(key, value, slot_mapping, kv_cache, num_seqs)
    if seq_lens.shape[0] != num_seqs or block_table.shape[0] < num_seqs:
        raise ValueError("seq_lens must be [num_seqs] and block_table [num_seqs, max_blocks]")
    if query.shape[2] != kv_cache.shape[4]:
        raise ValueError("query head_size does not match the cache")
    if out is None:
        out = torch.empty_like(query)
    else:
        _need(out, "out", _act(kv_cache), dev, 3)
        if out.shape != query.shape:
            raise ValueError("out must match query's shape")
    need = pa_decode_workspace_size(kv_cache, num_seqs, query.shape[1], int(max_seq_len),
                                    int(sliding_window), int(partition_size))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None and workspace.device != dev:
        raise ValueError("workspace must be on the cache's device")
    with (torch.cuda.device(dev) if dev.type == "cuda" else contextlib.nullcontext()):
        if validate:
            _v.check_decode_with_store(slot_mapping, seq_lens, block_table, int(max_seq_len), int(sliding_window),
                                       kv_cache.shape[1], kv_cache.shape[2])
        _check(lib.pa_decode_with_store(ctypes.byref(desc), _ptr(out), _ptr(query), _ptr(key), _ptr(value),
                                        _ptr(slot_mapping), _ptr(block_table), block_table.shape[1],
                                        _ptr(seq_lens), num_seqs, int(max_seq_len), query.shape[1],
                                        float(scale), int(sliding_window), _alibi(alibi_slopes, query, dev),
                                        int(partition_size), _ptr(workspace), ws_bytes, _stream(kv_cache)),
               "pa_decode_with_store")
    return out

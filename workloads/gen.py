"""Seeded synthetic inputs for paged-attention steps.

This module only draws inputs and lays out batch metadata (lengths, cumulative lengths,
block tables, slot mappings, copy maps).  It holds no attention arithmetic, and it imports
neither the oracle nor the HIP library: both of those consume what it returns.

Draw order for one workload, from ``numpy.random.default_rng(seed)``: the lengths (drawn
by the caller), a permutation of the physical block pool, the cache fill, the queries, the
new keys, the new values, then the copy map.  Gaussians are float32 N(0, 1) rounded to the
cache dtype once (bf16 by round-to-nearest-even), so every consumer sees the same bits.

A sequence's life is a timeline: ``ctx0`` keys already in the cache, then per phase a
query chunk of ``q`` new tokens that is either a prefill chunk or one decode token.  Each
phase is: optional copy_blocks, store every new token of the phase through slot_mapping
(prefill tokens first, then decode tokens, as in the vllm-npu 0.4.2 diff, ``xformers.py``
``XFormersImpl`` token layout), attention for the prefill chunks, attention for the decode
tokens.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "SeqSpec", "StoreOp", "CopyOp", "PrefillOp", "DecodeOp", "Workload",
    "cu_seqlens", "slot_mapping", "build", "config", "CONFIG_NAMES", "shared_prefix_decode",
    "shared_prefix_prefill",
]


@dataclass
class SeqSpec:
    """One sequence: ``ctx0`` cached keys, then per phase ``q[p]`` new tokens of ``kind[p]``."""
    ctx0: int
    q: List[int]
    kind: List[Optional[str]]          # "prefill", "decode" or None per phase


@dataclass
class StoreOp:
    key: torch.Tensor                  # [T, Hkv, D] (CPU, cache dtype)
    value: torch.Tensor
    slot_mapping: np.ndarray           # [T] int32, -1 = skip


@dataclass
class CopyOp:
    pairs: np.ndarray                  # [n, 2] int32 (src, dst)


@dataclass
class PrefillOp:
    query: torch.Tensor                # [Tq, H, D]
    block_table: np.ndarray            # [B, MB] int32, -1 = unallocated
    cu_seqlens_q: np.ndarray           # [B+1] int32
    cu_seqlens_k: np.ndarray           # [B+1] int32
    max_seqlen_q: int
    max_seqlen_k: int
    out_rows: slice                    # rows of the phase's packed output
    seq_ids: List[int]


@dataclass
class DecodeOp:
    query: torch.Tensor                # [B, H, D]
    block_table: np.ndarray            # [B, MB] int32
    seq_lens: np.ndarray               # [B] int32
    max_seq_len: int
    out_rows: slice
    seq_ids: List[int]


@dataclass
class Workload:
    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: torch.dtype
    scale: float
    sliding_window: int
    kv_cache: torch.Tensor             # [2, NB, BS, Hkv, D] initial contents (CPU)
    phases: List[list] = field(default_factory=list)
    seqs: List[SeqSpec] = field(default_factory=list)
    tables: np.ndarray = None          # [num_seqs, max blocks] physical block of every seq


def cu_seqlens(lengths: Sequence[int]) -> np.ndarray:
    """Cumulative lengths with a leading 0: ``[5, 7] -> [0, 5, 12]`` (MinivLLM API docs,
    section flash_attention_prefill, parameter cu_seqlens)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def slot_mapping(table_row: np.ndarray, context_len: int, query_len: int,
                 block_size: int) -> np.ndarray:
    """Flat cache slots of a sequence's ``query_len`` new tokens.

    vLLM learning book, "05. Attention Backends", section 10 question 2: token ``i`` of the
    chunk is logical position ``context_len + i``; its slot is the physical block of that
    position times ``block_size`` plus the position's offset in the block.
    """
    pos = context_len + np.arange(query_len, dtype=np.int64)
    blocks = table_row[pos // block_size].astype(np.int64)
    return (blocks * block_size + pos % block_size).astype(np.int32)


_CHUNK = 1 << 25


def _gauss(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """float32 N(0,1) draws rounded to ``dtype``, drawn in chunks of 2**25 in C order."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        x = torch.from_numpy(rng.standard_normal(size=stop - start, dtype=np.float32))
        out[start:stop] = x if dtype == torch.float32 else x.to(dtype)
    return out.view(shape)


def build(name: str, seed: int, seqs: List[SeqSpec], *, num_heads: int, num_kv_heads: int,
          head_size: int, block_size: int, dtype: torch.dtype, sliding_window: int = 0,
          scale: Optional[float] = None, num_blocks: Optional[int] = None,
          copy_fraction: float = 0.0, rng: Optional[np.random.Generator] = None,
          shared_prefix: int = 0, cache_dtype: Optional[torch.dtype] = None) -> Workload:
    """Draw the inputs of every phase of ``seqs`` (see the module docstring for the order).

    The pool is ``ceil(1.1 * total blocks)`` physical blocks unless ``num_blocks`` is given;
    sequences take blocks in order from one seeded permutation of the pool, and block-table
    rows are padded with -1.  ``shared_prefix`` (a multiple of ``block_size``, at most every
    ``ctx0``): the first that many keys of every sequence are the first sequence's, through
    the same physical blocks (a prefix-cache hit shared by the batch); the other sequences
    take blocks only for the rest.  ``cache_dtype`` (default ``dtype``): the cache fill is drawn
    in that dtype (``torch.float8_e4m3fn``: N(0,1) rounded by torch's conversion), the queries
    and new keys/values in ``dtype``.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    nphase = max(len(s.q) for s in seqs) if seqs else 0
    n_final = [s.ctx0 + sum(s.q) for s in seqs]
    nblk = [math.ceil(n / block_size) for n in n_final]
    assert shared_prefix % block_size == 0 and all(s.ctx0 >= shared_prefix for s in seqs)
    n_shared = shared_prefix // block_size
    own = [nb - (n_shared if i > 0 else 0) for i, nb in enumerate(nblk)]
    total = sum(own)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.1 * total))
    assert num_blocks >= total, "pool too small"
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max([1] + nblk)
    tables = np.full((len(seqs), width), -1, dtype=np.int32)
    cursor = 0
    for i, nb in enumerate(nblk):
        if i > 0 and n_shared:
            tables[i, :n_shared] = tables[0, :n_shared]
        tables[i, nb - own[i]:nb] = perm[cursor:cursor + own[i]]
        cursor += own[i]
    allocated = perm[:cursor]
    free = perm[cursor:]

    kv_cache = _gauss(rng, (2, num_blocks, block_size, num_kv_heads, head_size), cache_dtype or dtype)

    # per-phase token order: prefill chunks (sequence order) then decode tokens
    order = []
    for p in range(nphase):
        pre = [i for i, s in enumerate(seqs) if p < len(s.q) and s.kind[p] == "prefill" and s.q[p] > 0]
        dec = [i for i, s in enumerate(seqs) if p < len(s.q) and s.kind[p] == "decode"]
        order.append((pre, dec))
    total_tokens = sum(sum(seqs[i].q[p] for i in pre) + len(dec) for p, (pre, dec) in enumerate(order))
    q_all = _gauss(rng, (total_tokens, num_heads, head_size), dtype)
    k_all = _gauss(rng, (total_tokens, num_kv_heads, head_size), dtype)
    v_all = _gauss(rng, (total_tokens, num_kv_heads, head_size), dtype)

    pairs = None
    if copy_fraction > 0:
        n_copy = min(math.ceil(copy_fraction * num_blocks), len(allocated), len(free))
        src = rng.choice(allocated, size=n_copy, replace=False)
        dst = rng.choice(free, size=n_copy, replace=False)
        pairs = np.stack([src, dst], axis=1).astype(np.int32)

    if scale is None:
        scale = 1.0 / math.sqrt(head_size)
    wl = Workload(name=name, num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
                  block_size=block_size, num_blocks=num_blocks, dtype=dtype, scale=float(scale),
                  sliding_window=int(sliding_window), kv_cache=kv_cache, seqs=seqs, tables=tables)

    ctx = [s.ctx0 for s in seqs]
    tok = 0
    for p, (pre, dec) in enumerate(order):
        ops = []
        if p == 0 and pairs is not None:
            ops.append(CopyOp(pairs=pairs))
        n_pre = sum(seqs[i].q[p] for i in pre)
        n_tok = n_pre + len(dec)
        sl = []
        for i in pre:
            sl.append(slot_mapping(tables[i], ctx[i], seqs[i].q[p], block_size))
        for i in dec:
            sl.append(slot_mapping(tables[i], ctx[i], 1, block_size))
        slots = np.concatenate(sl).astype(np.int32) if sl else np.zeros(0, np.int32)
        ops.append(StoreOp(key=k_all[tok:tok + n_tok], value=v_all[tok:tok + n_tok], slot_mapping=slots))
        if pre:
            ql = [seqs[i].q[p] for i in pre]
            kl = [ctx[i] + seqs[i].q[p] for i in pre]
            mb = max(math.ceil(k / block_size) for k in kl)
            ops.append(PrefillOp(query=q_all[tok:tok + n_pre], block_table=np.ascontiguousarray(tables[pre, :max(mb, 1)]),
                                 cu_seqlens_q=cu_seqlens(ql), cu_seqlens_k=cu_seqlens(kl),
                                 max_seqlen_q=max(ql), max_seqlen_k=max(kl),
                                 out_rows=slice(0, n_pre), seq_ids=list(pre)))
        if dec:
            lens = np.array([ctx[i] + 1 for i in dec], dtype=np.int32)
            mb = max(math.ceil(int(n) / block_size) for n in lens)
            ops.append(DecodeOp(query=q_all[tok + n_pre:tok + n_tok], block_table=np.ascontiguousarray(tables[dec, :max(mb, 1)]),
                                seq_lens=lens, max_seq_len=int(lens.max()),
                                out_rows=slice(n_pre, n_tok), seq_ids=list(dec)))
        for i in pre:
            ctx[i] += seqs[i].q[p]
        for i in dec:
            ctx[i] += 1
        tok += n_tok
        wl.phases.append(ops)
    return wl


CONFIG_NAMES = {
    1: "fp32 smoke: 2 prompts (5, 13) + 4 decode steps, H 4/2, D 64, bs 16",
    2: "GQA paged decode: B 64, ctx U[512,4096], H 32/8, D 128, bs 16, bf16",
    3: "varlen causal prefill: B 16, L U[128,2048], H 32/8, D 128, bs 16, bf16",
    4: "chunked prefill 8x512 over ctx U[4096,32768], window 4096, H 40/8, D 128, + decode, bf16",
    5: "mixed step: copy_blocks 1% + 4x512 prefill chunks (ctx U[0,8192]) + 252 decodes (ctx U[256,8192]), H 64/8, D 128, bf16",
}


def config(n: int) -> Workload:
    """The five seeded workloads (seed = config number)."""
    rng = np.random.default_rng(n)
    if n == 1:
        seqs = [SeqSpec(0, [5, 1, 1, 1, 1], ["prefill"] + ["decode"] * 4),
                SeqSpec(0, [13, 1, 1, 1, 1], ["prefill"] + ["decode"] * 4)]
        return build("config1", n, seqs, num_heads=4, num_kv_heads=2, head_size=64, block_size=16,
                     dtype=torch.float32, num_blocks=8, rng=rng)
    if n == 2:
        ctx = rng.integers(512, 4096 + 1, size=64)
        seqs = [SeqSpec(int(c), [1], ["decode"]) for c in ctx]
        return build("config2", n, seqs, num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                     dtype=torch.bfloat16, rng=rng)
    if n == 3:
        lens = rng.integers(128, 2048 + 1, size=16)
        seqs = [SeqSpec(0, [int(L)], ["prefill"]) for L in lens]
        return build("config3", n, seqs, num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                     dtype=torch.bfloat16, rng=rng)
    if n == 4:
        ctx = rng.integers(4096, 32768 + 1, size=8)
        seqs = [SeqSpec(int(c), [512, 1], ["prefill", "decode"]) for c in ctx]
        return build("config4", n, seqs, num_heads=40, num_kv_heads=8, head_size=128, block_size=16,
                     dtype=torch.bfloat16, sliding_window=4096, rng=rng)
    if n == 5:
        pre_ctx = rng.integers(0, 8192 + 1, size=4)
        dec_ctx = rng.integers(256, 8192 + 1, size=252)
        seqs = [SeqSpec(int(c), [512], ["prefill"]) for c in pre_ctx]
        seqs += [SeqSpec(int(c), [1], ["decode"]) for c in dec_ctx]
        return build("config5", n, seqs, num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                     dtype=torch.bfloat16, copy_fraction=0.01, rng=rng)
    raise ValueError(f"no config {n}")


def shared_prefix_decode(seed: int = 6, num_seqs: int = 64, prefix: int = 1024, lo: int = 1024,
                         hi: int = 4096, num_heads: int = 32, num_kv_heads: int = 8,
                         head_size: int = 128, block_size: int = 16,
                         dtype: torch.dtype = torch.bfloat16,
                         cache_dtype: Optional[torch.dtype] = None) -> Workload:
    """One decode step of ``num_seqs`` sequences that share their first ``prefix`` keys (one
    system prompt, served from the prefix cache): contexts U[lo, hi] (at least ``prefix``),
    the GQA decode shape otherwise.  The vLLM learning book (self-check question 4) names a
    shared prefix of at least 256 tokens and at least two requests as the usual trigger."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(max(lo, prefix), hi + 1, size=num_seqs)
    seqs = [SeqSpec(int(c), [1], ["decode"]) for c in ctx]
    return build(f"shared_prefix{prefix}_b{num_seqs}", seed, seqs, num_heads=num_heads,
                 num_kv_heads=num_kv_heads, head_size=head_size, block_size=block_size, dtype=dtype,
                 rng=rng, shared_prefix=prefix, cache_dtype=cache_dtype)


def shared_prefix_prefill(seed: int = 7, num_seqs: int = 8, prefix: int = 2048, lo: int = 2048,
                          hi: int = 4096, chunk: int = 512, num_heads: int = 32, num_kv_heads: int = 8,
                          head_size: int = 128, block_size: int = 16,
                          dtype: torch.dtype = torch.bfloat16,
                          cache_dtype: Optional[torch.dtype] = None) -> Workload:
    """One chunked-prefill step of ``num_seqs`` sequences that share their first ``prefix``
    keys (one system prompt from the prefix cache): cached contexts U[lo, hi] (at least
    ``prefix``), each with a ``chunk``-token query chunk, the GQA shape otherwise."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(max(lo, prefix), hi + 1, size=num_seqs)
    seqs = [SeqSpec(int(c), [chunk], ["prefill"]) for c in ctx]
    return build(f"shared_prefix_prefill{prefix}_b{num_seqs}", seed, seqs, num_heads=num_heads,
                 num_kv_heads=num_kv_heads, head_size=head_size, block_size=block_size, dtype=dtype,
                 rng=rng, shared_prefix=prefix, cache_dtype=cache_dtype)


"""Helpers shared by the GPU parity tests: run a workload phase through the HIP library and
the same phase through the oracle, and compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_attention_block_amd as pa
import workloads as W

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-5, 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tol_for(dtype):
    return (F32_ATOL, F32_RTOL) if dtype == torch.float32 else (BF16_ATOL, BF16_RTOL)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype, what: str) -> float:
    """Elementwise |got - ref| <= atol + rtol*|ref|; returns the max abs error."""
    atol, rtol = tol_for(dtype)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"gpu {got[i]} oracle {ref[i]} (max abs err {err.max():.3e})")
    return float(err.max()) if err.size else 0.0


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a CPU tensor as an integer numpy array."""
    t = t.contiguous()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]).numpy()


def host_values(t: torch.Tensor) -> np.ndarray:
    """Exact float values of a (bf16 or fp32) CPU tensor as a float32 numpy array."""
    return t.float().numpy() if t.dtype != torch.float32 else t.numpy()


class GpuRun:
    """Owns the device copy of a workload's cache and runs its ops in order."""

    def __init__(self, wl: W.Workload, device: torch.device):
        self.wl = wl
        self.dev = device
        self.cache = wl.kv_cache.to(device)
        self.alibi = None        # optional np.ndarray [num_heads] ALiBi slopes
        self.kv_scale = 1.0      # the scale of an FP8 cache

    def _slopes(self):
        return None if self.alibi is None else torch.from_numpy(np.asarray(self.alibi, np.float32)).to(self.dev)

    def i32(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev)

    def run(self, op, partition_size: int = 0):
        wl = self.wl
        if isinstance(op, W.CopyOp):
            pa.pa_copy_blocks(self.cache, self.i32(op.pairs))
            return None
        if isinstance(op, W.StoreOp):
            pa.pa_store_kv(op.key.to(self.dev), op.value.to(self.dev), self.cache, self.i32(op.slot_mapping),
                           kv_scale=self.kv_scale)
            return None
        if isinstance(op, W.PrefillOp):
            return pa.pa_prefill_varlen(op.query.to(self.dev), self.cache, self.i32(op.block_table),
                                        self.i32(op.cu_seqlens_q), self.i32(op.cu_seqlens_k),
                                        op.max_seqlen_q, op.max_seqlen_k, wl.scale, wl.num_kv_heads,
                                        wl.sliding_window, alibi_slopes=self._slopes(), kv_scale=self.kv_scale)
        if isinstance(op, W.DecodeOp):
            return pa.pa_decode(op.query.to(self.dev), self.cache, self.i32(op.block_table),
                                self.i32(op.seq_lens), op.max_seq_len, wl.scale, wl.num_kv_heads,
                                wl.sliding_window, partition_size=partition_size,
                                alibi_slopes=self._slopes(), kv_scale=self.kv_scale)
        raise TypeError(op)

    def run_with_store(self, store, op, partition_size: int = 0):
        """The store of ``op``'s rows of ``store`` and the attention ``op``, as one call."""
        wl, d = self.wl, self.dev
        k = store.key[op.out_rows].to(d)
        v = store.value[op.out_rows].to(d)
        sl = self.i32(store.slot_mapping[op.out_rows])
        if isinstance(op, W.PrefillOp):
            return pa.pa_prefill_varlen_with_store(op.query.to(d), k, v, sl, self.cache, self.i32(op.block_table),
                                                   self.i32(op.cu_seqlens_q), self.i32(op.cu_seqlens_k),
                                                   op.max_seqlen_q, op.max_seqlen_k, wl.scale, wl.num_kv_heads,
                                                   wl.sliding_window, alibi_slopes=self._slopes(),
                                                   kv_scale=self.kv_scale)
        return pa.pa_decode_with_store(op.query.to(d), k, v, sl, self.cache, self.i32(op.block_table),
                                       self.i32(op.seq_lens), op.max_seq_len, wl.scale, wl.num_kv_heads,
                                       wl.sliding_window, partition_size=partition_size,
                                       alibi_slopes=self._slopes(), kv_scale=self.kv_scale)


def oracle_attention(wl: W.Workload, op, cache_vals: np.ndarray, picks=None, alibi=None) -> np.ndarray:
    """Oracle output for a prefill/decode op; ``picks`` = list of (row, head) to sample;
    ``alibi`` = optional ALiBi slopes [num_heads]."""
    q = host_values(op.query)
    if isinstance(op, W.PrefillOp):
        cu_q, cu_k = op.cu_seqlens_q, op.cu_seqlens_k
    else:
        cu_q = np.arange(len(op.seq_lens) + 1)
        cu_k = np.concatenate([[0], np.cumsum(op.seq_lens)])
    if picks is None:
        return oracle.prefill_varlen(q, cache_vals, op.block_table, cu_q, cu_k, wl.scale,
                                     wl.num_kv_heads, wl.sliding_window, alibi)
    return oracle.attention_rows(q, cache_vals, op.block_table, cu_q, cu_k, wl.scale,
                                 wl.num_kv_heads, wl.sliding_window, picks, alibi)


def sample_picks(op, num_heads: int, rng: np.random.Generator, n_random: int = 96):
    """Rows to check at full size: first/last rows of every sequence, rows at tile
    boundaries, and random rows; each with a few heads (first, last, random)."""
    if isinstance(op, W.PrefillOp):
        cu = op.cu_seqlens_q
    else:
        cu = np.arange(len(op.seq_lens) + 1)
    rows = set()
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for r in (a, b - 1, min(b - 1, a + 31), min(b - 1, a + 32), min(b - 1, a + 64)):
            rows.add(r)
    total = int(cu[-1])
    rows.update(int(x) for x in rng.integers(0, total, size=min(n_random, total)))
    picks = []
    for r in sorted(rows):
        for h in {0, num_heads - 1, int(rng.integers(0, num_heads))}:
            picks.append((r, h))
    return picks


def relayout(wl: W.Workload, block_size: int, seed: int) -> W.Workload:
    """Same logical keys/values, queries and new tokens, placed in a fresh pool of
    ``block_size``-slot blocks handed out in a seeded random order (tables, slots and cache
    rewritten together)."""
    import copy
    import math
    rng = np.random.default_rng(seed)
    n_final = [s.ctx0 + sum(s.q) for s in wl.seqs]
    nblk = [max(1, math.ceil(n / block_size)) for n in n_final]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    tables = np.full((len(wl.seqs), max(nblk)), -1, dtype=np.int32)
    cur = 0
    for s, k in enumerate(nblk):
        tables[s, :k] = perm[cur:cur + k]
        cur += k
    old_bs = wl.block_size
    cache = torch.zeros((2, nb, block_size) + tuple(wl.kv_cache.shape[3:]), dtype=wl.kv_cache.dtype)
    where = {}
    for s, n in enumerate(n_final):
        for j in range(n):
            ob, oo = int(wl.tables[s, j // old_bs]), j % old_bs
            cache[:, tables[s, j // block_size], j % block_size] = wl.kv_cache[:, ob, oo]
            where[ob * old_bs + oo] = (s, j)
    out = copy.copy(wl)
    out.block_size, out.num_blocks, out.kv_cache, out.tables = block_size, nb, cache, tables
    out.phases = []
    for ph in wl.phases:
        ops = []
        for op in ph:
            if isinstance(op, W.StoreOp):
                sl = [int(tables[where[int(x)][0], where[int(x)][1] // block_size]) * block_size
                      + where[int(x)][1] % block_size if x >= 0 else -1 for x in op.slot_mapping]
                ops.append(W.StoreOp(op.key, op.value, np.array(sl, dtype=np.int32)))
            elif isinstance(op, (W.PrefillOp, W.DecodeOp)):
                lens = (np.diff(op.cu_seqlens_k) if isinstance(op, W.PrefillOp) else op.seq_lens)
                mb = max(1, max(math.ceil(int(n) / block_size) for n in lens))
                ops.append(type(op)(**{**op.__dict__, "block_table": np.ascontiguousarray(tables[op.seq_ids, :mb])}))
            else:
                raise TypeError("relayout covers store/prefill/decode phases only")
        out.phases.append(ops)
    return out

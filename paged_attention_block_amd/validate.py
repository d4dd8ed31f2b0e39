"""Host-side checks of the device-content preconditions of the library's calls.

The C entry points check their scalar arguments but not the contents of index arrays (slot
values, block-table entries, cumulative lengths, sequence lengths): a bad value there is
an out-of-range access or a write race on the GPU.  These functions check those contents
on host copies, raising ``ValueError`` that names the first violation; the binding runs
them before the call when it is given ``validate=True`` (which copies the index arrays to
the host and so synchronises with the device).

Preconditions checked (as documented per entry point in ``include/pa.h``):
  * store: every non-negative slot < num_blocks * block_size, no slot repeated;
  * copy_blocks: block ids in [0, num_blocks), destinations unique and never a source;
  * prefill: cu_seqlens_q / cu_seqlens_k of num_seqs + 1 entries, starting at 0,
    non-decreasing, lengths within max_seqlen_q / max_seqlen_k, the queries' rows
    covering cu_seqlens_q[num_seqs]; block-table entries in [0, num_blocks) for every
    block holding a key some row attends (the union of the rows' key ranges, windowed);
  * decode: 0 <= seq_lens[s] <= max_seq_len, table entries of the live keys
    [max(0, n - window), n) (or [0, n)) in range;
  * the store-fused calls: both of the above, and each new token's non-negative slot
    equal to the block-table position of its key;
  * cascade decode: every seq_len >= common_prefix_len and the prefix's block-table
    entries the same physical blocks in every row.
Pure host logic on numpy arrays: no device access and none of the attention arithmetic.
"""

from __future__ import annotations

import numpy as np


def _host(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor (any device)
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def check_store(slot_mapping, num_blocks: int, block_size: int) -> None:
    slots = _host(slot_mapping).astype(np.int64).reshape(-1)
    live = slots[slots >= 0]
    cap = int(num_blocks) * int(block_size)
    bad = np.nonzero((slots >= cap))[0]
    if bad.size:
        t = int(bad[0])
        raise ValueError(f"slot_mapping[{t}] = {slots[t]} is not below num_blocks*block_size = {cap}")
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        s = int(uniq[np.argmax(counts > 1)])
        ts = np.nonzero(slots == s)[0][:2].tolist()
        raise ValueError(f"slot {s} is written by tokens {ts[0]} and {ts[1]} (a write race)")


def check_copy_blocks(block_pairs, num_blocks: int) -> None:
    pairs = _host(block_pairs).astype(np.int64).reshape(-1, 2)
    bad = np.nonzero(((pairs < 0) | (pairs >= num_blocks)).any(axis=1))[0]
    if bad.size:
        i = int(bad[0])
        raise ValueError(f"block_pairs[{i}] = {pairs[i].tolist()} has a block id outside [0, {num_blocks})")
    dst = pairs[:, 1]
    uniq, counts = np.unique(dst, return_counts=True)
    if (counts > 1).any():
        raise ValueError(f"block {int(uniq[np.argmax(counts > 1)])} is the destination of more than one pair")
    both = np.intersect1d(dst, pairs[:, 0])
    if both.size:
        raise ValueError(f"block {int(both[0])} is both a destination and a source")


def _check_table_range(table: np.ndarray, s: int, lo: int, hi: int, num_blocks: int,
                       block_size: int) -> None:
    """Entries of row s for the blocks of logical keys [lo, hi) exist and are in range."""
    if hi <= lo:
        return
    b0, b1 = lo // block_size, (hi - 1) // block_size
    if b1 >= table.shape[1]:
        raise ValueError(f"sequence {s}: key {hi - 1} needs block-table column {b1}, but the "
                         f"table has {table.shape[1]} columns")
    row = table[s, b0:b1 + 1]
    bad = np.nonzero((row < 0) | (row >= num_blocks))[0]
    if bad.size:
        c = b0 + int(bad[0])
        raise ValueError(f"sequence {s}: block_table[{s}, {c}] = {int(table[s, c])} is outside "
                         f"[0, {num_blocks}) but holds live keys")


def _check_cu(cu, name: str, num_seqs: int, max_len: int) -> np.ndarray:
    cu = _host(cu).astype(np.int64).reshape(-1)
    if cu.shape[0] != num_seqs + 1:
        raise ValueError(f"{name} has {cu.shape[0]} entries, expected num_seqs + 1 = {num_seqs + 1}")
    if num_seqs >= 0 and cu.shape[0] and cu[0] != 0:
        raise ValueError(f"{name}[0] = {int(cu[0])}, expected 0")
    d = np.diff(cu)
    if (d < 0).any():
        s = int(np.argmax(d < 0))
        raise ValueError(f"{name} decreases at sequence {s} ({int(cu[s])} -> {int(cu[s + 1])})")
    if (d > max_len).any():
        s = int(np.argmax(d > max_len))
        raise ValueError(f"sequence {s} has {int(d[s])} entries in {name}, above the maximum {max_len}")
    return cu


def check_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q: int, max_seqlen_k: int,
                  sliding_window: int, num_blocks: int, block_size: int, query_rows: int) -> None:
    table = _host(block_table).astype(np.int64)
    num_seqs = _host(cu_seqlens_q).reshape(-1).shape[0] - 1
    cq = _check_cu(cu_seqlens_q, "cu_seqlens_q", num_seqs, int(max_seqlen_q))
    ck = _check_cu(cu_seqlens_k, "cu_seqlens_k", num_seqs, int(max_seqlen_k))
    if table.ndim != 2 or table.shape[0] < num_seqs:
        raise ValueError(f"block_table must be [num_seqs, max_blocks], got {list(table.shape)}")
    if cq[-1] > query_rows:
        raise ValueError(f"cu_seqlens_q ends at {int(cq[-1])} but the query has {query_rows} rows")
    for s in range(num_seqs):
        sq, sk = int(cq[s + 1] - cq[s]), int(ck[s + 1] - ck[s])
        if sq == 0 or sk == 0:
            continue
        first = sk - sq  # position of the sequence's first query row
        lo = max(0, first - int(sliding_window) + 1) if sliding_window > 0 else 0
        _check_table_range(table, s, lo, sk, num_blocks, block_size)


def check_decode(seq_lens, block_table, max_seq_len: int, sliding_window: int, num_blocks: int,
                 block_size: int) -> None:
    table = _host(block_table).astype(np.int64)
    lens = _host(seq_lens).astype(np.int64).reshape(-1)
    if table.ndim != 2 or table.shape[0] < lens.shape[0]:
        raise ValueError(f"block_table must be [num_seqs, max_blocks], got {list(table.shape)}")
    bad = np.nonzero((lens < 0) | (lens > max_seq_len))[0]
    if bad.size:
        s = int(bad[0])
        raise ValueError(f"seq_lens[{s}] = {int(lens[s])} is outside [0, max_seq_len = {max_seq_len}]")
    for s, n in enumerate(lens.tolist()):
        lo = max(0, n - int(sliding_window)) if sliding_window > 0 else 0
        _check_table_range(table, s, lo, n, num_blocks, block_size)


def _check_slot_is_table_position(slot: int, table: np.ndarray, s: int, pos: int, block_size: int,
                                  what: str) -> None:
    if slot < 0:
        # a fused call attends every new token it stores: leaving one unstored is outside its
        # precondition (the rows attending that key would see the given row with a bf16 cache but
        # the old cache row with float32 and FP8 caches, which store before attending)
        raise ValueError(f"{what}: negative slot {slot}: the fused store-and-attend calls need a slot for every "
                         f"new token (key position {pos} of sequence {s})")
    want = int(table[s, pos // block_size]) * block_size + pos % block_size
    if slot != want:
        raise ValueError(f"{what}: slot {slot}, but key position {pos} of sequence {s} sits at slot "
                         f"{want} through the block table")


def check_prefill_with_store(slot_mapping, cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q: int,
                             max_seqlen_k: int, sliding_window: int, num_blocks: int, block_size: int,
                             query_rows: int) -> None:
    check_store(slot_mapping, num_blocks, block_size)
    check_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q, max_seqlen_k, sliding_window,
                  num_blocks, block_size, query_rows)
    slots = _host(slot_mapping).astype(np.int64).reshape(-1)
    cq = _host(cu_seqlens_q).astype(np.int64).reshape(-1)
    ck = _host(cu_seqlens_k).astype(np.int64).reshape(-1)
    table = _host(block_table).astype(np.int64)
    if slots.shape[0] != cq[-1]:
        raise ValueError(f"slot_mapping has {slots.shape[0]} entries, expected cu_seqlens_q[-1] = {int(cq[-1])}")
    for s in range(cq.shape[0] - 1):
        sq, sk = int(cq[s + 1] - cq[s]), int(ck[s + 1] - ck[s])
        if sq > sk:
            raise ValueError(f"sequence {s}: {sq} new tokens but only {sk} keys")
        for i in range(sq):
            t = int(cq[s]) + i
            _check_slot_is_table_position(int(slots[t]), table, s, sk - sq + i, block_size,
                                          f"slot_mapping[{t}]")


def check_decode_with_store(slot_mapping, seq_lens, block_table, max_seq_len: int, sliding_window: int,
                            num_blocks: int, block_size: int) -> None:
    check_store(slot_mapping, num_blocks, block_size)
    check_decode(seq_lens, block_table, max_seq_len, sliding_window, num_blocks, block_size)
    slots = _host(slot_mapping).astype(np.int64).reshape(-1)
    lens = _host(seq_lens).astype(np.int64).reshape(-1)
    table = _host(block_table).astype(np.int64)
    if slots.shape[0] != lens.shape[0]:
        raise ValueError(f"slot_mapping has {slots.shape[0]} entries, expected num_seqs = {lens.shape[0]}")
    for s, n in enumerate(lens.tolist()):
        if n == 0:
            if slots[s] >= 0:
                raise ValueError(f"sequence {s} has seq_len 0 but a new token at slot {int(slots[s])}")
            continue
        _check_slot_is_table_position(int(slots[s]), table, s, n - 1, block_size, f"slot_mapping[{s}]")


def check_cascade(seq_lens, block_table, max_seq_len: int, common_prefix_len: int, num_blocks: int,
                  block_size: int) -> None:
    check_decode(seq_lens, block_table, max_seq_len, 0, num_blocks, block_size)
    lens = _host(seq_lens).astype(np.int64).reshape(-1)
    table = _host(block_table).astype(np.int64)
    if common_prefix_len <= 0 or lens.shape[0] == 0:
        return
    short = np.nonzero(lens < common_prefix_len)[0]
    if short.size:
        s = int(short[0])
        raise ValueError(f"seq_lens[{s}] = {int(lens[s])} is below common_prefix_len = {common_prefix_len}")
    nb = common_prefix_len // block_size
    diff = np.nonzero((table[:lens.shape[0], :nb] != table[0, :nb]).any(axis=1))[0]
    if diff.size:
        s = int(diff[0])
        c = int(np.argmax(table[s, :nb] != table[0, :nb]))
        raise ValueError(f"block_table[{s}, {c}] = {int(table[s, c])} differs from row 0's "
                         f"{int(table[0, c])} inside the shared prefix")


def check_cascade_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q: int, max_seqlen_k: int,
                          common_prefix_len: int, num_blocks: int, block_size: int, query_rows: int) -> None:
    """pa_cascade_prefill_varlen's device-content preconditions: those of pa_prefill_varlen, every
    sequence's first query row at or after the prefix's last key, and the prefix blocks shared by
    every block-table row."""
    check_prefill(cu_seqlens_q, cu_seqlens_k, block_table, max_seqlen_q, max_seqlen_k, 0, num_blocks, block_size,
                  query_rows)
    if common_prefix_len <= 0:
        return
    cq = _host(cu_seqlens_q).astype(np.int64).reshape(-1)
    ck = _host(cu_seqlens_k).astype(np.int64).reshape(-1)
    table = _host(block_table).astype(np.int64)
    num_seqs = cq.shape[0] - 1
    first = (ck[1:] - ck[:-1]) - (cq[1:] - cq[:-1])
    early = np.nonzero(first + 1 < common_prefix_len)[0]
    if early.size:
        s = int(early[0])
        raise ValueError(f"sequence {s}: its first query row (position {int(first[s])}) lies inside the shared "
                         f"prefix of {common_prefix_len} keys")
    nb = common_prefix_len // block_size
    diff = np.nonzero((table[:num_seqs, :nb] != table[0, :nb]).any(axis=1))[0]
    if diff.size:
        s = int(diff[0])
        c = int(np.argmax(table[s, :nb] != table[0, :nb]))
        raise ValueError(f"block_table[{s}, {c}] = {int(table[s, c])} differs from row 0's "
                         f"{int(table[0, c])} inside the shared prefix")

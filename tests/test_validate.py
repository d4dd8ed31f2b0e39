"""Host checks of the calls' device-content preconditions (``paged_attention_block_amd.validate``).

Pure host logic, no GPU: the seeded workloads (which the parity tests run) must pass every
check, and each precondition broken on its own must raise ``ValueError`` naming it.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from paged_attention_block_amd import validate as V


def _phase_ops(phase):
    store = next((op for op in phase if isinstance(op, W.StoreOp)), None)
    return store, [op for op in phase if not isinstance(op, W.StoreOp)]


def _check_workload(wl, common_prefix_len=0):
    nb, bs = wl.num_blocks, wl.block_size
    for phase in wl.phases:
        store, ops = _phase_ops(phase)
        if store is not None:
            V.check_store(store.slot_mapping, nb, bs)
        for op in ops:
            if isinstance(op, W.CopyOp):
                V.check_copy_blocks(op.pairs, nb)
            elif isinstance(op, W.PrefillOp):
                V.check_prefill(op.cu_seqlens_q, op.cu_seqlens_k, op.block_table, op.max_seqlen_q,
                                op.max_seqlen_k, wl.sliding_window, nb, bs, op.query.shape[0])
                V.check_prefill_with_store(store.slot_mapping[op.out_rows], op.cu_seqlens_q, op.cu_seqlens_k,
                                           op.block_table, op.max_seqlen_q, op.max_seqlen_k,
                                           wl.sliding_window, nb, bs, op.query.shape[0])
            elif isinstance(op, W.DecodeOp):
                V.check_decode(op.seq_lens, op.block_table, op.max_seq_len, wl.sliding_window, nb, bs)
                if store is not None:
                    V.check_decode_with_store(store.slot_mapping[op.out_rows], op.seq_lens, op.block_table,
                                              op.max_seq_len, wl.sliding_window, nb, bs)
                if common_prefix_len:
                    V.check_cascade(op.seq_lens, op.block_table, op.max_seq_len, common_prefix_len, nb, bs)


def _small(seed, window=0, bs=16):
    seqs = [W.SeqSpec(0, [37, 1], ["prefill", "decode"]), W.SeqSpec(70, [5, 1], ["prefill", "decode"]),
            W.SeqSpec(130, [1, 1], ["decode", "decode"]), W.SeqSpec(0, [64, 1], ["prefill", "decode"])]
    return W.build(f"validate{seed}", seed, seqs, num_heads=4, num_kv_heads=2, head_size=64, block_size=bs,
                   dtype=torch.float32, sliding_window=window, copy_fraction=0.1)


@pytest.mark.parametrize("window,bs", [(0, 16), (40, 16), (0, 1), (17, 8)])
def test_seeded_workloads_pass(window, bs):
    _check_workload(_small(3, window, bs))


def test_config1_and_shared_prefix_pass():
    _check_workload(W.config(1))
    wl = W.shared_prefix_decode(seed=6, num_seqs=5, prefix=64, lo=64, hi=150, num_heads=4, num_kv_heads=2,
                                head_size=64)
    _check_workload(wl, common_prefix_len=64)


def test_store_violations():
    V.check_store(np.array([0, 1, 16, -1, -7], np.int32), 8, 16)   # negative slots skip
    with pytest.raises(ValueError, match="write race"):
        V.check_store(np.array([3, 5, 3], np.int32), 8, 16)
    with pytest.raises(ValueError, match=r"slot_mapping\[1\] = 128"):
        V.check_store(np.array([0, 128], np.int32), 8, 16)


def test_copy_violations():
    V.check_copy_blocks(np.array([[0, 3], [1, 4]], np.int32), 8)
    with pytest.raises(ValueError, match="outside"):
        V.check_copy_blocks(np.array([[0, 8]], np.int32), 8)
    with pytest.raises(ValueError, match="more than one pair"):
        V.check_copy_blocks(np.array([[0, 3], [1, 3]], np.int32), 8)
    with pytest.raises(ValueError, match="both a destination and a source"):
        V.check_copy_blocks(np.array([[0, 3], [3, 4]], np.int32), 8)


def test_prefill_violations():
    table = np.array([[2, 5, -1], [7, -1, -1]], np.int32)
    cq, ck = np.array([0, 3, 5], np.int32), np.array([0, 20, 22], np.int32)
    # sequence 1 has 2 keys but table row 1 only needs column 0
    V.check_prefill(cq, ck, table, 3, 20, 0, 8, 16, 5)
    with pytest.raises(ValueError, match=r"cu_seqlens_q\[0\] = 1"):
        V.check_prefill(np.array([1, 3, 5], np.int32), ck, table, 3, 20, 0, 8, 16, 5)
    with pytest.raises(ValueError, match="decreases"):
        V.check_prefill(np.array([0, 3, 2], np.int32), ck, table, 3, 20, 0, 8, 16, 5)
    with pytest.raises(ValueError, match="above the maximum"):
        V.check_prefill(cq, ck, table, 2, 20, 0, 8, 16, 5)
    with pytest.raises(ValueError, match="query has 4 rows"):
        V.check_prefill(cq, ck, table, 3, 20, 0, 8, 16, 4)
    with pytest.raises(ValueError, match="entries in cu_seqlens_k"):
        V.check_prefill(cq, np.array([0, 40, 42], np.int32), table, 3, 39, 0, 8, 16, 5)
    bad = table.copy()
    bad[0, 1] = 8
    with pytest.raises(ValueError, match=r"block_table\[0, 1\] = 8"):
        V.check_prefill(cq, ck, bad, 3, 20, 0, 8, 16, 5)
    # with a window the first block of sequence 0 holds no live key: -1 there is allowed
    bad[0, 0], bad[0, 1] = -1, 5
    with pytest.raises(ValueError, match=r"block_table\[0, 0\]"):
        V.check_prefill(cq, ck, bad, 3, 20, 0, 8, 16, 5)
    V.check_prefill(cq, ck, bad, 3, 20, 2, 8, 16, 5)   # rows at 17..19 attend keys 16..19
    with pytest.raises(ValueError, match=r"block_table\[0, 0\]"):
        V.check_prefill(cq, ck, bad, 3, 20, 3, 8, 16, 5)   # window 3: key 15 is live
    with pytest.raises(ValueError, match="needs block-table column 3"):
        V.check_prefill(np.array([0, 1], np.int32), np.array([0, 49], np.int32), table[:1], 1, 49, 0, 8, 16, 1)


def test_decode_violations():
    table = np.array([[2, 5], [7, -1]], np.int32)
    V.check_decode(np.array([20, 16], np.int32), table, 32, 0, 8, 16)
    with pytest.raises(ValueError, match=r"seq_lens\[1\] = 33"):
        V.check_decode(np.array([20, 33], np.int32), table, 32, 0, 8, 16)
    with pytest.raises(ValueError, match=r"block_table\[1, 1\] = -1"):
        V.check_decode(np.array([20, 17], np.int32), table, 32, 0, 8, 16)
    t2 = np.array([[-1, 5]], np.int32)
    V.check_decode(np.array([20], np.int32), t2, 32, 4, 8, 16)          # window: keys 16..19
    with pytest.raises(ValueError, match=r"block_table\[0, 0\]"):
        V.check_decode(np.array([20], np.int32), t2, 32, 5, 8, 16)      # window: key 15 is live


def test_store_fused_violations():
    table = np.array([[2, 5]], np.int32)
    # prefill of 3 new tokens at positions 17..19 of a 20-key sequence: slots 5*16 + 1..3
    cq, ck = np.array([0, 3], np.int32), np.array([0, 20], np.int32)
    V.check_prefill_with_store(np.array([81, 82, 83], np.int32), cq, ck, table, 3, 20, 0, 8, 16, 3)
    # a fused call stores every new token: a negative slot is outside its precondition
    with pytest.raises(ValueError, match=r"slot_mapping\[1\]: negative slot -1"):
        V.check_prefill_with_store(np.array([81, -1, 83], np.int32), cq, ck, table, 3, 20, 0, 8, 16, 3)
    with pytest.raises(ValueError, match="negative slot"):
        V.check_decode_with_store(np.array([-1], np.int32), np.array([20], np.int32), table, 32, 0, 8, 16)
    V.check_decode_with_store(np.array([83, -1], np.int32), np.array([20, 0], np.int32),
                              np.array([[2, 5], [1, 3]], np.int32), 32, 0, 8, 16)   # seq_len 0: no new token
    with pytest.raises(ValueError, match=r"slot_mapping\[2\]: slot 84"):
        V.check_prefill_with_store(np.array([81, 82, 84], np.int32), cq, ck, table, 3, 20, 0, 8, 16, 3)
    with pytest.raises(ValueError, match="new tokens but only"):
        V.check_prefill_with_store(np.array([0, 1, 2], np.int32), cq, np.array([0, 2], np.int32), table,
                                   3, 20, 0, 8, 16, 3)
    V.check_decode_with_store(np.array([83], np.int32), np.array([20], np.int32), table, 32, 0, 8, 16)
    with pytest.raises(ValueError, match="sits at slot 83"):
        V.check_decode_with_store(np.array([35], np.int32), np.array([20], np.int32), table, 32, 0, 8, 16)


def test_cascade_violations():
    table = np.array([[2, 5, 6], [2, 5, 1]], np.int32)
    V.check_cascade(np.array([40, 33], np.int32), table, 48, 32, 8, 16)
    with pytest.raises(ValueError, match="below common_prefix_len"):
        V.check_cascade(np.array([40, 20], np.int32), table, 48, 32, 8, 16)
    bad = table.copy()
    bad[1, 1] = 4
    with pytest.raises(ValueError, match=r"block_table\[1, 1\] = 4 differs"):
        V.check_cascade(np.array([40, 33], np.int32), bad, 48, 32, 8, 16)


def test_cascade_prefill_workload_passes_and_violations_raise():
    wl = W.shared_prefix_prefill(seed=7, num_seqs=3, prefix=64, lo=64, hi=150, chunk=20, num_heads=4,
                                 num_kv_heads=2, head_size=64)
    pre = wl.phases[0][1]
    args = (pre.cu_seqlens_q, pre.cu_seqlens_k, pre.block_table, pre.max_seqlen_q, pre.max_seqlen_k)
    V.check_cascade_prefill(*args, 64, wl.num_blocks, wl.block_size, pre.query.shape[0])
    table = np.array([[2, 5, 6], [2, 5, 1]], np.int32)
    cu_q = np.array([0, 4, 10], np.int32)
    V.check_cascade_prefill(cu_q, np.array([0, 40, 80], np.int32), table, 6, 40, 32, 8, 16, 10)
    # second sequence: 30 keys with 6 query rows -> first row at 24, inside a 32-key prefix
    with pytest.raises(ValueError, match="inside the shared prefix"):
        V.check_cascade_prefill(cu_q, np.array([0, 40, 70], np.int32), table, 6, 40, 32, 8, 16, 10)
    bad = table.copy()
    bad[1, 1] = 4
    with pytest.raises(ValueError, match=r"block_table\[1, 1\] = 4 differs"):
        V.check_cascade_prefill(cu_q, np.array([0, 40, 80], np.int32), bad, 6, 40, 32, 8, 16, 10)

"""Seeded input generators: the pages' cumulative-length examples, the slot formula, and
the structure of the five workloads (small ones built here; the big ones are only sized)."""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import workloads as W


def test_cu_seqlens_examples(golden_dir):
    with open(os.path.join(golden_dir, "cu_seqlens_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            lens, cu = line.split(":")
            got = W.cu_seqlens([int(x) for x in lens.split()])
            assert got.dtype == np.int32
            assert got.tolist() == [int(x) for x in cu.split()]


def test_slot_mapping_formula_walk():
    table = np.array([7, 2, 9, -1], dtype=np.int32)
    got = W.slot_mapping(table, context_len=14, query_len=5, block_size=8)
    expect = []
    for i in range(5):
        pos = 14 + i
        expect.append(int(table[pos // 8]) * 8 + pos % 8)
    assert got.tolist() == expect == [2 * 8 + 6, 2 * 8 + 7, 9 * 8 + 0, 9 * 8 + 1, 9 * 8 + 2]


def _check_structure(wl):
    nb = wl.num_blocks
    used = wl.tables[wl.tables >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < nb
    for ph in wl.phases:
        for op in ph:
            if isinstance(op, W.StoreOp):
                s = op.slot_mapping[op.slot_mapping >= 0]
                assert len(np.unique(s)) == len(s) and s.max() < nb * wl.block_size
                assert op.key.shape == op.value.shape == (len(op.slot_mapping), wl.num_kv_heads, wl.head_size)
            if isinstance(op, W.PrefillOp):
                assert op.query.shape == (op.cu_seqlens_q[-1], wl.num_heads, wl.head_size)
                assert (np.diff(op.cu_seqlens_k) >= np.diff(op.cu_seqlens_q)).all()
            if isinstance(op, W.DecodeOp):
                assert op.query.shape == (len(op.seq_lens), wl.num_heads, wl.head_size)
                for r, n in enumerate(op.seq_lens):
                    assert (op.block_table[r, :math.ceil(n / wl.block_size)] >= 0).all()
            if isinstance(op, W.CopyOp):
                src, dst = op.pairs[:, 0], op.pairs[:, 1]
                assert not np.isin(dst, used).any() and np.isin(src, used).all()
                assert len(np.unique(dst)) == len(dst)


def test_config1_structure():
    wl = W.config(1)
    assert wl.dtype == torch.float32 and wl.num_blocks == 8 and wl.scale == 1 / 8
    assert len(wl.phases) == 5
    pre = wl.phases[0][1]
    assert pre.cu_seqlens_q.tolist() == [0, 5, 18] == pre.cu_seqlens_k.tolist()
    lens = [ph[1].seq_lens.tolist() for ph in wl.phases[1:]]
    assert lens == [[6, 14], [7, 15], [8, 16], [9, 17]]
    _check_structure(wl)


def test_small_custom_build_is_deterministic():
    seqs = [W.SeqSpec(3, [4, 1], ["prefill", "decode"]), W.SeqSpec(0, [0, 1], [None, "decode"]),
            W.SeqSpec(20, [1], ["decode"])]
    a = W.build("t", 5, seqs, num_heads=4, num_kv_heads=2, head_size=64, block_size=16, dtype=torch.bfloat16)
    b = W.build("t", 5, seqs, num_heads=4, num_kv_heads=2, head_size=64, block_size=16, dtype=torch.bfloat16)
    assert torch.equal(a.kv_cache.view(torch.int16), b.kv_cache.view(torch.int16))
    _check_structure(a)
    dec = a.phases[0][-1]
    assert dec.seq_lens.tolist() == [21]
    assert a.phases[1][-1].seq_lens.tolist() == [8, 1]


@pytest.mark.slow
@pytest.mark.parametrize("n", [2, 3])
def test_headline_configs_structure(n):
    wl = W.config(n)
    _check_structure(wl)
    if n == 2:
        dec = wl.phases[0][-1]
        assert len(dec.seq_lens) == 64 and dec.seq_lens.min() >= 513 and dec.seq_lens.max() <= 4097
    else:
        pre = wl.phases[0][-1]
        assert len(pre.cu_seqlens_q) == 17 and (pre.cu_seqlens_q == pre.cu_seqlens_k).all()

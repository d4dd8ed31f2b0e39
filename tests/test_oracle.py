"""Pins for the fp64 oracle: the pages' worked examples, independent formulations of the
mask, textbook special cases, closed forms and invariants.  CPU only."""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import (hf_style_mask, paged_from_contiguous, parse_mask_golden,
                           sdpa_style_mask)


# ----------------------------------------------------------------------------- mask pins


@pytest.mark.parametrize("fname", ["mask_sk8_sq4_w6.txt", "mask_sk5_sq3_w2.txt"])
def test_mask_worked_examples(golden_dir, fname):
    meta, grids = parse_mask_golden(os.path.join(golden_dir, fname))
    sq, sk, w = meta["seqlen_q"], meta["seqlen_k"], meta["sliding_window"]
    assert grids["causal"].shape == (sq, sk)
    assert grids["window"].shape == (sq, sk)
    np.testing.assert_array_equal(oracle.allowed_mask(sq, sk, 0), grids["causal"])
    np.testing.assert_array_equal(oracle.allowed_mask(sq, sk, w), grids["combined"])
    # window grid alone = the lower bound of the oracle's key range
    for i in range(sq):
        lo, _ = oracle.key_range(i, sq, sk, w)
        np.testing.assert_array_equal(grids["window"][i], np.arange(sk) >= lo)


def test_mask_matches_triu_tril_construction():
    """Brute force: the range rule equals HF's triu/tril bias for every small shape with
    seqlen_q <= seqlen_k; HF's window of 1 means "no window", our 0."""
    for sk in range(1, 12):
        for sq in range(1, sk + 1):
            for w in [1] + list(range(2, 14)):
                ours = oracle.allowed_mask(sq, sk, w if w > 1 else 0)
                np.testing.assert_array_equal(ours, hf_style_mask(sq, sk, w), err_msg=f"{sq} {sk} {w}")


def test_mask_matches_sdpa_sliding_window_bias():
    for L in range(1, 12):
        np.testing.assert_array_equal(oracle.allowed_mask(L, L, 0), sdpa_style_mask(L, None))
        for w in range(1, 14):
            np.testing.assert_array_equal(oracle.allowed_mask(L, L, w), sdpa_style_mask(L, w))


def test_window_of_one_is_self_only_and_counts_w_keys():
    for sk in range(1, 10):
        for sq in range(1, sk + 1):
            m = oracle.allowed_mask(sq, sk, 1)
            assert (m.sum(axis=1) == 1).all()
            for w in range(1, 12):
                m = oracle.allowed_mask(sq, sk, w)
                off = sk - sq
                expect = np.minimum(w, off + np.arange(sq) + 1)
                np.testing.assert_array_equal(m.sum(axis=1), expect)


# ----------------------------------------------------------------------------- store / copy


def test_store_worked_example(golden_dir):
    meta, placed, slots = {}, [], None
    with open(os.path.join(golden_dir, "store_example.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "slot_mapping":
                slots = np.array([int(x) for x in parts[1:]], dtype=np.int32)
            elif parts[0] == "placed":
                placed.append(tuple(int(x) for x in parts[1:]))
            else:
                meta[parts[0]] = int(parts[1])
    T, H, D = meta["num_tokens"], meta["num_kv_heads"], meta["head_dim"]
    NB, BS = meta["num_blocks"], meta["block_size"]
    rng = np.random.default_rng(0)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    cache = np.zeros((2, NB, BS, H, D), dtype=np.float32)
    out = oracle.store_kv(cache, k, v, slots)
    expect = np.zeros_like(cache)
    for t, b, o in placed:
        expect[0, b, o] = k[t]
        expect[1, b, o] = v[t]
    np.testing.assert_array_equal(out, expect)
    assert not np.shares_memory(out, cache) and not cache.any()


def test_store_is_bitwise_and_skips_all_negative_slots():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=(2, 5, 4, 3, 8), dtype=np.uint16)   # includes NaN patterns
    k = rng.integers(0, 1 << 16, size=(6, 3, 8), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(6, 3, 8), dtype=np.uint16)
    slots = np.array([19, -1, 0, -2, 7, 12], dtype=np.int32)
    out = oracle.store_kv(bits, k, v, slots)
    exp = bits.copy()
    for t, s in enumerate(slots):
        if s >= 0:
            exp[0, s // 4, s % 4] = k[t]
            exp[1, s // 4, s % 4] = v[t]
    assert out.dtype == np.uint16
    np.testing.assert_array_equal(out, exp)


def test_copy_blocks_reads_pre_call_state():
    rng = np.random.default_rng(2)
    cache = rng.integers(0, 1 << 16, size=(2, 6, 4, 2, 8), dtype=np.uint16)
    out = oracle.copy_blocks(cache, np.array([[0, 3], [3, 5], [1, 4]]))
    np.testing.assert_array_equal(out[:, 3], cache[:, 0])
    np.testing.assert_array_equal(out[:, 5], cache[:, 3])      # old contents of block 3
    np.testing.assert_array_equal(out[:, 4], cache[:, 1])
    for b in (0, 1, 2):
        np.testing.assert_array_equal(out[:, b], cache[:, b])


# ----------------------------------------------------------------------------- attention cases


def _random_case(seed, seq_specs, H, Hkv, D, BS, extra_blocks=3, fill=0.0):
    """seq_specs = [(seqlen_q, seqlen_k)]; keys are positions 0..sk-1, queries the last sq."""
    rng = np.random.default_rng(seed)
    ks = [rng.standard_normal((sk, Hkv, D)) for _, sk in seq_specs]
    vs = [rng.standard_normal((sk, Hkv, D)) for _, sk in seq_specs]
    cache, table = paged_from_contiguous(ks, vs, BS, rng, extra_blocks=extra_blocks, fill=fill)
    tq = sum(sq for sq, _ in seq_specs)
    q = rng.standard_normal((tq, H, D))
    cu_q = np.concatenate([[0], np.cumsum([sq for sq, _ in seq_specs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([sk for _, sk in seq_specs])]).astype(np.int32)
    return dict(q=q, cache=cache, table=table, cu_q=cu_q, cu_k=cu_k, ks=ks, vs=vs)


def _sdpa(q, k, v, allowed, scale):
    """torch SDPA in float64 on contiguous K/V: q [sq, H, D], k/v [sk, H, D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(allowed), scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 2), (8, 1)])
@pytest.mark.parametrize("w", [0, 3, 7])
def test_matches_dense_sdpa_on_contiguous_kv(H, Hkv, w):
    specs = [(5, 5), (1, 9), (7, 20), (13, 13), (3, 17)]
    c = _random_case(10 + H + w, specs, H, Hkv, 16, 4)
    scale = 0.37
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], scale, Hkv, w)
    for s, (sq, sk) in enumerate(specs):
        q = c["q"][c["cu_q"][s]:c["cu_q"][s + 1]]
        k = np.repeat(c["ks"][s], H // Hkv, axis=1)
        v = np.repeat(c["vs"][s], H // Hkv, axis=1)
        ref = _sdpa(q, k, v, hf_style_mask(sq, sk, w if w > 0 else 1), scale)
        np.testing.assert_allclose(out[c["cu_q"][s]:c["cu_q"][s + 1]], ref, rtol=1e-12, atol=1e-12)


def test_square_causal_matches_sdpa_is_causal():
    c = _random_case(3, [(11, 11)], 4, 4, 8, 2)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 4, 0)
    qt = torch.from_numpy(c["q"]).permute(1, 0, 2)[None]
    kt = torch.from_numpy(c["ks"][0]).permute(1, 0, 2)[None]
    vt = torch.from_numpy(c["vs"][0]).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.5)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_closed_forms():
    H, Hkv, D, BS = 4, 2, 8, 4
    specs = [(3, 10), (6, 6), (1, 13)]
    for w in (0, 1, 2, 5):
        c = _random_case(20 + w, specs, H, Hkv, D, BS)
        # q = 0: plain mean of the allowed value rows (pins the window's extent)
        out = oracle.prefill_varlen(np.zeros_like(c["q"]), c["cache"], c["table"], c["cu_q"], c["cu_k"], 1.0, Hkv, w)
        for s, (sq, sk) in enumerate(specs):
            for i in range(sq):
                lo, hi = oracle.key_range(i, sq, sk, w)
                for h in range(H):
                    exp = c["vs"][s][lo:hi + 1, h // (H // Hkv)].mean(axis=0)
                    np.testing.assert_allclose(out[c["cu_q"][s] + i, h], exp, rtol=1e-13, atol=1e-13)
        # window of one: the value row at the query's own position
        if w == 1:
            out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.3, Hkv, 1)
            for s, (sq, sk) in enumerate(specs):
                for i in range(sq):
                    p = sk - sq + i
                    for h in range(H):
                        np.testing.assert_array_equal(out[c["cu_q"][s] + i, h], c["vs"][s][p, h // (H // Hkv)])
    # every allowed value row equal to a constant -> that constant
    c = _random_case(30, specs, H, Hkv, D, BS)
    const = np.arange(D, dtype=np.float64) - 2.5
    c["cache"][1, :, :, :, :] = const
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.7, Hkv, 0)
    np.testing.assert_allclose(out, np.broadcast_to(const, out.shape), rtol=1e-14, atol=1e-14)
    # a single key: its value row, whatever the query
    c = _random_case(31, [(1, 1)], H, Hkv, D, BS)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 3.0, Hkv, 0)
    for h in range(H):
        np.testing.assert_array_equal(out[0, h], c["vs"][0][0, h // (H // Hkv)])
    # very large scale with distinct scores: the value row of the best-scoring key
    c = _random_case(32, [(4, 9)], H, Hkv, D, BS)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 1e6, Hkv, 0)
    for i in range(4):
        lo, hi = oracle.key_range(i, 4, 9, 0)
        for h in range(H):
            g = h // (H // Hkv)
            best = lo + int(np.argmax(c["ks"][0][lo:hi + 1, g] @ c["q"][i, h]))
            np.testing.assert_allclose(out[i, h], c["vs"][0][best, g], rtol=1e-12, atol=1e-12)


def test_empty_rows_and_sequences_write_zero():
    # seqlen_q > seqlen_k: rows with p < 0 have no key (documented reading); zero-length seqs no-op
    c = _random_case(40, [(4, 2), (0, 5), (2, 2)], 2, 1, 8, 4)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 1.0, 1, 0)
    assert not out[0:2].any()
    assert out[2:4].any() and out[4:6].any()
    dec = oracle.decode(c["q"][:3], c["cache"], c["table"], np.array([2, 0, 2]), 1.0, 1)
    assert not dec[1].any() and dec[0].any()


# ----------------------------------------------------------------------------- invariants


def test_softmax_rows_sum_to_one_and_mask_is_exact_zero():
    c = _random_case(50, [(5, 12), (7, 7)], 4, 2, 8, 4)
    for w in (0, 4):
        for t in range(12):
            for h in range(4):
                p, s = oracle.attention_probs(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.6, 2, w, t, h)
                sq = c["cu_q"][s + 1] - c["cu_q"][s]
                sk = c["cu_k"][s + 1] - c["cu_k"][s]
                i = t - c["cu_q"][s]
                assert abs(p.sum() - 1.0) < 1e-12
                allowed = oracle.allowed_mask(sq, sk, w)[i]
                assert (p[~allowed] == 0).all() and (p[allowed] > 0).all()


def test_row_form_equals_batched_form():
    c = _random_case(51, [(5, 12), (7, 7), (1, 30)], 6, 3, 16, 4)
    full = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.25, 3, 6)
    picks = [(t, h) for t in range(13) for h in range(6)]
    rows = oracle.attention_rows(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.25, 3, 6, picks)
    np.testing.assert_allclose(rows, full.reshape(-1, 16), rtol=1e-12, atol=1e-13)


def test_block_relabelling_is_bitwise_invariant():
    c = _random_case(60, [(5, 23), (9, 9)], 4, 2, 8, 4, extra_blocks=4)
    base = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.4, 2, 5)
    perm = np.random.default_rng(7).permutation(c["cache"].shape[1])
    cache2 = np.empty_like(c["cache"])
    cache2[:, perm] = c["cache"]
    table2 = np.where(c["table"] >= 0, perm[np.maximum(c["table"], 0)], -1).astype(np.int32)
    again = oracle.prefill_varlen(c["q"], cache2, table2, c["cu_q"], c["cu_k"], 0.4, 2, 5)
    np.testing.assert_array_equal(base, again)


def test_block_size_invariance():
    rng = np.random.default_rng(61)
    specs = [(5, 23), (9, 9), (1, 17)]
    ks = [rng.standard_normal((sk, 2, 8)) for _, sk in specs]
    vs = [rng.standard_normal((sk, 2, 8)) for _, sk in specs]
    q = rng.standard_normal((15, 4, 8))
    cu_q = np.array([0, 5, 14, 15], dtype=np.int32)
    cu_k = np.array([0, 23, 32, 49], dtype=np.int32)
    outs = []
    for bs in (1, 4, 8, 16, 32):
        cache, table = paged_from_contiguous(ks, vs, bs, np.random.default_rng(bs), extra_blocks=2)
        outs.append(oracle.prefill_varlen(q, cache, table, cu_q, cu_k, 0.3, 2, 6))
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-14, atol=1e-14)


def test_chunked_prefill_equals_one_shot():
    rng = np.random.default_rng(62)
    L, H, Hkv, D = 29, 4, 2, 8
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((L, H, D))
    cache, table = paged_from_contiguous([k], [v], 4, rng)
    for w in (0, 5):
        one = oracle.prefill_varlen(q, cache, table, np.array([0, L]), np.array([0, L]), 0.5, Hkv, w)
        start = 0
        for chunk in (7, 1, 12, 9):
            part = oracle.prefill_varlen(q[start:start + chunk], cache, table, np.array([0, chunk]),
                                         np.array([0, start + chunk]), 0.5, Hkv, w)
            np.testing.assert_allclose(part, one[start:start + chunk], rtol=1e-13, atol=1e-13)
            start += chunk


def test_decode_equals_last_row_of_prefill():
    rng = np.random.default_rng(63)
    lens = [1, 16, 17, 40]
    ks = [rng.standard_normal((n, 2, 8)) for n in lens]
    vs = [rng.standard_normal((n, 2, 8)) for n in lens]
    cache, table = paged_from_contiguous(ks, vs, 16, rng)
    qd = rng.standard_normal((4, 6, 8))
    for w in (0, 3, 20):
        dec = oracle.decode(qd, cache, table, np.array(lens), 0.8, 2, w)
        for s, n in enumerate(lens):
            qp = np.zeros((n, 6, 8)); qp[-1] = qd[s]
            pre = oracle.prefill_varlen(qp, cache, table[s:s + 1], np.array([0, n]), np.array([0, n]), 0.8, 2, w)
            np.testing.assert_allclose(dec[s], pre[-1], rtol=1e-13, atol=1e-13)


def test_gqa_equals_explicitly_duplicated_kv_heads():
    c = _random_case(64, [(5, 11), (3, 3)], 6, 2, 8, 4)
    gqa = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, 0)
    dup = np.repeat(c["cache"], 3, axis=3)      # KV head g -> heads 3g, 3g+1, 3g+2
    mha = oracle.prefill_varlen(c["q"], dup, c["table"], c["cu_q"], c["cu_k"], 0.5, 6, 0)
    np.testing.assert_array_equal(gqa, mha)
    # a different head->KV-head assignment must change the result
    alt = np.tile(c["cache"], (1, 1, 1, 3, 1))  # head h -> KV head h % 2
    assert not np.allclose(oracle.prefill_varlen(c["q"], alt, c["table"], c["cu_q"], c["cu_k"], 0.5, 6, 0), gqa)


def test_shared_blocks_equal_private_copies():
    rng = np.random.default_rng(65)
    k = rng.standard_normal((20, 2, 8)); v = rng.standard_normal((20, 2, 8))
    cache, table = paged_from_contiguous([k, k], [v, v], 4, rng)
    shared = table.copy(); shared[1] = shared[0]
    q = rng.standard_normal((2, 4, 8))
    a = oracle.decode(q, cache, table, np.array([20, 18]), 0.5, 2)
    b = oracle.decode(q, cache, shared, np.array([20, 18]), 0.5, 2)
    np.testing.assert_array_equal(a, b)


def test_poison_outside_live_keys_is_never_read():
    c = _random_case(66, [(3, 13), (2, 6)], 4, 2, 8, 4, extra_blocks=3, fill=np.nan)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, 4)
    assert np.isfinite(out).all()
    # also NaN at keys before the window start of every row
    for s, (sq, sk) in enumerate([(3, 13), (2, 6)]):
        lo, _ = oracle.key_range(0, sq, sk, 4)
        for j in range(lo):
            c["cache"][:, c["table"][s, j // 4], j % 4] = np.nan
    out2 = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, 4)
    np.testing.assert_array_equal(out, out2)


def test_scale_enters_once_as_final_factor():
    c = _random_case(67, [(4, 9)], 2, 2, 8, 4)
    a = oracle.prefill_varlen(c["q"] * 2.0, c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.25, 2, 0)
    b = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, 0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    assert math.isclose(1 / math.sqrt(64), 0.125)


# ----------------------------------------------------------------------------- ALiBi pins


def _alibi_slopes(H):
    # the geometric slopes of the ALiBi paper for a power-of-two head count: 2^(-8 i / H)
    return np.array([2.0 ** (-8.0 * (i + 1) / H) for i in range(H)])


def _pages_alibi_attention(q, k, v, slopes, scale, hf_style=False):
    """Square causal prompt on contiguous K/V with the pages' bias construction: the
    position differences bias[i, j] = j - i (or HF's j, which the pages say gives the same
    result), times each head's slope, plus the -inf strict upper triangle, added to
    scale * q.K^T; then softmax and the value rows.  q [L, H, D], k/v [L, H, D]."""
    L, H, _ = q.shape
    pos = np.arange(L, dtype=np.float64)
    bias = np.broadcast_to(pos[None, :], (L, L)).copy() if hf_style else pos[None, :] - pos[:, None]
    bias = bias[None] * slopes[:, None, None]                              # [H, L, L]
    inf_mask = np.triu(np.full((L, L), -np.inf), k=1)
    z = scale * np.einsum("ihd,jhd->hij", q, k) + bias + inf_mask[None]
    w = np.exp(z - z.max(axis=2, keepdims=True))
    w /= w.sum(axis=2, keepdims=True)
    return np.einsum("hij,jhd->ihd", w, v)


def test_alibi_matches_the_pages_bias_construction():
    H, Hkv, D, BS = 8, 2, 16, 4
    specs = [(9, 9), (14, 14), (1, 1)]
    c = _random_case(40, specs, H, Hkv, D, BS)
    slopes = _alibi_slopes(H)
    out = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.25, Hkv, 0,
                                alibi_slopes=slopes)
    for s, (sq, sk) in enumerate(specs):
        q = c["q"][c["cu_q"][s]:c["cu_q"][s + 1]]
        k = np.repeat(c["ks"][s], H // Hkv, axis=1)
        v = np.repeat(c["vs"][s], H // Hkv, axis=1)
        for hf in (False, True):
            ref = _pages_alibi_attention(q, k, v, slopes, 0.25, hf_style=hf)
            np.testing.assert_allclose(out[c["cu_q"][s]:c["cu_q"][s + 1]], ref, rtol=1e-11, atol=1e-12)


def test_alibi_zero_slopes_is_plain_attention():
    specs = [(3, 10), (6, 6), (1, 13)]
    c = _random_case(41, specs, 4, 2, 8, 4)
    for w in (0, 3):
        a = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, w)
        b = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.5, 2, w,
                                  alibi_slopes=np.zeros(4))
        np.testing.assert_array_equal(a, b)


def test_alibi_closed_forms():
    """q = 0: the weights are exp(slope * (j - p)), a geometric sequence over the allowed
    keys j in [lo, p], so out = sum_j r^(p-j) v_j / sum_j r^(p-j) with r = exp(-slope); a
    huge slope leaves only the query's own key.  Chunked rows and a window included."""
    H, Hkv, D, BS = 4, 2, 8, 4
    specs = [(3, 10), (6, 6), (1, 13)]
    slopes = np.array([0.3, 1.1, 0.05, 2.0])
    for w in (0, 4):
        c = _random_case(42 + w, specs, H, Hkv, D, BS)
        out = oracle.prefill_varlen(np.zeros_like(c["q"]), c["cache"], c["table"], c["cu_q"], c["cu_k"],
                                    1.0, Hkv, w, alibi_slopes=slopes)
        for s, (sq, sk) in enumerate(specs):
            for i in range(sq):
                lo, hi = oracle.key_range(i, sq, sk, w)
                p = sk - sq + i
                assert hi == p
                for h in range(H):
                    r = math.exp(-slopes[h])
                    n = p - lo + 1
                    wts = r ** np.arange(n - 1, -1, -1)          # keys lo..p: r^(p-j)
                    denom = (1 - r ** n) / (1 - r)                # geometric series
                    exp = (wts[:, None] * c["vs"][s][lo:p + 1, h // (H // Hkv)]).sum(axis=0) / denom
                    np.testing.assert_allclose(out[c["cu_q"][s] + i, h], exp, rtol=1e-12, atol=1e-13)
        big = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.1, Hkv, w,
                                    alibi_slopes=np.full(H, 1e4))
        for s, (sq, sk) in enumerate(specs):
            for i in range(sq):
                p = sk - sq + i
                for h in range(H):
                    np.testing.assert_allclose(big[c["cu_q"][s] + i, h], c["vs"][s][p, h // (H // Hkv)],
                                               rtol=0, atol=1e-12)


def test_alibi_decode_and_rows_agree_with_prefill():
    specs = [(1, 7), (1, 1), (1, 20)]
    c = _random_case(43, specs, 4, 2, 8, 4)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    lens = np.array([sk for _, sk in specs])
    d = oracle.decode(c["q"], c["cache"], c["table"], lens, 0.4, 2, 5, alibi_slopes=slopes)
    p = oracle.prefill_varlen(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.4, 2, 5, alibi_slopes=slopes)
    np.testing.assert_array_equal(d, p)
    picks = [(t, h) for t in range(3) for h in range(4)]
    rows = oracle.attention_rows(c["q"], c["cache"], c["table"], c["cu_q"], c["cu_k"], 0.4, 2, 5, picks,
                                 alibi_slopes=slopes)
    np.testing.assert_allclose(rows, np.stack([p[t, h] for t, h in picks]), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- cascade pins


def _shared_prefix_case(seed, lens, P, H, Hkv, D, BS):
    """Sequences whose first ``P`` keys are the same rows, paged with the prefix blocks shared:
    every block-table row starts with the first sequence's prefix blocks."""
    rng = np.random.default_rng(seed)
    kp = rng.standard_normal((P, Hkv, D)); vp = rng.standard_normal((P, Hkv, D))
    ks = [np.concatenate([kp, rng.standard_normal((n - P, Hkv, D))]) for n in lens]
    vs = [np.concatenate([vp, rng.standard_normal((n - P, Hkv, D))]) for n in lens]
    cache, table = paged_from_contiguous(ks, vs, BS, rng, extra_blocks=2)
    table[1:, :P // BS] = table[0, :P // BS]
    q = rng.standard_normal((len(lens), H, D))
    return q, cache, table, ks, vs


@pytest.mark.parametrize("P,lens", [(8, [8, 9, 21, 30]), (12, [40, 12, 13]), (0, [5, 17]), (16, [16])])
def test_cascade_equals_dense_attention_and_plain_decode(P, lens):
    # vLLM learning book, section 8: the cascade split is mathematically equivalent to plain
    # attention; checked against torch SDPA on the contiguous keys and against plain decode
    H, Hkv, D, BS = 6, 2, 8, 4
    q, cache, table, ks, vs = _shared_prefix_case(80 + P, lens, P, H, Hkv, D, BS)
    out = oracle.cascade_decode(q, cache, table, np.array(lens), 0.4, Hkv, P)
    for s, n in enumerate(lens):
        k = np.repeat(ks[s], H // Hkv, axis=1); v = np.repeat(vs[s], H // Hkv, axis=1)
        ref = _sdpa(q[s:s + 1], k, v, np.ones((1, n), dtype=bool), 0.4)
        np.testing.assert_allclose(out[s], ref[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, oracle.decode(q, cache, table, np.array(lens), 0.4, Hkv),
                               rtol=1e-12, atol=1e-12)


def test_cascade_uniform_weights_closed_form():
    # q = 0 gives every key the same weight: each output is the mean of all n value rows,
    # so the prefix part must count P / n of it and the own part (n - P) / n
    H, Hkv, D, BS, P = 4, 4, 8, 4, 12
    lens = [13, 20, 40]
    q, cache, table, ks, vs = _shared_prefix_case(91, lens, P, H, Hkv, D, BS)
    out = oracle.cascade_decode(np.zeros_like(q), cache, table, np.array(lens), 0.7, Hkv, P)
    for s in range(len(lens)):
        np.testing.assert_allclose(out[s], vs[s].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_merge_partials_of_any_split_is_the_whole_softmax():
    rng = np.random.default_rng(92)
    k = rng.standard_normal((11, 8)); v = rng.standard_normal((11, 8)); q = rng.standard_normal(8)
    z = 0.6 * (k @ q)
    whole = (np.exp(z - z.max()) / np.exp(z - z.max()).sum()) @ v
    for cuts in ([0, 4, 11], [0, 0, 7, 11], [0, 1, 2, 11, 11]):
        parts = [oracle.partial_attention(q, k[a:b], v[a:b], 0.6) for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_allclose(oracle.merge_partials(parts), whole, rtol=1e-13, atol=1e-13)
    empty = oracle.partial_attention(q, k[:0], v[:0], 0.6)
    assert empty[1] == -np.inf and not empty[0].any()
    assert not oracle.merge_partials([empty, empty]).any()


def test_cascade_rejects_what_is_not_a_shared_prefix():
    H, Hkv, D, BS, P = 4, 2, 8, 4, 8
    q, cache, table, _, _ = _shared_prefix_case(93, [9, 12], P, H, Hkv, D, BS)
    with pytest.raises(ValueError):
        oracle.cascade_decode(q, cache, table, np.array([9, 12]), 0.5, Hkv, 6)      # not whole blocks
    with pytest.raises(ValueError):
        oracle.cascade_decode(q, cache, table, np.array([9, 12]), 0.5, Hkv, 12)     # 9 < 12
    bad = table.copy(); bad[1, 1] = table[1, 2]
    with pytest.raises(ValueError):
        oracle.cascade_decode(q, cache, bad, np.array([9, 12]), 0.5, Hkv, P)        # block not shared


# ----------------------------------------------------------------------------- cascade prefill pins


def _shared_prefix_chunks(seed, specs, P, H, Hkv, D, BS):
    """Query chunks over sequences that share their first ``P`` keys (prefix blocks shared by
    every block-table row): specs = [(seqlen_q, seqlen_k)], each with seqlen_k - seqlen_q >= P."""
    lens = [sk for _, sk in specs]
    q_all, cache, table, ks, vs = _shared_prefix_case(seed, lens, P, H, Hkv, D, BS)
    rng = np.random.default_rng(seed + 1000)
    q = rng.standard_normal((sum(sq for sq, _ in specs), H, D))
    cu_q = np.concatenate([[0], np.cumsum([sq for sq, _ in specs])]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, cache, table, cu_q, cu_k, ks, vs


CASCADE_PREFILL_SPECS = {
    # name: (P, [(seqlen_q, seqlen_k)])
    "chunks": (8, [(4, 12), (1, 9), (7, 30), (3, 11)]),
    "long_prefix": (16, [(5, 21), (2, 40)]),
    "no_prefix": (0, [(3, 3), (5, 9)]),
    "exact_context": (12, [(6, 18), (12, 24)]),
}


@pytest.mark.parametrize("name", sorted(CASCADE_PREFILL_SPECS))
def test_cascade_prefill_equals_sdpa_and_plain_prefill(name):
    # vLLM learning book, section 8: the split into the shared segment (all queries of the batch
    # together) and each request's own segment is mathematically equivalent to plain attention;
    # checked against torch SDPA on the contiguous keys with the bottom-right causal mask, and
    # against plain prefill_varlen on the same paged cache
    P, specs = CASCADE_PREFILL_SPECS[name]
    H, Hkv, D, BS = 6, 2, 8, 4
    q, cache, table, cu_q, cu_k, ks, vs = _shared_prefix_chunks(120 + P, specs, P, H, Hkv, D, BS)
    out = oracle.cascade_prefill_varlen(q, cache, table, cu_q, cu_k, 0.45, Hkv, P)
    for s, (sq, sk) in enumerate(specs):
        k = np.repeat(ks[s], H // Hkv, axis=1); v = np.repeat(vs[s], H // Hkv, axis=1)
        allowed = np.tril(np.ones((sq, sk), dtype=bool), k=sk - sq)
        ref = _sdpa(q[cu_q[s]:cu_q[s + 1]], k, v, allowed, 0.45)
        np.testing.assert_allclose(out[cu_q[s]:cu_q[s + 1]], ref, rtol=1e-12, atol=1e-12)
    plain = oracle.prefill_varlen(q, cache, table, cu_q, cu_k, 0.45, Hkv)
    np.testing.assert_allclose(out, plain, rtol=1e-12, atol=1e-12)


def test_cascade_prefill_uniform_weights_closed_form():
    # q = 0 gives every visible key the same weight: row i of a sequence (position p) is the
    # mean of value rows 0..p, so the shared segment counts P / (p + 1) of it
    H, Hkv, D, BS, P = 4, 4, 8, 4, 12
    specs = [(3, 15), (5, 20), (1, 13)]
    q, cache, table, cu_q, cu_k, ks, vs = _shared_prefix_chunks(131, specs, P, H, Hkv, D, BS)
    out = oracle.cascade_prefill_varlen(np.zeros_like(q), cache, table, cu_q, cu_k, 0.8, Hkv, P)
    for s, (sq, sk) in enumerate(specs):
        for i in range(sq):
            p = sk - sq + i
            np.testing.assert_allclose(out[cu_q[s] + i], vs[s][:p + 1].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_cascade_prefill_of_single_queries_is_cascade_decode():
    # one query per sequence: the decode form of the same split
    H, Hkv, D, BS, P = 6, 3, 8, 4, 8
    specs = [(1, 9), (1, 8), (1, 30)]
    q, cache, table, cu_q, cu_k, _, _ = _shared_prefix_chunks(141, specs, P, H, Hkv, D, BS)
    a = oracle.cascade_prefill_varlen(q, cache, table, cu_q, cu_k, 0.5, Hkv, P)
    b = oracle.cascade_decode(q, cache, table, np.array([sk for _, sk in specs]), 0.5, Hkv, P)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_cascade_prefill_rejects_what_is_not_a_shared_cached_prefix():
    H, Hkv, D, BS, P = 4, 2, 8, 4, 8
    q, cache, table, cu_q, cu_k, _, _ = _shared_prefix_chunks(151, [(2, 12), (4, 14)], P, H, Hkv, D, BS)
    with pytest.raises(ValueError):
        oracle.cascade_prefill_varlen(q, cache, table, cu_q, cu_k, 0.5, Hkv, 6)    # not whole blocks
    with pytest.raises(ValueError):
        oracle.cascade_prefill_varlen(q, cache, table, cu_q, cu_k, 0.5, Hkv, 12)   # 14 - 4 < 12
    bad = table.copy(); bad[1, 1] = table[1, 2]
    with pytest.raises(ValueError):
        oracle.cascade_prefill_varlen(q, cache, bad, cu_q, cu_k, 0.5, Hkv, P)      # block not shared

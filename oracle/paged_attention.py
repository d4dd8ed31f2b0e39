"""Plain, slow, fp64 CPU oracle for attention over a paged, block-structured KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.  It
shares no code with the HIP library (``paged_attention_block_amd``) and imports nothing
from it; both sides only consume the seeded inputs made by ``workloads``.

Every function takes numpy arrays and follows the pages' statement of the problem:

* Cache layout ``kv_cache[2, num_blocks, block_size, num_kv_heads, head_size]``; plane 0
  holds keys, plane 1 values (vLLM learning book, "05. Attention Backends",
  section 3 FlashAttentionBackend.get_kv_cache_shape; section 5 ``kv_cache.unbind(0)``).
* Store: a token whose slot is negative is skipped; otherwise the slot splits into
  ``block = slot // block_size`` and ``offset = slot % block_size`` (MinivLLM API docs,
  "Attention", section store_kvcache, parameter slot_mapping and its example).
* Block addressing: logical key ``j`` of sequence ``s`` lives in physical block
  ``block_table[s, j // block_size]`` at offset ``j % block_size`` (vLLM learning book,
  section 10 question 2, the slot_mapping / block_table formula; MinivLLM API docs,
  section paged_attention_decode, parameter block_tables).
* Mask: query row ``i`` of a sequence with ``seqlen_q`` queries and ``seqlen_k`` keys sits
  at absolute position ``p = seqlen_k - seqlen_q + i`` (bottom-right aligned causal
  diagonal of HF transformers continuous_batching ``input_ouputs.py``,
  ``build_attention_mask``); it may attend keys ``j <= p`` and, with a sliding window of
  ``W >= 1`` keys, only ``j >= p - W + 1`` (the window counts the query's own key; same
  function, and the vllm-npu 0.4.2 diff, ``torch_sdpa.py`` ``_make_sliding_window_bias``).
  ``W <= 0`` means no window.
* GQA: query head ``h`` reads KV head ``h // (num_heads // num_kv_heads)`` (vllm-npu 0.4.2
  diff, ``torch_sdpa.py`` forward, ``repeat_interleave(num_queries_per_kv, dim=1)``).
* Attention: ``out = softmax(scale * q K^T) V`` over the allowed keys; a row with no
  allowed key is written as zeros (vLLM learning book, section 5, the profile-run
  ``output.fill_(0)``; the pages leave the empty row otherwise undefined).

* ALiBi (optional ``alibi_slopes[num_heads]``): the score of query head ``h`` at position
  ``p`` for key ``j`` gets ``slope[h] * (j - p)`` added after the scale, before the softmax
  and the mask (vllm-npu 0.4.2 diff, ``torch_sdpa.py`` and ``xformers.py``
  ``_make_alibi_bias``: the bias matrix ``bias[i, j] = j - i`` times the per-head slope,
  added to the scores together with the causal ``-inf`` triangle).  Positions are the
  absolute ones of the mask above, so chunked prefill and decode use the same rule.

Decode is the same definition with one query per sequence and ``seqlen_k = seq_lens[s]``
(MinivLLM API docs, section paged_attention_decode: one query, ``context_lens`` valid
keys).  All floating-point work is fp64.

* Cascade (shared-prefix) decode: when the sequences of a batch share their first
  ``common_prefix_len`` keys through the same physical blocks, attention is taken in two
  parts, the shared prefix for all queries at once and then each sequence's own keys, and
  the parts are combined; the result equals plain decode (vLLM learning book, section 8
  Cascade Attention, the self-check question 4, and the cascade fields of section 4
  FlashAttentionMetadata).  The pages do not write out the
  combination; the one that makes the two parts equal to a softmax over their union is the
  log-sum-exp weighting of ``merge_partials``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "store_kv",
    "copy_blocks",
    "key_range",
    "allowed_mask",
    "kv_head_of",
    "gather_kv",
    "alibi_bias",
    "attention_probs",
    "attention_rows",
    "prefill_varlen",
    "decode",
    "partial_attention",
    "merge_partials",
    "cascade_split",
    "cascade_decode",
    "cascade_prefill_varlen",
]


# ----------------------------------------------------------------------------- store / copy


def store_kv(kv_cache: np.ndarray, key: np.ndarray, value: np.ndarray,
             slot_mapping: np.ndarray) -> np.ndarray:
    """Return a copy of ``kv_cache`` with token ``t``'s key/value rows written to its slot.

    MinivLLM API docs, "Attention", section store_kvcache: ``slot // block_size`` picks
    the block, ``slot % block_size`` the offset, and a slot of -1 skips the token (any
    negative slot is skipped here).  The copy is bitwise: the arrays keep their dtype.
    ``key``/``value`` are ``[num_tokens, num_kv_heads, head_size]``.
    """
    out = kv_cache.copy()
    block_size = kv_cache.shape[2]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        out[0, block, offset] = key[t]
        out[1, block, offset] = value[t]
    return out


def copy_blocks(kv_cache: np.ndarray, block_pairs) -> np.ndarray:
    """Return a copy of ``kv_cache`` in which block ``dst`` of both planes holds block ``src``.

    vllm-npu 0.4.2 diff, ``torch_sdpa.py`` / ``xformers.py``, ``copy_blocks(kv_caches,
    src_to_dists)`` (signature only on the pages).  Reading: every copy reads the cache
    as it was before the call.
    """
    before = kv_cache.copy()
    out = kv_cache.copy()
    for src, dst in block_pairs:
        out[:, int(dst)] = before[:, int(src)]
    return out


# ----------------------------------------------------------------------------- the mask


def key_range(row: int, seqlen_q: int, seqlen_k: int, sliding_window: int):
    """Inclusive key range ``(lo, hi)`` that query ``row`` may attend; empty when ``hi < lo``.

    HF transformers ``input_ouputs.py``, ``build_attention_mask``: the causal diagonal is
    offset by ``seqlen_k - seqlen_q`` so the last query sees every key; the sliding window
    keeps the ``W`` keys ending at the query's own position.
    """
    p = seqlen_k - seqlen_q + row
    hi = min(p, seqlen_k - 1)
    lo = max(0, p - sliding_window + 1) if sliding_window > 0 else 0
    return lo, hi


def allowed_mask(seqlen_q: int, seqlen_k: int, sliding_window: int) -> np.ndarray:
    """Boolean ``[seqlen_q, seqlen_k]`` matrix, True where query row ``i`` may attend key ``j``."""
    mask = np.zeros((seqlen_q, seqlen_k), dtype=bool)
    for i in range(seqlen_q):
        lo, hi = key_range(i, seqlen_q, seqlen_k, sliding_window)
        if hi >= lo:
            mask[i, lo:hi + 1] = True
    return mask


# ----------------------------------------------------------------------------- attention


def kv_head_of(head: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``head``: consecutive query heads share one KV head
    (vllm-npu 0.4.2 diff, ``torch_sdpa.py`` forward, ``repeat_interleave`` on dim 1)."""
    return head // (num_heads // num_kv_heads)


def gather_kv(kv_cache: np.ndarray, table_row: np.ndarray, positions, kv_head: int):
    """Key and value rows (fp64, ``[len(positions), head_size]``) of logical keys ``positions``.

    vLLM learning book, section 10 question 2: physical block ``table_row[j // block_size]``,
    offset ``j % block_size``.
    """
    block_size = kv_cache.shape[2]
    n = len(positions)
    head_size = kv_cache.shape[4]
    k = np.empty((n, head_size), dtype=np.float64)
    v = np.empty((n, head_size), dtype=np.float64)
    for r, j in enumerate(positions):
        block = int(table_row[j // block_size])
        offset = j % block_size
        k[r] = kv_cache[0, block, offset, kv_head]
        v[r] = kv_cache[1, block, offset, kv_head]
    return k, v


def alibi_bias(slope, key_pos, query_pos):
    """ALiBi bias ``slope * (j - p)`` for key positions ``j`` and query positions ``p``
    (numpy broadcasting; vllm-npu 0.4.2 diff, ``_make_alibi_bias``)."""
    return slope * (key_pos - query_pos)


def _locate(cu_seqlens_q: np.ndarray, token: int) -> int:
    """Sequence that owns packed query ``token`` (zero-length sequences own nothing)."""
    s = int(np.searchsorted(cu_seqlens_q, token, side="right")) - 1
    assert cu_seqlens_q[s] <= token < cu_seqlens_q[s + 1]
    return s


def attention_probs(query, kv_cache, block_table, cu_seqlens_q, cu_seqlens_k, scale,
                    num_kv_heads, sliding_window, token, head, alibi_slopes=None):
    """Softmax weights of packed query ``token``, head ``head`` over keys ``[0, seqlen_k)``.

    Masked keys get weight exactly 0.  Returns ``(probs, seq)``; ``probs`` is all zeros
    for a row with no allowed key.  ``alibi_slopes`` adds ``slope[head] * (j - p)``.
    """
    s = _locate(cu_seqlens_q, token)
    seqlen_q = int(cu_seqlens_q[s + 1] - cu_seqlens_q[s])
    seqlen_k = int(cu_seqlens_k[s + 1] - cu_seqlens_k[s])
    row = token - int(cu_seqlens_q[s])
    g = kv_head_of(head, query.shape[1], num_kv_heads)
    probs = np.zeros(seqlen_k, dtype=np.float64)
    lo, hi = key_range(row, seqlen_q, seqlen_k, sliding_window)
    if hi < lo:
        return probs, s
    k, _ = gather_kv(kv_cache, block_table[s], range(lo, hi + 1), g)
    z = float(scale) * (k @ np.asarray(query[token, head], dtype=np.float64))
    if alibi_slopes is not None:
        p = seqlen_k - seqlen_q + row
        z = z + alibi_bias(float(alibi_slopes[head]), np.arange(lo, hi + 1, dtype=np.float64), p)
    w = np.exp(z - z.max())
    probs[lo:hi + 1] = w / w.sum()
    return probs, s


def attention_rows(query, kv_cache, block_table, cu_seqlens_q, cu_seqlens_k, scale,
                   num_kv_heads, sliding_window, picks, alibi_slopes=None) -> np.ndarray:
    """Output rows ``out[token, head, :]`` (fp64) for each ``(token, head)`` in ``picks``.

    The definition, one row at a time: softmax weights from ``attention_probs`` times the
    value rows gathered through the block table.  Used at sizes where computing every
    row would take too long.
    """
    rows = []
    num_heads = query.shape[1]
    for token, head in picks:
        probs, s = attention_probs(query, kv_cache, block_table, cu_seqlens_q, cu_seqlens_k,
                                   scale, num_kv_heads, sliding_window, int(token), int(head),
                                   alibi_slopes)
        nz = np.nonzero(probs)[0]
        if len(nz) == 0:
            rows.append(np.zeros(query.shape[2], dtype=np.float64))
            continue
        lo, hi = int(nz.min()), int(nz.max())
        g = kv_head_of(int(head), num_heads, num_kv_heads)
        _, v = gather_kv(kv_cache, block_table[s], range(lo, hi + 1), g)
        rows.append(probs[lo:hi + 1] @ v)
    return np.stack(rows) if rows else np.zeros((0, query.shape[2]))


def prefill_varlen(query, kv_cache, block_table, cu_seqlens_q, cu_seqlens_k, scale,
                   num_kv_heads, sliding_window=0, alibi_slopes=None) -> np.ndarray:
    """Every output row of varlen paged attention, ``[total_q, num_heads, head_size]`` fp64.

    Same definition as ``attention_rows``, evaluated per (sequence, KV head) over the
    union of the rows' key ranges with the element mask of ``allowed_mask``: only
    numpy's summation order differs.  Covers prefill (``seqlen_q == seqlen_k``) and
    chunked prefill (``seqlen_q < seqlen_k``, MinivLLM API docs, section
    flash_attention_prefill; HF ``build_attention_mask``).
    """
    q = np.asarray(query, dtype=np.float64)
    total_q, num_heads, head_size = q.shape
    out = np.zeros((total_q, num_heads, head_size), dtype=np.float64)
    num_seqs = len(cu_seqlens_q) - 1
    for s in range(num_seqs):
        q0 = int(cu_seqlens_q[s])
        seqlen_q = int(cu_seqlens_q[s + 1]) - q0
        seqlen_k = int(cu_seqlens_k[s + 1] - cu_seqlens_k[s])
        if seqlen_q <= 0 or seqlen_k <= 0:
            continue
        mask = allowed_mask(seqlen_q, seqlen_k, sliding_window)
        cols = np.nonzero(mask.any(axis=0))[0]
        if len(cols) == 0:
            continue
        lo, hi = int(cols.min()), int(cols.max())
        mask = mask[:, lo:hi + 1]
        live_rows = mask.any(axis=1)
        for g in range(num_kv_heads):
            k, v = gather_kv(kv_cache, block_table[s], range(lo, hi + 1), g)
            heads = [h for h in range(num_heads) if kv_head_of(h, num_heads, num_kv_heads) == g]
            qg = q[q0:q0 + seqlen_q, heads, :].transpose(1, 0, 2)   # [group, seqlen_q, D]
            z = float(scale) * (qg @ k.T)                           # [group, seqlen_q, n]
            if alibi_slopes is not None:
                pos = seqlen_k - seqlen_q + np.arange(seqlen_q, dtype=np.float64)   # query positions
                keys = np.arange(lo, hi + 1, dtype=np.float64)
                sl = np.asarray(alibi_slopes, dtype=np.float64)[heads]
                z = z + alibi_bias(sl[:, None, None], keys[None, None, :], pos[None, :, None])
            z = np.where(mask[None], z, -np.inf)
            zmax = np.where(live_rows[None, :, None], z.max(axis=2, keepdims=True), 0.0)
            w = np.where(mask[None], np.exp(z - zmax), 0.0)
            denom = w.sum(axis=2, keepdims=True)
            p = np.divide(w, denom, out=np.zeros_like(w), where=denom > 0)
            out[q0:q0 + seqlen_q, heads, :] = (p @ v).transpose(1, 0, 2)
    return out


def decode(query, kv_cache, block_table, seq_lens, scale, num_kv_heads,
           sliding_window=0, alibi_slopes=None) -> np.ndarray:
    """Paged decode, ``[num_seqs, num_heads, head_size]`` fp64: one query per sequence.

    MinivLLM API docs, section paged_attention_decode: sequence ``s`` attends its
    ``seq_lens[s]`` cached keys; this is ``prefill_varlen`` with ``seqlen_q = 1``, so the
    sliding window applies to the single query too.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cu_q = np.arange(len(seq_lens) + 1, dtype=np.int64)
    cu_k = np.concatenate([[0], np.cumsum(seq_lens)])
    return prefill_varlen(query, kv_cache, block_table, cu_q, cu_k, scale, num_kv_heads,
                          sliding_window, alibi_slopes)


# ----------------------------------------------------------------------------- cascade


def partial_attention(q_row, k, v, scale):
    """Attention of one query over one part of its keys: ``(o, lse)``.

    ``o = softmax(scale * k q) v`` over the part's rows and ``lse = log sum exp(scale * k q)``;
    a part with no key gives ``(0, -inf)``.
    """
    if len(k) == 0:
        return np.zeros(v.shape[1], dtype=np.float64), -np.inf
    z = float(scale) * (k @ np.asarray(q_row, dtype=np.float64))
    zmax = z.max()
    w = np.exp(z - zmax)
    return (w / w.sum()) @ v, zmax + np.log(w.sum())


def merge_partials(parts):
    """Combine ``[(o_i, lse_i)]`` of disjoint key sets into the attention over their union.

    A softmax over the union weights part ``i`` by ``exp(lse_i)`` relative to the others:
    ``o = sum_i exp(lse_i - L) o_i`` with ``L = log sum_i exp(lse_i)``.  All parts empty gives
    the zero row of an empty softmax.
    """
    lses = np.array([lse for _, lse in parts], dtype=np.float64)
    if not np.isfinite(lses).any():
        return np.zeros_like(parts[0][0])
    top = lses[np.isfinite(lses)].max()
    w = np.exp(lses - top)
    w = w / w.sum()
    return sum(wi * o for wi, (o, _) in zip(w, parts))


def cascade_split(seq_len, common_prefix_len):
    """Key positions of the shared part and of the sequence's own part: ``[0, P)`` and
    ``[P, seq_len)`` (vLLM learning book, self-check question 4: the shared segment, then each
    request's later segment)."""
    return range(0, common_prefix_len), range(common_prefix_len, seq_len)


def cascade_decode(query, kv_cache, block_table, seq_lens, scale, num_kv_heads,
                   common_prefix_len) -> np.ndarray:
    """Shared-prefix decode, ``[num_seqs, num_heads, head_size]`` fp64.

    vLLM learning book, section 8 (Cascade Attention) and self-check question 4: (1) every
    query of the batch attends the one shared prefix, read once through the first
    sequence's block table; (2) each query attends its own sequence's keys after the prefix;
    (3) the two parts are combined (``merge_partials``).  The prefix is a whole number of
    blocks (the scheduler counts common prefix blocks), every sequence holds at least the
    prefix, and every block-table row starts with the same prefix blocks; anything else
    raises ``ValueError``.  No sliding window and no ALiBi (every prefix key is visible to
    every query with the same weight rule).
    """
    q = np.asarray(query, dtype=np.float64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_seqs, num_heads, head_size = q.shape
    block_size = kv_cache.shape[2]
    P = int(common_prefix_len)
    if P < 0 or P % block_size != 0:
        raise ValueError("common_prefix_len must be a non-negative multiple of block_size")
    nb = P // block_size
    if num_seqs and (seq_lens < P).any():
        raise ValueError("every sequence must hold the whole common prefix")
    for s in range(num_seqs):
        if not np.array_equal(block_table[s, :nb], block_table[0, :nb]):
            raise ValueError(f"sequence {s} does not share the prefix blocks")
    out = np.zeros((num_seqs, num_heads, head_size), dtype=np.float64)
    for h in range(num_heads):
        g = kv_head_of(h, num_heads, num_kv_heads)
        # (1) the shared part, for every query at once
        pre_pos, _ = cascade_split(P, P)
        kp, vp = gather_kv(kv_cache, block_table[0], pre_pos, g)
        shared = [partial_attention(q[s, h], kp, vp, scale) for s in range(num_seqs)]
        for s in range(num_seqs):
            # (2) the sequence's own part, (3) the combination
            _, own_pos = cascade_split(int(seq_lens[s]), P)
            ko, vo = gather_kv(kv_cache, block_table[s], own_pos, g)
            own = partial_attention(q[s, h], ko, vo, scale)
            out[s, h] = merge_partials([shared[s], own])
    return out


def cascade_prefill_varlen(query, kv_cache, block_table, cu_seqlens_q, cu_seqlens_k, scale,
                           num_kv_heads, common_prefix_len) -> np.ndarray:
    """Shared-prefix varlen attention, ``[total_q, num_heads, head_size]`` fp64.

    vLLM learning book, section 8 (Cascade Attention) and self-check question 4, with the
    cascade fields of section 4 FlashAttentionMetadata (``cu_prefix_query_lens``,
    ``prefix_kv_lens``, ``suffix_kv_lens``): (1) the shared segment: every query row of the
    batch, taken together as one block of rows, attends the one prefix ``[0, P)``, read once
    through the first sequence's block table; (2) each sequence's own segment: its rows attend
    its keys from ``P`` on under the causal rule of ``prefill_varlen`` (diagonal offset by
    ``seqlen_k - seqlen_q``); (3) the two parts are combined (``merge_partials``).

    Reading: the pages give the shared segment no mask.  That holds because every query row
    sits at or after the prefix's last key (``seqlen_k - seqlen_q >= P - 1``: the prefix lies in
    the sequence's cached context, or ends at its first new token; for one query per sequence
    this is ``seq_lens >= P`` as in ``cascade_decode``), so it may attend all of the prefix.  The
    prefix is whole blocks and every block-table row starts with the same prefix blocks;
    anything else raises ``ValueError``.  No sliding window and no ALiBi.
    """
    q = np.asarray(query, dtype=np.float64)
    total_q, num_heads, head_size = q.shape
    block_size = kv_cache.shape[2]
    P = int(common_prefix_len)
    if P < 0 or P % block_size != 0:
        raise ValueError("common_prefix_len must be a non-negative multiple of block_size")
    num_seqs = len(cu_seqlens_q) - 1
    nb = P // block_size
    for s in range(num_seqs):
        seqlen_q = int(cu_seqlens_q[s + 1] - cu_seqlens_q[s])
        seqlen_k = int(cu_seqlens_k[s + 1] - cu_seqlens_k[s])
        if seqlen_k - seqlen_q + 1 < P:
            raise ValueError(f"sequence {s}: its first query row lies inside the shared prefix")
        if not np.array_equal(block_table[s, :nb], block_table[0, :nb]):
            raise ValueError(f"sequence {s} does not share the prefix blocks")
    out = np.zeros((total_q, num_heads, head_size), dtype=np.float64)
    # (1) the shared segment's keys, once for the whole batch
    pre_pos, _ = cascade_split(P, P)
    shared_kv = [gather_kv(kv_cache, block_table[0], pre_pos, g) for g in range(num_kv_heads)]
    for s in range(num_seqs):
        q0 = int(cu_seqlens_q[s])
        seqlen_q = int(cu_seqlens_q[s + 1]) - q0
        seqlen_k = int(cu_seqlens_k[s + 1] - cu_seqlens_k[s])
        own_kv = [gather_kv(kv_cache, block_table[s], range(P, seqlen_k), g) for g in range(num_kv_heads)]
        for i in range(seqlen_q):
            lo, hi = key_range(i, seqlen_q, seqlen_k, 0)
            for h in range(num_heads):
                g = kv_head_of(h, num_heads, num_kv_heads)
                kp, vp = shared_kv[g]
                ko, vo = own_kv[g]
                prefix_pos, own_pos = cascade_split(hi + 1, P)
                # the parts are ranges of positions: the rows gathered above, sliced
                shared = partial_attention(q[q0 + i, h], kp[prefix_pos.start:prefix_pos.stop],
                                           vp[prefix_pos.start:prefix_pos.stop], scale)
                own = partial_attention(q[q0 + i, h], ko[own_pos.start - P:own_pos.stop - P],
                                        vo[own_pos.start - P:own_pos.stop - P], scale)
                out[q0 + i, h] = merge_partials([shared, own])
    return out


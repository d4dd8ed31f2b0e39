"""Test-side helpers: paged layouts built from contiguous K/V, golden-file parsing."""

from __future__ import annotations

import numpy as np

ALLOW, MASK = "█", "░"


def paged_from_contiguous(k_seqs, v_seqs, block_size, perm_rng=None, extra_blocks=0,
                          fill=0.0, dtype=np.float64):
    """Lay per-sequence contiguous keys/values ``[L_s, Hkv, D]`` into a paged cache.

    Returns ``(kv_cache [2, NB, BS, Hkv, D], block_table [B, MB] int32)``; physical blocks
    are handed out in the order of a permutation drawn from ``perm_rng`` (identity when
    None), unused slots and blocks hold ``fill``, table padding is -1.
    """
    hkv, d = k_seqs[0].shape[1], k_seqs[0].shape[2]
    nblk = [max(1, -(-len(k) // block_size)) for k in k_seqs]
    nb = sum(nblk) + extra_blocks
    order = np.arange(nb) if perm_rng is None else perm_rng.permutation(nb)
    cache = np.full((2, nb, block_size, hkv, d), fill, dtype=dtype)
    table = np.full((len(k_seqs), max(nblk)), -1, dtype=np.int32)
    cur = 0
    for s, (k, v) in enumerate(zip(k_seqs, v_seqs)):
        for lb in range(nblk[s]):
            pb = int(order[cur]); cur += 1
            table[s, lb] = pb
            rows = slice(lb * block_size, min(len(k), (lb + 1) * block_size))
            n = rows.stop - rows.start
            if n > 0:
                cache[0, pb, :n] = k[rows]
                cache[1, pb, :n] = v[rows]
    return cache, table


def parse_mask_golden(path):
    """Read a transcribed mask example: header ints plus [causal]/[window]/[combined] grids.

    Window rows drop the cells printed left of ``|`` (outside the key range).
    """
    meta, grids, cur = {}, {}, None
    with open(path, encoding="utf-8") as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                grids[cur] = []
                continue
            if cur is None:
                key, val = line.split()
                meta[key] = int(val)
                continue
            if "|" in line:
                line = line.split("|", 1)[1]
            cells = line.split()
            assert all(c in (ALLOW, MASK) for c in cells), line
            grids[cur].append([c == ALLOW for c in cells])
    return meta, {k: np.array(v, dtype=bool) for k, v in grids.items()}


def hf_style_mask(seqlen_q, seqlen_k, sliding_window):
    """Allowed-key matrix built the way HF ``build_attention_mask`` builds its bias:
    ``triu`` of -inf from the causal diagonal, plus ``tril`` of -inf up to the sliding
    diagonal when the window exceeds 1.  An independent formulation of the mask rule."""
    minus_inf = np.full((seqlen_q, seqlen_k), -np.inf)
    if 1 <= seqlen_q < seqlen_k:
        causal_diagonal = seqlen_k - seqlen_q + 1
    else:
        causal_diagonal = 1
    masked = np.triu(minus_inf, k=causal_diagonal)
    if sliding_window > 1:
        masked = masked + np.tril(minus_inf, k=seqlen_k - seqlen_q - sliding_window)
    return masked == 0


def sdpa_style_mask(seq_len, window):
    """Allowed-key matrix of the vllm-npu SDPA backend's sliding-window bias (square case):
    ``tril`` of ones at diagonal 0, then ``triu`` at ``-window + 1``."""
    m = np.tril(np.ones((seq_len, seq_len)), k=0)
    if window is not None:
        m = np.triu(m, k=-window + 1)
    return m == 1

"""Seeded randomized GPU parity sweeps.  (1) One store + prefill or store + decode step per case, at
shapes drawn from a seeded generator so that combinations the fixed cases do not list get
checked too (group sizes 1-16, head size 64/128, block sizes 1-256, windows, chunked prefill
offsets, ALiBi, FP8 caches with a kv_scale, the fused store, decode partition sizes), against
the oracle on every output element and every cache byte.  (2) Shared-prefix (cascade) decode at
random prefix lengths, batches on both sides of the prefix-pass switch, bf16 and FP8 caches,
against the oracle's cascade decode.  (3) Large prefill chunks (256-2048 rows over contexts up to
8192 keys) on sampled rows."""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
import workloads as W
from tests.gpu_helpers import GpuRun, assert_close, bits, host_values, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
F8 = torch.float8_e4m3fn
# case counts (PA_RANDOM_CASES / PA_RANDOM_CASCADE_CASES widen a run; the defaults are what the
# suite runs); PA_RANDOM_SEED0 starts every sweep at another seed, so a run can draw cases the
# default range does not
N_CASES = int(os.environ.get("PA_RANDOM_CASES", "160"))
SEED0 = int(os.environ.get("PA_RANDOM_SEED0", "0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_attention_block_amd as pa
    pa.load()  # fails loudly when libpa.so is missing
    yield
    torch.cuda.synchronize()


def draw_case(seed: int) -> dict:
    """The configuration of sweep case ``seed`` (pure host logic, deterministic)."""
    rng = np.random.default_rng(1000 + seed)
    dtype = torch.float32 if rng.random() < 0.15 else torch.bfloat16
    fp8_cache = dtype == torch.bfloat16 and rng.random() < 0.25
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
    while Hkv * G > 64:
        Hkv = max(1, Hkv // 2)
    bs_choices = [1, 4, 16, 32, 128] if dtype == torch.float32 else [16, 32, 64, 128, 256]
    BS = int(rng.choice(bs_choices))
    window = int(rng.integers(1, 300)) if rng.random() < 0.35 else 0
    kind = "prefill" if rng.random() < 0.5 else "decode"
    B = int(rng.integers(1, 7))
    if kind == "prefill":
        seqs = [(int(rng.integers(0, 500)) if rng.random() < 0.6 else 0, int(rng.integers(1, 260)))
                for _ in range(B)]
    else:
        top = 20000 if rng.random() < 0.15 else 2500  # a few long contexts: many chunks per sequence
        seqs = [(int(rng.integers(0, top)), 1) for _ in range(B)]
    c = {
        "seed": seed, "dtype": dtype, "fp8": fp8_cache, "D": D, "Hkv": Hkv, "H": Hkv * G, "BS": BS,
        "window": window, "kind": kind, "seqs": seqs,
        "alibi": bool(rng.random() < 0.3),
        "fused": bool(rng.random() < 0.35),
        "kv_scale": float(rng.choice([1.0, 0.5, 2.0, 0.3])) if fp8_cache else 1.0,
        "part": int(rng.choice([0, 0, 32, 64, 256])) if kind == "decode" else 0,
    }
    _widen_heads(rng, c, G)
    return c


def _widen_heads(rng, c, G):
    """Now and then more than 8 KV heads (the decode kernel then runs several head groups per
    chunk, the last one partly idle); drawn after everything else, so the rest of a case is the
    same as without this draw."""
    if rng.random() < 0.12:
        wide = int(rng.choice([12, 16]))
        if wide * G <= 64:
            c["Hkv"], c["H"] = wide, wide * G


def test_sweep_draws_cover_the_options():
    cases = [draw_case(i) for i in range(SEED0, SEED0 + N_CASES)]
    for key in ("fp8", "alibi", "fused"):
        assert any(c[key] for c in cases) and not all(c[key] for c in cases), key
    assert {c["kind"] for c in cases} == {"prefill", "decode"}
    assert any(c["window"] for c in cases)
    assert any(c["Hkv"] > 8 and c["kind"] == "decode" for c in cases)
    assert any(c["dtype"] == torch.float32 for c in cases)
    assert len({c["H"] // c["Hkv"] for c in cases}) >= 5
    assert len({c["BS"] for c in cases}) >= 5


@pytest.mark.parametrize("seed", range(SEED0, SEED0 + N_CASES))
def test_random_step(seed):
    c = draw_case(seed)
    say(f"[random {seed}] {c['kind']} {str(c['dtype'])[6:]}{' fp8' if c['fp8'] else ''} H {c['H']}/{c['Hkv']} "
        f"D {c['D']} BS {c['BS']} W {c['window']} alibi {c['alibi']} fused {c['fused']} part {c['part']} "
        f"seqs {c['seqs']}")
    specs = [W.SeqSpec(ctx, [q], [c["kind"]]) for ctx, q in c["seqs"]]
    wl = W.build(f"random{seed}", 2000 + seed, specs, num_heads=c["H"], num_kv_heads=c["Hkv"], head_size=c["D"],
                 block_size=c["BS"], dtype=c["dtype"], sliding_window=c["window"],
                 cache_dtype=F8 if c["fp8"] else None)
    run = GpuRun(wl, DEV)
    run.kv_scale = c["kv_scale"]
    if c["alibi"]:
        run.alibi = np.array([2.0 ** (-8.0 * (i + 1) / c["H"]) for i in range(c["H"])])
    store, op = wl.phases[0]
    before = bits(wl.kv_cache)
    if c["fused"]:
        out = run.run_with_store(store, op, partition_size=c["part"])
    else:
        run.run(store)
        out = run.run(op, partition_size=c["part"])
    torch.cuda.synchronize()
    # the cache after the store, byte for byte
    if c["fp8"]:
        ref_cache = fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                     store.slot_mapping, c["kv_scale"])
        vals = fp8.dequantize(ref_cache, c["kv_scale"])
    else:
        ref_cache = oracle.store_kv(before, bits(store.key), bits(store.value), store.slot_mapping)
    got_cache = bits(run.cache.cpu())
    np.testing.assert_array_equal(got_cache, ref_cache)
    if not c["fp8"]:
        vals = host_values(run.cache.cpu())
    # the attention output against the oracle over that cache
    q = host_values(op.query)
    if isinstance(op, W.PrefillOp):
        cu_q, cu_k = op.cu_seqlens_q, op.cu_seqlens_k
    else:
        cu_q = np.arange(len(op.seq_lens) + 1)
        cu_k = np.concatenate([[0], np.cumsum(op.seq_lens)])
    ref = oracle.prefill_varlen(q, vals, op.block_table, cu_q, cu_k, wl.scale, wl.num_kv_heads,
                                wl.sliding_window, run.alibi)
    err = assert_close(out.float().cpu().numpy(), ref, c["dtype"], f"random {seed}")
    say(f"[random {seed}] max abs err {err:.3e}")


N_CASCADE = int(os.environ.get("PA_RANDOM_CASCADE_CASES", "40"))


def draw_cascade(seed: int) -> dict:
    """Sweep case ``seed`` of shared-prefix (cascade) decode (host logic, deterministic)."""
    rng = np.random.default_rng(5000 + seed)
    fp8_cache = bool(rng.random() < 0.3)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 5, 8, 16]))
    while Hkv * G > 64:
        Hkv = max(1, Hkv // 2)
    BS = int(rng.choice([16, 32, 64, 128, 256]))
    prefix = BS * int(rng.integers(1, max(2, 2048 // BS)))
    # (a prefix of at most 2048 keys; B up to ~535 sequences when G is 1)
    # batches large enough for a KV head to have >= 512 (sequence, query head) rows take the
    # prefix pass on the prefill kernel
    big = bool(rng.random() < 0.35)
    B = -(-512 // G) + int(rng.integers(0, 24)) if big else int(rng.integers(1, 12))
    own = [0 if rng.random() < 0.15 else int(rng.integers(1, 300 if big else 1500)) for _ in range(B)]
    c = {"seed": seed, "fp8": fp8_cache, "D": D, "Hkv": Hkv, "H": Hkv * G, "BS": BS, "prefix": prefix,
         "ctx": [prefix + o for o in own],
         "kv_scale": float(rng.choice([1.0, 0.5, 2.0])) if fp8_cache else 1.0,
         "part": int(rng.choice([0, 0, 64, 256]))}
    _widen_heads(rng, c, G)
    return c


def test_cascade_draws_reach_both_prefix_passes():
    cases = [draw_cascade(i) for i in range(N_CASCADE)]
    rows = [len(c["ctx"]) * (c["H"] // c["Hkv"]) for c in cases]
    assert any(r >= 512 for r in rows) and any(r < 512 for r in rows)
    assert any(c["fp8"] for c in cases) and not all(c["fp8"] for c in cases)


@pytest.mark.parametrize("seed", range(SEED0, SEED0 + N_CASCADE))
def test_random_cascade(seed):
    import paged_attention_block_amd as pa
    c = draw_cascade(seed)
    P = c["prefix"]
    say(f"[random cascade {seed}] {'fp8' if c['fp8'] else 'bf16'} H {c['H']}/{c['Hkv']} D {c['D']} BS {c['BS']} "
        f"prefix {P} B {len(c['ctx'])} part {c['part']} ctx {c['ctx'][:8]}")
    specs = [W.SeqSpec(ctx, [1], ["decode"]) for ctx in c["ctx"]]
    wl = W.build(f"rcascade{seed}", 3000 + seed, specs, num_heads=c["H"], num_kv_heads=c["Hkv"], head_size=c["D"],
                 block_size=c["BS"], dtype=torch.bfloat16, shared_prefix=P, cache_dtype=F8 if c["fp8"] else None)
    run = GpuRun(wl, DEV)
    run.kv_scale = c["kv_scale"]
    store, dec = wl.phases[0]
    before = bits(wl.kv_cache)
    run.run(store)
    out = pa.pa_cascade_decode(dec.query.to(DEV), run.cache, run.i32(dec.block_table), run.i32(dec.seq_lens),
                               int(dec.max_seq_len), wl.scale, wl.num_kv_heads, P, partition_size=c["part"],
                               kv_scale=c["kv_scale"])
    torch.cuda.synchronize()
    if c["fp8"]:
        ref_cache = fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                     store.slot_mapping, c["kv_scale"])
        np.testing.assert_array_equal(bits(run.cache.cpu()), ref_cache)
        vals = fp8.dequantize(ref_cache, c["kv_scale"])
    else:
        np.testing.assert_array_equal(bits(run.cache.cpu()),
                                      oracle.store_kv(before, bits(store.key), bits(store.value), store.slot_mapping))
        vals = host_values(run.cache.cpu())
    ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale,
                                wl.num_kv_heads, P)
    err = assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, f"random cascade {seed}")
    say(f"[random cascade {seed}] max abs err {err:.3e}")


N_LARGE = int(os.environ.get("PA_RANDOM_LARGE_CASES", "16"))


def draw_large(seed: int) -> dict:
    """Sweep case ``seed`` of large prefill chunks (host logic, deterministic)."""
    rng = np.random.default_rng(7000 + seed)
    G = int(rng.choice([1, 2, 4, 5, 8]))
    Hkv = int(rng.choice([1, 2, 8])) if G < 8 else int(rng.choice([1, 2]))
    B = int(rng.integers(1, 5))
    seqs = [(int(rng.integers(0, 8193)) if rng.random() < 0.6 else 0, int(rng.integers(256, 2049))) for _ in range(B)]
    return {"seed": seed, "G": G, "Hkv": Hkv, "H": G * Hkv, "D": int(rng.choice([64, 128])),
            "BS": int(rng.choice([16, 64, 256])), "window": int(rng.choice([0, 0, 1024, 4096])),
            "seqs": seqs, "fp8": bool(rng.random() < 0.25), "alibi": bool(rng.random() < 0.25),
            "kv_scale": 0.5}


@pytest.mark.parametrize("seed", range(SEED0, SEED0 + N_LARGE))
def test_random_large_prefill_sampled(seed):
    """Chunks of 256-2048 rows over contexts up to 8192 keys: many q-tiles and key tiles per
    sequence; sampled rows (tile edges, first/last rows, random) against the oracle."""
    from tests.gpu_helpers import sample_picks
    c = draw_large(seed)
    say(f"[random large {seed}] H {c['H']}/{c['Hkv']} D {c['D']} BS {c['BS']} W {c['window']} fp8 {c['fp8']} "
        f"alibi {c['alibi']} seqs {c['seqs']}")
    specs = [W.SeqSpec(ctx, [q], ["prefill"]) for ctx, q in c["seqs"]]
    wl = W.build(f"rlarge{seed}", 4000 + seed, specs, num_heads=c["H"], num_kv_heads=c["Hkv"], head_size=c["D"],
                 block_size=c["BS"], dtype=torch.bfloat16, sliding_window=c["window"],
                 cache_dtype=F8 if c["fp8"] else None)
    run = GpuRun(wl, DEV)
    if c["fp8"]:
        run.kv_scale = c["kv_scale"]
    if c["alibi"]:
        run.alibi = np.array([2.0 ** (-8.0 * (i + 1) / c["H"]) for i in range(c["H"])])
    store, op = wl.phases[0]
    before = bits(wl.kv_cache)
    run.run(store)
    out = run.run(op)
    torch.cuda.synchronize()
    if c["fp8"]:
        vals = fp8.dequantize(fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                               store.slot_mapping, c["kv_scale"]), c["kv_scale"])
    else:
        vals = host_values(run.cache.cpu())
    picks = sample_picks(op, wl.num_heads, np.random.default_rng(seed), n_random=64)
    ref = oracle.attention_rows(host_values(op.query), vals, op.block_table, op.cu_seqlens_q, op.cu_seqlens_k,
                                wl.scale, wl.num_kv_heads, wl.sliding_window, picks, run.alibi)
    got = out.float().cpu().numpy()
    err = assert_close(np.stack([got[r, h] for r, h in picks]), ref, torch.bfloat16, f"random large {seed}")
    say(f"[random large {seed}] {len(picks)} rows, max abs err {err:.3e}")

"""GPU parity of the FP8 (E4M3) KV cache: the quantizing store bit for bit against the
oracle (every finite bf16 value, and random rows at several scales), and decode, cascade
decode and prefill over FP8 caches against the oracle's attention over the dequantized
cache."""

from __future__ import annotations

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_attention_block_amd as pa
    pa.load()  # fails loudly when libpa.so is missing
    yield
    torch.cuda.synchronize()


def _store_and_compare(key_bf16: torch.Tensor, value_bf16: torch.Tensor, kv_scale: float, label: str):
    import paged_attention_block_amd as pa
    T, Hkv, D = key_bf16.shape
    BS = 16
    nb = (T + BS - 1) // BS + 1
    rng = np.random.default_rng(T)
    slots = rng.permutation(nb * BS)[:T].astype(np.int32)
    slots[::7] = -1
    cache = torch.zeros((2, nb, BS, Hkv, D), dtype=F8, device=DEV)
    say(f"[fp8 store {label}] tokens {T} kv_scale {kv_scale}")
    pa.pa_store_kv(key_bf16.to(DEV), value_bf16.to(DEV), cache, torch.from_numpy(slots).to(DEV), kv_scale=kv_scale)
    torch.cuda.synchronize()
    ref = fp8.store_kv_fp8(np.zeros((2, nb, BS, Hkv, D), np.uint8), key_bf16.float().numpy(),
                           value_bf16.float().numpy(), slots, kv_scale)
    got = bits(cache.cpu())
    bad = got != ref
    assert not bad.any(), f"{label}: {int(bad.sum())} codes differ; first at {np.argwhere(bad)[0]}: gpu {got[bad][0]:#x} oracle {ref[bad][0]:#x}"


def test_store_every_finite_bf16_value():
    """All 2^16 bf16 bit patterns except NaNs (zeros there), as key rows and, reversed, as
    value rows, stored with kv_scale 1: every rounding tie, subnormal, saturation and signed
    zero of the E4M3 conversion."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16)
    vals[torch.isnan(vals)] = 0
    key = vals.reshape(64, 8, 128)
    value = vals.flip(0).reshape(64, 8, 128)
    _store_and_compare(key, value, 1.0, "all bf16")


@pytest.mark.parametrize("kv_scale", [0.05, 0.3, 2.0, 7.0])
def test_store_random_rows_at_scales(kv_scale):
    g = torch.Generator().manual_seed(int(kv_scale * 100))
    key = (torch.randn((300, 4, 64), generator=g) * 4).to(torch.bfloat16)
    value = (torch.randn((300, 4, 64), generator=g) * 30).to(torch.bfloat16)
    _store_and_compare(key, value, kv_scale, f"scale {kv_scale}")


def _fp8_decode_workload(name, seed, ctxs, H, Hkv, D, BS, window=0, shared_prefix=0):
    seqs = [W.SeqSpec(c, [1], ["decode"]) for c in ctxs]
    return W.build(name, seed, seqs, num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=BS,
                   dtype=torch.bfloat16, sliding_window=window, cache_dtype=F8, shared_prefix=shared_prefix)


def _store_then(run: GpuRun, store, kv_scale):
    """GPU store of the step's new tokens, checked against the oracle's store bit for bit;
    returns the oracle's dequantized cache after it."""
    before = bits(run.wl.kv_cache)
    run.run(store)
    torch.cuda.synchronize()
    ref = fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(), store.slot_mapping,
                           kv_scale)
    np.testing.assert_array_equal(bits(run.cache.cpu()), ref)
    return fp8.dequantize(ref, kv_scale)


DECODE_CASES = {
    # name: (H, Hkv, D, BS, window, [ctx0 ...])
    "g4_d128": (32, 8, 128, 16, 0, [0, 4, 31, 32, 100, 700, 2000]),
    "g5_d128_window": (10, 2, 128, 16, 40, [0, 39, 41, 300]),
    "g8_d64": (16, 2, 64, 16, 0, [5, 64, 900]),
    "g4_d64_bs256": (16, 4, 64, 256, 0, [0, 255, 256, 300, 1000]),
}


@pytest.mark.parametrize("kv_scale", [1.0, 0.25])
@pytest.mark.parametrize("part", [0, 64])
@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_fp8_decode(name, part, kv_scale):
    import paged_attention_block_amd as pa
    H, Hkv, D, BS, win, ctxs = DECODE_CASES[name]
    wl = _fp8_decode_workload(name, 500, ctxs, H, Hkv, D, BS, win)
    run = GpuRun(wl, DEV)
    run.kv_scale = kv_scale
    store, dec = wl.phases[0]
    vals = _store_then(run, store, kv_scale)
    say(f"[fp8 decode {name} p{part} s{kv_scale}]")
    out = run.run(dec, partition_size=part)
    torch.cuda.synchronize()
    cu_q = np.arange(len(dec.seq_lens) + 1)
    cu_k = np.concatenate([[0], np.cumsum(dec.seq_lens)])
    ref = oracle.prefill_varlen(host_values(dec.query), vals, dec.block_table, cu_q, cu_k, wl.scale,
                                wl.num_kv_heads, win)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, f"fp8 decode {name} p{part}")


def test_fp8_decode_alibi_and_with_store():
    import paged_attention_block_amd as pa
    wl = _fp8_decode_workload("fa", 501, [0, 33, 500, 1200], 16, 4, 128, 16)
    slopes = np.array([2.0 ** (-8.0 * (i + 1) / 16) for i in range(16)])
    run = GpuRun(wl, DEV)
    run.kv_scale = 0.5
    run.alibi = slopes
    store, dec = wl.phases[0]
    before = bits(wl.kv_cache)
    say("[fp8 decode alibi with store]")
    out = run.run_with_store(store, dec, partition_size=64)
    torch.cuda.synchronize()
    ref_cache = fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                 store.slot_mapping, 0.5)
    np.testing.assert_array_equal(bits(run.cache.cpu()), ref_cache)
    cu_q = np.arange(len(dec.seq_lens) + 1)
    cu_k = np.concatenate([[0], np.cumsum(dec.seq_lens)])
    ref = oracle.prefill_varlen(host_values(dec.query), fp8.dequantize(ref_cache, 0.5), dec.block_table, cu_q,
                                cu_k, wl.scale, wl.num_kv_heads, 0, slopes)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "fp8 decode alibi")


@pytest.mark.parametrize("part", [0, 64])
def test_fp8_cascade_decode(part):
    import paged_attention_block_amd as pa
    P = 256
    wl = _fp8_decode_workload("fc", 502, [256, 300, 1000, 257, 2000, 256], 32, 8, 128, 16, shared_prefix=P)
    run = GpuRun(wl, DEV)
    run.kv_scale = 2.0
    store, dec = wl.phases[0]
    vals = _store_then(run, store, 2.0)
    say(f"[fp8 cascade p{part}]")
    out = pa.pa_cascade_decode(dec.query.to(DEV), run.cache, run.i32(dec.block_table), run.i32(dec.seq_lens),
                               int(dec.max_seq_len), wl.scale, wl.num_kv_heads, P, partition_size=part,
                               kv_scale=2.0)
    torch.cuda.synchronize()
    ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale,
                                wl.num_kv_heads, P)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, f"fp8 cascade p{part}")


def test_fp8_decode_gqa_full_size():
    """The GQA decode shape (B 64, contexts U[512, 4096], H 32/8, D 128) over an FP8 cache:
    every output against the oracle."""
    rng = np.random.default_rng(2)
    ctx = rng.integers(512, 4096 + 1, size=64)
    wl = _fp8_decode_workload("fp8_gqa", 503, [int(c) for c in ctx], 32, 8, 128, 16)
    run = GpuRun(wl, DEV)
    run.kv_scale = 0.7
    store, dec = wl.phases[0]
    vals = _store_then(run, store, 0.7)
    say("[fp8 decode full size]")
    out = run.run(dec)
    torch.cuda.synchronize()
    ref = oracle.decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale, wl.num_kv_heads)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "fp8 decode full")


PREFILL_CASES = {
    # name: (H, Hkv, D, BS, window, [(ctx0, q) ...])
    "g4_d128": (32, 8, 128, 16, 0, [(0, 1), (0, 37), (0, 200), (150, 90)]),
    "g5_d128_window": (10, 2, 128, 16, 70, [(0, 130), (300, 64), (20, 5)]),
    "g8_d64_chunked": (16, 2, 64, 32, 0, [(64, 100), (1000, 33)]),
    "g4_d128_bs256": (16, 4, 128, 256, 0, [(0, 300), (500, 70)]),
}


@pytest.mark.parametrize("kv_scale", [1.0, 0.5])
@pytest.mark.parametrize("name", sorted(PREFILL_CASES))
def test_fp8_prefill(name, kv_scale):
    H, Hkv, D, BS, win, spec = PREFILL_CASES[name]
    seqs = [W.SeqSpec(c, [q], ["prefill"]) for c, q in spec]
    wl = W.build(name, 505, seqs, num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=BS,
                 dtype=torch.bfloat16, sliding_window=win, cache_dtype=F8)
    run = GpuRun(wl, DEV)
    run.kv_scale = kv_scale
    store, pre = wl.phases[0]
    vals = _store_then(run, store, kv_scale)
    say(f"[fp8 prefill {name} s{kv_scale}]")
    out = run.run(pre)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(host_values(pre.query), vals, pre.block_table, pre.cu_seqlens_q, pre.cu_seqlens_k,
                                wl.scale, wl.num_kv_heads, win)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, f"fp8 prefill {name}")


def test_fp8_prefill_with_store_alibi():
    """The fused call over an FP8 cache: the store runs first, so the attention reads the
    quantized new rows; cache contents and output match the oracle's store then prefill."""
    wl = W.build("fpws", 506, [W.SeqSpec(0, [150], ["prefill"]), W.SeqSpec(200, [70], ["prefill"])],
                 num_heads=16, num_kv_heads=4, head_size=128, block_size=16, dtype=torch.bfloat16,
                 cache_dtype=F8)
    slopes = np.array([2.0 ** (-8.0 * (i + 1) / 16) for i in range(16)])
    run = GpuRun(wl, DEV)
    run.kv_scale = 0.25
    run.alibi = slopes
    store, pre = wl.phases[0]
    before = bits(wl.kv_cache)
    say("[fp8 prefill with store alibi]")
    out = run.run_with_store(store, pre)
    torch.cuda.synchronize()
    ref_cache = fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                 store.slot_mapping, 0.25)
    np.testing.assert_array_equal(bits(run.cache.cpu()), ref_cache)
    ref = oracle.prefill_varlen(host_values(pre.query), fp8.dequantize(ref_cache, 0.25), pre.block_table,
                                pre.cu_seqlens_q, pre.cu_seqlens_k, wl.scale, wl.num_kv_heads, 0, slopes)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "fp8 prefill with store")


def test_fp8_prefill_varlen_full_size():
    """16 prompts U[128, 2048], H 32/8, D 128 over an FP8 cache: every output."""
    rng = np.random.default_rng(3)
    lens = rng.integers(128, 2048 + 1, size=16)
    wl = W.build("fp8_prefill", 507, [W.SeqSpec(0, [int(n)], ["prefill"]) for n in lens], num_heads=32,
                 num_kv_heads=8, head_size=128, block_size=16, dtype=torch.bfloat16, cache_dtype=F8)
    run = GpuRun(wl, DEV)
    run.kv_scale = 1.5
    store, pre = wl.phases[0]
    vals = _store_then(run, store, 1.5)
    say("[fp8 prefill full size]")
    out = run.run(pre)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(host_values(pre.query), vals, pre.block_table, pre.cu_seqlens_q, pre.cu_seqlens_k,
                                wl.scale, wl.num_kv_heads, 0)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "fp8 prefill full")


def test_fp8_cascade_decode_prefill_kernel_prefix():
    """FP8 cache, 130 sequences x 4 query heads per KV head (the prefix pass on the prefill
    kernel), prefix 192 keys."""
    import paged_attention_block_amd as pa
    P = 192
    rng = np.random.default_rng(508)
    ctxs = [int(c) for c in rng.integers(192, 500, size=130)]
    wl = _fp8_decode_workload("fcm", 508, ctxs, 32, 8, 128, 16, shared_prefix=P)
    run = GpuRun(wl, DEV)
    run.kv_scale = 0.5
    store, dec = wl.phases[0]
    vals = _store_then(run, store, 0.5)
    say("[fp8 cascade mfma prefix]")
    out = pa.pa_cascade_decode(dec.query.to(DEV), run.cache, run.i32(dec.block_table), run.i32(dec.seq_lens),
                               int(dec.max_seq_len), wl.scale, wl.num_kv_heads, P, kv_scale=0.5)
    torch.cuda.synchronize()
    ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale,
                                wl.num_kv_heads, P)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "fp8 cascade mfma")

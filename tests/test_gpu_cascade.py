"""GPU parity of shared-prefix (cascade) decode: pa_cascade_decode through the C ABI against
the oracle's cascade decode (pinned to plain attention), at small sizes on every output and
at the GQA decode shape with a 1024-key shared prefix on sampled rows."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import GpuRun, assert_close, bits, host_values, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_attention_block_amd as pa
    pa.load()  # fails loudly when libpa.so is missing
    yield
    torch.cuda.synchronize()


def _cascade(run: GpuRun, dec, prefix, lens=None, partition_size=0, workspace=None):
    import paged_attention_block_amd as pa
    wl = run.wl
    lens = dec.seq_lens if lens is None else lens
    return pa.pa_cascade_decode(dec.query.to(DEV), run.cache, run.i32(dec.block_table), run.i32(lens),
                                int(dec.max_seq_len), wl.scale, wl.num_kv_heads, prefix,
                                partition_size=partition_size, workspace=workspace)


CASES = {
    # name: (H, Hkv, D, BS, shared prefix, [ctx0 ...]); ctx0 >= prefix, the new token follows
    "g4_d128_p48": (32, 8, 128, 16, 48, [48, 49, 63, 64, 95, 96, 200, 700]),
    "g4_d128_p64": (32, 8, 128, 16, 64, [64, 65, 127, 128, 300, 1000, 64, 90]),
    "g5_d128_p256": (10, 2, 128, 16, 256, [256, 300, 257, 600]),
    "g8_d64_p32": (16, 2, 64, 32, 32, [32, 33, 100, 31 + 32]),
    "g16_d128_p512": (16, 1, 128, 16, 512, [512, 520, 900]),
    "g2_d128_hkv12_p128": (24, 12, 128, 16, 128, [128, 129, 400, 2000, 160]),
    "g4_d128_b1_p1024": (8, 2, 128, 16, 1024, [1500]),
    "g4_d128_bs256_p512": (32, 8, 128, 256, 512, [512, 600, 1000, 2000]),
}


@pytest.mark.parametrize("part", [0, 64, 256])
@pytest.mark.parametrize("name", sorted(CASES))
def test_small_cascade_decode(name, part):
    H, Hkv, D, BS, P, ctxs = CASES[name]
    seqs = [W.SeqSpec(c, [1], ["decode"]) for c in ctxs]
    wl = W.build(name, 400, seqs, num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=BS,
                 dtype=torch.bfloat16, shared_prefix=P)
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    say(f"[cascade {name} p{part}] B {len(ctxs)} prefix {P}")
    out = _cascade(run, dec, P, partition_size=part)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale,
                                wl.num_kv_heads, P)
    assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"cascade {name} p{part}")


def test_cascade_sequences_with_no_own_key_and_prefix_zero():
    """Sequences whose whole context is the shared prefix (seq_len == prefix) get the
    prefix's attention; prefix 0 is plain decode, bit for bit."""
    import paged_attention_block_amd as pa
    P = 96
    seqs = [W.SeqSpec(c, [1], ["decode"]) for c in (96, 100, 96, 400, 130)]
    wl = W.build("own0", 401, seqs, num_heads=16, num_kv_heads=4, head_size=128, block_size=16,
                 dtype=torch.bfloat16, shared_prefix=P)
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    lens = dec.seq_lens.copy()
    lens[[0, 2]] = P
    vals = host_values(run.cache.cpu())
    for part in (0, 64):
        say(f"[cascade no-own-key p{part}]")
        out = _cascade(run, dec, P, lens=lens, partition_size=part)
        torch.cuda.synchronize()
        ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, lens, wl.scale,
                                    wl.num_kv_heads, P)
        assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"no own key p{part}")
        plain = pa.pa_decode(dec.query.to(DEV), run.cache, run.i32(dec.block_table), run.i32(dec.seq_lens),
                             int(dec.max_seq_len), wl.scale, wl.num_kv_heads, partition_size=part)
        zero = _cascade(run, dec, 0, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(plain.view(torch.int16), zero.view(torch.int16))


def test_cascade_workspace_contents_need_no_init():
    seqs = [W.SeqSpec(c, [1], ["decode"]) for c in (256, 300, 1000, 257, 600, 2000)]
    wl = W.build("cws", 402, seqs, num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                 dtype=torch.bfloat16, shared_prefix=256)
    import paged_attention_block_amd as pa
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    need = pa.pa_cascade_decode_workspace_size(run.cache, len(seqs), 32, int(dec.max_seq_len), 256, 64)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    a = _cascade(run, dec, 256, partition_size=64, workspace=ws)
    b = _cascade(run, dec, 256, partition_size=64)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("part", [0, 128])
def test_shared_prefix_decode_full_size(part):
    """B 64, shared prefix 1024, contexts U[1024, 4096], H 32/8, D 128: every output against
    the oracle's plain decode definition (which the cascade oracle is pinned to equal)."""
    wl = W.shared_prefix_decode()
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    say(f"[cascade full p{part}]")
    out = _cascade(run, dec, 1024, partition_size=part)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale, wl.num_kv_heads)
    assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"shared prefix full p{part}")


# With at least 512 (sequence, query head) rows per KV head the prefix pass runs on the
# prefill kernel (64-key tiles, 32 rows per wave); the cases above have fewer rows and run
# the split-key prefix kernel.
MFMA_CASES = {
    # name: (H, Hkv, D, BS, shared prefix, batch, context range)
    "g4_d128_p80": (32, 8, 128, 16, 80, 160, (80, 300)),
    "g5_d64_p128": (10, 2, 64, 32, 128, 110, (128, 400)),
    "g8_d128_p1024": (16, 2, 128, 16, 1024, 64, (1024, 1300)),
}


@pytest.mark.parametrize("part", [0, 64])
@pytest.mark.parametrize("name", sorted(MFMA_CASES))
def test_cascade_decode_prefill_kernel_prefix(name, part):
    H, Hkv, D, BS, P, B, (lo, hi) = MFMA_CASES[name]
    assert B * (H // Hkv) >= 512
    rng = np.random.default_rng(403)
    ctxs = rng.integers(lo, hi + 1, size=B)
    seqs = [W.SeqSpec(int(c), [1], ["decode"]) for c in ctxs]
    wl = W.build(name, 403, seqs, num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=BS,
                 dtype=torch.bfloat16, shared_prefix=P)
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    say(f"[cascade mfma prefix {name} p{part}] B {B} prefix {P}")
    out = _cascade(run, dec, P, partition_size=part)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale,
                                wl.num_kv_heads, P)
    assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"cascade mfma {name} p{part}")


def test_shared_prefix_b256_p4096_full():
    """The large shared-prefix batch (B 256, prefix 4096, contexts U[4096, 8192], H 32/8):
    every output against the plain decode definition."""
    wl = W.shared_prefix_decode(num_seqs=256, prefix=4096, lo=4096, hi=8192)
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    say("[cascade b256 p4096]")
    out = _cascade(run, dec, 4096)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale, wl.num_kv_heads)
    assert_close(out.float().cpu().numpy(), ref, wl.dtype, "shared prefix b256")


def test_cascade_empty_batch_and_all_context_shared():
    """An empty batch is a no-op; a batch whose every context is exactly the shared prefix (no
    own key anywhere: the own-keys pass has no step) gets the prefix attention alone, on both
    prefix passes (split-key at B 6, the prefill kernel at B 160 x G 4 rows)."""
    import paged_attention_block_amd as pa
    wl = W.build("e0", 404, [W.SeqSpec(64, [1], ["decode"])], num_heads=8, num_kv_heads=2, head_size=128,
                 block_size=16, dtype=torch.bfloat16, shared_prefix=64)
    run = GpuRun(wl, DEV)
    say("[cascade empty batch]")
    q0 = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    out0 = pa.pa_cascade_decode(q0, run.cache, torch.zeros((0, 4), dtype=torch.int32, device=DEV),
                                torch.zeros((0,), dtype=torch.int32, device=DEV), 0, wl.scale, wl.num_kv_heads, 64)
    torch.cuda.synchronize()
    assert out0.shape == (0, 8, 128)
    for B, P in ((6, 256), (160, 512)):
        seqs = [W.SeqSpec(P - 1, [1], ["decode"]) for _ in range(B)]
        wl = W.build(f"allshared{B}", 405, seqs, num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                     dtype=torch.bfloat16, shared_prefix=P - 16)
        run = GpuRun(wl, DEV)
        store, dec = wl.phases[0]
        run.run(store)
        lens = np.full(B, P - 16, dtype=np.int32)  # every context = the shared blocks only
        for part in (0, 64):
            say(f"[cascade all shared B {B} P {P - 16} p{part}]")
            out = _cascade(run, dec, P - 16, lens=lens, partition_size=part)
            torch.cuda.synchronize()
            vals = host_values(run.cache.cpu())
            ref = oracle.cascade_decode(host_values(dec.query), vals, dec.block_table, lens, wl.scale,
                                        wl.num_kv_heads, P - 16)
            assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"all shared B {B} p{part}")


# ----------------------------------------------------------------------------- query chunks


CASCADE_PREFILL_CASES = {
    # name: (H, Hkv, D, BS, shared prefix, [(context, query rows)])
    "g4_d128_p48": (32, 8, 128, 16, 48, [(48, 1), (60, 37), (300, 64), (49, 130)]),
    "g5_d128_p256": (10, 2, 128, 16, 256, [(256, 90), (500, 33), (270, 1), (1000, 200)]),
    "g8_d64_bs32_p128": (16, 2, 64, 32, 128, [(128, 70), (200, 1), (129, 64)]),
    "g1_d128_p64": (4, 4, 128, 16, 64, [(64, 100), (80, 31)]),
    "g4_d128_many_rows_p512": (32, 8, 128, 16, 512, [(512 + 7 * i, 40 + 3 * i) for i in range(8)]),
}


def _cascade_prefill(run, op, P, workspace=None):
    import paged_attention_block_amd as pa
    wl = run.wl
    return pa.pa_cascade_prefill_varlen(op.query.to(DEV), run.cache, run.i32(op.block_table),
                                        run.i32(op.cu_seqlens_q), run.i32(op.cu_seqlens_k), op.max_seqlen_q,
                                        op.max_seqlen_k, wl.scale, wl.num_kv_heads, P, workspace=workspace,
                                        kv_scale=run.kv_scale, validate=True)


def _prefill_case(name, seed, cache_dtype=None):
    H, Hkv, D, BS, P, spec = CASCADE_PREFILL_CASES[name]
    seqs = [W.SeqSpec(c, [q], ["prefill"]) for c, q in spec]
    return W.build(name, seed, seqs, num_heads=H, num_kv_heads=Hkv, head_size=D, block_size=BS,
                   dtype=torch.bfloat16, shared_prefix=P, cache_dtype=cache_dtype), P


@pytest.mark.parametrize("name", sorted(CASCADE_PREFILL_CASES))
def test_cascade_prefill_small(name):
    """Every output against the cascade oracle (pinned to plain prefill and SDPA), and against
    pa_prefill_varlen on the same cache.  The cases run both prefix passes (split-key below 512
    (row, head) pairs per KV head, the prefill kernel above), prefixes that end inside a 64-key
    tile, single-row chunks next to long ones, and head sizes 64 / 128."""
    import paged_attention_block_amd as pa
    wl, P = _prefill_case(name, 410)
    run = GpuRun(wl, DEV)
    store, pre = wl.phases[0]
    run.run(store)
    say(f"[cascade prefill {name}] rows {int(pre.cu_seqlens_q[-1])} prefix {P}")
    out = _cascade_prefill(run, pre, P)
    plain = run.run(pre)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.cascade_prefill_varlen(host_values(pre.query), vals, pre.block_table, pre.cu_seqlens_q,
                                        pre.cu_seqlens_k, wl.scale, wl.num_kv_heads, P)
    err = assert_close(out.float().cpu().numpy(), ref, wl.dtype, f"cascade prefill {name}")
    assert_close(plain.float().cpu().numpy(), ref, wl.dtype, f"plain prefill {name}")
    say(f"[cascade prefill {name}] max abs err {err:.3e}")


def test_cascade_prefill_fp8():
    from oracle import fp8
    wl, P = _prefill_case("g5_d128_p256", 411, cache_dtype=torch.float8_e4m3fn)
    run = GpuRun(wl, DEV)
    run.kv_scale = 0.5
    store, pre = wl.phases[0]
    before = bits(wl.kv_cache)
    run.run(store)
    say("[cascade prefill fp8]")
    out = _cascade_prefill(run, pre, P)
    torch.cuda.synchronize()
    vals = fp8.dequantize(fp8.store_kv_fp8(before, store.key.float().numpy(), store.value.float().numpy(),
                                           store.slot_mapping, 0.5), 0.5)
    ref = oracle.cascade_prefill_varlen(host_values(pre.query), vals, pre.block_table, pre.cu_seqlens_q,
                                        pre.cu_seqlens_k, wl.scale, wl.num_kv_heads, P)
    assert_close(out.float().cpu().numpy(), ref, torch.bfloat16, "cascade prefill fp8")


def test_cascade_prefill_full_size():
    """8 sequences sharing a 2048-key prefix, cached contexts U[2048, 4096], a 512-row chunk
    each, H 32/8, D 128: every output against the oracle's plain prefill definition (which the
    cascade oracle is pinned to equal; the row-by-row cascade oracle takes minutes here)."""
    wl = W.shared_prefix_prefill()
    run = GpuRun(wl, DEV)
    store, pre = wl.phases[0]
    run.run(store)
    say("[cascade prefill full size] 8 x 512 rows, prefix 2048")
    out = _cascade_prefill(run, pre, 2048)
    torch.cuda.synchronize()
    vals = host_values(run.cache.cpu())
    ref = oracle.prefill_varlen(host_values(pre.query), vals, pre.block_table, pre.cu_seqlens_q,
                                pre.cu_seqlens_k, wl.scale, wl.num_kv_heads)
    err = assert_close(out.float().cpu().numpy(), ref, wl.dtype, "cascade prefill full size")
    say(f"[cascade prefill full size] max abs err {err:.3e}")


def test_cascade_prefill_workspace_needs_no_init_and_zero_prefix_is_plain():
    import paged_attention_block_amd as pa
    wl, P = _prefill_case("g4_d128_p48", 412)
    run = GpuRun(wl, DEV)
    store, pre = wl.phases[0]
    run.run(store)
    rows = int(pre.cu_seqlens_q[-1])
    need = pa.pa_cascade_prefill_varlen_workspace_size(run.cache, rows, wl.num_heads, P)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    a = _cascade_prefill(run, pre, P, workspace=ws)
    b = _cascade_prefill(run, pre, P)
    zero = _cascade_prefill(run, pre, 0)
    plain = run.run(pre)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(zero.view(torch.int16), plain.view(torch.int16))

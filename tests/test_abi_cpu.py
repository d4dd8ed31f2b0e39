"""C ABI on the CPU: the library loads, exports every function include/pa.h declares, and
rejects bad arguments on the host before any HIP call (no kernel ever runs here)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import paged_attention_block_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation or has zero work


def _declared():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.lib_path()):
        pytest.skip("libpa.so not built")
    return pa.load()


def desc(nb=64, bs=16, hkv=2, d=128, dtype=1, ptr=FAKE, kv_scale=1.0):
    return ctypes.byref(pa._CacheDesc(ptr, nb, bs, hkv, d, dtype, kv_scale))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"pa_store_kv", "pa_copy_blocks", "pa_prefill_varlen", "pa_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.pa_status_string(0) == b"ok"
    assert b"argument" in lib.pa_status_string(1)
    assert b"unknown" in lib.pa_status_string(99)


def test_zero_work_is_ok_without_launch(lib):
    assert lib.pa_store_kv(desc(), None, None, None, 0, None) == 0
    assert lib.pa_copy_blocks(desc(), None, 0, None) == 0
    assert lib.pa_prefill_varlen(desc(), None, None, None, 1, None, None, 0, 0, 0, 8, 1.0, 0, None, None) == 0
    assert lib.pa_decode(desc(), None, None, None, 1, None, 0, 0, 8, 1.0, 0, None, 0, None, 0, None) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(d=96), 2, b"head_size"),
    (dict(bs=12), 2, b"block_size"),
    (dict(bs=512), 2, b"block_size"),
    (dict(dtype=7), 2, b"dtype"),
    (dict(nb=0), 1, b"num_blocks"),
    (dict(hkv=0), 1, b"num_kv_heads"),
    (dict(ptr=0), 1, b"kv_cache"),
    (dict(nb=1 << 28, bs=16), 1, b"2^31"),
])
def test_cache_descriptor_checks(lib, kw, status, needle):
    assert lib.pa_store_kv(desc(**kw), FAKE, FAKE, FAKE, 4, None) == status
    assert needle in lib.pa_last_error()


def test_null_cache_descriptor(lib):
    assert lib.pa_store_kv(None, FAKE, FAKE, FAKE, 4, None) == 1


def test_store_and_copy_argument_checks(lib):
    assert lib.pa_store_kv(desc(), None, FAKE, FAKE, 4, None) == 1
    assert lib.pa_store_kv(desc(), FAKE, FAKE, FAKE, -1, None) == 1
    assert lib.pa_copy_blocks(desc(), None, 3, None) == 1
    assert lib.pa_copy_blocks(desc(), FAKE, -2, None) == 1


def test_prefill_argument_checks(lib):
    args = lambda **k: dict(dict(out=FAKE, q=FAKE, tab=FAKE, mb=4, cuq=FAKE, cuk=FAKE, b=2, msq=10, msk=60, h=8,  # noqa: E731
                                  scale=0.1, w=0), **k)

    def call(d=None, **k):
        a = args(**k)
        return lib.pa_prefill_varlen(d or desc(), a["out"], a["q"], a["tab"], a["mb"], a["cuq"], a["cuk"],
                                     a["b"], a["msq"], a["msk"], a["h"], a["scale"], a["w"], None, None)
    assert call(h=7) == 1 and b"multiple" in lib.pa_last_error()
    assert call(h=0) == 1
    assert call(h=2 * 17) == 2 and b"16" in lib.pa_last_error()          # group 17 > 16 for bf16
    assert call(out=None) == 1
    assert call(mb=0) == 1
    assert call(msk=65) == 1 and b"max_blocks_per_seq" in lib.pa_last_error()
    # the kernels need a finite scale > 0 (a masked score times a zero or infinite scale is NaN)
    for bad in (float("nan"), -0.5, 0.0, float("inf")):
        assert call(scale=bad) == 1 and b"scale" in lib.pa_last_error(), bad
    assert call(d=desc(bs=8)) == 2                                      # bf16 needs block_size >= 16
    assert call(b=-1) == 1


def test_decode_argument_and_workspace_checks(lib):
    d = desc(nb=1000, bs=16, hkv=8, d=128)
    # partition_size 128 = chunks of at least 4 steps of 32 keys: 64 sequences of at most
    # ceil(4097 / 32) = 129 steps -> ceil(64 * 129 / 4) chunks, two partial slots each
    need = lib.pa_decode_workspace_size(d, 64, 32, 4097, 0, 128)
    assert need == -(-64 * 129 // 4) * 2 * 32 * (128 + 2) * 4
    # too small a workspace is rejected before any launch
    assert lib.pa_decode(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, 128, FAKE, need - 1, None) == 3
    assert lib.pa_decode(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, 128, None, need, None) == 3
    assert lib.pa_decode(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, 48, FAKE, need, None) == 1
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.pa_decode(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, bad, 0, None, 128, FAKE, need, None) == 1
        assert b"scale" in lib.pa_last_error()
    assert lib.pa_decode(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, -32, FAKE, need, None) == 1
    assert lib.pa_decode(d, FAKE, FAKE, FAKE, 200, FAKE, 64, 4097, 32, 0.1, 0, None, 128, FAKE, need, None) == 1
    assert lib.pa_decode(d, None, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, 128, FAKE, need, None) == 1
    # a batch that fits one chunk needs no workspace; float32 never needs one
    assert lib.pa_decode_workspace_size(d, 1, 32, 100, 0, 128) == 0
    assert lib.pa_decode_workspace_size(d, 64, 32, 0, 0, 0) == 0
    assert lib.pa_decode_workspace_size(desc(dtype=0), 64, 32, 4097, 0, 128) == 0
    # a window bounds the key span: at most 4096 + 31 keys = 129 steps per sequence
    assert lib.pa_decode_workspace_size(d, 8, 40, 33281, 4096, 128) == -(-8 * 129 // 4) * 2 * 40 * 130 * 4


def test_decode_auto_chunks_without_device(lib):
    # with no device to ask, the automatic split assumes 256 resident workgroups, shared by
    # the groups of 8 KV heads, and never cuts below 4 steps (128 keys) per chunk
    d8 = desc(nb=1000, bs=16, hkv=8, d=128)
    assert lib.pa_decode_workspace_size(d8, 64, 32, 4097, 0, 0) == 256 * 2 * 32 * 130 * 4
    d16 = desc(nb=1000, bs=16, hkv=16, d=64)
    assert lib.pa_decode_workspace_size(d16, 64, 32, 4097, 0, 0) == 128 * 2 * 32 * 66 * 4
    # 4 sequences of at most 100 keys: 16 steps -> 4 chunks; one sequence: 4 steps -> 1 chunk
    assert lib.pa_decode_workspace_size(d8, 4, 32, 100, 0, 0) == 4 * 2 * 32 * 130 * 4
    assert lib.pa_decode_workspace_size(d8, 1, 32, 100, 0, 0) == 0


def test_fused_store_entry_points_check_arguments(lib):
    d = desc(nb=64, bs=16, hkv=2, d=128)
    # prefill with store: key/value/slot_mapping required once there are rows
    args = (d, FAKE, FAKE, None, FAKE, FAKE, 40, FAKE, 4, FAKE, FAKE, 2, 20, 30, 8, 0.1, 0, None, None)
    assert lib.pa_prefill_varlen_with_store(*args) == 1 and b"key" in lib.pa_last_error()
    args = (d, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 4, FAKE, FAKE, 2, 20, 30, 8, 0.1, 0, None, None)
    assert lib.pa_prefill_varlen_with_store(*args) == 1
    args = (d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 4, FAKE, FAKE, 2, 20, 30, 8, 0.1, 0, None, None)
    assert lib.pa_prefill_varlen_with_store(*args) == 1                  # rows but no tokens
    args = (d, None, None, None, None, None, 0, None, 1, None, None, 0, 0, 0, 8, 0.1, 0, None, None)
    assert lib.pa_prefill_varlen_with_store(*args) == 0                  # empty batch
    # decode with store
    args = (d, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, FAKE, 3, 60, 8, 0.1, 0, None, 0, FAKE, 1 << 20, None)
    assert lib.pa_decode_with_store(*args) == 1 and b"key" in lib.pa_last_error()
    args = (d, None, None, None, None, None, None, 1, None, 0, 0, 8, 0.1, 0, None, 0, None, 0, None)
    assert lib.pa_decode_with_store(*args) == 0                          # no sequences


def test_cascade_decode_checks_and_workspace(lib):
    d = desc(nb=1000, bs=16, hkv=8, d=128)
    # own keys after a 1024-key prefix: at most 4097 - 1024 = 3073 keys = 97 steps; chunks
    # of at least 4 steps -> ceil(64 * 97 / 4) chunks; the prefix (32 steps) over 16-row
    # groups: 64 * 4 / 16 = 16 groups x 8 KV heads = 128 units -> 2 prefix chunks
    need = lib.pa_cascade_decode_workspace_size(d, 64, 32, 4097, 1024, 128)
    assert need == -(-64 * 97 // 4) * 2 * 32 * 130 * 4 + 2 * 64 * 32 * 130 * 4
    # automatic split without a device: 256 chunks
    assert lib.pa_cascade_decode_workspace_size(d, 64, 32, 4097, 1024, 0) == 256 * 2 * 32 * 130 * 4 + 2 * 64 * 32 * 130 * 4
    # no prefix: exactly pa_decode's workspace
    assert lib.pa_cascade_decode_workspace_size(d, 64, 32, 4097, 0, 128) == lib.pa_decode_workspace_size(d, 64, 32, 4097, 0, 128)
    args = lambda P, ws=need, dd=d: (dd, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, P, 128, FAKE, ws, None)  # noqa: E731
    assert lib.pa_cascade_decode(*args(1000)) == 1 and b"multiple of block_size" in lib.pa_last_error()
    assert lib.pa_cascade_decode(*args(-16)) == 1
    assert lib.pa_cascade_decode(*args(4112)) == 1 and b"max_seq_len" in lib.pa_last_error()
    assert lib.pa_cascade_decode(*args(1024, need - 1)) == 3
    assert lib.pa_cascade_decode(*args(1024, need, desc(dtype=0))) == 2 and b"bf16" in lib.pa_last_error()
    # a misaligned workspace is refused
    a = list(args(1024)); a[12] = FAKE + 8
    assert lib.pa_cascade_decode(*a) == 1 and b"aligned" in lib.pa_last_error()
    assert lib.pa_cascade_decode(d, None, None, None, 1, None, 0, 0, 32, 0.1, 0, 0, None, 0, None) == 0


def test_fp8_cache_checks(lib):
    # the descriptor gained kv_scale in what was padding: same size as before
    assert ctypes.sizeof(pa._CacheDesc) == 32
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.pa_store_kv(desc(dtype=2, kv_scale=bad), FAKE, FAKE, FAKE, 4, None) == 1
        assert b"kv_scale" in lib.pa_last_error()
    d = desc(dtype=2, kv_scale=0.5)
    assert lib.pa_store_kv(d, FAKE, FAKE, FAKE, 0, None) == 0
    # prefill over an FP8 cache takes the same argument checks (and the kv_scale one)
    assert lib.pa_prefill_varlen(d, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 2, 10, 65, 8, 0.1, 0, None, None) == 1
    assert b"max_blocks_per_seq" in lib.pa_last_error()
    bad = desc(dtype=2, kv_scale=-2.0)
    assert lib.pa_prefill_varlen(bad, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 2, 10, 60, 8, 0.1, 0, None, None) == 1
    args = (d, FAKE, FAKE, None, FAKE, FAKE, 40, FAKE, 4, FAKE, FAKE, 2, 20, 30, 8, 0.1, 0, None, None)
    assert lib.pa_prefill_varlen_with_store(*args) == 1 and b"key" in lib.pa_last_error()
    # decode plans the same split as for bf16
    d8 = desc(nb=1000, bs=16, hkv=8, d=128, dtype=2, kv_scale=0.5)
    b8 = desc(nb=1000, bs=16, hkv=8, d=128, dtype=1)
    assert lib.pa_decode_workspace_size(d8, 64, 32, 4097, 0, 128) == lib.pa_decode_workspace_size(b8, 64, 32, 4097, 0, 128) > 0
    assert lib.pa_cascade_decode_workspace_size(d8, 64, 32, 4097, 1024, 0) == lib.pa_cascade_decode_workspace_size(b8, 64, 32, 4097, 1024, 0)
    # bf16-kernel limits apply: block_size >= 16
    assert lib.pa_decode(desc(bs=8, dtype=2, kv_scale=1.0), FAKE, FAKE, FAKE, 4, FAKE, 2, 30, 4, 0.1, 0, None, 0, FAKE, 1 << 20, None) == 2


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libpa.so every entry point raises (no CPU or oracle fallback on the product path)."""
    import torch
    import paged_attention_block_amd as pa
    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "lib_path", lambda: str(tmp_path / "libpa.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        pa.load()
    cache = torch.zeros((2, 4, 16, 2, 64), dtype=torch.bfloat16)
    key = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="is missing"):
        pa.pa_store_kv(key, key, cache, torch.zeros(3, dtype=torch.int32))
    with pytest.raises(RuntimeError, match="is missing"):
        pa.pa_decode(torch.zeros((1, 4, 64), dtype=torch.bfloat16), cache, torch.zeros((1, 4), dtype=torch.int32),
                     torch.ones(1, dtype=torch.int32), 1, 0.125, 2)


def test_decode_no_alloc_refuses_splits_beyond_its_scratch(lib):
    """pa_decode_no_alloc holds PA_DECODE_NO_ALLOC_SCRATCH_BYTES of scratch per GPU: a split
    needing more is refused on the host (workspace status) before any HIP call; zero work is
    a no-op."""
    d = desc(nb=1000, bs=16, hkv=8, d=128)
    need = lib.pa_decode_workspace_size(d, 512, 128, 4096, 0, 32)
    assert need == 512 * 128 * 2 * 128 * 130 * 4 > pa.DECODE_NO_ALLOC_SCRATCH_BYTES
    assert lib.pa_decode_no_alloc(d, FAKE, FAKE, FAKE, 300, FAKE, 512, 4096, 128, 0.1, 0, None, 32, None) == 3
    assert b"scratch" in lib.pa_last_error()
    assert lib.pa_decode_no_alloc(d, None, None, None, 1, None, 0, 0, 32, 1.0, 0, None, 0, None) == 0
    # bad scalars are still rejected as by pa_decode
    assert lib.pa_decode_no_alloc(d, FAKE, FAKE, FAKE, 300, FAKE, 64, 4097, 32, 0.1, 0, None, 48, None) == 1


def test_cascade_prefill_checks_and_workspace(lib):
    """pa_cascade_prefill_varlen: host-side rejections before any HIP call, and the workspace
    formula (states of every packed row and head per prefix chunk)."""
    d = desc(nb=1000, bs=16, hkv=8, d=128)
    P = ctypes.c_void_p
    def call(dd=None, prefix=64, tokens=100, ws=None, nbytes=0, max_k=300, nseq=2, scale=0.1):
        return lib.pa_cascade_prefill_varlen(dd or d, FAKE, FAKE, FAKE, 64, FAKE, FAKE, nseq, 80, max_k, 32,
                                             scale, prefix, tokens, ws, nbytes, None)
    assert call(desc(dtype=0)) == 2 and b"bf16" in lib.pa_last_error()
    assert call(prefix=24) == 1 and b"multiple of block_size" in lib.pa_last_error()
    assert call(prefix=320) == 1 and b"exceeds max_seqlen_k" in lib.pa_last_error()
    assert call(scale=-1.0) == 1
    assert call(tokens=-1) == 1
    assert call(tokens=0) == 1 and b"num_tokens is 0" in lib.pa_last_error()
    assert call(nseq=0, tokens=0) == 0                       # empty batch: no-op
    need = lib.pa_cascade_prefill_varlen_workspace_size(d, 100, 32, 64)
    assert need > 0 and need % (100 * 32 * 130 * 4) == 0     # whole prefix chunks of states
    assert call(ws=FAKE, nbytes=need - 1) == 3
    assert call(ws=None, nbytes=0) == 3
    assert call(ws=FAKE + 4, nbytes=need) == 1 and b"aligned" in lib.pa_last_error()
    assert lib.pa_cascade_prefill_varlen_workspace_size(d, 100, 32, 0) == 0
    assert lib.pa_cascade_prefill_varlen_workspace_size(desc(dtype=0), 100, 32, 64) == 0

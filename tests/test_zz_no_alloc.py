"""pa_decode_no_alloc (the decode entry point that allocates nothing, for callers that
cannot allocate device memory) against pa_decode with a caller-owned workspace: the same
kernels on the same split, so the outputs are compared bit for bit, and both against the
oracle within the bf16 tolerance.  Two calls in a row share the library's scratch, the
second with a smaller batch; a split too large for the scratch is refused before any launch.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import GpuRun, assert_close, host_values, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_attention_block_amd as pa
    pa.load()
    yield
    torch.cuda.synchronize()


def _decode_both(wl, partition_size, alibi=None):
    import paged_attention_block_amd as pa
    run = GpuRun(wl, DEV)
    store, dec = wl.phases[0]
    run.run(store)
    q = dec.query.to(DEV)
    table, lens = run.i32(dec.block_table), run.i32(dec.seq_lens)
    slopes = None if alibi is None else torch.from_numpy(np.asarray(alibi, np.float32)).to(DEV)
    ref_gpu = pa.pa_decode(q, run.cache, table, lens, int(dec.max_seq_len), wl.scale, wl.num_kv_heads,
                           wl.sliding_window, partition_size=partition_size, alibi_slopes=slopes)
    out = torch.full_like(q, float("nan"))
    got = pa.pa_decode_no_alloc(q, run.cache, table, lens, int(dec.max_seq_len), wl.scale, wl.num_kv_heads,
                                wl.sliding_window, out=out, partition_size=partition_size, alibi_slopes=slopes)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref_gpu.view(torch.int16)), "differs from pa_decode"
    vals = host_values(run.cache.cpu())
    ref = oracle.decode(host_values(dec.query), vals, dec.block_table, dec.seq_lens, wl.scale, wl.num_kv_heads,
                        wl.sliding_window, alibi)
    return assert_close(got.float().cpu().numpy(), ref, wl.dtype, "no_alloc decode")


def test_no_alloc_decode_two_calls_second_smaller():
    """The GQA decode batch (B 64, contexts U[512, 4096], H 32/8, D 128), then a smaller
    windowed batch with more heads per KV head and a fixed partition size: the second call
    reuses the scratch the first one left filled."""
    big = W.config(2)
    say("[no_alloc] B 64 GQA decode, automatic split")
    err = _decode_both(big, 0)
    say(f"[no_alloc] max abs err {err:.3e}")
    small = W.build("no_alloc_small", 77, [W.SeqSpec(c, [1], ["decode"]) for c in (300, 17, 1200, 64, 999)],
                    num_heads=16, num_kv_heads=2, head_size=128, block_size=16, dtype=torch.bfloat16,
                    sliding_window=500)
    slopes = np.array([2.0 ** (-8.0 * (i + 1) / 16) for i in range(16)])
    say("[no_alloc] B 5 windowed decode, partition 64, ALiBi")
    err = _decode_both(small, 64, slopes)
    say(f"[no_alloc] max abs err {err:.3e}")


def test_no_alloc_rejects_a_split_beyond_the_scratch():
    import paged_attention_block_amd as pa
    # 512 sequences x 128 heads with 32-key partitions: far more partial states than 32 MiB
    cache = torch.zeros(2, 64, 16, 8, 128, dtype=torch.bfloat16, device=DEV)
    need = pa.pa_decode_workspace_size(cache, 512, 128, 4096, 0, 32)
    assert need > pa.DECODE_NO_ALLOC_SCRATCH_BYTES
    q = torch.zeros(512, 128, 128, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(512, 256, dtype=torch.int32, device=DEV)
    lens = torch.full((512,), 4096, dtype=torch.int32, device=DEV)
    with pytest.raises(pa.PaError, match="scratch"):
        pa.pa_decode_no_alloc(q, cache, table, lens, 4096, 0.1, 8, partition_size=32)
    torch.cuda.synchronize()

"""fp64 CPU oracle for paged attention (and, in ``oracle.fp8``, an FP8 KV cache): test
infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package.  It holds no C sources, so there is nothing to compile for it.
"""

from .paged_attention import (  # noqa: F401
    alibi_bias,
    allowed_mask,
    attention_probs,
    attention_rows,
    cascade_decode,
    cascade_prefill_varlen,
    cascade_split,
    copy_blocks,
    decode,
    gather_kv,
    key_range,
    kv_head_of,
    merge_partials,
    partial_attention,
    prefill_varlen,
    store_kv,
)
from . import fp8  # noqa: F401,E402

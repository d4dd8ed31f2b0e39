"""Seeded synthetic workloads shared by the tests, the bench and the smoke check."""

from .gen import (  # noqa: F401
    CONFIG_NAMES, CopyOp, DecodeOp, PrefillOp, SeqSpec, StoreOp, Workload, build, config,
    cu_seqlens, shared_prefix_decode, shared_prefix_prefill, slot_mapping,
)

"""Benchmark of the paged-attention hot path on one MI355X.

Default run (one JSON line on stdout):
  * headline, ``value``: GQA paged decode, B 64, contexts U[512, 4096], H 32 / Hkv 8,
    D 128, block 16, bf16.  One step = store the 64 new tokens through slot_mapping, then
    decode.  ``value`` = algorithmic bytes of the step / time of the step (GB/s).
  * Before every timed step an untimed read of a 1 GiB buffer evicts the 256 MB last-level
    cache (MALL) and the L2s, so the step's data comes from HBM (a read leaves clean lines:
    an eviction by writing would leave dirty ones whose write-back lands inside the timed
    step); the step is timed with HIP events around its ops (``--flush-mb 0`` turns the
    eviction off and times back-to-back steps).
  * ``prefill``: varlen causal prefill, 16 prompts of U[128, 2048] tokens, same heads;
    one step = store every prompt token, then prefill.  TFLOP/s of algorithmic FLOPs.
  * ``secondary``: chunked prefill of 512-token chunks over long contexts with a 4096-key
    window and the decode after it (8 sequences, contexts U[4096, 32768], H 40/8), and the mixed
    step copy_blocks -> store -> prefill -> decode (4 chunks + 252 decodes, H 64/8); every op
    with its roofline.
  * ``roofline`` per op: algorithmic bytes (decode) or FLOPs (prefill) of one launch over
    its mean duration, timed with HIP events on the stream the library launches on.
  * ``cpu_baseline``: the fp64 numpy oracle on the host, on a bounded sample of the same
    workload, in the same unit (``cpu_baseline_1thread``: the decode one with one BLAS thread;
    ``config1.cpu_baseline_1thread``: the fp32 smoke workload's calls on one thread).
  * ``config1``: the fp32 smoke workload (prefill step, then one decode step): times only,
    the fp32 path makes no roofline claim.
  * ``fp8``: the headline decode step with the cache in FP8 (E4M3, kv_scale 1): half the
    K/V bytes.
  * ``shared_prefix``: decode of a batch whose sequences share a prefix of cached blocks,
    as plain decode and as cascade decode (the shared prefix attended once for all
    queries): 64 sequences sharing 1024 keys (contexts U[1024, 4096]) and 256 sequences
    sharing 4096 keys (contexts U[4096, 8192]), same heads.

Algorithmic work (not the work the kernels actually do):
  decode bytes  = sum_s keys(s) * Hkv * D * 2 (K and V) * 2 B + q + out + 4 B per block-table
                  entry read and per seq_len
  prefill FLOPs = sum over (query row, allowed key, head) of 4 * D
  store bytes   = 2 * T * Hkv * D * (bytes per element read + per element stored) + 4 B per slot
  cascade bytes = decode bytes with the shared prefix's K/V and block-table entries counted
                  once for the batch

Usage: python bench.py [--steps K] [--warmup W] [--workload decode|prefill|chunked|mixed]
"""

from __future__ import annotations

import argparse
import functools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
METRIC = "paged decode HBM GB/s (% peak); varlen prefill bf16 TFLOP/s (% MFMA peak)"

WORKLOAD_CONFIG = {"decode": 2, "prefill": 3, "chunked": 4, "chunked_decode": 4, "mixed": 5,
                   "smoke": 1, "smoke_decode": 1}


# ----------------------------------------------------------------------------- algorithmic work


def key_span(sq, sk, i, window):
    p = sk - sq + i
    hi = min(p, sk - 1)
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, hi


def decode_bytes(op, wl) -> float:
    import numpy as np
    elt = 2 if wl.dtype.itemsize == 2 else 4
    row = wl.num_kv_heads * wl.head_size * wl.kv_cache.element_size()   # 1 B per element for FP8
    total = 0
    for n in op.seq_lens.astype(np.int64):
        lo = max(0, int(n) - wl.sliding_window) if wl.sliding_window > 0 else 0
        keys = int(n) - lo
        total += 2 * keys * row
        if keys > 0:
            total += 4 * ((int(n) - 1) // wl.block_size - lo // wl.block_size + 1)
    b = len(op.seq_lens)
    total += 2 * b * wl.num_heads * wl.head_size * elt + 4 * b
    return float(total)


def cascade_bytes(op, wl, prefix: int) -> float:
    """Decode bytes when the first ``prefix`` keys of every sequence are one shared prefix,
    read once: the prefix K/V and table entries once, each sequence's own keys and entries."""
    import numpy as np
    elt = 2 if wl.dtype.itemsize == 2 else 4
    row = wl.num_kv_heads * wl.head_size * wl.kv_cache.element_size()
    total = 2 * prefix * row + 4 * (prefix // wl.block_size)
    for n in op.seq_lens.astype(np.int64):
        own = int(n) - prefix
        total += 2 * own * row
        if own > 0:
            total += 4 * ((int(n) - 1) // wl.block_size - prefix // wl.block_size + 1)
    b = len(op.seq_lens)
    total += 2 * b * wl.num_heads * wl.head_size * elt + 4 * b
    return float(total)


def prefill_flops(op, wl) -> float:
    import numpy as np
    cu_q, cu_k = op.cu_seqlens_q.astype(np.int64), op.cu_seqlens_k.astype(np.int64)
    total = 0
    for s in range(len(cu_q) - 1):
        sq, sk = int(cu_q[s + 1] - cu_q[s]), int(cu_k[s + 1] - cu_k[s])
        i = np.arange(sq)
        p = sk - sq + i
        hi = np.minimum(p, sk - 1)
        lo = np.maximum(0, p - wl.sliding_window + 1) if wl.sliding_window > 0 else np.zeros_like(p)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return float(total) * wl.num_heads * 4 * wl.head_size


def store_bytes(op, wl) -> float:
    elt = 2 if wl.dtype.itemsize == 2 else 4      # the new rows as passed in
    celt = wl.kv_cache.element_size()             # as stored (1 B for FP8)
    t = len(op.slot_mapping)
    return float(2 * t * wl.num_kv_heads * wl.head_size * (elt + celt) + 4 * t)


def copy_bytes(op, wl) -> float:
    elt = wl.kv_cache.element_size()
    return float(2 * len(op.pairs) * 2 * wl.block_size * wl.num_kv_heads * wl.head_size * elt)


# ----------------------------------------------------------------------------- GPU timing


class Step:
    """Device-resident inputs of one phase and a callable that runs it."""

    def __init__(self, wl, ops, dev, partition_size=0, fused=False, alibi=False, cascade=0):
        """fused: every attention op runs as its *_with_store call on its own rows of the
        phase's store (the separate store op is dropped).  cascade > 0: decode runs as
        pa_cascade_decode over a shared prefix of that many keys."""
        import numpy as np
        import torch
        import paged_attention_block_amd as pa
        self.pa, self.torch = pa, torch
        self.wl, self.ops, self.dev = wl, ops, dev
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
        self.cache = wl.kv_cache.to(dev)
        # ALiBi: the ALiBi paper's geometric slopes 2^(-8 i / H)
        self.slopes = (torch.tensor([2.0 ** (-8.0 * (i + 1) / wl.num_heads) for i in range(wl.num_heads)],
                                    dtype=torch.float32, device=dev) if alibi else None)
        self.prepared = []
        store = next((op for op in ops if type(op).__name__ == "StoreOp"), None)
        for op in ops:
            d = {"op": op}
            name = type(op).__name__
            if fused and name == "StoreOp":
                continue
            if fused and name in ("PrefillOp", "DecodeOp"):
                d["fused"] = True
                d.update(nk=store.key[op.out_rows].to(dev), nv=store.value[op.out_rows].to(dev),
                         nslots=i32(store.slot_mapping[op.out_rows]))
            if name == "CopyOp":
                d["pairs"] = i32(op.pairs)
            elif name == "StoreOp":
                d.update(k=op.key.to(dev), v=op.value.to(dev), slots=i32(op.slot_mapping))
            elif name == "PrefillOp":
                d.update(q=op.query.to(dev), table=i32(op.block_table), cuq=i32(op.cu_seqlens_q),
                         cuk=i32(op.cu_seqlens_k))
                d["out"] = torch.empty_like(d["q"])
                d["cascade"] = cascade
                if cascade:
                    need = pa.pa_cascade_prefill_varlen_workspace_size(self.cache, op.query.shape[0],
                                                                       wl.num_heads, cascade)
                    d["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            elif name == "DecodeOp":
                d.update(q=op.query.to(dev), table=i32(op.block_table), lens=i32(op.seq_lens))
                d["out"] = torch.empty_like(d["q"])
                d["part"] = partition_size
                d["cascade"] = cascade
                if cascade:
                    need = pa.pa_cascade_decode_workspace_size(self.cache, len(op.seq_lens), wl.num_heads,
                                                               op.max_seq_len, cascade, d["part"])
                else:
                    need = pa.pa_decode_workspace_size(self.cache, len(op.seq_lens), wl.num_heads,
                                                       op.max_seq_len, wl.sliding_window, d["part"])
                d["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            self.prepared.append(d)
        self.names = [type(d["op"]).__name__ for d in self.prepared]

    def run_op(self, d):
        pa, wl, op = self.pa, self.wl, d["op"]
        name = type(op).__name__
        if name == "CopyOp":
            pa.pa_copy_blocks(self.cache, d["pairs"])
        elif name == "StoreOp":
            pa.pa_store_kv(d["k"], d["v"], self.cache, d["slots"])
        elif name == "PrefillOp" and d.get("fused"):
            pa.pa_prefill_varlen_with_store(d["q"], d["nk"], d["nv"], d["nslots"], self.cache, d["table"],
                                            d["cuq"], d["cuk"], op.max_seqlen_q, op.max_seqlen_k, wl.scale,
                                            wl.num_kv_heads, wl.sliding_window, out=d["out"],
                                            alibi_slopes=self.slopes)
        elif name == "PrefillOp" and d.get("cascade"):
            pa.pa_cascade_prefill_varlen(d["q"], self.cache, d["table"], d["cuq"], d["cuk"], op.max_seqlen_q,
                                         op.max_seqlen_k, wl.scale, wl.num_kv_heads, d["cascade"], out=d["out"],
                                         workspace=d["ws"])
        elif name == "PrefillOp":
            pa.pa_prefill_varlen(d["q"], self.cache, d["table"], d["cuq"], d["cuk"], op.max_seqlen_q,
                                 op.max_seqlen_k, wl.scale, wl.num_kv_heads, wl.sliding_window, out=d["out"],
                                 alibi_slopes=self.slopes)
        elif name == "DecodeOp" and d.get("fused"):
            pa.pa_decode_with_store(d["q"], d["nk"], d["nv"], d["nslots"], self.cache, d["table"], d["lens"],
                                    op.max_seq_len, wl.scale, wl.num_kv_heads, wl.sliding_window,
                                    out=d["out"], workspace=d["ws"], partition_size=d["part"],
                                    alibi_slopes=self.slopes)
        elif name == "DecodeOp" and d.get("cascade"):
            pa.pa_cascade_decode(d["q"], self.cache, d["table"], d["lens"], op.max_seq_len, wl.scale,
                                 wl.num_kv_heads, d["cascade"], out=d["out"], workspace=d["ws"],
                                 partition_size=d["part"])
        elif name == "DecodeOp":
            pa.pa_decode(d["q"], self.cache, d["table"], d["lens"], op.max_seq_len, wl.scale,
                         wl.num_kv_heads, wl.sliding_window, out=d["out"], workspace=d["ws"],
                         partition_size=d["part"], alibi_slopes=self.slopes)

    def time(self, steps: int, warmup: int, flush_bytes: int = 0):
        """Mean step time, mean HIP-event duration of every op, and wall time per step
        (eviction writes included) over the timed steps.  With flush_bytes > 0 each step is
        preceded by an untimed read of that many bytes (cache eviction)."""
        torch = self.torch
        scratch = torch.ones(flush_bytes // 4, dtype=torch.int32, device=self.dev) if flush_bytes else None
        sink = torch.zeros(1, dtype=torch.int32, device=self.dev)
        for w in range(warmup):
            if scratch is not None:
                torch.amax(scratch, dim=0, keepdim=True, out=sink)
            for d in self.prepared:
                self.run_op(d)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(self.dev)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.prepared) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            if scratch is not None:
                torch.amax(scratch, dim=0, keepdim=True, out=sink)
            evs[k][0].record(stream)
            for i, d in enumerate(self.prepared):
                self.run_op(d)
                evs[k][i + 1].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        n_ops = len(self.prepared)
        step_t = sum(evs[k][0].elapsed_time(evs[k][n_ops]) for k in range(steps)) / steps / 1e3
        per_op = [sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)) / steps / 1e3
                  for i in range(n_ops)]
        # median and minimum of every op over the timed steps
        self.op_stats = []
        for i in range(n_ops):
            ts = sorted(evs[k][i].elapsed_time(evs[k][i + 1]) / 1e3 for k in range(steps))
            self.op_stats.append((ts[len(ts) // 2], ts[0]))
        return step_t, per_op, wall


# ----------------------------------------------------------------------------- CPU baseline


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        return int(n)
    except Exception:
        return 1


def cpu_baseline_decode(wl, op, budget_s: float = 10.0, threads: int = 0):
    """Oracle decode of the sequences in order (wrapping around) until ~budget_s, in GB/s
    (threads > 0: BLAS limited to that many threads)."""
    if threads > 0:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            r = cpu_baseline_decode(wl, op, budget_s)
        r["cores"] = threads
        return r
    import oracle
    vals = wl.kv_cache.float().numpy()
    q = op.query.float().numpy()
    done, bytes_done, t_used = 0, 0.0, 0.0
    b = len(op.seq_lens)
    while t_used < budget_s or done < 4:
        s = done % b
        sub = type(op)(query=op.query[s:s + 1], block_table=op.block_table[s:s + 1],
                       seq_lens=op.seq_lens[s:s + 1], max_seq_len=int(op.seq_lens[s]),
                       out_rows=op.out_rows, seq_ids=[s])
        t0 = time.perf_counter()
        oracle.decode(q[s:s + 1], vals, op.block_table[s:s + 1], op.seq_lens[s:s + 1], wl.scale,
                      wl.num_kv_heads, wl.sliding_window)
        t_used += time.perf_counter() - t0
        bytes_done += decode_bytes(sub, wl)
        done += 1
    return {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle decode of {done} sequence decodes (the batch of {b} in order, "
                      f"repeated) ({bytes_done / 1e6:.1f} MB algorithmic, {t_used:.1f} s)"}


def cpu_baseline_prefill(wl, op, budget_s: float = 10.0):
    """Oracle prefill of whole sequences, shortest first, until ~budget_s; TFLOP/s."""
    import numpy as np
    import oracle
    vals = wl.kv_cache.float().numpy()
    q = op.query.float().numpy()
    lens = np.diff(op.cu_seqlens_q)
    order = np.argsort(lens)
    flops, t_used, n = 0.0, 0.0, 0
    k = 0
    while t_used < budget_s or n < 1:
        s = order[k % len(order)]
        k += 1
        a, b = int(op.cu_seqlens_q[s]), int(op.cu_seqlens_q[s + 1])
        cu_q = np.array([0, b - a]); cu_k = np.array([0, int(op.cu_seqlens_k[s + 1] - op.cu_seqlens_k[s])])
        t0 = time.perf_counter()
        oracle.prefill_varlen(q[a:b], vals, op.block_table[s:s + 1], cu_q, cu_k, wl.scale,
                              wl.num_kv_heads, wl.sliding_window)
        t_used += time.perf_counter() - t0
        sub = type(op)(query=op.query[a:b], block_table=op.block_table[s:s + 1], cu_seqlens_q=cu_q,
                       cu_seqlens_k=cu_k, max_seqlen_q=b - a, max_seqlen_k=int(cu_k[1]),
                       out_rows=op.out_rows, seq_ids=[int(s)])
        flops += prefill_flops(sub, wl)
        n += 1
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle prefill of {n} sequences, shortest first (the batch of "
                      f"{len(lens)}, repeated) "
                      f"({flops / 1e9:.1f} GFLOP algorithmic, {t_used:.1f} s)"}


def cpu_config1_1thread(budget_s: float = 2.0):
    """Oracle times of the fp32 smoke workload's attention calls with one BLAS thread: the
    prefill of both prompts, and one decode step (ms per call, mean over repeats)."""
    import workloads as W
    import oracle
    from threadpoolctl import threadpool_limits
    wl = W.config(1)
    vals = wl.kv_cache.double().numpy()
    pre = [op for op in wl.phases[0] if isinstance(op, W.PrefillOp)][0]
    dec = [op for op in wl.phases[1] if isinstance(op, W.DecodeOp)][0]
    calls = {
        "prefill": lambda: oracle.prefill_varlen(pre.query.double().numpy(), vals, pre.block_table, pre.cu_seqlens_q,
                                                 pre.cu_seqlens_k, wl.scale, wl.num_kv_heads, wl.sliding_window),
        "decode": lambda: oracle.decode(dec.query.double().numpy(), vals, dec.block_table, dec.seq_lens, wl.scale,
                                        wl.num_kv_heads, wl.sliding_window),
    }
    out = {}
    with threadpool_limits(limits=1):
        for name, fn in calls.items():
            n, t_used = 0, 0.0
            while t_used < budget_s / len(calls) or n < 3:
                t0 = time.perf_counter()
                fn()
                t_used += time.perf_counter() - t0
                n += 1
            out[name] = {"ms": round(1e3 * t_used / n, 4), "calls": n}
    return {"ops": out, "cores": 1, "kind": "oracle",
            "sample": "fp64 numpy oracle, one BLAS thread: the prefill of the two prompts (5 and 13 tokens) "
                      "and the first decode step, each repeated"}


# ----------------------------------------------------------------------------- traffic (PMC)


def source_digest(names) -> str:
    """First 16 hex digits of the sha256 over the named csrc files (in order)."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_attention_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag: str):
    """HBM bytes per launch from a committed counter summary, if it still matches the sources.

    ``profiles/<tag>_traffic.txt`` holds ``key = value`` lines: ``sources`` (csrc files the
    kernels are built from), ``source_sha256_16`` (their digest when the counters were taken)
    and ``hbm_bytes_per_launch``.  Returns None when the file is missing or the sources changed.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    try:
        names = kv["sources"].split()
        if source_digest(names) != kv.get("source_sha256_16"):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


# ----------------------------------------------------------------------------- main


def roofline(achieved, peak, unit, bound, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# shared-prefix batches: name -> (sequences, shared prefix keys, context range, query rows per
# sequence: 1 = a decode step, more = a chunked-prefill step)
SHARED_PREFIX = {"b64_p1024": (64, 1024, 1024, 4096, 1), "b256_p4096": (256, 4096, 4096, 8192, 1),
                 "prefill_b8_p2048": (8, 2048, 2048, 4096, 512)}


def shared_prefix_name(key):
    b, p, lo, hi, rows = SHARED_PREFIX[key]
    if rows > 1:
        return (f"shared-prefix chunked prefill: B {b} x {rows}-row chunks, prefix {p} keys shared, "
                f"ctx U[{lo},{hi}], H 32/8, D 128, bs 16, bf16")
    return f"shared-prefix decode: B {b}, prefix {p} keys shared, ctx U[{lo},{hi}], H 32/8, D 128, bs 16, bf16"


@functools.lru_cache(maxsize=1)
def _workload(n):
    import torch
    import workloads as W
    if n == "fp8_decode":
        # the headline decode sequences (B 64, contexts U[512, 4096]) with an FP8 cache
        c2 = W.config(2)
        return W.build("config2_fp8", 2, c2.seqs, num_heads=c2.num_heads, num_kv_heads=c2.num_kv_heads,
                       head_size=c2.head_size, block_size=c2.block_size, dtype=torch.bfloat16,
                       cache_dtype=torch.float8_e4m3fn)
    if isinstance(n, str) and n in SHARED_PREFIX:
        b, p, lo, hi, rows = SHARED_PREFIX[n]
        if rows > 1:
            return W.shared_prefix_prefill(num_seqs=b, prefix=p, lo=lo, hi=hi, chunk=rows)
        return W.shared_prefix_decode(num_seqs=b, prefix=p, lo=lo, hi=hi)
    return W.config(n)


def bench_workload(name, steps, warmup, dev, with_cpu, partition_size=0, flush_mb=1024, fused=False,
                   alibi=False, cascade=False):
    import workloads as W
    shared = name in SHARED_PREFIX
    wl = _workload(name if shared or name == "fp8_decode" else WORKLOAD_CONFIG[name])
    prefix = SHARED_PREFIX[name][1] if shared else 0
    phase = wl.phases[-1] if name == "chunked_decode" else (wl.phases[1] if name == "smoke_decode" else wl.phases[0])
    step = Step(wl, phase, dev, partition_size, fused, alibi, prefix if cascade else 0)
    step_t, per_op, wall = step.time(steps, warmup, flush_mb * 1024 * 1024)
    ops = [d["op"] for d in step.prepared]
    if shared:
        wname = shared_prefix_name(name)
    elif name == "fp8_decode":
        wname = W.CONFIG_NAMES[2] + ", cache FP8 E4M3 (kv_scale 1)"
    else:
        wname = W.CONFIG_NAMES[WORKLOAD_CONFIG[name]]
    res = {"workload": wname, "ms_per_step": round(step_t * 1e3, 4),
           "wall_ms_per_step": round(wall * 1e3, 4), "cache_eviction_MiB_per_step": flush_mb, "ops": {}}
    total_bytes, total_flops = 0.0, 0.0
    def traffic(kind):
        # committed counter summary of this op in this workload (plain calls only)
        if fused or alibi or cascade:
            return None
        return read_traffic(kind if name == kind else f"{kind}_{name}")

    for op, t, d in zip(ops, per_op, step.prepared):
        n = type(op).__name__
        fused = bool(d.get("fused"))
        # a fused call also does the store of its rows: its bytes count toward the step
        sb = 0.0
        if fused:
            rows = d["nk"].shape[0]
            elt = 2 if wl.dtype.itemsize == 2 else 4
            sb = float(2 * 2 * rows * wl.num_kv_heads * wl.head_size * elt + 4 * rows)
            total_bytes += sb
        if n == "DecodeOp" and cascade:
            b = cascade_bytes(op, wl, prefix)
            total_bytes += b
            res["ops"]["cascade_decode"] = {
                "ms": round(t * 1e3, 4), "GB/s": round(b / t / 1e9, 1), "bytes": b,
                "plain_decode_bytes": decode_bytes(op, wl), "tokens_per_s": round(len(op.seq_lens) / t, 1),
                "partition_size": d["part"] or "auto",
                "roofline": roofline(b / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm")}
        elif n == "DecodeOp":
            b = decode_bytes(op, wl)
            total_bytes += b
            res["ops"]["decode_with_store" if fused else "decode"] = {
                "ms": round(t * 1e3, 4), "GB/s": round((b + sb) / t / 1e9, 1),
                "bytes": b + sb, "tokens_per_s": round(len(op.seq_lens) / t, 1),
                "partition_size": d["part"] or "auto",
                "roofline": roofline((b + sb) / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm", traffic("decode"))}
        elif n == "PrefillOp":
            f = prefill_flops(op, wl)
            total_flops += f
            res["ops"]["prefill_with_store" if fused else ("cascade_prefill" if cascade else "prefill")] = {
                "ms": round(t * 1e3, 4), "TFLOP/s": round(f / t / 1e12, 2), "flops": f,
                "roofline": roofline(f / t / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma", traffic("prefill"))}
        elif n == "StoreOp":
            b = store_bytes(op, wl)
            total_bytes += b
            res["ops"]["store"] = {"ms": round(t * 1e3, 4), "GB/s": round(b / t / 1e9, 1), "bytes": b,
                                   "roofline": roofline(b / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm", traffic("store"))}
        elif n == "CopyOp":
            b = copy_bytes(op, wl)
            total_bytes += b
            res["ops"]["copy_blocks"] = {"ms": round(t * 1e3, 4), "GB/s": round(b / t / 1e9, 1), "bytes": b,
                                         "roofline": roofline(b / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                                                              traffic("copy_blocks"))}
    for (med, lo), (opname, r) in zip(step.op_stats, res["ops"].items()):
        r["ms_median"] = round(med * 1e3, 4)
        r["ms_min"] = round(lo * 1e3, 4)
    res["step_GB/s"] = round(total_bytes / step_t / 1e9, 2)
    res["step_TFLOP/s"] = round(total_flops / step_t / 1e12, 3)
    if with_cpu:
        for op in ops:
            if type(op).__name__ == "DecodeOp" and name == "decode":
                res["cpu_baseline"] = cpu_baseline_decode(wl, op)
            if type(op).__name__ == "PrefillOp" and name == "prefill":
                res["cpu_baseline"] = cpu_baseline_prefill(wl, op)
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOAD_CONFIG))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition-size", type=int, default=0, help="decode split-K: fewest keys per chunk (0 = auto: one chunk per resident workgroup)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB megabytes (3 times): the "
                         "reference kernel for scaling HBM byte counters")
    ap.add_argument("--no-prefill", action="store_true", help="skip the secondary prefill measurement")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the chunked-prefill and mixed-step measurements")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="untimed read of this many MiB before every step to evict the caches (0 = off)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * 1000 * 1000
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return 0
    with_cpu = not args.no_cpu_baseline
    main_res = bench_workload(args.workload, args.steps, args.warmup, dev, with_cpu, args.partition_size,
                              args.flush_mb)
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": main_res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16, seeded lengths and block tables)"}
    if "decode" in main_res["ops"]:
        line.update(value=main_res["step_GB/s"], unit="GB/s")
        line["roofline"] = main_res["ops"]["decode"]["roofline"]
        if line["roofline"]["traffic"] is not None:
            line["traffic_note"] = ("roofline.traffic (here and in every op that has one): HBM bytes per call "
                                    "from the committed FETCH_SIZE/WRITE_SIZE summary profiles/<op>[_<workload>]"
                                    "_traffic.txt, used only while its source digest matches the built "
                                    "sources (not counted in this run)")
    else:
        line.update(value=main_res["step_TFLOP/s"], unit="TFLOP/s")
        line["roofline"] = main_res["ops"]["prefill"]["roofline"]
    wl_cfg = WORKLOAD_CONFIG[args.workload]
    line["config"] = {"workload": main_res["workload"], "config_index": wl_cfg, "ops": main_res["ops"],
                      "cache_eviction_MiB_per_step": args.flush_mb,
                      "wall_ms_per_step": main_res["wall_ms_per_step"]}
    line["cpu_baseline"] = main_res.get("cpu_baseline")
    if with_cpu and args.workload == "decode":
        wl2 = _workload(2)
        line["cpu_baseline_1thread"] = cpu_baseline_decode(wl2, wl2.phases[0][-1], budget_s=5.0, threads=1)
    if args.workload == "decode" and not args.no_prefill:
        pre = bench_workload("prefill", max(10, args.steps // 2), max(3, args.warmup // 2), dev, with_cpu,
                             flush_mb=args.flush_mb)
        call = pre["ops"]["prefill"]
        # the prefill call alone (the store of the prompts is its own op in the step): its
        # roofline and the oracle's rate also sit at the top level of the line, beside the
        # decode ones, with flat copies of the figures inside "prefill"
        line["prefill_roofline"] = call["roofline"]
        line["prefill_cpu_baseline"] = pre.get("cpu_baseline")
        line["prefill"] = {"workload": pre["workload"], "value": call["TFLOP/s"], "unit": "TFLOP/s",
                           "ms_per_call": call["ms"], "roofline_frac": call["roofline"]["frac"],
                           "roofline_achieved": call["roofline"]["achieved"],
                           "roofline_peak": call["roofline"]["peak"],
                           "cpu_baseline_value": (pre.get("cpu_baseline") or {}).get("value"),
                           "step_value": pre["step_TFLOP/s"], "ms_per_step": pre["ms_per_step"],
                           "ops": pre["ops"], "roofline": call["roofline"],
                           "cpu_baseline": pre.get("cpu_baseline")}
    if args.workload == "decode" and not args.no_secondary:
        # the same two steps with the store fused into the attention call
        line["with_store"] = {}
        for name in ("decode", "prefill"):
            r = bench_workload(name, 20, 5, dev, False, flush_mb=args.flush_mb, fused=True)
            line["with_store"][name] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"],
                                        "step_GB/s" if name == "decode" else "step_TFLOP/s":
                                        r["step_GB/s"] if name == "decode" else r["step_TFLOP/s"],
                                        "ops": r["ops"]}
        # the same two steps with ALiBi slopes
        line["alibi"] = {}
        for name in ("decode", "prefill"):
            r = bench_workload(name, 20, 5, dev, False, flush_mb=args.flush_mb, alibi=True)
            line["alibi"][name] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"], "ops": r["ops"]}
        # the fp32 smoke workload (correctness path): times only
        line["config1"] = {}
        for name in ("smoke", "smoke_decode"):
            r = bench_workload(name, 20, 5, dev, False, flush_mb=args.flush_mb)
            for op in r["ops"].values():
                op.pop("roofline", None)
            line["config1"][name] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"], "ops": r["ops"]}
        if with_cpu:
            line["config1"]["cpu_baseline_1thread"] = cpu_config1_1thread()
        # the other two workloads, every op with its roofline (no CPU baseline): chunked prefill
        # with a 4096-key window and the decode after it, and the mixed step
        # copy_blocks -> store -> prefill -> decode
        # the headline decode step over an FP8 cache
        r = bench_workload("fp8_decode", 30, 5, dev, False, flush_mb=args.flush_mb)
        line["fp8"] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"], "step_GB/s": r["step_GB/s"],
                       "ops": r["ops"]}
        # batches sharing a prefix of cached blocks: plain decode / prefill, then the cascade form
        line["shared_prefix"] = {}
        for key in SHARED_PREFIX:
            line["shared_prefix"][key] = {}
            for kind, casc in (("plain", False), ("cascade", True)):
                r = bench_workload(key, 20, 5, dev, False, flush_mb=args.flush_mb, cascade=casc)
                line["shared_prefix"][key][kind] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"],
                                                    "ops": r["ops"]}
        line["secondary"] = {}
        for name in ("chunked", "chunked_decode", "mixed"):
            r = bench_workload(name, 10, 3, dev, False, flush_mb=args.flush_mb)
            line["secondary"][name] = {"workload": r["workload"], "ms_per_step": r["ms_per_step"], "ops": r["ops"]}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

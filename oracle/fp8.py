"""Plain CPU oracle of an 8-bit floating-point (FP8) KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same rules as ``oracle.paged_attention``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it).

The pages give an FP8 view of the cache and one ``kv_scale`` per call: vllm-npu 0.4.2 diff,
``torch_sdpa.py`` forward (``write_to_paged_cache(..., kv_cache_dtype, kv_scale)`` and the
decode call with ``kv_cache_dtype`` and ``kv_scale``); vLLM learning book, "05. Attention
Backends", section 5 (the cache planes viewed as an FP8 dtype when the cache is quantized).
They do not fix the format nor how the scale enters.  Readings (each pinned where a pin
exists, see the tests):

* Format: E4M3 as in the OCP 8-bit floating-point specification (the FP8 type of MI355X's
  conversion instructions): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals at exponent field 0 (steps of 2^-9), no infinities, the all-ones exponent and
  mantissa is NaN, largest finite value 448.  Encoding rounds to nearest, ties to even, and
  saturates magnitudes above 448 (infinities included) to 448.
* Scale: the cache holds ``x / kv_scale``.  The store computes ``y = fp32(x) * r`` in float32
  with ``r = fp32(1 / kv_scale)`` (both float32 operations correctly rounded) and stores
  ``encode(y)``; attention reads ``decode(code) * kv_scale``.  Which way the scale goes (divide
  at the store, multiply at the read, or the reverse) is not on the pages: parity unpinned for
  that choice alone; the pairing itself (the read undoes the store) is pinned.

Attention over an FP8 cache is the plain attention of ``oracle.paged_attention`` over the
dequantized cache.
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_encode", "e4m3_decode", "quantize", "dequantize", "store_kv_fp8"]

E4M3_MAX = 448.0
_BIAS = 7
_MANT_BITS = 3
_MIN_NORMAL_EXP = 1 - _BIAS          # -6: exponent of the smallest normal value
_SUB_QUANTUM = 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS)   # 2^-9


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of E4M3 codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> _MANT_BITS) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - _BIAS)
    sub = m * _SUB_QUANTUM
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of float32 values: nearest, ties to even; magnitudes above 448
    (infinities included) saturate to 448; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)                 # exact
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # exponent of the binade holding a (normal range), or the subnormal exponent
    _, ex = np.frexp(a)                              # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    quantum = np.exp2(e - _MANT_BITS)
    m = np.rint(a / quantum).astype(np.int64)        # round half to even
    # a carry out of the mantissa moves to the next binade (m == 16 -> 8 of the next)
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    normal = m >= 8
    code = np.where(normal, ((e + _BIAS) << _MANT_BITS) | (m - 8), m)
    code = np.where(a == 0, 0, code)
    code = np.where(nan, 0x7F, code) | sign
    return code.astype(np.uint8)


def quantize(x, kv_scale: float) -> np.ndarray:
    """Codes the store writes for values ``x``: ``encode(fp32(x) * fp32(1 / kv_scale))``."""
    r = np.float32(1.0) / np.float32(kv_scale)
    y = np.asarray(x, dtype=np.float32) * r
    return e4m3_encode(y)


def dequantize(codes, kv_scale: float) -> np.ndarray:
    """Values attention reads from an FP8 cache: ``decode(code) * kv_scale`` (fp64)."""
    return e4m3_decode(codes) * float(np.float32(kv_scale))


def store_kv_fp8(kv_codes: np.ndarray, key, value, slot_mapping, kv_scale: float) -> np.ndarray:
    """Return a copy of the code cache (uint8 ``[2, NB, BS, Hkv, D]``) with token ``t``'s
    quantized key/value rows at its slot (negative slots skipped, as the plain store)."""
    out = kv_codes.copy()
    block_size = kv_codes.shape[2]
    kq = quantize(key, kv_scale)
    vq = quantize(value, kv_scale)
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        out[0, block, offset] = kq[t]
        out[1, block, offset] = vq[t]
    return out

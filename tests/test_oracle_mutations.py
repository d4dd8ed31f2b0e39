"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Every mutation replaces one oracle helper for the duration of a test; the pins from
``test_oracle.py`` are then run and at least one of them must fail.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle.paged_attention as pa
from tests import test_oracle as pins

PIN_FUNCS = [
    lambda gd: pins.test_mask_worked_examples(gd, "mask_sk8_sq4_w6.txt"),
    lambda gd: pins.test_mask_worked_examples(gd, "mask_sk5_sq3_w2.txt"),
    lambda gd: pins.test_matches_dense_sdpa_on_contiguous_kv(4, 2, 3),
    lambda gd: pins.test_matches_dense_sdpa_on_contiguous_kv(6, 2, 0),
    lambda gd: pins.test_square_causal_matches_sdpa_is_causal(),
    lambda gd: pins.test_closed_forms(),
    lambda gd: pins.test_chunked_prefill_equals_one_shot(),
    lambda gd: pins.test_decode_equals_last_row_of_prefill(),
    lambda gd: pins.test_block_size_invariance(),
    lambda gd: pins.test_gqa_equals_explicitly_duplicated_kv_heads(),
    lambda gd: pins.test_store_worked_example(gd),
    lambda gd: pins.test_alibi_matches_the_pages_bias_construction(),
    lambda gd: pins.test_alibi_closed_forms(),
    lambda gd: pins.test_cascade_equals_dense_attention_and_plain_decode(8, [8, 9, 21, 30]),
    lambda gd: pins.test_cascade_uniform_weights_closed_form(),
    lambda gd: pins.test_merge_partials_of_any_split_is_the_whole_softmax(),
    lambda gd: pins.test_cascade_prefill_equals_sdpa_and_plain_prefill("chunks"),
    lambda gd: pins.test_cascade_prefill_uniform_weights_closed_form(),
]


def _window_off_by_one(row, sq, sk, w):
    p = sk - sq + row
    return (max(0, p - w) if w > 0 else 0), min(p, sk - 1)


def _causal_exclusive(row, sq, sk, w):
    p = sk - sq + row
    return (max(0, p - w + 1) if w > 0 else 0), min(p - 1, sk - 1)


def _top_left_aligned(row, sq, sk, w):
    p = row
    return (max(0, p - w + 1) if w > 0 else 0), min(p, sk - 1)


def _gqa_modulo(head, num_heads, num_kv_heads):
    return head % num_kv_heads


def _gather_swapped_planes(kv_cache, table_row, positions, kv_head):
    k, v = _orig_gather(kv_cache, table_row, positions, kv_head)
    return v, k


def _gather_wrong_offset(kv_cache, table_row, positions, kv_head):
    bs = kv_cache.shape[2]
    k = np.stack([kv_cache[0, int(table_row[j // bs]), (bs - 1 - j % bs), kv_head] for j in positions])
    v = np.stack([kv_cache[1, int(table_row[j // bs]), (bs - 1 - j % bs), kv_head] for j in positions])
    return k.astype(np.float64), v.astype(np.float64)


def _store_offset_swapped(kv_cache, key, value, slot_mapping):
    out = kv_cache.copy()
    bs = kv_cache.shape[2]
    for t, slot in enumerate(slot_mapping):
        if slot < 0:
            continue
        out[0, slot % bs, slot // bs] = key[t]
        out[1, slot % bs, slot // bs] = value[t]
    return out


def _alibi_sign_flipped(slope, key_pos, query_pos):
    return slope * (query_pos - key_pos)


def _alibi_half_slope(slope, key_pos, query_pos):
    return 0.5 * slope * (key_pos - query_pos)


def _merge_equal_weights(parts):
    live = [o for o, lse in parts if np.isfinite(lse)]
    return sum(live) / len(live) if live else np.zeros_like(parts[0][0])


def _split_overlapping(seq_len, common_prefix_len):
    return range(0, common_prefix_len), range(max(0, common_prefix_len - 1), seq_len)


_orig_gather = pa.gather_kv
_orig_split = pa.cascade_split


def _shared_segment_causal(seq_len, common_prefix_len):
    # the shared segment cut at the row's own position relative to the prefix, as if the
    # prefix were the start of each query chunk
    pre, own = _orig_split(seq_len, common_prefix_len)
    return range(0, min(common_prefix_len, max(1, seq_len - common_prefix_len))), own

MUTATIONS = {
    "window_off_by_one": ("key_range", _window_off_by_one),
    "causal_excludes_self": ("key_range", _causal_exclusive),
    "top_left_alignment": ("key_range", _top_left_aligned),
    "gqa_modulo_mapping": ("kv_head_of", _gqa_modulo),
    "k_v_planes_swapped": ("gather_kv", _gather_swapped_planes),
    "block_offset_reversed": ("gather_kv", _gather_wrong_offset),
    "store_block_offset_swapped": ("store_kv", _store_offset_swapped),
    "alibi_sign_flipped": ("alibi_bias", _alibi_sign_flipped),
    "alibi_half_slope": ("alibi_bias", _alibi_half_slope),
    "cascade_merge_equal_weights": ("merge_partials", _merge_equal_weights),
    "cascade_parts_overlap": ("cascade_split", _split_overlapping),
    "cascade_shared_segment_causal": ("cascade_split", _shared_segment_causal),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch, golden_dir):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(pa, attr, fn)
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failures = 0
    for pin in PIN_FUNCS:
        try:
            pin(golden_dir)
        except (AssertionError, IndexError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


# ----------------------------------------------------------------------------- FP8 cache


from oracle import fp8 as _fp8  # noqa: E402
from tests import test_oracle_fp8 as fp8_pins  # noqa: E402

FP8_PINS = [
    fp8_pins.test_decode_of_every_code_matches_torch,
    fp8_pins.test_encode_matches_torch_inside_the_range,
    fp8_pins.test_round_trip_error_bound,
    lambda: fp8_pins.test_power_of_two_scales_are_exact(2),
    lambda: fp8_pins.test_attention_over_grid_values_is_lossless(8.0),
]

_orig_encode, _orig_decode = _fp8.e4m3_encode, _fp8.e4m3_decode


def _encode_truncating(x):
    # round toward zero instead of to nearest: step just above each code
    x = np.asarray(x, np.float32)
    codes = _orig_encode(x)
    back = _orig_decode(codes)
    down = np.abs(back) > np.abs(x.astype(np.float64))
    return np.where(down & (codes & 0x7F > 0), codes - 1, codes).astype(np.uint8)


def _decode_bias_8(codes):
    return _orig_decode(codes) / 2.0


def _dequantize_divides(codes, kv_scale):
    return _orig_decode(codes) / float(np.float32(kv_scale))


FP8_MUTATIONS = {
    "fp8_round_toward_zero": ("e4m3_encode", _encode_truncating),
    "fp8_exponent_bias_8": ("e4m3_decode", _decode_bias_8),
    "fp8_read_divides_by_scale": ("dequantize", _dequantize_divides),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_fp8_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = FP8_MUTATIONS[name]
    monkeypatch.setattr(_fp8, attr, fn)
    failures = 0
    for pin in FP8_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"

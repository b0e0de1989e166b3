"""Planted mistakes: each mutant of the oracle must fail at least one pin.

A mutant is the oracle's source with one plausible mistake written into it (a
dropped term, a wrong sign or index, a wrong rounding rule), loaded as a fresh
module on the CPU. The pins of ``test_oracle_pins.py`` then run against the
mutant's functions; if none of them fails, the pins would not have noticed
that mistake in the real oracle either.
"""

from __future__ import annotations

import inspect
import sys
import types

import pytest

import oracle
import oracle.paged_attention as base
import tests.test_oracle_pins as pins

SRC = inspect.getsource(base)

MUTANTS = {
    "drop_scale": ("s = s64 * (K[:m_keys, k, :] @ q[r, h, :])", "s = (K[:m_keys, k, :] @ q[r, h, :])"),
    "gqa_modulo": ("return h // (num_q_heads // num_kv_heads)", "return h % num_kv_heads"),
    "causal_off_by_one": ("int(positions[r]) + 1))", "int(positions[r])))"),
    "lse_without_max": ("lse[r, h] = m + math.log(den)", "lse[r, h] = math.log(den)"),
    "no_max_subtraction_sign": ("w = np.exp(s - m)\n", "w = np.exp(m - s)\n"),
    "values_of_wrong_head": ("out[r, h, :] = (w @ V[:m_keys, k, :]) / den", "out[r, h, :] = (w @ V[:m_keys, (k + 1) % Hkv, :]) / den"),
    "gather_offset": ("    off = t % bs\n", "    off = (t + 1) % bs\n"),
    "gather_block_index": ("blk = np.asarray(table_row, np.int64)[t // bs]", "blk = np.asarray(table_row, np.int64)[t // (2 * bs)]"),
    "scatter_offset": ("off = s % pool.block_size", "off = (s + 1) % pool.block_size"),
    "bf16_shift": ("astype(np.uint32) << np.uint32(16)", "astype(np.uint32) << np.uint32(15)"),
    "round_half_up": ("np.rint(quot)", "np.floor(quot + np.float32(0.5))"),
    "scale_over_128": ("(safe / np.float32(127.0))", "(safe / np.float32(128.0))"),
    "quot_by_reciprocal": ("quot = (x32 / scale[..., None])", "quot = (x32 * (np.float32(1.0) / scale[..., None]))"),
    "int8_no_scale": ("np.asarray(raw, np.int8).astype(np.float64) * np.asarray(scale", "np.asarray(raw, np.int8).astype(np.float64) + 0 * np.asarray(scale"),
    "decode_position": ("np.array([n - 1])", "np.array([n - 2])"),
    "chunk_not_offset": ("n - L + np.arange(L)", "np.arange(L)"),
    "online_no_rescale": ("acc = acc * corr + p @ V[t0:t0 + block]", "acc = acc + p @ V[t0:t0 + block]"),
    "combine_no_shift": ("w = np.where(live, np.exp(np.where(live, lse_parts, M) - M), 0.0)",
                         "w = np.where(live, np.exp(np.where(live, lse_parts, M)), 0.0) * 0 + live"),
    "split_not_block_aligned": ("tps = block_size * (-(-per // block_size))", "tps = per"),
    "fp8_bias_8": ("(1.0 + m / 8.0) * np.power(2.0, e - 7)", "(1.0 + m / 8.0) * np.power(2.0, e - 8)"),
    "fp8_subnormal_step": ("np.where(e == 0, m * 2.0 ** -9,", "np.where(e == 0, m * 2.0 ** -10,"),
    "fp8_ties_to_odd": ("np.where(hi % 2 == 0, hi, lo)", "np.where(hi % 2 == 0, lo, hi)"),
    "fp8_truncate": ("pick = np.where(d_hi < d_lo, hi,", "pick = np.where(d_hi < 0, hi,"),
    "fp8_scale_over_240": ("(safe / np.float32(448.0))", "(safe / np.float32(240.0))"),
}

# every pin, with the arguments its pytest parametrisation would give it
PIN_CALLS = [
    (pins.test_bf16_decoding_matches_format, ()),
    (pins.test_int8_decoding_is_code_times_scale, ()),
    (pins.test_quantizer_against_exact_rational_arithmetic, ()),
    (pins.test_quantizer_bounds_and_special_cases, ()),
    (pins.test_quantizer_near_half_way_quotients, ()),
    (pins.test_fp8_decoding_matches_format, ()),
    (pins.test_fp8_decoding_matches_library, ()),
    (pins.test_fp8_encoder_matches_library_rounding, ()),
    (pins.test_fp8_quantizer_bounds_and_special_cases, ()),
    (pins.test_fp8_scatter_stores_quantized_rows, ()),
    (pins.test_gather_of_scatter_is_identity, ("f32",)),
    (pins.test_gather_of_scatter_is_identity, ("bf16",)),
    (pins.test_int8_scatter_stores_quantized_rows, ()),
    (pins.test_piecewise_chunk_writes_equal_one_shot, ("i8",)),
    (pins.test_negative_slots_are_skipped_and_bad_slots_raise, ()),
    (pins.test_output_invariant_under_block_placement, ("f32",)),
    (pins.test_direct_matches_brute_force, ()),
    (pins.test_paged_matches_library_sdpa_on_contiguous_kv, ()),
    (pins.test_tiny_decode_config_against_sdpa, ()),
    (pins.test_closed_forms, ()),
    (pins.test_one_hot_key_selects_its_value_exactly, ()),
    (pins.test_decode_equals_last_row_of_full_causal_attention, ()),
    (pins.test_chunk_row_equals_decode_at_its_position, ()),
    (pins.test_online_and_split_k_agree_with_direct, (40,)),
    (pins.test_online_softmax_rescales_when_the_max_grows, ()),
    (pins.test_split_bounds_partition_the_context, ()),
    (pins.test_lse_combine_ignores_empty_splits, ()),
]


def load_mutant(old: str, new: str) -> types.ModuleType:
    assert SRC.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    name = "oracle_mutant"
    mod = types.ModuleType(name)
    sys.modules[name] = mod        # dataclasses look their module up by name
    try:
        exec(compile(SRC.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def test_unmutated_oracle_passes_every_pin():
    for fn, args in PIN_CALLS:
        fn(*args)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mut = load_mutant(*MUTANTS[name])
    for attr in dir(oracle):
        if not attr.startswith("_") and hasattr(mut, attr):
            monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    caught = []
    for fn, args in PIN_CALLS:
        try:
            fn(*args)
        except KeyboardInterrupt:
            raise
        except BaseException:      # pytest.raises reports "did not raise" as a BaseException
            caught.append(fn.__name__)
    assert caught, f"no pin noticed mutant {name}"

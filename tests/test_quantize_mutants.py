"""Planted-mistake check for the quantizer reference's pins (CPU only).

Each case copies ``oracle/quantize.py``, plants one plausible mistake (the
grid end off by one, ties to even, sign(0) = -1, codes from the unrounded
scale, a double rounding of the 1-bit mean, a wrong tier edge, ...), loads
the copy as a module and runs the pins of ``test_quantize_pins.py`` against
it. Every mutant must fail at least one pin.
"""
import importlib.util
import os

import pytest

from tests import test_quantize_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "quantize.py")

MUTANTS = {
    "grid_end_off_by_one": ("qmax = np.float32(2 ** (width - 1) - 1)", "qmax = np.float32(2 ** (width - 1))"),
    "ties_to_even": ("return np.sign(r) * np.floor(a + 0.5)", "return np.round(r)"),
    "ties_in_fp32": ("a = np.abs(r).astype(np.float64)", "a = np.abs(r)"),
    "sign_of_zero_negative": ("codes[one] = np.where(g[one] < 0, -1, 1)", "codes[one] = np.where(g[one] <= 0, -1, 1)"),
    "codes_from_unrounded_scale": ("r = g[sel] / s32[:, None]",
                                   "r = g[sel] / (mag[sel].max(axis=1) / qmax)[:, None]"),
    "one_bit_mean_through_fp32": ("mean = mag[one].astype(np.float64).sum(axis=1) / 64.0",
                                  "mean = (mag[one].astype(np.float64).sum(axis=1) / 64.0).astype(np.float32)"),
    "one_bit_mean_count": ("mean = mag[one].astype(np.float64).sum(axis=1) / 64.0", "mean = mag[one].astype(np.float64).sum(axis=1) / 63.0"),
    "absmean_for_wide_groups": ("s16 = _stored_scale(mag[sel].max(axis=1) / qmax)",
                                "s16 = _stored_scale(mag[sel].mean(axis=1) / qmax)"),
    "no_saturation": ("return np.where(np.isinf(s16), FP16_MAX, s16)", "return s16"),
    "zero_scale_codes_kept": ("q = np.where(s32[:, None] == 0, 0, q)", "q = np.where(s32[:, None] == 0, q, q)"),
    "tiers_not_cumulative": ("for per_mille in (5, 20, 120)", "for per_mille in (5, 15, 100)"),
    "tier_edges_floor": ("cut = [(per_mille * rows + 500) // 1000", "cut = [(per_mille * rows) // 1000"),
    "ties_to_higher_row": ("np.lexsort((np.arange(rows), -freq.astype(np.float64)))",
                           "np.lexsort((-np.arange(rows), -freq.astype(np.float64)))"),
    "ascending_frequency": ("np.lexsort((np.arange(rows), -freq.astype(np.float64)))",
                            "np.lexsort((np.arange(rows), freq.astype(np.float64)))"),
    "first_block_flipped": ("return 4 if first_block_mlp else 2", "return 2 if first_block_mlp else 4"),
    "soft_tau_ignored": ("np.asarray(gumbel, np.float64).reshape(-1, 4)) / tau", "np.asarray(gumbel, np.float64).reshape(-1, 4))"),
    "soft_noise_dropped": ("(np.asarray(logits, np.float64).reshape(-1, 4) + np.asarray(gumbel, np.float64).reshape(-1, 4))",
                           "(np.asarray(logits, np.float64).reshape(-1, 4) + 0 * np.asarray(gumbel, np.float64).reshape(-1, 4))"),
    "soft_widths_reversed": ("recon = [training_reconstruction(w, b).reshape(-1, 64) for b in WIDTHS]",
                             "recon = [training_reconstruction(w, b).reshape(-1, 64) for b in WIDTHS[::-1]]"),
    "soft_cost_uses_index": ("bits = float((pi * np.array(WIDTHS, np.float64)).sum(axis=1).mean())",
                             "bits = float((pi * np.arange(1, 5, dtype=np.float64)).sum(axis=1).mean())"),
    "training_scale_rounded_to_half": ("        s = mag.max(axis=1) / qmax\n",
                                       "        s = (mag.max(axis=1) / qmax).astype(np.float16).astype(np.float32)\n"),
}

PINS = [(P.test_codes_are_the_nearest_grid_point_of_the_stored_scale, (b,)) for b in (2, 4, 8)] + \
       [(P.test_scale_is_the_nearest_half_of_max_over_grid_end, (b,)) for b in (2, 4, 8)] + \
       [(f, ()) for f in (P.test_one_bit_is_sign_and_mean_magnitude, P.test_one_bit_scale_is_rounded_once_from_the_mean,
                          P.test_ties_round_away_from_zero, P.test_rounding_just_below_a_half,
                          P.test_codes_use_the_stored_half_scale, P.test_zero_group_and_tiny_and_huge_scales,
                          P.test_mixed_widths_pick_each_groups_rule, P.test_head_recipe_mean_is_the_pages_1_18_bits,
                          P.test_head_recipe_ties_go_to_the_lower_row,
                          P.test_head_recipe_rounds_tier_edges_half_up, P.test_projection_recipe,
                          P.test_dequantize_error_bound,
                          P.test_training_reconstruction_is_the_nearest_grid_point_with_fp32_scale,
                          P.test_soft_quantizer_limits_and_bit_cost)]


def load_variant(text, path):
    path.write_text(text)
    spec = importlib.util.spec_from_file_location(f"quantize_variant_{abs(hash(text))}", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def failed_pins(mod):
    saved = P.Q
    P.Q = mod
    bad = []
    try:
        for fn, args in PINS:
            try:
                fn(*args)
            except Exception:     # an assertion, or an error the mistake causes
                bad.append(f"{fn.__name__}{args}")
    finally:
        P.Q = saved
    return bad


def test_unmutated_reference_passes_every_pin(tmp_path):
    assert failed_pins(load_variant(open(SRC).read(), tmp_path / "q.py")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site of {name} not found once"
    assert failed_pins(load_variant(text.replace(old, new), tmp_path / "q.py")), f"{name} passes every pin"

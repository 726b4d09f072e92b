"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, swaps it in, and checks that the pin
tests named for it fail.  The real oracle is restored afterwards.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_a8 as A8
from tests import test_oracle_format as F
from tests import test_oracle_linear as L
from tests import test_oracle_moe as M
from tests import test_oracle_route_sort as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "mx_oracle.c")

MUTATIONS = {
    "nibble_order": ("return (i & 1) ? (b >> 4) : (b & 15);", "return (i & 1) ? (b & 15) : (b >> 4);"),
    "scale_block_16": ("s[r * (K / 32) + k / 32]", "s[r * (K / 32) + k / 16 % (K / 32)]"),
    "e8m0_bias": ("ldexp(1.0, (s & 0xFF) - 127)", "ldexp(1.0, (s & 0xFF) - 128)"),
    "magnitude_table": ("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 4.0}"),
    "drop_up_projection": ("return gd / (1.0 + exp(-gd)) * (double)u;", "return gd / (1.0 + exp(-gd));"),
    "swap_gate_up": ("float g = dot_vals(xa + (p / k) * H, W, S, H, n, &ga);\n      float u = dot_vals(xa + (p / k) * H, W, S, H, I + n, &ua);",
                     "float u = dot_vals(xa + (p / k) * H, W, S, H, n, &ga);\n      float g = dot_vals(xa + (p / k) * H, W, S, H, I + n, &ua);"),
    "combine_wrong_gate": ("float gd = (float)((double)gates[p] * (double)d);", "float gd = (float)((double)gates[i * k] * (double)d);"),
    "tie_to_higher_id": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    "unstable_sort": ("for (int64_t f = 0; f < F; ++f) {\n    int32_t e = ids[f];", "for (int64_t f = F - 1; f >= 0; --f) {\n    int32_t e = ids[f];"),
    "softmax_over_all": ("for (int64_t j = 0; j < k; ++j) den += exp((double)l[ids[t * k + j]] - m);",
                         "for (int64_t j = 0; j < E; ++j) den += exp((double)l[j] - m);"),
    "rounding_truncates": ("double n = nearbyint(a / q);", "double n = floor(a / q);"),
    "e4m3_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "mxfp8_scale_emax": ("sbyte = (e - 1) - 8 + 127;", "sbyte = (e - 1) - 7 + 127;"),
    "e4m3_no_saturation": ("if (a >= 448.0) return 0x7E;", "if (a >= 480.0) return 0x7E;"),
    "e4m3_subnormal_spacing": ("if (a == 0.0 || lead < -6) lead = -6;", "if (a == 0.0 || lead < -7) lead = -7;"),
    "a8_h_not_quantized": ("activation_row(h + p * I, I, act8, ha + p * I);", "activation_row(h + p * I, I, 0, ha + p * I);"),
    "active_lists_idle_experts": ("if (counts[e] > 0) active[na++] = (int32_t)e;", "if (counts[e] >= 0) active[na++] = (int32_t)e;"),
    "silu_sign": ("return gd / (1.0 + exp(-gd)) * (double)u;", "return gd / (1.0 + exp(gd)) * (double)u;"),
    "combine_drops_last_slot": ("      for (int64_t j = 0; j < k; ++j) {\n        int64_t p = i * k + j;",
                                "      for (int64_t j = 0; j < k - 1; ++j) {\n        int64_t p = i * k + j;"),
    "down_uses_first_slot_expert": ("        int64_t p = i * k + j;\n        int64_t e = ids[p];",
                                    "        int64_t p = i * k + j;\n        int64_t e = ids[i * k];"),
    "gate_up_wrong_token": ("float g = dot_vals(xa + (p / k) * H, W, S, H, n, &ga);",
                            "float g = dot_vals(xa + (p % k) * H, W, S, H, n, &ga);"),
    "bound_term_ungated": ("        sm += (double)gates[p] * as;", "        sm += as;"),
    "gates_not_normalized": ("gates[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - m) / den);",
                             "gates[t * k + j] = (float)(exp((double)l[ids[t * k + j]] - m));"),
    "offsets_missing_last": ("for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];",
                             "for (int64_t e = 0; e + 1 < E; ++e) offsets[e + 1] = offsets[e] + counts[e];"),
}

# pin tests expected to catch each mutation (each entry: callable(tmp_fixture_args) -> runs asserts)
def _fmt():
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_format.json")) as f:
        return json.load(f)


def _mags():
    return _fmt()["magnitudes"]


CATCHERS = {
    "nibble_order": [lambda: L.test_one_hot_extracts_weight_column(_mags())],
    "scale_block_16": [lambda: L.test_one_hot_extracts_weight_column(_mags())],
    "e8m0_bias": [lambda: F.test_e8m0_all_bytes(_fmt())],
    "magnitude_table": [lambda: F.test_e2m1_magnitudes_match_page(_fmt())],
    "drop_up_projection": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "swap_gate_up": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "combine_wrong_gate": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "tie_to_higher_id": [lambda: R.test_route_ties_go_to_lower_id()],
    "unstable_sort": [lambda: R.test_sort_matches_stable_argsort(4, 256, 8)],
    "softmax_over_all": [lambda: R.test_route_matches_lexsort_and_softmax(4, 256, 8)],
    "rounding_truncates": [lambda: F.test_bf16_rne_matches_torch_cast_on_floats()],
    "e4m3_bias": [lambda: A8.test_e4m3_decode_matches_torch()],
    "mxfp8_scale_emax": [lambda: A8.test_quantize_rounds_like_torch_over_all_bf16(0, 1.75)],
    "e4m3_no_saturation": [lambda: A8.test_quantize_rounds_like_torch_over_all_bf16(0, 2 - 2.0 ** -7)],
    "e4m3_subnormal_spacing": [lambda: A8.test_quantize_rounds_like_torch_over_all_bf16(0, 1.75)],
    "a8_h_not_quantized": [lambda: A8.test_a8_moe_single_expert_reduces_to_a8_linear()],
    "active_lists_idle_experts": [lambda: R.test_sort_matches_stable_argsort(32, 256, 8)],
    "silu_sign": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "combine_drops_last_slot": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "down_uses_first_slot_expert": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "gate_up_wrong_token": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "bound_term_ungated": [lambda: M.test_brute_force_tiny_moe(0, _mags())],
    "gates_not_normalized": [lambda: R.test_route_matches_lexsort_and_softmax(4, 256, 8)],
    "offsets_missing_last": [lambda: R.test_sort_matches_stable_argsort(4, 256, 8)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mx_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(so), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    for catch in CATCHERS[name]:
        with pytest.raises(AssertionError):
            catch()
    # the real oracle still passes the same pins
    monkeypatch.undo()
    oracle._lib = None
    for catch in CATCHERS[name]:
        catch()

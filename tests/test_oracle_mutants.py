"""Plant plausible mistakes in a copy of the oracle and check a pin fails.

Each mutant is the oracle's own source with one textual change, loaded as a
separate module on the CPU; the pin tests of ``test_oracle_pins`` are then
run against it.  A pin set that lets a mutant pass would not have caught
that mistake in the real oracle.
"""
import importlib.util
import os
import types

import numpy as np
import pytest

import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "stce_oracle.py")

MUTANTS = {
    "tie-break by descending id": ("np.lexsort((ids, -s))", "np.lexsort((-ids, -s))",
                                   ["test_order_matches_pairwise_definition"]),
    "top-p drops the crossing token": ("n_p = r + 1", "n_p = max(r, 1)",
                                       ["test_top_p_includes_crossing_token"]),
    "min-p compared in the wrong space": ("thr = math.log(mp)", "thr = -mp",
                                          ["test_min_p_closed_form_matches_probability_space"]),
    "temperature by reciprocal multiply": ("q = z32.astype(np.float64) / t[:, None]",
                                           "q = z32 * (np.float32(1) / t.astype(np.float32))[:, None]",
                                           ["test_temperature_division_is_correctly_rounded"]),
    "gradient misses the 1/T factor": ("dz[i] = g[i] * (onehot - q) / t64[i]", "dz[i] = g[i] * (onehot - q)",
                                       ["test_gradients_match_central_differences"]),
    "gradient sign flipped": ("dz[i] = g[i] * (onehot - q) / t64[i]", "dz[i] = g[i] * (q - onehot) / t64[i]",
                              ["test_gradients_match_torch_autograd", "test_loss_sign_convention"]),
    "lse over the unfiltered row": ("lse = mx + math.log(np.exp(u[i, S] - mx).sum())",
                                    "lse = u[i].max() + math.log(np.exp(u[i] - u[i].max()).sum())",
                                    ["test_filtered_logprob_closed_form"]),
    "out-of-support rows keep a gradient": ("        if not fwd[\"in_support\"][i]:\n            continue\n", "",
                                            ["test_out_of_support_has_minus_inf_and_zero_gradient"]),
    "top-k keeps one token too many": ("n_k = k if 0 < k < V else V", "n_k = min(k + 1, V) if 0 < k < V else V",
                                       ["test_support_matches_brute_force", "test_tie_group_split_by_token_id"]),
    "min-p against the second-largest key": ("gap = s64[pi] - m ", "gap = s64[pi] - s64[pi[min(1, V - 1)]] ",
                                             ["test_min_p_one_keeps_the_whole_max_tie_group",
                                              "test_min_p_closed_form_matches_probability_space"]),
    "dW uses the wrong operand": ("return np.asarray(dz @ W64), np.asarray(dz.T @ h64)",
                                  "return np.asarray(dz @ W64), np.asarray(dz.T @ (h64 * 0.5))",
                                  ["test_gradients_match_central_differences"]),
    "CISPO weight not a stop-gradient": ("            g[t] = -A[t] * wgt\n",
                                         "            g[t] = -A[t] * wgt - (A[t] * r * lp[t] if r < 1.0 + eh else 0.0)\n",
                                         ["test_policy_gradient_matches_autograd_of_objective"]),
    "clipped surrogate takes the max": ("            if unclipped <= clipped:", "            if unclipped >= clipped:",
                                        ["test_policy_loss_special_cases",
                                         "test_clipped_policy_gradient_matches_central_differences"]),
    "support entropy over the full row": ('        out["entropy_support"][i] = _entropy(u[i, S])[1]',
                                          '        out["entropy_support"][i] = _entropy(u[i])[1]',
                                          ["test_entropy_closed_forms", "test_entropy_matches_scipy_and_bounds"]),
    "entropy with a plus sign": ("    return lse, float(-(np.exp(logp) * logp).sum())",
                                 "    return lse, float((np.exp(logp) * logp).sum())",
                                 ["test_entropy_closed_forms", "test_entropy_matches_scipy_and_bounds"]),
    "ignored rows score -inf": ("        lp = 0.0 if ignored[i] else", "        lp = -math.inf if ignored[i] else",
                                ["test_ignored_rows_score_zero_and_get_no_gradient"]),
    "policy gradient in the objective's sign": ("    return dict(loss=loss * sc, g=g * sc, ratio=ratio)",
                                                "    return dict(loss=loss * sc, g=-g * sc, ratio=ratio)",
                                                ["test_policy_gradient_matches_autograd_of_objective",
                                                 "test_clipped_policy_gradient_matches_central_differences"]),
    "pre-GEMM gradient misses the 1/T": ("    return dH / float(np.float32(temperature)), dW",
                                         "    return dH, dW",
                                         ["test_pre_gemm_temperature_equals_post_gemm_for_a_power_of_two",
                                          "test_pre_gemm_gradient_matches_autograd"]),
    "pre-GEMM hidden not rounded to the operand": ('    return round_to_bf16(q) if operand == "bf16" else q',
                                                   "    return q",
                                                   ["test_pre_gemm_hidden_matches_torch_division_and_rounding"]),
    "bf16 rounding half up": ("    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000",
                              "    b = (b + 0x8000) & 0xFFFF0000",
                              ["test_round_to_bf16_matches_torch_and_ties_to_even"]),
    "bf16 lane skips the projection's rounding": (
        "    zb = round_to_bf16(np.asarray(z, np.float64).astype(np.float32))",
        "    zb = np.asarray(z, np.float64).astype(np.float32)",
        ["test_bf16_lane_keys_follow_the_value_program_exactly"]),
    "bf16 lane logprob not rounded": (
        "            lp = float(round_to_bf16(np.float32(lp)))             # the lane's logprob dtype",
        "            lp = float(lp)",
        ["test_bf16_lane_logprob_is_the_bf16_log_softmax_of_the_keys"]),
    "bf16 lane gradient from the fp64 logits": (
        '    u = fwd["keys"].astype(np.float64) if lane == "bf16" else z / t64[:, None]',
        "    u = z / t64[:, None]",
        ["test_bf16_lane_gradient_is_the_straight_through_vjp"]),
    "e4m3 rounding ties away from zero": (
        "    q = np.rint(a * np.exp2(3.0 - e))                                   # 8 .. 16, exact scaling",
        "    q = np.floor(a * np.exp2(3.0 - e) + 0.5)",
        ["test_e4m3_encode_matches_torch_and_ties_to_even"]),
    "fp8 dW from the unquantized hidden rows": (
        "        hr = fp8_dequant_rows(hr)\n", "",
        ["test_fp8_lane_gradient_is_the_straight_through_vjp"]),
    "fp8 logits miss the row scale": (
        "    return acc * np.asarray(w_scale, np.float32).astype(np.float64)[None, :] * a.astype(np.float64)[:, None]",
        "    return acc * np.asarray(w_scale, np.float32).astype(np.float64)[None, :]",
        ["test_fp8_logits_reduce_to_the_plain_product_on_exact_operands"]),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    old, new, tests = MUTANTS[name]
    mutant = _load_mutant(old, new)
    monkeypatch.setattr(pins, "oracle", mutant)
    caught = []
    for t in tests:
        rng = np.random.Generator(np.random.PCG64(20261203))
        fn = getattr(pins, t)
        try:
            args = fn.__code__.co_varnames[: fn.__code__.co_argcount]
            if "objective" in args:
                for obj in ("cispo", "clip"):
                    fn(np.random.Generator(np.random.PCG64(20261203)), obj)
            else:
                fn(rng) if args else fn()
        except Exception:  # noqa: BLE001 -- any failure of the pin counts
            caught.append(t)
    assert caught, f"mutant '{name}' survived {tests}"

"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of the oracle source with one plausible mistake (a dropped term, a wrong
sign, index or operand), compiled with gcc into a temporary directory. The pin suite is run
against it and at least one pin must fail. Mistakes are planted only in a copy of the oracle,
never in the product library.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "tie_order_reversed": [("(xu == xv && u < v)", "(xu == xv && u > v)")],
    "topk_smallest_first": [("return xu > xv ||", "return xu < xv ||")],
    "insertion_never_displaces_first": [("while (pos > 0 && comes_before", "while (pos > 1 && comes_before")],
    "lse_drops_max": [("const double row_lse = m + log(sum + comp);", "const double row_lse = log(sum + comp);")],
    "lse_drops_log": [("const double row_lse = m + log(sum + comp);", "const double row_lse = m + (sum + comp);")],
    "lse_drops_first_term": [("for (int v = 0; v < V; ++v) {\n            double t = exp", "for (int v = 1; v < V; ++v) {\n            double t = exp")],
    "unary_sign_flipped": [("best_x[j] - row_lse", "row_lse - best_x[j]")],
    "bf16_wrong_shift": [("<< 16;", "<< 15;")],
    "gate_transposed_weight": [("(size_t)h * r + d", "(size_t)d * H + h")],
    "gate_drops_first_term": [("for (int h = 0; h < H; ++h)", "for (int h = 1; h < H; ++h)")],
    "lattice_prev_from_current_position": [("cand_ids[(row - 1) * k + i]", "cand_ids[row * k + i]")],
    "lattice_codebooks_swapped": [("oracle_value(pred_cb, cb_dtype, (size_t)prev", "oracle_value(@@S, cb_dtype, (size_t)prev"),
                                  ("oracle_value(succ_cb, cb_dtype, (size_t)cand", "oracle_value(pred_cb, cb_dtype, (size_t)cand"),
                                  ("@@S", "succ_cb")],
    "lattice_pred_table_for_both": [("oracle_value(pred_cb, cb_dtype, (size_t)prev", "oracle_value(succ_cb, cb_dtype, (size_t)prev")],
    "lattice_drops_gate": [(" *\n                               g[row * r + d];", ";")],
    "lattice_drops_last_rank": [("for (int d = 0; d < r; ++d)", "for (int d = 0; d < r - 1; ++d)")],
    "lattice_anchor_of_first_sequence": [("anchor_ids[b] : cand_ids", "anchor_ids[0] : cand_ids")],
    "lattice_unary_of_predecessor": [("unary[row * k + j] + acc", "unary[row * k + i] + acc")],
    "walk_tie_to_highest_index": [("if (e[j] > e[best])", "if (e[j] >= e[best])")],
    "walk_ignores_predecessor": [("edges + (row * k + prev) * k", "edges + (row * k + 0) * k")],
    "walk_margin_sign": [("e[best] - second", "second - e[best]")],
    "walk_score_wrong_edge": [("total += e[best];", "total += e[0];")],
    "sample_temperature_inverted": [("exp((e[j] - m) / temperature)", "exp((e[j] - m) * temperature)")],
    "sample_drops_max_shift_sign": [("exp((e[j] - m) / temperature)", "exp((m - e[j]) / temperature)")],
    "sample_ignores_predecessor": [("edges + (row * k + prev) * k;\n            double m", "edges + (row * k + 0) * k;\n            double m")],
    "sample_uniform_complement": [("uniforms[row] * total", "(1.0 - uniforms[row]) * total")],
    "pmin_confidence_scaled": [("z += exp(e[j] - m);", "z += exp((e[j] - m) / (temperature > 0 ? temperature : 1));")],
    "pmin_stops_at_equality": [("c < p_min", "c <= p_min")],
    "pmin_length_off_by_one": [("stop = p;", "stop = p + 1;")],
    "conv_tap_reads_ahead": [("((size_t)b * T + (t - tap)) * C + c)", "((size_t)b * T + (t + tap < T ? t + tap : t)) * C + c)")],
    "conv_dyn_at_source_row": [("(((size_t)b * T + t) * K + tap) * ng + c / G)", "(((size_t)b * T + (t - tap)) * K + tap) * ng + c / G)")],
    "conv_group_index_modulo": [("* ng + c / G)", "* ng + c % ng)")],
    "conv_crosses_blocks": [("if (t - tap < 0)\n                        continue;", "if (b == 0 && t - tap < 0)\n                        continue;")],
    "conv_drops_base": [("oracle_value(base, dtype, (size_t)tap * C + c) +", "0.0 +")],
    "lmhead_transposed_weight": [("oracle_value(W_lm, dtype, (size_t)v * H + h)", "oracle_value(W_lm, dtype, (size_t)h * V + v)")],
    "lmhead_drops_first_h": [("for (int h = 0; h < H; ++h)\n                dot +=", "for (int h = 1; h < H; ++h)\n                dot +=")],
    "lmhead_first_row_only": [("oracle_value(hidden, dtype, (size_t)row * H + h)", "oracle_value(hidden, dtype, (size_t)h)")],
    "lmhead_unary_without_lse": [("top_x[j] - x_lse", "top_x[j]")],
    "lmhead_lse_drops_max": [("const double x_lse = mx + log(total + carry);", "const double x_lse = log(total + carry);")],
}


def _build(name, tmp_path_factory):
    src = open(oracle.SOURCE).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutant {name}: pattern not found: {old!r}"
        src = src.replace(old, new, 1)
    d = tmp_path_factory.mktemp(name)
    path = os.path.join(d, "dflash2_oracle.c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.Oracle(oracle.compile_oracle(path, os.path.join(d, "libmutant.so")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path_factory):
    mutant = _build(name, tmp_path_factory)
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"

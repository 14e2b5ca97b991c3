"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case rewrites one line of the oracle's source into a plausible mistake (a dropped term, a
swapped operand, an off-by-one index, an inverted comparison), loads the result as a separate
module, and runs the pins of tests/test_oracle_pins.py against it: at least one must fail.
The real oracle module is never modified.
"""
import sys
import types

import pytest

import oracle.sv_oracle as real
import tests.test_oracle_pins as pins

SRC = open(real.__file__).read()

MUTATIONS = {
    "temperature_dropped": (
        "z = np.asarray(logits, dtype=np.float64) / float(tau)",
        "z = np.asarray(logits, dtype=np.float64)"),
    "ratio_inverted": ("return min(1.0, a / c)", "return min(1.0, c / max(a, 1e-300))"),
    "residual_sign_swapped": ("return np.maximum(0.0, p - q)", "return np.maximum(0.0, q - p)"),
    "accept_test_inverted": ("if not u < thresholds[i]:", "if u < thresholds[i]:"),
    "scan_does_not_stop": ("            n = i\n            break\n\n    if n < k:",
                           "            n = i\n\n    if n < k:"),
    "bonus_row_off_by_one": ("w = p_rows[k]", "w = p_rows[max(k - 1, 0)]"),
    "draft_rows_from_target": (
        "q_rows = [softmax_fp64(decode_logits(draft_rows[i], dtype), tau)",
        "q_rows = [softmax_fp64(decode_logits(target_rows[i], dtype), tau)"),
    "commits_rejected_draft": (
        "committed = [int(tokens[i]) for i in range(n)] + [y] + [-1] * (K - n)",
        "committed = [int(tokens[i]) for i in range(n)] + "
        "[int(tokens[n]) if n < k else y] + [-1] * (K - n)"),
    "cdf_index_off_by_one": ("y = int(above[0])", "y = max(int(above[0]) - 1, 0)"),
    "bf16_shift_wrong": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "greedy_match_inverted": ("if int(tokens[i]) != g[i]:", "if int(tokens[i]) == g[i]:"),
    "greedy_commits_previous_argmax": (
        "committed = [int(tokens[i]) for i in range(n)] + [g[n]] + [-1] * (K - n)",
        "committed = [int(tokens[i]) for i in range(n)] + [g[max(n - 1, 0)]] + [-1] * (K - n)"),
    "ragged_target_start_off_by_one": (
        "t_rows = target_flat[ts:ts + k + 1]", "t_rows = target_flat[ts + 1:ts + k + 2]"),
    "ragged_draft_rows_from_target_start": (
        "d_rows = draft_flat[ds:ds + k] if k > 0", "d_rows = draft_flat[ts:ts + k] if k > 0"),
    "ragged_greedy_flag_inverted": ("        if tau == 0.0:\n            acc[b], com[b]",
                                    "        if tau != 0.0:\n            acc[b], com[b]"),
    "ragged_temperature_of_request_0": ("tau = float(temperatures[b])",
                                        "tau = float(temperatures[0])"),
    "ragged_draft_bound_unchecked": ("if tau != 0.0 and k > 0 and (ds < 0 or ds + k > n_draft_rows):",
                                     "if tau != 0.0 and k > 0 and ds < 0:"),
    "greedy_ties_to_highest_index": (
        "best = int(np.argmax(values))",
        "best = int(len(values) - 1 - np.argmax(np.asarray(values)[::-1]))"),
}

CHECKS = [
    pins.check_decode, pins.check_softmax, pins.check_accept_threshold,
    pins.check_identical_rows_accept_all, pins.check_golden, pins.check_masking_and_edges,
    pins.check_inverse_cdf, pins.check_greedy_argmax, pins.check_greedy_decode_equals_target_only,
    pins.check_ragged_golden, pins.check_ragged_invalid_requests,
    lambda: pins.check_single_slot_lossless(Vs=(3, 5), seeds=range(3)),
    lambda: pins.check_multi_slot_law(cases=((3, 2), (3, 3))),
]


def _mutant(name, monkeypatch):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation {name} does not apply exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = f"<mutant {name}>"
    monkeypatch.setitem(sys.modules, mod.__name__, mod)  # dataclasses look the module up
    exec(compile(SRC.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    mutant = _mutant(name, monkeypatch)
    monkeypatch.setattr(pins, "O", mutant)
    caught = []
    for chk in CHECKS:
        try:
            chk()
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_oracle_passes_the_same_checks():
    for chk in CHECKS:
        chk()

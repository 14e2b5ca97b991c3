"""Pins of the Markov-head oracle (CPU only).

Checked against the pages' worked example (tests/golden/markov/of_course.json), closed forms
(zero factors leave the base logits; rank-1 factors give a_prev * b_v), a brute-force double
loop for the bias, and the anchor rule. The top-K variant: the same example with 1, 2 and all
candidates (tests/golden/markov/of_course_topk.json: with one candidate the proposal differs
from the full head's, a restriction the Metal article warns about), kc = V equal to the full
head, a brute-force sort for the selection (ties, NaN, -inf), and a bias that would lift a
non-candidate. Planted mistakes must be caught.
"""
import json
import os
import sys
import types

import numpy as np
import pytest

import oracle.markov_oracle as real
from workloads import to_bf16_bits

M = real
HERE = os.path.dirname(__file__)


def bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def check_golden():
    g = json.load(open(os.path.join(HERE, "golden", "markov", "of_course.json")))
    base = np.asarray(g["base_logits"], np.float32)
    L, R = bits(g["left_factor"]), bits(g["right_factor"])
    t, c, gaps = M.markov_draft_request(base, "f32", L, R, g["anchor"])
    assert t.tolist() == g["expected"]["tokens"]
    assert np.allclose(c, g["expected"]["corrected_logits"])
    z = np.zeros_like(np.asarray(g["left_factor"]), dtype=np.float32)
    t0, _, _ = M.markov_draft_request(base, "f32", bits(z), bits(z), g["anchor"])
    assert t0.tolist() == g["expected"]["tokens_without_head"]


def check_closed_forms():
    rng = np.random.default_rng(3)
    K, V, R = 4, 37, 8
    base = rng.normal(0, 2, size=(K, V)).astype(np.float32)
    zero = bits(np.zeros((V, R)))
    t, c, _ = M.markov_draft_request(base, "f32", zero, zero, 5)
    assert np.array_equal(c, base.astype(np.float64))
    assert t.tolist() == [int(np.argmax(base[k])) for k in range(K)]
    # rank 1: bias_k[v] = a[prev] * b[v]
    a = np.round(rng.normal(0, 1, V), 2).astype(np.float32)
    bv = np.round(rng.normal(0, 1, V), 2).astype(np.float32)
    La, Rb = bits(a[:, None]), bits(bv[:, None])
    a64 = M.bf16_factor(La)[:, 0]
    b64 = M.bf16_factor(Rb)[:, 0]
    t, c, _ = M.markov_draft_request(base, "f32", La, Rb, 7)
    prev = 7
    for k in range(K):
        want = base[k].astype(np.float64) + a64[prev] * b64
        assert np.allclose(c[k], want, rtol=0, atol=1e-12)
        assert t[k] == int(np.argmax(want))
        prev = t[k]


def check_bruteforce_bias():
    rng = np.random.default_rng(4)
    K, V, R = 3, 11, 5
    base = to_bf16_bits(rng.normal(0, 1, size=(K, V)).astype(np.float32))
    L = bits(rng.normal(0, 1, size=(V, R)))
    Rf = bits(rng.normal(0, 1, size=(V, R)))
    t, c, _ = M.markov_draft_request(base, "bf16", L, Rf, 2)
    Ld, Rd = M.bf16_factor(L), M.bf16_factor(Rf)
    prev = 2
    for k in range(K):
        for v in range(V):
            s = 0.0
            for j in range(R):
                s += Ld[prev, j] * Rd[v, j]
            want = float(M.decode_logits(base[k], "bf16")[v]) + s
            assert abs(c[k, v] - want) <= 1e-12
        prev = int(t[k])


def check_anchor_rule():
    rng = np.random.default_rng(5)
    K, V, R = 2, 9, 3
    base = rng.normal(0, 1, size=(K, V)).astype(np.float32)
    L = bits(rng.normal(0, 3, size=(V, R)))
    Rf = bits(rng.normal(0, 3, size=(V, R)))
    _, c_none, _ = M.markov_draft_request(base, "f32", L, Rf, -1)
    _, c_out, _ = M.markov_draft_request(base, "f32", L, Rf, V)
    assert np.array_equal(c_none[0], base[0].astype(np.float64))
    assert np.array_equal(c_out[0], c_none[0])
    _, c_4, _ = M.markov_draft_request(base, "f32", L, Rf, 4)
    want = base[0].astype(np.float64) + M.bf16_factor(Rf) @ M.bf16_factor(L)[4]
    assert np.allclose(c_4[0], want)


def check_ties_lowest_index():
    base = np.array([[1.0, 3.0, 3.0, 0.0]], np.float32)
    z = bits(np.zeros((4, 2)))
    t, _, gaps = M.markov_draft_request(base, "f32", z, z, -1)
    assert t.tolist() == [1] and gaps[0] == 0.0
    _, _, amb = M.markov_draft(base[None], "f32", z, z)
    assert amb[0]


def check_topk_golden():
    g = json.load(open(os.path.join(HERE, "golden", "markov", "of_course_topk.json")))
    base = np.asarray(g["base_logits"], np.float32)
    L, R = bits(g["left_factor"]), bits(g["right_factor"])
    for kc, want in g["expected"].items():
        t, c, z, _ = M.markov_topk_request(base, "f32", L, R, g["anchor"], int(kc))
        assert t.tolist() == want["tokens"], kc
        assert c.tolist() == want["candidates"], kc
        assert np.allclose(z, want["corrected"]), kc


def check_topk_full_vocabulary_is_the_head():
    rng = np.random.default_rng(6)
    K, V, R = 5, 23, 6
    base = to_bf16_bits(rng.normal(0, 1, size=(K, V)).astype(np.float32))
    L = bits(rng.normal(0, 1, size=(V, R)))
    Rf = bits(rng.normal(0, 1, size=(V, R)))
    for anchor in (-1, 3):
        t, c, z, _ = M.markov_topk_request(base, "bf16", L, Rf, anchor, V)
        tf, cf, _ = M.markov_draft_request(base, "bf16", L, Rf, anchor)
        assert np.array_equal(t, tf)
        assert np.array_equal(c, np.tile(np.arange(V), (K, 1)))
        assert np.array_equal(z, cf)


def check_topk_selection_bruteforce():
    rng = np.random.default_rng(7)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        z = rng.choice([-2.0, -1.0, 0.0, 0.5, 1.0, 3.0], size=V)  # many ties
        z[rng.random(V) < 0.1] = np.nan
        z[rng.random(V) < 0.1] = -np.inf
        kc = int(rng.integers(1, V + 1))
        order = sorted(range(V), key=lambda v: (bool(np.isnan(z[v])),
                                                0.0 if np.isnan(z[v]) else -z[v], v))
        assert M.topk_candidates(z, kc).tolist() == sorted(order[:kc]), (z, kc)
        if kc < V:  # nested: one more candidate keeps every earlier one
            assert set(M.topk_candidates(z, kc)) <= set(M.topk_candidates(z, kc + 1))


def check_topk_zero_head_and_restriction():
    rng = np.random.default_rng(8)
    K, V = 3, 30
    base = rng.normal(0, 1, size=(K, V)).astype(np.float32)
    zero = bits(np.zeros((V, 4)))
    t, c, z, _ = M.markov_topk_request(base, "f32", zero, zero, 2, 4)
    assert t.tolist() == [int(np.argmax(base[k])) for k in range(K)]
    assert np.array_equal(z, np.take_along_axis(base.astype(np.float64), c, 1))
    # a bias that lifts a token outside the candidates: the full head takes it, top-K cannot
    base = np.zeros((2, 6), np.float32)
    base[:, 0] = 1.0
    base[:, 1] = 0.9
    Lm = np.zeros((6, 1), np.float32)
    Lm[0, 0] = 1.0
    Rm = np.zeros((6, 1), np.float32)
    Rm[5, 0] = 4.0
    tf, _, _ = M.markov_draft_request(base, "f32", bits(Lm), bits(Rm), -1)
    tk, ck, _, _ = M.markov_topk_request(base, "f32", bits(Lm), bits(Rm), -1, 2)
    assert tf.tolist() == [0, 5] and tk.tolist() == [0, 0] and ck[1].tolist() == [0, 1]


def check_sampled_golden():
    g = json.load(open(os.path.join(HERE, "golden", "markov", "of_course_sampled.json")))
    base = np.asarray(g["base_logits"], np.float32)
    L, R = bits(g["left_factor"]), bits(g["right_factor"])
    z = bits(np.zeros((g["V"], g["R"])))
    for case in g["cases"]:
        u = np.asarray(case["uniforms"])
        t, _, amb = M.markov_sampled_request(base, "f32", L, R, g["anchor"], g["temperature"], u)
        assert t.tolist() == case["tokens"] and not amb.any(), case
        t0, _, _ = M.markov_sampled_request(base, "f32", z, z, g["anchor"], g["temperature"], u)
        assert t0.tolist() == case["tokens_without_head"], case


def check_sampled_law():
    """Stratified uniforms u_i = (i + 0.5) / N through an inverse CDF give each token
    N p_v draws up to rounding. Logits ln(1..4): p = (1, 2, 3, 4) / 10 at temperature 1,
    (1, 4, 9, 16) / 30 at 1/2 and sqrt(1..4) / sum at 2; ascending order puts the lowest
    uniforms on token 0."""
    base = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    zero = bits(np.zeros((4, 16)))
    N = 600
    laws = {1.0: np.array([1, 2, 3, 4]) / 10.0, 0.5: np.array([1, 4, 9, 16]) / 30.0,
            2.0: np.sqrt([1.0, 2.0, 3.0, 4.0]) / np.sum(np.sqrt([1.0, 2.0, 3.0, 4.0]))}
    for tau, p in laws.items():
        counts = np.zeros(4, dtype=np.int64)
        seq = []
        for i in range(N):
            t, _, _ = M.markov_sampled_request(base, "f32", zero, zero, -1, tau,
                                               np.array([(i + 0.5) / N]))
            counts[t[0]] += 1
            seq.append(int(t[0]))
        assert np.all(np.abs(counts - N * p) <= 1.0), (tau, counts, N * p)
        assert seq == sorted(seq), tau  # ascending uniforms draw ascending tokens


def check_sampled_chain_and_tau_zero():
    rng = np.random.default_rng(9)
    K, V, R = 6, 40, 8
    base = to_bf16_bits(rng.normal(0, 1, size=(K, V)).astype(np.float32))
    L = bits(rng.normal(0, 1.5, size=(V, R)))
    Rf = bits(rng.normal(0, 1.5, size=(V, R)))
    u = rng.random(K)
    t0, c0, _ = M.markov_sampled_request(base, "bf16", L, Rf, 3, 0.0, u)
    td, cd, _ = M.markov_draft_request(base, "bf16", L, Rf, 3)
    assert np.array_equal(t0, td) and np.array_equal(c0, cd)
    t, c, _ = M.markov_sampled_request(base, "bf16", L, Rf, 3, 1.0, u)
    Ld, Rd = M.bf16_factor(L), M.bf16_factor(Rf)
    prev = 3
    for k in range(K):  # each position biased by the previous draw, not by an argmax
        want = M.decode_logits(base[k], "bf16") + Rd @ Ld[prev]
        assert np.allclose(c[k], want, rtol=0, atol=1e-12)
        prev = int(t[k])
    assert any(t[k] != int(np.argmax(c[k])) for k in range(K))


def check_sampled_extremes():
    ninf = -np.inf
    zero = bits(np.zeros((6, 16)))
    row = np.array([[ninf, ninf, 0.5, np.nan, 0.25, ninf]], np.float32)

    def draw(r, u, tau=1.0):
        t, _, _ = M.markov_sampled_request(np.asarray(r, np.float32), "f32", zero, zero, -1, tau,
                                           np.array([u]))
        return int(t[0])

    assert draw(row, 0.0) == 2 and draw(row, -0.5) == 2 and draw(row, np.nan) == 2
    assert draw(row, 0.999999) == 4 and draw(row, 1.0) == 4 and draw(row, 7.0) == 4
    assert {draw(row, (i + 0.5) / 200) for i in range(200)} == {2, 4}
    assert draw([[ninf, np.nan, ninf, ninf, ninf, ninf]], 0.7) == 0  # no mass: token 0
    inf_row = [[1.0, np.inf, 3.0, np.inf, 0.0, 2.0]]
    assert draw(inf_row, 0.2) == 1 and draw(inf_row, 0.7) == 3
    # a near-zero temperature is the argmax
    distinct = [[0.3, -1.0, 2.25, 2.0, 0.0, 1.0]]
    assert {draw(distinct, (i + 0.5) / 100, tau=1e-4) for i in range(100)} == {2}


def check_sampled_invalid_temperature():
    rng = np.random.default_rng(10)
    K, V, R = 3, 12, 4
    base = rng.normal(0, 1, size=(K, V)).astype(np.float32)
    L = bits(rng.normal(0, 1, size=(V, R)))
    Rf = bits(rng.normal(0, 1, size=(V, R)))
    for tau in (-1.0, np.nan, np.inf, M.TAU_MIN / 2):
        t, c, _ = M.markov_sampled_request(base, "f32", L, Rf, 5, tau, np.full(K, 0.5))
        assert t.tolist() == [M.MARKOV_INVALID] * K, tau
        assert np.allclose(c[0], base[0] + M.bf16_factor(Rf) @ M.bf16_factor(L)[5])
        assert np.array_equal(c[1:], base[1:].astype(np.float64))
    t, _, _ = M.markov_sampled_request(base, "f32", L, Rf, 5, M.TAU_MIN, np.full(K, 0.5))
    assert np.all((t >= 0) & (t < V))


def check_sampled_draws_from_stored_rows():
    """bf16 rows: the draw uses the rounded logits. 1 + 2^-9 rounds to 1 in bf16, so two
    tokens at 1 and 1 + 2^-9 are equally likely: u = 0.4997 draws token 0 (the unrounded
    CDF would put the boundary at 0.49951 and draw token 1)."""
    base = to_bf16_bits(np.array([[1.0, 1.0]], np.float32))
    Lm = bits(np.array([[1.0], [0.0]]))
    Rm = bits(np.array([[0.0], [2.0 ** -9]]))
    t, c, amb = M.markov_sampled_request(base, "bf16", Lm, Rm, 0, 1.0, np.array([0.4997]))
    assert c[0, 1] == 1.0 + 2.0 ** -9 and t.tolist() == [0] and not amb[0]
    t, _, _ = M.markov_sampled_request(base, "bf16", Lm, Rm, 0, 1.0, np.array([0.5001]))
    assert t.tolist() == [1]
    x = np.random.default_rng(11).normal(0, 4, 5000).astype(np.float32)
    from workloads import bf16_bits_to_f32
    assert np.array_equal(M.round_stored(x, "bf16"), bf16_bits_to_f32(to_bf16_bits(x)))
    assert M.round_stored(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]), "bf16").tolist() == \
        [1.0, 1.015625]  # ties to even


def check_sampled_ambiguity():
    """A uniform on a CDF boundary is ambiguous; one far from every boundary is not; a bf16
    value on a rounding midpoint widens the band, one far from it does not."""
    zero = bits(np.zeros((2, 16)))
    base = np.log(np.array([[1.0, 1.0]])).astype(np.float32)
    _, _, amb = M.markov_sampled_request(base, "f32", zero, zero, -1, 1.0, np.array([0.5]))
    assert amb[0]
    _, _, amb = M.markov_sampled_request(base, "f32", zero, zero, -1, 1.0, np.array([0.3]))
    assert not amb[0]
    assert M.stored_uncertainty(np.array([1.5, 1.25]), "bf16", 1.0) == 0.0
    assert M.stored_uncertainty(np.array([1.0 + 2.0 ** -8, 1.25]), "bf16", 1.0) > 1e-3
    f32 = M.stored_uncertainty(np.array([1.0, 0.0]), "f32", 1.0)
    assert 1e-5 < f32 < 1e-4
    # through the request: 1 + 2^-8 is a bf16 rounding midpoint (stored as 1.0, ties to even),
    # so a float32 kernel may store either neighbour and u = 0.501 is too close to call
    base = to_bf16_bits(np.array([[1.0, 1.0]], np.float32))
    Lm = bits(np.array([[1.0], [0.0]]))
    Rm = bits(np.array([[2.0 ** -8], [0.0]]))
    t, _, amb = M.markov_sampled_request(base, "bf16", Lm, Rm, 0, 1.0, np.array([0.501]))
    assert t.tolist() == [1] and amb[0]
    t, _, amb = M.markov_sampled_request(base, "bf16", Lm, Rm, 0, 1.0, np.array([0.6]))
    assert t.tolist() == [1] and not amb[0]


def check_valid_token_sets():
    """The valid set of a draw: the draw itself at band 0, both neighbours of a boundary the
    uniform sits on, every token whose CDF interval meets the band otherwise; the argmax's: the
    entries within AMBIGUOUS_GAP of the top."""
    y = np.log(np.array([1.0, 2.0, 3.0, 4.0]))  # CDF 0.1, 0.3, 0.6, 1.0
    assert M.draw_valid_tokens(y, 1.0, 0.45, 0.0).tolist() == [2]
    assert M.draw_valid_tokens(y, 1.0, 0.3, 1e-9).tolist() == [1, 2]
    assert M.draw_valid_tokens(y, 1.0, 0.25, 0.06).tolist() == [1, 2]
    assert M.draw_valid_tokens(y, 1.0, 0.25, 0.2).tolist() == [0, 1, 2]
    assert M.draw_valid_tokens(y, 1.0, 0.05, 0.01).tolist() == [0]
    assert M.draw_valid_tokens(y, 1.0, 7.0, 0.0).tolist() == [3]
    ninf = np.array([-np.inf, 0.0, -np.inf, 0.0])
    assert M.draw_valid_tokens(ninf, 1.0, 0.5, 0.1).tolist() == [1, 3]
    z = np.array([1.0, 3.0, 3.0 - 0.5 * M.AMBIGUOUS_GAP, 3.0 - 2 * M.AMBIGUOUS_GAP])
    assert M.argmax_valid_tokens(z).tolist() == [1, 2]


def check_choose_follows_a_valid_branch():
    """At a draw that sits on the 'of' / 'no' boundary of the golden example, either token is
    valid; choosing 'no' makes the next position follow 'no' (its bias), choosing a token
    outside the valid set changes nothing."""
    g = json.load(open(os.path.join(HERE, "golden", "markov", "of_course_sampled.json")))
    base = np.asarray(g["base_logits"], np.float32)
    L, R = bits(g["left_factor"]), bits(g["right_factor"])
    w0 = np.exp(np.asarray(g["base_logits"][0], np.float64))
    edge = float(w0[0] / w0.sum())  # CDF boundary between 'of' and 'no'
    u = np.array([edge, 0.5])
    t, _, amb = M.markov_sampled_request(base, "f32", L, R, -1, 1.0, u)
    assert amb[0] and t[0] in (0, 1)
    t1, c1, _ = M.markov_sampled_request(base, "f32", L, R, -1, 1.0, u, choose=[1, -9])
    assert t1.tolist() == [1, 3]
    assert np.allclose(c1[1], [0.0, 0.0, 0.0, 2.2, 0.3])
    t0, c0, _ = M.markov_sampled_request(base, "f32", L, R, -1, 1.0, u, choose=[0, -9])
    assert t0.tolist() == [0, 2] and np.allclose(c0[1], [0.0, 0.0, 2.0, 0.2, 0.3])
    tx, _, _ = M.markov_sampled_request(base, "f32", L, R, -1, 1.0, u, choose=[4, -9])
    assert tx.tolist() == t.tolist()
    # an unambiguous position ignores choose
    ty, _, amb = M.markov_sampled_request(base, "f32", L, R, -1, 1.0, np.array([0.3, 0.5]),
                                          choose=[1, 1])
    assert not amb.any() and ty.tolist() == [0, 2]


CHECKS = [check_golden, check_closed_forms, check_bruteforce_bias, check_anchor_rule,
          check_ties_lowest_index, check_topk_golden, check_topk_full_vocabulary_is_the_head,
          check_topk_selection_bruteforce, check_topk_zero_head_and_restriction,
          check_sampled_golden, check_sampled_law, check_sampled_chain_and_tau_zero,
          check_sampled_extremes, check_sampled_invalid_temperature,
          check_sampled_draws_from_stored_rows, check_sampled_ambiguity,
          check_valid_token_sets, check_choose_follows_a_valid_branch]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda f: f.__name__)
def test_markov_oracle_pins(chk):
    chk()


SRC = open(real.__file__).read()
MUTATIONS = {
    "factors_swapped": ("z = z + Rf @ L[prev]", "z = z + L @ Rf[prev]"),
    "bias_from_own_position": ("        tokens[k] = y\n        prev = y\n    return tokens, corrected, gaps",
                               "        tokens[k] = y\n        prev = prev\n    return tokens, corrected, gaps"),
    "sample_bias_from_own_position": ("        tokens[k] = y\n        prev = y\n    return tokens, corrected, amb",
                                      "        tokens[k] = y\n        prev = prev\n    return tokens, corrected, amb"),
    "no_anchor_bias": (
        "    prev = int(anchor)\n    for k in range(K):\n        z = correct_row(base[k], dtype, L, Rf, prev)\n"
        "        corrected[k] = z\n        y, gaps[k]",
        "    prev = -1\n    for k in range(K):\n        z = correct_row(base[k], dtype, L, Rf, prev)\n"
        "        corrected[k] = z\n        y, gaps[k]"),
    "sample_no_anchor_bias": (
        "    prev = int(anchor)\n    for k in range(K):\n        z = correct_row(base[k], dtype, L, Rf, prev)\n"
        "        corrected[k] = z\n        if not valid:",
        "    prev = -1\n    for k in range(K):\n        z = correct_row(base[k], dtype, L, Rf, prev)\n"
        "        corrected[k] = z\n        if not valid:"),
    "topk_no_anchor_bias": (
        "    prev = int(anchor)\n    for k in range(K):\n        z = decode_logits(base[k], dtype)\n",
        "    prev = -1\n    for k in range(K):\n        z = decode_logits(base[k], dtype)\n"),
    "bias_sign_flipped": ("z = z + Rf @ L[prev]", "z = z - Rf @ L[prev]"),
    "ties_highest_index": ("y = argmax_lowest(z)", "y = int(len(z) - 1 - np.argmax(z[::-1]))"),
    "topk_ties_to_higher_index": ("order = np.lexsort((np.arange(z.shape[0]),",
                                  "order = np.lexsort((-np.arange(z.shape[0]),"),
    "topk_nan_preferred": ("-np.where(nan, 0.0, z), nan))", "-np.where(nan, 0.0, z), ~nan))"),
    "topk_candidates_from_corrected": ("cand = topk_candidates(z, kc)",
                                       "cand = topk_candidates(z + (Rf @ L[prev] if 0 <= prev < V "
                                       "else 0.0), kc)"),
    "topk_bias_wrong_rows": ("zc = zc + Rf[cand] @ L[prev]", "zc = zc + Rf[:kc] @ L[prev]"),
    "topk_token_is_position": ("tokens[k] = int(cand[j])", "tokens[k] = int(j)"),
    "sample_biased_by_argmax": ("        tokens[k] = y\n        prev = y\n    return tokens, corrected, amb",
                                "        tokens[k] = y\n        prev = argmax_lowest(z) if valid else y\n"
                                "    return tokens, corrected, amb"),
    "sample_from_unrounded": ("stored = round_stored(z, dtype)", "stored = z"),
    "sample_temperature_dropped": ("np.exp((np.where(valid, y, m) - m) / tau)",
                                   "np.exp(np.where(valid, y, m) - m)"),
    "sample_descending_cdf": ("    return inverse_cdf(w, clamp_uniform(u))\n",
                              "    y, mg = inverse_cdf(w[::-1], clamp_uniform(u))\n"
                              "    return len(w) - 1 - y, mg\n"),
    "sample_nan_has_mass": ("valid = ~np.isnan(y) & (y > -np.inf)\n    if not valid.any():\n"
                            "        return np.zeros_like(y)",
                            "valid = ~(y == -np.inf)\n    if not valid.any():\n"
                            "        return np.zeros_like(y)"),
    "sample_uniform_unclamped": ("return 0.0 if not u > 0.0 else min(float(u), 1.0)",
                                 "return float(u)"),
    "sample_invalid_tau_accepted": ("valid = greedy or (TAU_MIN <= tau < np.inf)",
                                    "valid = greedy or tau > 0.0"),
    "sample_bf16_truncates": ("np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)",
                              "np.ldexp(np.trunc(np.ldexp(mant, 8)), expo - 8)"),
    "sample_uncertainty_ignored": ("band = SAMPLE_EPS + stored_uncertainty(z, dtype, tau)",
                                   "band = SAMPLE_EPS"),
    "valid_set_misses_lower_neighbour": ("hit = (w > 0.0) & (c >= r - band) & (lo <= r + band)",
                                         "hit = (w > 0.0) & (c >= r) & (lo <= r + band)"),
    "valid_set_ignores_band": ("hit = (w > 0.0) & (c >= r - band) & (lo <= r + band)",
                               "hit = (w > 0.0) & (c > r) & (lo <= r)"),
    "choose_outside_valid_set": ("int(choose[k]) in draw_valid_tokens(stored, tau, float(uniforms[k]), band)",
                                 "True"),
    "argmax_valid_gap_ignored": ("return np.nonzero(z >= z[argmax_lowest(z)] - AMBIGUOUS_GAP)[0]",
                                 "return np.array([argmax_lowest(z)])"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    mod = types.ModuleType(f"oracle.markov_mutant_{name}")
    mod.__package__ = "oracle"
    monkeypatch.setitem(sys.modules, mod.__name__, mod)
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    monkeypatch.setattr(sys.modules[__name__], "M", mod)
    caught = False
    for chk in CHECKS:
        try:
            chk()
        except Exception:
            caught = True
            break
    assert caught, name

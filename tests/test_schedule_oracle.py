"""Pins of the confidence-scheduling oracle (CPU only).

The scheduler's choice is checked against exhaustive enumeration of every per-request
allocation on small cases (the ranked, full-table search must reach the best expected tokens
per unit time over all prefix allocations), against the pages' worked threshold example, and
against properties the pages state: prefixes only, shorter drafts under heavier load. Planted
mistakes in the oracle's source must be caught.
"""
import itertools
import sys
import types

import numpy as np
import pytest

import oracle.schedule_oracle as real

O = real


def brute_force(conf, table):
    s = O.prefix_survival(conf)
    B, K = s.shape
    best = (-np.inf, None)
    for alloc in itertools.product(range(K + 1), repeat=B):
        n = sum(alloc)
        t = table[B + n]
        if not (np.isfinite(t) and t > 0):
            continue
        exp = float(B) + sum(float(s[b, k]) for b in range(B) for k in range(alloc[b]))
        rate = exp / t
        if rate > best[0] * (1 + 1e-12):
            best = (rate, alloc)
    return best


def jumpy_table(rng, B, K, base=1.0):
    """Step time of a target step over n tokens: a base, a per-token slope, and jumps every
    few tokens (tile quantisation)."""
    n = np.arange(B + B * K + 1)
    slope = rng.uniform(0.005, 0.2)
    tile = int(rng.integers(2, 6))
    jump = rng.uniform(0.0, 0.5)
    return base + slope * n + jump * np.ceil(n / tile)


def check_bruteforce(cases=30):
    rng = np.random.default_rng(5)
    for _ in range(cases):
        B, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        conf = rng.uniform(0.0, 1.0, size=(B, K)).astype(np.float32)
        table = jumpy_table(rng, B, K)
        num, n, rate = O.schedule_hardware_aware(conf, table)
        brate, balloc = brute_force(conf, table)
        assert n == int(num.sum())
        assert abs(rate - brate) <= 1e-12 * brate, (conf, table, num, balloc)
        s = O.prefix_survival(conf)
        exp = B + sum(float(s[b, k]) for b in range(B) for k in range(num[b]))
        assert abs(exp / table[B + n] - rate) <= 1e-12 * rate


def check_threshold_examples():
    # "Accelerating Large-Model Inference ...", section 1 DSpark table, prefix-scheduler row:
    # the first score below the threshold cuts that position and everything after it. The DSpark
    # review, 4.2: the scheduler keeps "jumps over a" and cuts "lazy".
    conf = np.array([[0.95, 0.9, 0.8, 0.2],    # jumps over a | lazy
                     [0.9, 0.3, 0.99, 0.99],    # cut at the 2nd although later scores are high
                     [0.1, 0.9, 0.9, 0.9],      # cut at once
                     [0.6, 0.6, 0.6, 0.6]], np.float32)  # nothing below: keep all
    assert O.schedule_threshold(conf, 0.5).tolist() == [3, 1, 0, 4]


def check_load_sensitivity():
    rng = np.random.default_rng(7)
    B, K = 8, 6
    conf = rng.uniform(0.3, 1.0, size=(B, K)).astype(np.float32)
    n = np.arange(B + B * K + 1)
    # no marginal cost: every token with positive survival is worth verifying
    num, N, _ = O.schedule_hardware_aware(conf, np.full(n.shape, 2.0))
    assert N == B * K and num.tolist() == [K] * B
    # heavier load = a larger marginal cost per verified token: never more tokens
    prev = B * K
    for slope in (0.001, 0.01, 0.05, 0.2, 1.0, 10.0):
        _, N, _ = O.schedule_hardware_aware(conf, 1.0 + slope * n)
        assert N <= prev
        prev = N
    assert prev == 0  # a very steep table verifies no drafts


def check_prefix_and_survival():
    rng = np.random.default_rng(9)
    conf = rng.uniform(0, 1, size=(5, 7)).astype(np.float32)
    # exact ties: confidence 1 keeps the survival flat, confidence 0 makes it 0 from there on
    conf[1, :3] = 1.0
    conf[2, 2:4] = 0.0
    conf[3] = conf[4] = 1.0
    s = O.prefix_survival(conf)
    assert np.all(np.diff(s, axis=1) <= 0)
    assert np.allclose(s, np.cumprod(conf.astype(np.float64), axis=1), rtol=1e-6)
    order = O.rank_tokens(s)
    for n in range(len(order) + 1):  # every ranked prefix is a prefix of every request
        taken = {}
        for b, k in order[:n]:
            taken.setdefault(b, []).append(k)
        for b, ks in taken.items():
            assert ks == list(range(len(ks))), (n, b, ks)


def check_clamping_and_row_starts():
    conf = np.array([[np.nan, 0.9], [1.5, -0.2]], np.float32)
    assert O.clamp_confidence(conf).tolist() == [[0.0, np.float32(0.9)], [1.0, 0.0]]
    ts, ds = O.row_starts([2, 0, 3])
    assert ts.tolist() == [0, 3, 4] and ds.tolist() == [0, 2, 2]


CHECKS = [check_bruteforce, check_threshold_examples, check_load_sensitivity,
          check_prefix_and_survival, check_clamping_and_row_starts]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda f: f.__name__)
def test_schedule_oracle_pins(chk):
    chk()


SRC = open(real.__file__).read()
MUTATIONS = {
    "survival_not_cumulative": ("acc = np.float32(acc * c[b, k])", "acc = np.float32(c[b, k])"),
    "ranked_ascending": ("items = [(-float(survival[b, k]), k, b)",
                        "items = [(float(survival[b, k]), k, b)"),
    "target_token_not_counted": ("expected = float(B)  # every", "expected = 0.0  # every"),
    "table_index_without_B": ("tn = t[B + n]", "tn = t[n]"),
    "stops_at_first_drop": ("            if rate > best_rate:\n                best_n, best_rate = n, rate",
                            "            if rate > best_rate:\n                best_n, best_rate = n, rate\n"
                            "            elif n > 0:\n                break"),
    "threshold_not_strict_cut": ("out[b] = k\n                break", "out[b] = k + 1\n                break"),
    "ties_to_later_position": ("items.sort()", "items.sort(key=lambda x: (x[0], -x[1], x[2]))"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    mod = types.ModuleType(f"schedule_mutant_{name}")
    monkeypatch.setitem(sys.modules, mod.__name__, mod)
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    monkeypatch.setattr(sys.modules[__name__], "O", mod)
    caught = False
    for chk in CHECKS:
        try:
            chk()
        except Exception:
            caught = True
            break
    assert caught, name

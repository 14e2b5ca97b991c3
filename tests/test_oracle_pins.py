"""Pins of the fp64 oracle to what the pages and the mathematics fix (CPU only).

Every check here compares the oracle with something other than itself: a library routine the
oracle does not call (scipy's softmax, numpy's searchsorted, torch's bf16 widening), a closed
form (the acceptance law of "From draft-then-verify to DSpark", section "How speculative
decoding works", and its consequences), exhaustive enumeration on tiny vocabularies, a
Monte-Carlo chi-square test, or hand-derived worked examples (tests/golden).

The checks are plain functions so that tests/test_oracle_mutations.py can plant a mistake in the
oracle and show that at least one of them fails.
"""
import glob
import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle.sv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# helpers that build inputs (no verification arithmetic)


def logits_from_probs(probs):
    """Natural-log logits, stored as float32 (softmax at tau=1 gives back probs to ~1e-7)."""
    return np.log(np.asarray(probs, dtype=np.float64)).astype(np.float32)


def scipy_probs(logits, tau):
    return scipy.special.softmax(np.asarray(logits, dtype=np.float64) / tau)


def residual_intervals(w):
    """[(v, lo, hi)] CDF intervals (normalised) of every token with positive mass."""
    z = float(np.sum(w))
    out, lo = [], 0.0
    for v, wv in enumerate(w):
        if wv > 0:
            out.append((v, lo / z, (lo + wv) / z))
            lo += wv
    return out


def call(target_logits, draft_logits, x, u, r, tau, k=None, K=None):
    target_logits = np.asarray(target_logits, dtype=np.float32)
    draft_logits = np.asarray(draft_logits, dtype=np.float32)
    K = len(x) if K is None else K
    k = K if k is None else k
    return O.verify_request(target_logits, draft_logits, "f32", np.asarray(x, dtype=np.int32),
                            np.asarray(u, dtype=np.float64), r, tau, k, K)


# ---------------------------------------------------------------------------------------------
# checks


def check_decode():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]  # finite patterns only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_logits(bits, "bf16")
    assert np.array_equal(got, ref)
    f = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(O.decode_logits(f, "f32"), f.astype(np.float64))


def check_softmax():
    rng = np.random.default_rng(1)
    for V in (1, 2, 7, 1000, 151936):
        for tau in (0.3, 0.7, 1.0, 2.5):
            z = rng.normal(0, 4, size=V).astype(np.float32)
            if V > 3:
                z[rng.integers(0, V, size=2)] = -np.inf
            got = O.softmax_fp64(z, tau)
            ref = scipy_probs(z, tau)
            fin = ref > 0
            assert np.all(got[~fin] == 0.0)
            assert np.allclose(got[fin], ref[fin], rtol=1e-13, atol=0)
            assert abs(np.sum(got) - 1.0) < 1e-13


def check_accept_threshold():
    cases = [(0.5, 0.25, 1.0), (0.25, 0.5, 0.5), (0.1, 0.4, 0.25), (0.3, 0.3, 1.0),
             (0.0, 0.2, 0.0), (0.2, 0.0, 1.0), (0.0, 0.0, 0.0)]
    for a, c, t in cases:
        assert abs(O.accept_threshold(a, c) - t) < 1e-15, (a, c)


def check_identical_rows_accept_all():
    """p == q at every slot: every draft is accepted whatever u < 1, and the extra token is the
    inverse-CDF draw from the row after the last draft."""
    rng = np.random.default_rng(2)
    for trial in range(20):
        K, V = int(rng.integers(1, 9)), int(rng.integers(2, 300))
        tau = float(rng.choice([0.5, 1.0, 1.7]))
        T = rng.normal(0, 3, size=(K + 1, V)).astype(np.float32)
        x = rng.integers(0, V, size=K)
        u = rng.random(K)
        u[0] = 1.0 - 2.0 ** -24  # the largest float32 below 1
        r = float(rng.random())
        res = call(T, T[:K], x, u, r, tau)
        assert res.n == K
        p_last = scipy_probs(T[K], tau)
        cdf = np.cumsum(p_last)
        y = int(np.searchsorted(cdf, r * cdf[-1], side="right"))
        assert res.committed == list(x) + [y]
        for i in range(K):
            pi = scipy_probs(T[i], tau)[x[i]]
            assert abs(res.target_prob[i] - pi) <= 1e-14
            assert res.target_prob[i] == res.draft_prob[i]


def check_single_slot_lossless(Vs=(2, 3, 5, 8), seeds=range(6)):
    """Brute force over the proposal x in [V] and over the accept / residual intervals: the law
    of the committed token equals the target distribution (the losslessness claim)."""
    for V in Vs:
        for seed in seeds:
            rng = np.random.default_rng(100 + 10 * V + seed)
            tau = float(rng.choice([0.6, 1.0, 1.4]))
            T = rng.normal(0, 2, size=(2, V)).astype(np.float32)
            D = (T[:1] + rng.normal(0, 1.5, size=(1, V))).astype(np.float32)
            if seed == 0:
                D[0, 0] = -np.inf  # a token the draft never proposes
            p = scipy_probs(T[0], tau)
            q = scipy_probs(D[0], tau)
            law = np.zeros(V)
            for x in range(V):
                if q[x] == 0.0:
                    continue
                t = min(1.0, p[x] / q[x])
                if t > 0:
                    res = call(T, D, [x], [t / 2], 0.5, tau)
                    assert res.n == 1 and res.committed[0] == x
                    assert abs(res.target_prob[0] - p[x]) < 1e-14
                    assert abs(res.draft_prob[0] - q[x]) < 1e-14
                    law[x] += q[x] * t
                if t < 1:
                    w = np.maximum(0.0, p - q)
                    for v, lo, hi in residual_intervals(w):
                        res = call(T, D, [x], [(1 + t) / 2], (lo + hi) / 2, tau)
                        assert res.n == 0 and res.committed == [v, -1], (V, seed, x, v)
                        law[v] += q[x] * (1 - t) * (hi - lo)
            assert np.allclose(law, p, atol=1e-12, rtol=0), (V, seed)


def _enumerate_law(T, D, tau, K):
    """Exact law of (n, committed) by enumerating proposals and decision intervals, calling the
    oracle at interval midpoints. Returns reach[i] = P(n >= i) and token[i][v] =
    P(committed[i] = v and n >= i)."""
    V = T.shape[1]
    p = [scipy_probs(T[i], tau) for i in range(K + 1)]
    q = [scipy_probs(D[i], tau) for i in range(K)]
    reach = np.zeros(K + 1)
    token = np.zeros((K + 1, V))
    for xs in np.ndindex(*([V] * K)):
        wx = float(np.prod([q[i][xs[i]] for i in range(K)]))
        if wx == 0.0:
            continue
        t = [min(1.0, p[i][xs[i]] / q[i][xs[i]]) for i in range(K)]
        acc_measure = 1.0
        for s in range(K + 1):  # s = first rejected slot (K: none)
            if s < K:
                rej = acc_measure * (1.0 - t[s])
                if rej > 0:
                    w = np.maximum(0.0, p[s] - q[s])
                    for v, lo, hi in residual_intervals(w):
                        u = [t[j] / 2 for j in range(s)] + [(1 + t[s]) / 2] + [0.5] * (K - s - 1)
                        res = call(T, D, xs, u, (lo + hi) / 2, tau)
                        exp = list(xs[:s]) + [v] + [-1] * (K - s)
                        assert res.n == s and res.committed == exp
                        m = wx * rej * (hi - lo)
                        reach[: s + 1] += m
                        for j in range(s):
                            token[j][xs[j]] += m
                        token[s][v] += m
                acc_measure *= t[s]
                if acc_measure == 0:
                    break
            else:
                for v, lo, hi in residual_intervals(p[K]):
                    u = [t[j] / 2 for j in range(K)]
                    res = call(T, D, xs, u, (lo + hi) / 2, tau)
                    assert res.n == K and res.committed == list(xs) + [v]
                    m = wx * acc_measure * (hi - lo)
                    reach += m
                    for j in range(K):
                        token[j][xs[j]] += m
                    token[K][v] += m
    return p, q, reach, token


def check_multi_slot_law(cases=((2, 1), (3, 2), (4, 2), (3, 3), (4, 3))):
    """Closed forms of the product structure: P(n >= i) = prod_{j<i} beta_j with
    beta_j = sum_v min(p_j, q_j); given the round reaches slot i, the token committed there has
    law p_i; E[n + 1] = sum_i prod_{j<i} beta_j."""
    for V, K in cases:
        rng = np.random.default_rng(7 * V + K)
        tau = 0.8
        T = rng.normal(0, 1.5, size=(K + 1, V)).astype(np.float32)
        D = (T[:K] + rng.normal(0, 1.0, size=(K, V))).astype(np.float32)
        p, q, reach, token = _enumerate_law(T, D, tau, K)
        beta = [float(np.sum(np.minimum(p[j], q[j]))) for j in range(K)]
        for i in range(K + 1):
            closed = float(np.prod(beta[:i]))
            assert abs(reach[i] - closed) < 1e-12, (V, K, i)
            assert np.allclose(token[i], closed * p[i], atol=1e-12, rtol=0), (V, K, i)
        assert abs(np.sum(reach) - sum(np.prod(beta[:i]) for i in range(K + 1))) < 1e-12


def check_monte_carlo(cases=((5, 1), (8, 2), (6, 3)), trials=12000, pmin=1e-3):
    """Seeded Monte-Carlo chi-square: committed tokens at each reached slot against p_i, and the
    accepted length against its closed-form law."""
    for V, K in cases:
        rng = np.random.default_rng(1000 + 10 * V + K)
        tau = 1.0
        T = rng.normal(0, 1.5, size=(K + 1, V)).astype(np.float32)
        D = (T[:K] + rng.normal(0, 1.0, size=(K, V))).astype(np.float32)
        p = [scipy_probs(T[i], tau) for i in range(K + 1)]
        q = [scipy_probs(D[i], tau) for i in range(K)]
        counts = np.zeros((K + 1, V))
        ncount = np.zeros(K + 1)
        for _ in range(trials):
            x = [int(rng.choice(V, p=q[i])) for i in range(K)]
            u = rng.random(K, dtype=np.float32)
            r = float(rng.random(dtype=np.float32))
            res = call(T, D, x, u, r, tau)
            ncount[res.n] += 1
            for i in range(res.n + 1):
                counts[i][res.committed[i]] += 1
        beta = [float(np.sum(np.minimum(p[j], q[j]))) for j in range(K)]
        pn = [np.prod(beta[:i]) * ((1 - beta[i]) if i < K else 1.0) for i in range(K + 1)]
        assert scipy.stats.chisquare(ncount, np.array(pn) * trials).pvalue > pmin, (V, K)
        for i in range(K + 1):
            tot = counts[i].sum()
            if tot < 200:
                continue
            keep = p[i] * tot > 5
            obs = np.append(counts[i][keep], counts[i][~keep].sum())
            expd = np.append(p[i][keep] * tot, p[i][~keep].sum() * tot)
            if expd[-1] == 0:
                obs, expd = obs[:-1], expd[:-1]
            assert scipy.stats.chisquare(obs, expd).pvalue > pmin, (V, K, i)


def check_inverse_cdf():
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if not np.any(w > 0):
            w[int(rng.integers(0, V))] = 0.3
        r = float(rng.random())
        y, margin = O.inverse_cdf(w, r)
        cdf = np.cumsum(w)
        assert y == int(np.searchsorted(cdf, r * cdf[-1], side="right"))
        assert w[y] > 0
        # brute force: y is the first index whose cumulative mass exceeds r * Z
        acc = 0.0
        for v in range(V):
            acc += w[v]
            if acc > r * cdf[-1]:
                assert v == y
                break
        assert margin >= 0


def check_greedy_argmax():
    rng = np.random.default_rng(4)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        row = rng.integers(-3, 4, size=V).astype(np.float32)  # many ties
        best, bi = -np.inf, -1
        for v in range(V):
            if row[v] > best:
                best, bi = row[v], v
        assert O.argmax_lowest(O.decode_logits(row, "f32")) == bi
    # drafts equal to the target argmax are all accepted; the bonus is the last row's argmax
    for trial in range(30):
        K, V = int(rng.integers(1, 9)), int(rng.integers(2, 100))
        T = rng.normal(size=(K + 1, V)).astype(np.float32)
        x = np.argmax(T[:K], axis=1).astype(np.int32)
        n, com = O.verify_greedy_request(T, "f32", x, K)
        assert n == K and com == list(x) + [int(np.argmax(T[K]))]
        if K > 1:
            j = int(rng.integers(0, K))
            x2 = x.copy()
            x2[j] = (x2[j] + 1) % V
            n, com = O.verify_greedy_request(T, "f32", x2, K)
            assert n == j and com == list(x[:j]) + [int(np.argmax(T[j]))] + [-1] * (K - j)


def check_greedy_decode_equals_target_only():
    """Speculative greedy decoding emits exactly the target-only greedy stream ("Bringing DSpark
    to vLLM Metal": output ids equal target-only serving). The target is a fixed synthetic
    next-token table (logits depend on the last token only); the drafter is a noisy copy."""
    rng = np.random.default_rng(5)
    V, K, steps = 37, 5, 120
    table = rng.normal(0, 2, size=(V, V)).astype(np.float32)  # logits of next token | last
    noisy = (table + rng.normal(0, 1.5, size=(V, V))).astype(np.float32)

    ref, last = [], 3
    for _ in range(steps):
        last = int(np.argmax(table[last]))
        ref.append(last)

    out, last = [], 3
    while len(out) < steps:
        x, prev = [], last  # the drafter proposes K tokens greedily from its own table
        for _ in range(K):
            prev = int(np.argmax(noisy[prev]))
            x.append(prev)
        ctx = [last] + x  # the target scores K+1 positions in one pass
        rows = np.stack([table[c] for c in ctx])
        n, com = O.verify_greedy_request(rows, "f32", np.asarray(x, dtype=np.int32), K)
        emitted = com[: n + 1]
        out.extend(emitted)
        last = emitted[-1]
    assert out[:steps] == ref


def check_golden():
    files = sorted(glob.glob(os.path.join(GOLDEN, "*.json")))
    assert files
    for f in files:
        g = json.load(open(f))
        K = g["K"]
        exp = g["expected"]
        if g["mode"] == "sample":
            T = logits_from_probs(g["target_probs"])
            D = logits_from_probs(g["draft_probs"])
            res = call(T, D, g["tokens"], g["uniforms"], g["residual"], g["tau"])
            assert res.n == exp["accepted_len"], f
            assert res.committed == exp["committed"], f
            assert np.allclose(res.target_prob, exp["target_prob"], atol=1e-6), f
            assert np.allclose(res.draft_prob, exp["draft_prob"], atol=1e-6), f
            assert not res.ambiguous
        else:
            T = np.asarray(g["target_logits"], dtype=np.float32)
            n, com = O.verify_greedy_request(T, "f32", np.asarray(g["tokens"], np.int32), K)
            assert n == exp["accepted_len"] and com == exp["committed"], f


def golden_flat_batch():
    """Every golden worked example as one request of a single flattened, mixed batch.

    Vocabularies are padded to the largest V with -inf logits (probability 0: no probability,
    argmax or draw changes), K to the largest K (num_draft keeps each request's own k), requests
    are packed in reverse file order with a NaN row between them, and each request keeps its own
    temperature (0 for the greedy example). Returns the batch and the expected outputs."""
    gs = [json.load(open(f)) for f in sorted(glob.glob(os.path.join(GOLDEN, "*.json")))]
    V = max(g["V"] for g in gs)
    K = max(g["K"] for g in gs)
    B = len(gs)

    def pad(rows):
        rows = np.asarray(rows, dtype=np.float32)
        out = np.full((rows.shape[0], V), -np.inf, dtype=np.float32)
        out[:, :rows.shape[1]] = rows
        return out

    t_rows, d_rows = [], []
    ts, ds = np.zeros(B, np.int32), np.zeros(B, np.int32)
    tokens = np.full((B, K), -1, np.int32)
    uni = np.full((B, K), np.nan)
    res = np.zeros(B)
    taus = np.zeros(B)
    nd = np.zeros(B, np.int32)
    expected = []
    gap = np.full((1, V), np.nan, dtype=np.float32)
    for b in reversed(range(B)):
        g = gs[b]
        k = g["K"] if g["num_draft"] is None else g["num_draft"]
        nd[b] = k
        tokens[b, :len(g["tokens"])] = g["tokens"]
        if g["mode"] == "sample":
            T = pad(logits_from_probs(g["target_probs"]))
            D = pad(logits_from_probs(g["draft_probs"]))
            uni[b, :len(g["uniforms"])] = g["uniforms"]
            res[b] = g["residual"]
            taus[b] = g["tau"]
            ds[b] = sum(len(r) for r in d_rows)
            d_rows += [D[:k], gap]
        else:
            T = pad(g["target_logits"])
        ts[b] = sum(len(r) for r in t_rows)
        t_rows += [T[:k + 1], gap]
    for b, g in enumerate(gs):
        e = g["expected"]
        com = list(e["committed"]) + [-1] * (K + 1 - len(e["committed"]))
        tp = list(e.get("target_prob", [])) + [0.0] * (K - len(e.get("target_prob", [])))
        dp = list(e.get("draft_prob", [])) + [0.0] * (K - len(e.get("draft_prob", [])))
        expected.append((e["accepted_len"], com, tp, dp))
    batch = dict(target_flat=np.concatenate(t_rows), draft_flat=np.concatenate(d_rows),
                 dtype="f32", tokens=tokens, uniforms=uni, residual=res, temperatures=taus,
                 num_draft=nd, target_row_start=ts, draft_row_start=ds)
    return batch, expected


def check_ragged_golden():
    batch, expected = golden_flat_batch()
    out = O.verify_ragged(**batch)
    for b, (n, com, tp, dp) in enumerate(expected):
        assert out.accepted_len[b] == n, b
        assert out.committed[b].tolist() == com, b
        assert np.allclose(out.target_prob[b], tp, atol=1e-6), b
        assert np.allclose(out.draft_prob[b], dp, atol=1e-6), b


def check_ragged_invalid_requests():
    batch, expected = golden_flat_batch()
    rows_t = batch["target_flat"].shape[0]
    B = len(expected)
    cases = [("target_row_start", 0, -1), ("target_row_start", 0, rows_t - 1),
             ("temperatures", 1, -0.5), ("temperatures", 1, np.nan),
             ("temperatures", 1, np.inf), ("temperatures", 1, O.TAU_MIN / 2),
             ("num_draft", 2, batch["tokens"].shape[1] + 1), ("num_draft", 2, -1)]
    samp = [b for b in range(B) if batch["temperatures"][b] > 0][0]
    cases.append(("draft_row_start", samp, batch["draft_flat"].shape[0]))
    for key, b, val in cases:
        bad = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in batch.items()}
        bad[key][b] = val
        out = O.verify_ragged(**bad)
        assert out.accepted_len[b] == O.RAGGED_INVALID, (key, val)
        assert out.committed[b].tolist() == [-1] * (bad["tokens"].shape[1] + 1)
        assert not out.target_prob[b].any() and not out.draft_prob[b].any()
        for o in range(B):  # the other requests are untouched
            if o != b:
                assert out.accepted_len[o] == expected[o][0], (key, o)
                assert out.committed[o].tolist() == expected[o][1], (key, o)


def check_masking_and_edges():
    rng = np.random.default_rng(6)
    K, V = 6, 50
    T = rng.normal(0, 2, size=(K + 1, V)).astype(np.float32)
    D = (T[:K] + rng.normal(0, 1, size=(K, V))).astype(np.float32)
    x = rng.integers(0, V, size=K).astype(np.int32)
    u = rng.random(K)
    r = 0.37
    # k = 0: a plain draw from target row 0
    res = call(T, D, x, u, r, 1.0, k=0)
    cdf = np.cumsum(scipy_probs(T[0], 1.0))
    assert res.n == 0
    assert res.committed == [int(np.searchsorted(cdf, r * cdf[-1], side="right"))] + [-1] * K
    assert res.target_prob == [0.0] * K
    # rows past k are never read: NaN there changes nothing
    for k in range(K + 1):
        T2, D2 = T.copy(), D.copy()
        T2[k + 1:] = np.nan
        D2[k:] = np.nan
        a = call(T, D, x, u, r, 1.0, k=k)
        b = call(T2, D2, x, u, r, 1.0, k=k)
        assert a.committed == b.committed and a.target_prob == b.target_prob
        assert a.committed[a.n + 1:] == [-1] * (K - a.n)
        assert all(v == 0.0 for v in a.target_prob[k:])
    # a token outside [0, V) is rejected with p(x) = q(x) = 0
    x3 = x.copy()
    x3[0] = V + 5
    res = call(T, D, x3, [0.0] * K, r, 1.0)
    assert res.n == 0 and res.target_prob[0] == 0.0 and res.draft_prob[0] == 0.0
    # the residual excludes tokens where q >= p
    x4 = x.copy()
    p0, q0 = scipy_probs(T[0], 1.0), scipy_probs(D[0], 1.0)
    x4[0] = int(np.argmax(q0 - p0))
    for rr in np.linspace(0.01, 0.99, 25):
        res = call(T, D, x4, [0.999999] + [0.5] * (K - 1), float(rr), 1.0)
        assert res.n == 0 and p0[res.committed[0]] > q0[res.committed[0]]


# ---------------------------------------------------------------------------------------------
# tests


def test_decode_matches_torch_bf16_widening():
    check_decode()


def test_softmax_matches_scipy():
    check_softmax()


def test_accept_threshold_closed_form():
    check_accept_threshold()


def test_identical_rows_accept_every_draft():
    check_identical_rows_accept_all()


def test_single_slot_losslessness_bruteforce():
    check_single_slot_lossless()


def test_multi_slot_law_exact_enumeration():
    check_multi_slot_law()


def test_multi_slot_law_monte_carlo_chi2():
    check_monte_carlo()


def test_inverse_cdf_matches_searchsorted_and_bruteforce():
    check_inverse_cdf()


def test_greedy_is_lowest_index_argmax():
    check_greedy_argmax()


def test_greedy_speculative_decode_equals_target_only_greedy():
    check_greedy_decode_equals_target_only()


def test_golden_worked_examples():
    check_golden()


def test_masking_k0_out_of_range_and_residual_support():
    check_masking_and_edges()


def test_tokens_without_mass_under_one_distribution():
    """The accept rule min(1, p/q) at its limits (a -inf logit is probability 0): a token the
    draft gives no mass (q = 0) is kept whenever the target gives it mass, for any u in [0, 1);
    a token the target gives no mass (p = 0) is always rejected, its target probability is 0,
    and the residual draw then follows max(0, p - q) without it."""
    T = np.array([[0.5, -1.0, 2.0, 0.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    D = np.array([[-np.inf, 0.3, 1.0, 0.2]], np.float32)
    for u in (0.0, 0.5, 0.999999):
        res = call(T, D, [0], [u], 0.5, 1.0)
        assert res.n == 1 and res.committed[0] == 0
        assert res.draft_prob[0] == 0.0 and res.target_prob[0] > 0.0
    T2 = T.copy()
    T2[0, 1] = -np.inf
    p = scipy_probs(T2[0], 1.0)
    q = scipy_probs(D[0], 1.0)
    w = np.maximum(0.0, p - q)
    assert w[1] == 0.0
    for u in (0.0, 0.5):
        for v, lo, hi in residual_intervals(w):
            res = call(T2, D, [1], [u], (lo + hi) / 2, 1.0)
            assert res.n == 0 and res.committed == [v, -1] and v != 1
            assert res.target_prob[0] == 0.0 and res.draft_prob[0] > 0.0


def test_batch_driver_matches_per_request():
    from workloads import TINY, generate

    inp = generate(TINY.replace(B=3, K=3, V=64, seed=77))
    w = inp.workload
    res = O.verify_batch(inp.target, inp.draft, w.dtype, inp.tokens, inp.uniforms,
                         inp.residual, w.temperature)
    for b in range(w.B):
        one = O.verify_request(inp.target[b], inp.draft[b], w.dtype, inp.tokens[b],
                               inp.uniforms[b], float(inp.residual[b]), w.temperature, w.K)
        assert res.committed[b].tolist() == one.committed
        assert res.accepted_len[b] == one.n


def test_ragged_mixed_batch_reproduces_the_golden_examples():
    check_ragged_golden()


def test_ragged_invalid_requests_are_flagged_and_isolated():
    check_ragged_invalid_requests()


def test_ragged_driver_matches_padded_drivers():
    """Flattening a padded batch (used rows only, packed in a shuffled order) changes nothing."""
    from workloads import HEAVY, generate

    inp = generate(HEAVY.replace(B=6, K=4, V=96, dtype="f32", seed=91))
    w = inp.workload
    B, K, V = w.B, w.K, w.V
    order = [3, 0, 5, 1, 4, 2]
    t_rows, d_rows, ts, ds = [], [], np.zeros(B, np.int32), np.zeros(B, np.int32)
    for b in order:
        k = inp.k_of(b)
        ts[b] = sum(len(r) for r in t_rows)
        ds[b] = sum(len(r) for r in d_rows)
        t_rows.append(inp.target[b, :k + 1])
        d_rows.append(inp.draft[b, :k])
    tf, df = np.concatenate(t_rows), np.concatenate(d_rows)
    taus = np.full(B, w.temperature)
    out = O.verify_ragged(tf, df, w.dtype, inp.tokens, inp.uniforms, inp.residual, taus,
                          inp.num_draft, ts, ds)
    ref = O.verify_batch(inp.target, inp.draft, w.dtype, inp.tokens, inp.uniforms,
                         inp.residual, w.temperature, inp.num_draft)
    assert np.array_equal(out.accepted_len, ref.accepted_len)
    assert np.array_equal(out.committed, ref.committed)
    assert np.array_equal(out.target_prob, ref.target_prob)
    out_g = O.verify_ragged(tf, df, w.dtype, inp.tokens, inp.uniforms, inp.residual,
                            np.zeros(B), inp.num_draft, ts, ds)
    ref_g = O.verify_greedy(inp.target, w.dtype, inp.tokens, inp.num_draft)
    assert np.array_equal(out_g.accepted_len, ref_g.accepted_len)
    assert np.array_equal(out_g.committed, ref_g.committed)

"""Top-K Markov drafting on the GPU against the Markov oracle.

Parity bar: candidates bit-exact at every position whose earlier tokens agree (they depend only
on the stored base logits); tokens bit-exact at every position whose oracle top-2 gap among the
candidates is at least AMBIGUOUS_GAP; corrected candidate logits (float32) within
2e-5 + 1e-6 |z| of the fp64 values (R products of bf16 factors are exact in float32; only the
accumulation rounds).
"""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

import lossless_draft_verification_sv_amd as sv  # noqa: E402
import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.gpu_util import abs_err, say, to_dev  # noqa: E402

HERE = os.path.dirname(__file__)


def run(base, left, right, kc, anchor):
    out = sv.sv_markov_topk(to_dev(base), to_dev(left), to_dev(right), kc,
                            None if anchor is None else to_dev(anchor))
    torch.cuda.synchronize()
    return out.tokens.cpu().numpy(), out.candidates.cpu().numpy(), out.cand_logits.cpu().numpy()


def check(name, base, dtype, left, right, kc, anchor, requests=None):
    B, K, V = base.shape
    say(f"[gpu] markov topk {name}: B={B} K={K} V={V} R={left.shape[1]} kc={kc} {dtype}")
    tok, cand, z = run(base, left, right, kc, anchor)
    assert tok.shape == (B, K) and cand.shape == (B, K, kc)
    n_amb = 0
    idx = range(B) if requests is None else requests
    for b in idx:
        a = -1 if anchor is None else int(anchor[b])
        rt, rc, rz, gaps = oracle.markov_topk_request(base[b], dtype, left, right, a, kc)
        for k in range(K):
            assert np.array_equal(cand[b, k], rc[k]), (name, b, k, cand[b, k][:8], rc[k][:8])
            err = abs_err(z[b, k], rz[k])
            tol = 2e-5 + 1e-6 * np.abs(rz[k])
            assert np.all(err <= tol), (name, b, k, float(err.max()))
            if gaps[k] < oracle.AMBIGUOUS_GAP:
                n_amb += 1
                say(f"[gpu] markov topk {name}: request {b} position {k} ambiguous")
                break
            assert tok[b, k] == rt[k], (name, b, k, tok[b, k], rt[k])
    say(f"[gpu] markov topk {name}: {len(list(idx))} requests, {n_amb} ambiguous")
    return tok, cand, z


def test_topk_golden_of_course():
    g = json.load(open(os.path.join(HERE, "golden", "markov", "of_course_topk.json")))
    V, R = g["V"], g["R"]
    left = np.zeros((V, 16), np.float32)
    right = np.zeros((V, 16), np.float32)
    left[:, :R] = np.asarray(g["left_factor"], np.float32)
    right[:, :R] = np.asarray(g["right_factor"], np.float32)
    base = np.asarray(g["base_logits"], np.float32)[None]
    for kc, want in g["expected"].items():
        tok, cand, z = run(base, workloads.to_bf16_bits(left), workloads.to_bf16_bits(right),
                           int(kc), np.array([g["anchor"]], np.int32))
        assert tok[0].tolist() == want["tokens"], kc
        assert cand[0].tolist() == want["candidates"], kc
        np.testing.assert_allclose(z[0], np.asarray(want["corrected"]), rtol=0, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,K,V,R,kc", [
    (70, 5, 1000, 256, 64),    # two blocks of requests; one chunk
    (3, 4, 300, 64, 17),       # kc not a multiple of anything
    (9, 11, 40000, 32, 64),    # three chunks; more positions than one walk block
    (5, 3, 777, 48, 8),        # rows not 16-byte aligned in bf16 and f32: element loads
    (4, 2, 64, 16, 64),        # every entry a candidate
])
def test_topk_parity(dtype, B, K, V, R, kc):
    base = workloads.markov_base(B, K, V, dtype, seed=31 + V)
    left, right = workloads.markov_factors(V, R, seed=32 + R)
    rng = np.random.default_rng(33 + B)
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    anchor[rng.random(B) < 0.25] = -1
    check(f"{dtype} B{B} K{K} V{V} R{R} kc{kc}", base, dtype, left, right, kc, anchor)


def test_topk_all_candidates_is_the_full_head():
    B, K, V, R = 6, 4, 64, 64
    base = workloads.markov_base(B, K, V, "f32", seed=41)
    left, right = workloads.markov_factors(V, R, seed=42)
    anchor = np.arange(B, dtype=np.int32)
    tok, cand, z = run(base, left, right, V, anchor)
    full_tok, full_z = sv.sv_markov_draft(to_dev(base), to_dev(left), to_dev(right),
                                          to_dev(anchor))
    torch.cuda.synchronize()
    assert np.all(cand == np.arange(V))
    np.testing.assert_array_equal(tok, full_tok.cpu().numpy())
    np.testing.assert_allclose(z, full_z.cpu().numpy(), rtol=0, atol=1e-4)


def test_topk_ties_nan_and_inf():
    """Tie-heavy rows (the selection's fallback over every entry), NaN and -inf entries: NaN is
    never a candidate while enough numbers remain, ties go to the lower index."""
    B, K, V, R, kc = 4, 3, 20000, 32, 64
    rng = np.random.default_rng(43)
    base = rng.choice(np.array([0.0, 1.0, 2.0], np.float32), size=(B, K, V), p=[0.9, 0.09, 0.01])
    base[0] = 0.0  # every entry tied
    base[1, :, ::7] = np.nan
    base[2, :, ::5] = -np.inf
    left, right = workloads.markov_factors(V, R, seed=44)
    tok, cand, z = check("ties", base.astype(np.float32), "f32", left, right, kc, None)
    # request 0, position 0: every logit 0 and no anchor, an exact tie: the lowest index
    assert cand[0, 0].tolist() == list(range(kc)) and tok[0, 0] == 0 and np.all(z[0, 0] == 0)
    check("ties bf16", workloads.to_bf16_bits(np.nan_to_num(base, nan=-1.0)), "bf16", left,
          right, kc, np.zeros(B, np.int32))


def test_topk_full_size_sampled():
    """The benchmarked shape: 64 requests, 8 positions, the Qwen3 vocabulary, rank 256, 64
    candidates, bf16; every request checked one by one."""
    B, K, V, R = 64, 8, workloads.QWEN3_VOCAB, 256
    base = workloads.markov_base(B, K, V, "bf16")
    left, right = workloads.markov_factors(V, R)
    anchor = np.random.default_rng(26).integers(0, V, size=B).astype(np.int32)
    check("full", base, "bf16", left, right, 64, anchor)

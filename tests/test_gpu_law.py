"""Losslessness of the GPU path on tiny vocabularies (GPU), measured statistically.

"From draft-then-verify to DSpark" ("How speculative decoding works") states that tokens
committed by the acceptance rule are distributed exactly as the target. With fixed tiny target
and draft rows replicated over a large batch, proposals drawn from q and fresh uniforms per
request, the committed token at every reached slot must follow p_i, and the number of kept
drafts must follow P(n >= i) = prod_{j<i} sum_v min(p_j, q_j). Chi-square tests at p >= 1e-3
with fixed seeds; the expected laws come from scipy's softmax, not from the kernel or the oracle.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

pytestmark = pytest.mark.gpu

from tests.gpu_util import run_sample, say  # noqa: E402


@pytest.mark.parametrize("V,K,tau,seed", [(5, 1, 1.0, 1), (8, 2, 0.8, 2), (6, 3, 1.3, 3)])
def test_committed_tokens_follow_the_target(V, K, tau, seed):
    rng = np.random.default_rng(seed)
    B, calls = 50_000, 4  # 200000 rounds in four batches
    T1 = rng.normal(0, 1.5, size=(K + 1, V)).astype(np.float32)
    D1 = (T1[:K] + rng.normal(0, 1.0, size=(K, V))).astype(np.float32)
    p = [scipy.special.softmax(T1[i].astype(np.float64) / tau) for i in range(K + 1)]
    q = [scipy.special.softmax(D1[i].astype(np.float64) / tau) for i in range(K)]
    T = np.ascontiguousarray(np.broadcast_to(T1, (B, K + 1, V)))
    D = np.ascontiguousarray(np.broadcast_to(D1, (B, K, V)))
    say(f"[gpu] law V={V} K={K} tau={tau} rounds={B * calls}")
    accs, coms = [], []
    for _ in range(calls):
        x = np.stack([rng.choice(V, size=B, p=q[i]) for i in range(K)], axis=1).astype(np.int32)
        u = rng.random((B, K), dtype=np.float32)
        r = rng.random(B, dtype=np.float32)
        a_, c_, _, _ = run_sample(T, D, x, u, r, tau)
        accs.append(a_)
        coms.append(c_)
    acc, com = np.concatenate(accs), np.concatenate(coms)
    B = B * calls

    beta = [float(np.sum(np.minimum(p[j], q[j]))) for j in range(K)]
    pn = np.array([np.prod(beta[:i]) * ((1 - beta[i]) if i < K else 1.0) for i in range(K + 1)])
    ncount = np.bincount(acc, minlength=K + 1)
    pv = scipy.stats.chisquare(ncount, pn * B).pvalue
    say(f"[gpu] law accepted-length counts {ncount.tolist()} p-value {pv:.4f}")
    assert pv > 1e-3
    for i in range(K + 1):
        reached = acc >= i
        tok = com[reached, i]
        cnt = np.bincount(tok, minlength=V)
        exp = p[i] * reached.sum()
        keep = exp > 5
        obs = np.append(cnt[keep], cnt[~keep].sum())
        ex = np.append(exp[keep], exp[~keep].sum())
        if ex[-1] == 0:
            obs, ex = obs[:-1], ex[:-1]
        pv = scipy.stats.chisquare(obs, ex).pvalue
        say(f"[gpu] law slot {i}: reached {int(reached.sum())} p-value {pv:.4f}")
        assert pv > 1e-3

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


def _chisq(cnt, exp):
    keep = exp > 5
    obs = np.append(cnt[keep], cnt[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return scipy.stats.chisquare(obs, ex * obs.sum() / ex.sum()).pvalue


@pytest.mark.parametrize("seed", [7, 8])
def test_markov_drafts_verified_follow_the_target(seed):
    """The sampled Markov head feeding sampling verification, end to end: proposals drawn by
    sv_markov_draft_sampled (position 1 biased by the token drawn at position 0) and verified by
    sv_verify_batch against the draft rows the head wrote. The drafts' joint law is
    softmax(base_0 + bias(anchor)) x softmax(base_1 + bias(x_0)) ("From draft-then-verify to
    DSpark", Recovering sequential dependencies); the committed token at every reached slot
    follows the target row ("How speculative decoding works")."""
    import torch

    import lossless_draft_verification_sv_amd as sv
    from tests.gpu_util import to_dev
    from workloads import bf16_bits_to_f32, to_bf16_bits

    V, K, R, tau, anchor0 = 6, 2, 16, 1.0, 2
    rng = np.random.default_rng(seed)
    base1 = rng.normal(0, 1.0, size=(K, V)).astype(np.float32)
    T1 = rng.normal(0, 1.5, size=(K + 1, V)).astype(np.float32)
    Lh = np.zeros((V, R), np.float32)
    Rh = np.zeros((V, R), np.float32)
    ang = np.arange(V)
    Lh[:, 0], Lh[:, 1] = np.cos(ang), np.sin(ang)
    Rh[:, 0], Rh[:, 1] = 1.5 * np.cos(2 * ang), 1.5 * np.sin(2 * ang)
    Lb, Rb = to_bf16_bits(Lh), to_bf16_bits(Rh)
    Ld = bf16_bits_to_f32(Lb).astype(np.float64)
    Rd = bf16_bits_to_f32(Rb).astype(np.float64)
    q0 = scipy.special.softmax((base1[0] + Rd @ Ld[anchor0]) / tau)
    q1 = np.stack([scipy.special.softmax((base1[1] + Rd @ Ld[v]) / tau) for v in range(V)])
    p = [scipy.special.softmax(T1[i].astype(np.float64) / tau) for i in range(K + 1)]
    B, calls = 16384, 16
    say(f"[gpu] markov -> verify law V={V} K={K} seed={seed} rounds={B * calls}")
    base = to_dev(np.ascontiguousarray(np.broadcast_to(base1, (B, K, V))))
    target = to_dev(np.ascontiguousarray(np.broadcast_to(T1, (B, K + 1, V))))
    left, right = to_dev(Lb), to_dev(Rb)
    taus = to_dev(np.full(B, tau, np.float32))
    anc = to_dev(np.full(B, anchor0, np.int32))
    xs, accs, coms = [], [], []
    for _ in range(calls):
        ud = to_dev(rng.random((B, K), dtype=np.float32))
        tok, q = sv.sv_markov_draft_sampled(base, left, right, taus, ud, anc)
        uv = to_dev(rng.random((B, K), dtype=np.float32))
        r = to_dev(rng.random(B, dtype=np.float32))
        out = sv.sv_verify_batch(target, q, tok, uv, r, tau)
        torch.cuda.synchronize()
        xs.append(tok.cpu().numpy())
        accs.append(out.accepted_len.cpu().numpy())
        coms.append(out.committed.cpu().numpy())
    x, acc, com = np.concatenate(xs), np.concatenate(accs), np.concatenate(coms)
    N = x.shape[0]
    joint = np.bincount(x[:, 0] * V + x[:, 1], minlength=V * V).astype(np.float64)
    pv = _chisq(joint, (q0[:, None] * q1).reshape(-1) * N)
    say(f"[gpu] markov drafts joint law p-value {pv:.4f}")
    assert pv > 1e-3
    for i in range(K + 1):
        reached = acc >= i
        cnt = np.bincount(com[reached, i], minlength=V).astype(np.float64)
        pv = _chisq(cnt, p[i] * reached.sum())
        say(f"[gpu] markov -> verify slot {i}: reached {int(reached.sum())} p-value {pv:.4f} "
            f"counts {cnt.astype(int).tolist()} expected {np.round(p[i] * reached.sum()).tolist()}")
        assert pv > 1e-3

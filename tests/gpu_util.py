"""Helpers for the GPU tests: upload seeded host inputs, call the C-ABI through the binding,
and compare with the fp64 oracle to the parity bar.

Parity bar (sampling mode): |target_prob - oracle| <= 1e-5 and |draft_prob - oracle| <= 1e-5 on
every request; accepted lengths and committed tokens identical on every request whose oracle
margins are all >= 1e-6 (ambiguous requests are counted and reported, not compared). Greedy mode:
accepted lengths and committed tokens bit-exact on every request.
"""
import sys

import numpy as np
import torch

import lossless_draft_verification_sv_amd as sv
import oracle

PROB_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def abs_err(got, ref) -> np.ndarray:
    """|got - ref| elementwise, with equal infinities and NaN on both sides counted as no error
    and a NaN on one side only as an infinite one (so that it never passes a tolerance check)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        err = np.abs(got - ref)
    err[((got == ref) & np.isinf(ref)) | (np.isnan(got) & np.isnan(ref))] = 0.0
    err[np.isnan(err)] = np.inf
    return err


def to_dev(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    if a is None:
        return None
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device())
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def run_sample(target, draft, tokens, uniforms, residual, tau, num_draft=None):
    out = sv.sv_verify_batch(to_dev(target), to_dev(draft), to_dev(tokens), to_dev(uniforms),
                             to_dev(residual), tau,
                             None if num_draft is None else to_dev(num_draft),
                             return_draft_prob=True)
    torch.cuda.synchronize()
    return (out.accepted_len.cpu().numpy(), out.committed.cpu().numpy(),
            out.target_prob.cpu().numpy(), out.draft_prob.cpu().numpy())


def run_greedy(target, tokens, num_draft=None):
    out = sv.sv_verify_greedy(to_dev(target), to_dev(tokens),
                              None if num_draft is None else to_dev(num_draft))
    torch.cuda.synchronize()
    return out.accepted_len.cpu().numpy(), out.committed.cpu().numpy()


def check_sample_parity(name, target, draft, dtype, tokens, uniforms, residual, tau,
                        num_draft=None, requests=None):
    """Run GPU and oracle on the same inputs; assert the parity bar. Returns a summary dict."""
    say(f"[gpu] sample {name}: target {target.shape} {dtype} tau={tau}")
    acc, com, tp, dp = run_sample(target, draft, tokens, uniforms, residual, tau, num_draft)
    ref = oracle.verify_batch(target, draft, dtype, tokens, uniforms, residual, tau, num_draft,
                              requests=requests)
    idx = np.arange(tokens.shape[0]) if requests is None else np.asarray(requests)
    amb = np.array([ref.requests[b].ambiguous for b in idx], dtype=bool)
    tp_err = float(np.max(np.abs(tp[idx] - ref.target_prob[idx])))
    dp_err = float(np.max(np.abs(dp[idx] - ref.draft_prob[idx])))
    ok = idx[~amb]
    bad_n = ok[acc[ok] != ref.accepted_len[ok]]
    bad_c = ok[np.any(com[ok] != ref.committed[ok], axis=1)]
    summary = dict(requests=len(idx), ambiguous=int(amb.sum()), max_target_prob_err=tp_err,
                   max_draft_prob_err=dp_err, accepted_mismatch=len(bad_n),
                   token_mismatch=len(bad_c),
                   mean_accepted_plus_one=float(np.mean(acc[idx] + 1)))
    say(f"[gpu] sample {name}: {summary}")
    assert tp_err <= PROB_TOL, (name, tp_err)
    assert dp_err <= PROB_TOL, (name, dp_err)
    assert len(bad_n) == 0, (name, bad_n[:10], acc[bad_n[:10]], ref.accepted_len[bad_n[:10]])
    assert len(bad_c) == 0, (name, bad_c[:10], com[bad_c[:5]], ref.committed[bad_c[:5]])
    # outputs of every request are well formed, ambiguous or not
    K = tokens.shape[1]
    for b in idx:
        k = K if num_draft is None else int(num_draft[b])
        n = int(acc[b])
        assert 0 <= n <= k
        assert list(com[b, :n]) == list(tokens[b, :n])
        assert 0 <= com[b, n] < target.shape[-1]
        assert np.all(com[b, n + 1:] == -1)
        assert np.all(tp[b, k:] == 0.0)
    return summary


def check_greedy_parity(name, target, dtype, tokens, num_draft=None, requests=None):
    say(f"[gpu] greedy {name}: target {target.shape} {dtype}")
    acc, com = run_greedy(target, tokens, num_draft)
    ref = oracle.verify_greedy(target, dtype, tokens, num_draft, requests=requests)
    idx = np.arange(tokens.shape[0]) if requests is None else np.asarray(requests)
    assert np.array_equal(acc[idx], ref.accepted_len[idx]), name
    assert np.array_equal(com[idx], ref.committed[idx]), name
    say(f"[gpu] greedy {name}: {len(idx)} requests bit-exact, "
        f"mean accepted+1 {np.mean(acc[idx] + 1):.3f}")

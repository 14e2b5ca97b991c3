"""Confidence-scheduled prefix selection on the GPU against the scheduling oracle.

The kernel's lengths must equal the oracle's; where the two pick different N, the rates must be
a tie to fp64 rounding (the expected-token sums are added in a different order). Row starts
must be the exclusive sums of the lengths, and the scheduler's output must drive a flattened
verify call directly.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

import lossless_draft_verification_sv_amd as sv  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_util import say, to_dev  # noqa: E402


def table(rng, B, K, slope, tile, jump, base=1.0):
    n = np.arange(B + B * K + 1 + int(rng.integers(0, 5)))
    return (base + slope * n + jump * np.ceil(n / tile)).astype(np.float32)


def confidences(rng, B, K):
    c = rng.beta(5, 1.5, size=(B, K)).astype(np.float32)
    c[rng.random((B, K)) < 0.05] = 1.0  # exact ties in survival
    c[rng.random((B, K)) < 0.02] = 0.0
    c[rng.random((B, K)) < 0.01] = np.nan
    return c


def rates(conf, tab):
    s = oracle.prefix_survival(conf)
    B = s.shape[0]
    order = oracle.rank_tokens(s)
    exp = float(B)
    out = []
    for n in range(len(order) + 1):
        if n:
            b, k = order[n - 1]
            exp += float(s[b, k])
        t = float(tab[B + n])
        out.append(exp / t if np.isfinite(t) and t > 0 else -np.inf)
    return np.array(out), order


def check(conf, tab):
    B, K = conf.shape
    out = sv.sv_schedule_prefix(to_dev(conf), to_dev(tab))
    torch.cuda.synchronize()
    num = out.num_draft.cpu().numpy()
    n_gpu = int(round(float(out.summary[0].item())))
    ref_num, n_ref, rate_ref = oracle.schedule_hardware_aware(conf, tab.astype(np.float64))
    if n_gpu != n_ref:  # only a tie to rounding may differ
        r, order = rates(conf, tab.astype(np.float64))
        assert abs(r[n_gpu] - rate_ref) <= 1e-12 * rate_ref, (n_gpu, n_ref)
        ref_num = np.zeros(B, np.int32)
        for b, k in order[:n_gpu]:
            ref_num[b] += 1
    assert np.array_equal(num, ref_num)
    assert int(num.sum()) == n_gpu
    ts, ds = oracle.row_starts(num)
    assert np.array_equal(out.target_row_start.cpu().numpy(), ts)
    assert np.array_equal(out.draft_row_start.cpu().numpy(), ds)
    return num, n_gpu


@pytest.mark.parametrize("B,K,seed", [(1, 1, 1), (3, 4, 2), (16, 8, 3), (64, 8, 4), (100, 7, 5),
                                      (256, 16, 6), (4096, 1, 7), (64, 64, 8)])
def test_hardware_aware_matches_oracle(B, K, seed):
    rng = np.random.default_rng(seed)
    conf = confidences(rng, B, K)
    for slope, tile, jump in ((0.0, 4, 0.0), (0.002, 16, 0.05), (0.02, 64, 0.3), (1.0, 8, 2.0)):
        num, n = check(conf, table(rng, B, K, slope, tile, jump))
        say(f"[gpu] schedule B={B} K={K} slope={slope}: N={n} of {B * K}")


def test_unusable_table_entries_are_skipped():
    rng = np.random.default_rng(11)
    B, K = 32, 8
    conf = confidences(rng, B, K)
    tab = table(rng, B, K, 0.01, 8, 0.1)
    tab[B + 5::7] = np.nan
    tab[B + 3::11] = 0.0
    check(conf, tab)
    tab[:] = -1.0  # nothing usable: no drafts
    out = sv.sv_schedule_prefix(to_dev(conf), to_dev(tab))
    assert not out.num_draft.cpu().numpy().any()


@pytest.mark.parametrize("threshold", [0.0, 0.3, 0.7, 1.0, 1.5])
def test_threshold_mode_matches_oracle(threshold):
    rng = np.random.default_rng(13)
    conf = confidences(rng, 200, 12)
    out = sv.sv_schedule_prefix(to_dev(conf), None, threshold)
    num = out.num_draft.cpu().numpy()
    assert np.array_equal(num, oracle.schedule_threshold(conf, threshold))
    ts, ds = oracle.row_starts(num)
    assert np.array_equal(out.target_row_start.cpu().numpy(), ts)


def test_scheduled_lengths_drive_a_flattened_verify():
    """Drafter confidences -> scheduler -> verify on exactly the scheduled rows, with no host
    round trip between the two calls (the host only builds the test's expected values)."""
    from workloads import BATCHED, generate

    w = BATCHED.replace(B=24, K=8, V=20000, seed=77)
    inp = generate(w)
    rng = np.random.default_rng(3)
    conf = confidences(rng, w.B, w.K)
    tab = table(rng, w.B, w.K, 0.01, 16, 0.05)
    out = sv.sv_schedule_prefix(to_dev(conf), to_dev(tab))
    num = out.num_draft.cpu().numpy()
    ts, ds = oracle.row_starts(num)
    # the flattened rows the target would have produced for exactly these lengths
    tflat = np.concatenate([inp.target[b, :num[b] + 1] for b in range(w.B)])
    dparts = [inp.draft[b, :num[b]] for b in range(w.B) if num[b] > 0]
    dflat = np.concatenate(dparts) if dparts else np.zeros((0, w.V), inp.draft.dtype)
    temps = np.full(w.B, w.temperature, np.float32)
    res = sv.sv_verify_ragged(to_dev(tflat), to_dev(dflat) if len(dflat) else None,
                              to_dev(inp.tokens), to_dev(inp.uniforms), to_dev(inp.residual),
                              to_dev(temps), out.num_draft, out.target_row_start,
                              out.draft_row_start)
    torch.cuda.synchronize()
    ref = oracle.verify_ragged(tflat, dflat, w.dtype, inp.tokens, inp.uniforms, inp.residual,
                               temps, num, ts, ds)
    ok = ~ref.ambiguous
    assert np.array_equal(res.accepted_len.cpu().numpy()[ok], ref.accepted_len[ok])
    assert np.array_equal(res.committed.cpu().numpy()[ok], ref.committed[ok])


def test_step_time_table_from_the_verify_kernel():
    from lossless_draft_verification_sv_amd.schedule import (step_time_table,
                                                              synthetic_target_step_us)

    B, K, V = 16, 8, 32768
    tab = step_time_table(B, K, V)
    say(f"[gpu] step table B={B} K={K}: {tab[B]:.0f} .. {tab[-1]:.0f} us")
    assert tab.shape == (B + B * K + 1,) and np.all(np.isfinite(tab)) and np.all(tab > 0)
    verify = tab - synthetic_target_step_us(np.arange(len(tab))).astype(np.float32)
    assert verify[B] > 0 and verify[-1] >= 0.8 * verify[B]  # more rows never much faster
    conf = confidences(np.random.default_rng(21), B, K)
    check(conf, tab)

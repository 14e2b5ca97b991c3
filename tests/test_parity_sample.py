"""Sampling-mode parity of the HIP path with the fp64 oracle (GPU).

Small shapes span several work-groups, vector and scalar row paths and ragged chunk tails; the
full-size cases are the workloads the benchmark times, in the same launch configuration.
"""
import glob
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from tests.gpu_util import check_sample_parity, run_sample, say  # noqa: E402
from workloads import (BATCHED, HEAVY, INTERACTIVE, TINY, generate, to_bf16_bits)  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check(inp, requests=None, name=None):
    w = inp.workload
    return check_sample_parity(name or w.name, inp.target, inp.draft, w.dtype, inp.tokens,
                               inp.uniforms, inp.residual, w.temperature, inp.num_draft,
                               requests=requests)


def test_tiny_workload_exact():
    s = _check(generate(TINY))
    assert s["ambiguous"] == 0


SMALL = [
    # (B, K, V, dtype, tau, ragged, identical_even)
    (3, 4, 1000, "f32", 1.0, False, False),  # 16-byte rows: vector loads
    (5, 3, 4099, "f32", 0.8, False, False),  # odd V: scalar path
    (4, 6, 4099, "bf16", 1.3, False, True),  # scalar bf16, half identical
    (6, 8, 16400, "bf16", 0.7, False, True),  # vector bf16, several chunks per row
    (7, 5, 12288, "f32", 2.0, True, False),  # ragged k_b, NaN rows past k_b
    (9, 16, 6000, "bf16", 1.0, True, False),  # ragged, K=16
    (2, 1, 70000, "bf16", 0.5, False, False),  # K=1
    (3, 64, 520, "f32", 1.0, False, False),  # K=64: every slot in one wave
]


@pytest.mark.parametrize("B,K,V,dtype,tau,ragged,ident", SMALL)
def test_small_shapes(B, K, V, dtype, tau, ragged, ident):
    w = HEAVY.replace(name=f"small_B{B}_K{K}_V{V}_{dtype}_t{tau}", B=B, K=K, V=V, dtype=dtype,
                      temperature=tau, ragged=ragged, identical_even=ident,
                      seed=3000 + B * 7 + K * 3 + V)
    _check(generate(w))


def test_identical_rows_accept_every_draft():
    inp = generate(BATCHED.replace(B=8, V=20000, seed=31))
    even = np.arange(0, 8, 2)
    s = _check(inp)
    acc, _, _, _ = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                              inp.workload.temperature)
    assert np.all(acc[even] == inp.workload.K)


@pytest.mark.parametrize("V,dtype", [
    (300000, "bf16"),  # 16-byte rows: 147 segments of 2048 logits, the bonus draw reads one
    (300001, "f32"),   # scalar rows: 1172 segments of 256 logits, more than the workspace keeps,
                       # so bonus tokens take the tile draw over the whole row
])
def test_bonus_draw_segments_and_tile_fallback(V, dtype):
    inp = generate(BATCHED.replace(name=f"bonus_V{V}_{dtype}", B=4, K=2, V=V, dtype=dtype,
                                   seed=37 + V % 7))
    _check(inp)
    acc, _, _, _ = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                              inp.workload.temperature)
    assert np.all(acc[0::2] == 2)  # identical draft rows: every draft kept, a bonus token drawn


def test_zero_drafts_and_out_of_range_tokens():
    w = TINY.replace(B=6, K=5, V=3000, seed=41)
    inp = generate(w)
    nd = np.array([0, 5, 2, 0, 5, 1], dtype=np.int32)
    inp.num_draft = nd
    inp.tokens[1, 0] = 3000 + 7  # past the vocabulary: rejected, p = 0
    inp.tokens[4, 2] = -3
    s = _check(inp, name="k0_and_out_of_range")
    acc, com, tp, _ = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                                 w.temperature, nd)
    assert acc[0] == 0 and acc[3] == 0 and acc[1] == 0 and tp[1, 0] == 0.0
    assert acc[4] <= 2


def test_misaligned_rows_take_the_scalar_path():
    import torch

    import lossless_draft_verification_sv_amd as sv
    import oracle

    inp = generate(TINY.replace(B=3, K=4, V=4096, seed=51))
    w = inp.workload
    dev = torch.device("cuda:0")

    def shifted(a):  # same values, device pointer 4 bytes past a 16-byte boundary
        flat = torch.empty(a.size + 1, dtype=torch.float32, device=dev)
        view = flat[1:].view(a.shape)
        view.copy_(torch.from_numpy(a))
        return view

    t, d = shifted(inp.target), shifted(inp.draft)
    assert t.data_ptr() % 16 != 0
    out = sv.sv_verify_batch(t, d, torch.from_numpy(inp.tokens).to(dev),
                             torch.from_numpy(inp.uniforms).to(dev),
                             torch.from_numpy(inp.residual).to(dev), w.temperature)
    torch.cuda.synchronize()
    ref = oracle.verify_batch(inp.target, inp.draft, "f32", inp.tokens, inp.uniforms,
                              inp.residual, w.temperature)
    ok = ~ref.ambiguous
    assert np.array_equal(out.committed.cpu().numpy()[ok], ref.committed[ok])
    assert np.max(np.abs(out.target_prob.cpu().numpy() - ref.target_prob)) <= 1e-5


@pytest.mark.parametrize("V,dtype", [(20000, "f32"), (20000, "bf16"), (4099, "f32"),
                                     (4099, "bf16")])
def test_masked_vocabulary(V, dtype):
    """Rows with most entries at -inf (a filtered vocabulary: probability 0). Odd requests draw
    the target and draft masks independently, so that draft tokens can fall where p or q is 0;
    even requests (identical target and draft rows) share one mask, keep every draft and draw
    the bonus token from a masked row. One target row and one draft row keep a single finite
    entry (p, then q, a point mass). Vector and scalar row paths."""
    inp = generate(BATCHED.replace(name=f"masked_V{V}_{dtype}", B=6, K=4, V=V, dtype=dtype,
                                   seed=81 + V % 11))
    rng = np.random.default_rng(83 + V)
    neg_inf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    keep_t = rng.random(inp.target.shape) < 0.4
    keep_d = rng.random(inp.draft.shape) < 0.4
    K = inp.workload.K
    for b in range(0, inp.workload.B, 2):
        keep_t[b, np.arange(K), inp.tokens[b]] = True  # the drafted tokens keep their mass
    keep_t[..., rng.integers(0, V)] = True  # every row keeps at least one finite entry
    keep_d[1::2, :, rng.integers(0, V)] = True
    keep_d[0::2] = keep_t[0::2, :-1]
    inp.target[~keep_t] = neg_inf
    inp.draft[~keep_d] = neg_inf

    def value(x):
        v = np.array([x], dtype=np.float32)
        return to_bf16_bits(v)[0] if dtype == "bf16" else v[0]

    inp.target[1, 0, :] = neg_inf
    inp.target[1, 0, int(rng.integers(0, V))] = value(1.5)
    inp.draft[5, 0, :] = neg_inf  # q is a point mass at the drafted token
    inp.draft[5, 0, inp.tokens[5, 0]] = value(2.0)
    _check(inp)
    acc, _, _, _ = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                              inp.workload.temperature)
    assert np.all(acc[0::2] == K)  # identical masked rows: every draft kept


@pytest.mark.parametrize("V,dtype", [(4096, "f32"), (4096, "bf16"), (4099, "f32")])
def test_tokens_without_mass_under_one_distribution(V, dtype):
    """Slot 0's token has a -inf draft logit (q = 0) and a finite target logit: kept for any
    uniform; slot 1's token has a -inf target logit (p = 0): rejected, with target probability
    0 and the residual draw avoiding it. Probabilities are 0, never NaN."""
    inp = generate(TINY.replace(name=f"zero_mass_V{V}_{dtype}", B=4, K=3, V=V, dtype=dtype,
                                seed=91 + V % 5))
    neg_inf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    for b in range(4):
        inp.draft[b, 0, inp.tokens[b, 0]] = neg_inf
        inp.target[b, 1, inp.tokens[b, 1]] = neg_inf
    inp.uniforms[:, 0] = np.array([0.0, 0.5, 0.9, 0.999], np.float32)
    inp.uniforms[:, 1] = 0.3
    s = _check(inp)
    assert s["ambiguous"] == 0
    acc, com, tp, dp = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                                  inp.workload.temperature)
    assert np.all(acc == 1) and np.all(dp[:, 0] == 0.0) and np.all(tp[:, 0] > 0.0)
    assert np.all(tp[:, 1] == 0.0) and np.all(com[:, 1] != inp.tokens[:, 1])
    assert not np.isnan(tp).any() and not np.isnan(dp).any()


@pytest.mark.parametrize("tau", [0.05, 20.0])
def test_extreme_temperatures(tau):
    w = TINY.replace(name=f"temperature_{tau}", B=6, K=4, V=8000, dtype="bf16",
                     temperature=tau, seed=61)
    _check(generate(w))


def test_golden_worked_examples_on_gpu():
    for f in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        g = json.load(open(f))
        if g["mode"] != "sample":
            continue
        T = np.log(np.asarray(g["target_probs"], dtype=np.float64)).astype(np.float32)[None]
        D = np.log(np.asarray(g["draft_probs"], dtype=np.float64)).astype(np.float32)[None]
        x = np.asarray([g["tokens"]], dtype=np.int32)
        u = np.asarray([g["uniforms"]], dtype=np.float32)
        r = np.asarray([g["residual"]], dtype=np.float32)
        acc, com, tp, dp = run_sample(T, D, x, u, r, g["tau"])
        e = g["expected"]
        say(f"[gpu] golden {os.path.basename(f)}: {acc.tolist()} {com.tolist()}")
        assert acc[0] == e["accepted_len"] and com[0].tolist() == e["committed"], f
        assert np.allclose(tp[0], e["target_prob"], atol=1e-6), f
        assert np.allclose(dp[0], e["draft_prob"], atol=1e-6), f


def test_repeat_calls_are_bitwise_deterministic():
    inp = generate(BATCHED.replace(B=6, V=30000, seed=71))
    w = inp.workload
    a = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual, w.temperature)
    for _ in range(5):
        b = run_sample(inp.target, inp.draft, inp.tokens, inp.uniforms, inp.residual,
                       w.temperature)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


# ----- full sizes (V = 151936), the configurations the benchmark times ---------------------


def test_full_interactive_B1_K8_f32():
    _check(generate(INTERACTIVE))


def test_full_vocabulary_f32_chunks_of_whole_rounds():
    """Float32 rows of the Qwen3 vocabulary at B = 4: an even split into the plan's 37 chunks
    leaves each a round and a three-group tail, so the launch cuts 38 chunks of whole rounds, the
    last one shorter (the bonus rows' segments among them); half the requests keep every draft."""
    w = INTERACTIVE.replace(name="whole_rounds_B4_K8_V151936_f32", B=4, identical_even=True,
                            seed=3701)
    s = _check(generate(w))
    assert s["requests"] == 4


def test_full_batched_B64_K8_bf16():
    s = _check(generate(BATCHED))
    assert s["requests"] == 64


def test_full_heavy_B256_K16_bf16():
    s = _check(generate(HEAVY))
    assert s["requests"] == 256


def test_one_workspace_reused_across_shapes_and_modes():
    """A single zero-filled workspace serves calls of different shapes and both modes in
    sequence, each matching the oracle: partials left by earlier calls are never taken for the
    current call's."""
    import torch

    import lossless_draft_verification_sv_amd as sv
    import oracle
    from tests.gpu_util import to_dev

    lib = sv.load_library()
    dev = torch.device("cuda:0")
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    shapes = [(5, 8, 30000, "bf16"), (2, 3, 4099, "f32"), (9, 16, 20000, "bf16"),
              (1, 4, 1000, "f32"), (5, 8, 30000, "bf16")]
    for i, (B, K, V, dt) in enumerate(shapes * 2):
        w = BATCHED.replace(name=f"reuse{i}", B=B, K=K, V=V, dtype=dt, temperature=1.0,
                            seed=900 + i)
        inp = generate(w)
        T, D = to_dev(inp.target), to_dev(inp.draft)
        x, u, r = to_dev(inp.tokens), to_dev(inp.uniforms), to_dev(inp.residual)
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        com = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
        tp = torch.empty(B, K, dtype=torch.float32, device=dev)
        code = sv.SV_DTYPE_BF16 if dt == "bf16" else sv.SV_DTYPE_F32
        if i % 2 == 0:
            st = lib.sv_verify_batch(T.data_ptr(), D.data_ptr(), code, B, K, V, 1.0,
                                     x.data_ptr(), None, u.data_ptr(), r.data_ptr(),
                                     acc.data_ptr(), com.data_ptr(), tp.data_ptr(), None,
                                     ws.data_ptr(), ws.numel(), s)
            assert st == 0, sv.sv_last_error()
            torch.cuda.synchronize()
            ref = oracle.verify_batch(inp.target, inp.draft, dt, inp.tokens, inp.uniforms,
                                      inp.residual, 1.0)
            ok = ~ref.ambiguous
            assert np.array_equal(com.cpu().numpy()[ok], ref.committed[ok]), i
        else:
            st = lib.sv_verify_greedy(T.data_ptr(), code, B, K, V, x.data_ptr(), None,
                                      acc.data_ptr(), com.data_ptr(), ws.data_ptr(), ws.numel(),
                                      s)
            assert st == 0, sv.sv_last_error()
            torch.cuda.synchronize()
            ref = oracle.verify_greedy(inp.target, dt, inp.tokens)
            assert np.array_equal(com.cpu().numpy(), ref.committed), i

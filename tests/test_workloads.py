"""The seeded input generator (CPU only): determinism, storage rounding, structure."""
import numpy as np
import torch

from workloads import (BATCHED, GREEDY, HEAVY, TINY, bf16_bits_to_f32, generate, to_bf16_bits)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 5, 100000), rng.normal(0, 1e-3, 1000),
                        [0.0, -0.0, 1.0, 3.0e38, -3.0e38]]).astype(np.float32)
    # exact ties: the low 16 bits are 0x8000
    ties = (rng.integers(0, 1 << 16, 1000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)
    ties = ties.view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_bits_to_f32(ref), back)


def test_generation_is_deterministic_and_request_local():
    w = BATCHED.replace(B=4, V=2048)
    a, b = generate(w), generate(w, threads=1)
    for f in ("target", "draft", "tokens", "uniforms", "residual"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    # request b depends only on (seed, b): a smaller batch reproduces the first requests
    c = generate(w.replace(B=2))
    assert np.array_equal(c.target, a.target[:2]) and np.array_equal(c.tokens, a.tokens[:2])


def test_batched_structure():
    w = BATCHED.replace(B=4, V=4096)
    inp = generate(w)
    assert inp.target.dtype == np.uint16 and inp.target.shape == (4, 9, 4096)
    assert np.array_equal(inp.draft[0], inp.target[0, :8])  # even request: identical rows
    assert not np.array_equal(inp.draft[1], inp.target[1, :8])
    assert inp.tokens.min() >= 0 and inp.tokens.max() < 4096
    assert np.all((inp.uniforms >= 0) & (inp.uniforms < 1))


def test_heavy_masks_rows_past_k():
    inp = generate(HEAVY.replace(B=6, V=512))
    for b in range(6):
        k = inp.k_of(b)
        assert 1 <= k <= 16
        t = bf16_bits_to_f32(inp.target[b])
        d = bf16_bits_to_f32(inp.draft[b])
        assert np.all(np.isfinite(t[: k + 1])) and np.all(np.isnan(t[k + 1:]))
        assert np.all(np.isfinite(d[:k])) and np.all(np.isnan(d[k:]))
        assert np.all(inp.tokens[b, k:] == -1) and np.all(inp.tokens[b, :k] >= 0)


def test_greedy_tokens_are_draft_argmax():
    inp = generate(GREEDY.replace(B=3, V=1000))
    assert inp.draft is None and inp.target.dtype == np.float32
    assert inp.tokens.min() >= 0


def test_sampled_tokens_follow_the_draft_distribution():
    """Gumbel-max draws: frequency of each token over many seeds against softmax(d / tau)."""
    import scipy.special
    import scipy.stats
    w = TINY.replace(B=4000, K=1, V=6, draft_sigma=(0.5,), seed=5, target_sigma=1.0)
    inp = generate(w, threads=1)
    # every request has its own draft row; pool by expected probability of the drawn token
    p = scipy.special.softmax(inp.draft[:, 0, :].astype(np.float64), axis=1)
    probs = p[np.arange(w.B), inp.tokens[:, 0]]
    # E[p(x)] under x ~ p is sum p^2; compare means
    expect = np.sum(p * p, axis=1)
    z = (probs.mean() - expect.mean()) / (probs.std() / np.sqrt(w.B))
    assert abs(z) < 4


def test_mixed_workload_and_flatten():
    from workloads import MIXED, flatten

    w = MIXED.replace(B=9, K=5, V=300, seed=12)
    inp = generate(w)
    assert list(inp.temperatures) == [w.temperature_of(b) for b in range(w.B)]
    for b in range(w.B):  # greedy requests propose the argmax of their draft rows
        if inp.temperatures[b] == 0:
            k = inp.k_of(b)
            d = bf16_bits_to_f32(inp.draft[b, :k]).astype(np.float64)
            assert list(inp.tokens[b, :k]) == list(np.argmax(d, axis=1))
    order = [4, 2, 8, 0, 1, 7, 3, 6, 5]
    f = flatten(inp, order)
    ks = [inp.k_of(b) for b in range(w.B)]
    assert f.target.shape[0] == sum(k + 1 for k in ks)
    assert f.draft.shape[0] == sum(k for b, k in enumerate(ks) if inp.temperatures[b] > 0)
    for b in range(w.B):
        k = ks[b]
        assert np.array_equal(f.target[f.target_row_start[b]:f.target_row_start[b] + k + 1],
                              inp.target[b, :k + 1])
        if inp.temperatures[b] > 0:
            assert np.array_equal(f.draft[f.draft_row_start[b]:f.draft_row_start[b] + k],
                                  inp.draft[b, :k])
    # requests are packed in the order given
    starts = [f.target_row_start[b] for b in order]
    assert starts == sorted(starts)

"""Seeded synthetic inputs for batched draft verification.

This module only draws random inputs: target and draft logits, draft tokens, per-slot
uniforms, the residual uniform and the per-request number of drafts to verify. It holds none
of the verification arithmetic (no softmax, no acceptance test, no residual sampling), so that
the oracle and the GPU path can both consume its output without sharing any of the method.

Draft tokens for sampling requests are drawn from softmax(d / tau) with the exponential-race
form of the Gumbel-max construction: x = argmax_v (d_v / tau - log E_v), E_v ~ Exp(1) i.i.d.
Since -log E_v is standard Gumbel, x has exactly the categorical law softmax(d / tau) of the
stored (already rounded) draft row. Greedy requests take x = argmax_v d_v (lowest index on
ties), the proposal a greedy drafter makes. In a mixed workload request b has temperature
temperatures[b % len(temperatures)], 0 marking a greedy request.

Shapes and value distributions stand in for the pages' workloads (no dataset is used):
  * vocabulary 151936, the size of the Qwen3-8B target used for the single-H100 comparison in
    "From draft-then-verify to DSpark" and for the vLLM demo in the DSpark paper review;
  * draft blocks of 4-16 tokens ("Accelerating Large-Model Inference ...", section 4 setup;
    block_size 8 in its section 8 config table; 7 speculative tokens in the DSpark review);
  * one request in flight vs 64 in flight vs a heavily loaded batch (DSpark review, section 6);
  * per-request verify lengths that differ inside one batch (DSpark review, 4.2.2 and 5.3);
  * later draft slots agreeing less with the target ("suffix decay", DSpark review 3.2 and
    "From draft-then-verify to DSpark", DFlash section);
  * batches flattened to the rows each request uses, with greedy and sampling requests mixed
    (DSpark review 4.2.2; "Bringing DSpark to vLLM Metal", greedy-only serving).

Randomness: every request b of a workload draws from its own generator
numpy.random.default_rng(SeedSequence([seed, b])), in this fixed order:
  1. target normals [K+1, V] (float32);  2. spike indices [K+1] (if the workload has a spike);
  3. draft noise [K, V] (float32);       4. draft-token exponentials [K, V] (sampling requests);
  5. per-slot uniforms u [K] (float32);  6. residual uniform r (float32);
  7. the number of drafts k_b (ragged workloads only).
Noise is added in float32; bf16 storage rounds to nearest, ties to even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

QWEN3_VOCAB = 151936


@dataclasses.dataclass(frozen=True)
class Workload:
    """A seeded synthetic verify workload (one batch of B requests)."""

    name: str
    B: int
    K: int
    V: int
    dtype: str  # "f32" or "bf16": storage type of both logit tensors
    temperature: float
    mode: str  # "sample", "greedy" or "mixed" (per-request temperatures, 0 = greedy)
    target_sigma: float
    spike: float  # added to one random vocabulary entry per target row; 0 = none
    draft_sigma: Sequence[float]  # per draft slot, length K
    identical_even: bool = False  # even requests: draft rows = target rows bitwise
    ragged: bool = False  # k_b ~ U{1..K}; rows past k_b are NaN-filled
    seed: int = 0
    temperatures: Sequence[float] = ()  # mixed mode: request b has temperatures[b % len]

    @property
    def rows_per_request(self) -> int:
        return 2 * self.K + 1 if self.mode == "sample" else self.K + 1

    def temperature_of(self, b: int) -> float:
        """Temperature of request b: 0 for a greedy request."""
        if self.mode == "mixed":
            return float(self.temperatures[b % len(self.temperatures)])
        return 0.0 if self.mode == "greedy" else float(self.temperature)

    def replace(self, **kw) -> "Workload":
        if "K" in kw and "draft_sigma" not in kw:
            s = self.draft_sigma
            if len(set(s)) == 1:
                kw["draft_sigma"] = (s[0],) * kw["K"]
            else:  # keep the linear ramp shape from first to last slot
                k = kw["K"]
                kw["draft_sigma"] = tuple(
                    s[0] + (s[-1] - s[0]) * (i / (k - 1) if k > 1 else 0.0) for i in range(k)
                )
        return dataclasses.replace(self, **kw)


def _ramp(lo: float, hi: float, k: int) -> tuple:
    return tuple(lo + (hi - lo) * i / (k - 1) for i in range(k)) if k > 1 else (lo,)


# The five workloads: tiny correctness case, interactive, batched (the throughput headline),
# heavy ragged load, and greedy mode.
TINY = Workload("tiny_sample_B1_K4_V1000_f32", 1, 4, 1000, "f32", 1.0, "sample",
                2.0, 0.0, (0.5,) * 4, seed=1001)
INTERACTIVE = Workload("interactive_sample_B1_K8_V151936_f32", 1, 8, QWEN3_VOCAB, "f32", 1.0,
                       "sample", 3.0, 12.0, (1.0,) * 8, seed=1002)
BATCHED = Workload("batched_sample_B64_K8_V151936_bf16_t0.7", 64, 8, QWEN3_VOCAB, "bf16", 0.7,
                   "sample", 3.0, 12.0, (1.5,) * 8, identical_even=True, seed=1003)
HEAVY = Workload("heavy_ragged_sample_B256_K16_V151936_bf16", 256, 16, QWEN3_VOCAB, "bf16",
                 1.0, "sample", 3.0, 12.0, _ramp(0.5, 3.0, 16), ragged=True, seed=1004)
GREEDY = Workload("greedy_B512_K8_V151936_f32", 512, 8, QWEN3_VOCAB, "f32", 1.0, "greedy",
                  3.0, 12.0, (1.0,) * 8, seed=1005)

# Heavy ragged load with greedy and sampling requests mixed, verified from flattened rows.
MIXED = Workload("mixed_flat_B256_K16_V151936_bf16", 256, 16, QWEN3_VOCAB, "bf16", 1.0, "mixed",
                 3.0, 12.0, _ramp(0.5, 3.0, 16), ragged=True, seed=1006,
                 temperatures=(0.0, 0.7, 1.0, 1.3))

WORKLOADS = {w.name: w for w in (TINY, INTERACTIVE, BATCHED, HEAVY, GREEDY, MIXED)}
BY_NUMBER = {1: TINY, 2: INTERACTIVE, 3: BATCHED, 4: HEAVY, 5: GREEDY}


def sweep_workload(K: int, B: int, dtype: str, mode: str = "sample") -> Workload:
    """K x B sweep point: batched-workload distributions, temperature 1."""
    return BATCHED.replace(name=f"sweep_{mode}_B{B}_K{K}_V{QWEN3_VOCAB}_{dtype}", K=K, B=B,
                           dtype=dtype, temperature=1.0, mode=mode,
                           draft_sigma=(1.5,) * K, seed=2000 + 100 * K + B)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only (the generator never rounds a NaN or an infinity)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload.

    target: [B, K+1, V] float32 or uint16 (bf16 bits); draft: [B, K, V] same type, or None for
    greedy workloads (draft logits are only used on the host to choose the proposals).
    tokens [B, K] int32; uniforms [B, K] float32; residual [B] float32;
    num_draft [B] int32 (None when every request verifies all K drafts).
    Masked slots (s >= k_b) hold token -1, uniform NaN and NaN logit rows.
    """

    workload: Workload
    target: np.ndarray
    draft: Optional[np.ndarray]
    tokens: np.ndarray
    uniforms: np.ndarray
    residual: np.ndarray
    num_draft: Optional[np.ndarray]
    temperatures: Optional[np.ndarray] = None  # [B] float32, mixed workloads

    @property
    def B(self):
        return self.workload.B

    @property
    def K(self):
        return self.workload.K

    @property
    def V(self):
        return self.workload.V

    def k_of(self, b: int) -> int:
        return self.workload.K if self.num_draft is None else int(self.num_draft[b])


def _stored(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == "bf16" else x32


def _as_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    return (bf16_bits_to_f32(stored) if dtype == "bf16" else stored).astype(np.float64)


def _gen_request(w: Workload, b: int, out: Inputs) -> None:
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b]))
    K, V = w.K, w.V
    t32 = rng.standard_normal((K + 1, V), dtype=np.float32)
    t32 *= np.float32(w.target_sigma)
    if w.spike != 0.0:
        idx = rng.integers(0, V, size=K + 1)
        t32[np.arange(K + 1), idx] += np.float32(w.spike)
    noise = rng.standard_normal((K, V), dtype=np.float32)
    noise *= np.asarray(w.draft_sigma, dtype=np.float32)[:, None]
    t_st = _stored(t32, w.dtype)
    if w.identical_even and b % 2 == 0:
        d_st = t_st[:K].copy()
    else:
        d_st = _stored(t32[:K] + noise, w.dtype)
    d64 = _as_f64(d_st, w.dtype)
    tau = w.temperature_of(b)
    if tau > 0.0:
        e = rng.standard_exponential((K, V))  # float64: never exactly 0
        keys = d64 / tau - np.log(e)
        x = np.argmax(keys, axis=1).astype(np.int32)
    else:
        x = np.argmax(d64, axis=1).astype(np.int32)
    u = rng.random(K, dtype=np.float32)
    r = rng.random(1, dtype=np.float32)[0]
    k = int(rng.integers(1, K + 1)) if w.ragged else K
    if k < K:
        nan = BF16_NAN if w.dtype == "bf16" else np.float32(np.nan)
        t_st[k + 1:] = nan
        d_st[k:] = nan
        x[k:] = -1
        u[k:] = np.nan
    out.target[b] = t_st
    if out.draft is not None:
        out.draft[b] = d_st
    out.tokens[b] = x
    out.uniforms[b] = u
    out.residual[b] = r
    if out.num_draft is not None:
        out.num_draft[b] = k
    if out.temperatures is not None:
        out.temperatures[b] = tau


def generate(w: Workload, threads: Optional[int] = None) -> Inputs:
    """Generate all B requests of workload `w` (requests are independent; threads share work)."""
    st = np.uint16 if w.dtype == "bf16" else np.float32
    out = Inputs(
        workload=w,
        target=np.empty((w.B, w.K + 1, w.V), dtype=st),
        draft=np.empty((w.B, w.K, w.V), dtype=st) if w.mode != "greedy" else None,
        tokens=np.empty((w.B, w.K), dtype=np.int32),
        uniforms=np.empty((w.B, w.K), dtype=np.float32),
        residual=np.empty((w.B,), dtype=np.float32),
        num_draft=np.empty((w.B,), dtype=np.int32) if w.ragged else None,
        temperatures=np.empty((w.B,), dtype=np.float32) if w.mode == "mixed" else None,
    )
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or w.B == 1:
        for b in range(w.B):
            _gen_request(w, b, out)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda b: _gen_request(w, b, out), range(w.B)))
    return out


@dataclasses.dataclass
class FlatInputs:
    """A workload with its logit rows packed: request b's k_b+1 target rows start at
    target_row_start[b] of target [rows_t, V], and, for a sampling request, its k_b draft rows at
    draft_row_start[b] of draft [rows_d, V] (None when no request samples). Greedy requests have
    temperature 0 and no draft rows. Small per-request arrays stay [B, K] / [B]."""

    workload: Workload
    target: np.ndarray
    draft: Optional[np.ndarray]
    target_row_start: np.ndarray
    draft_row_start: np.ndarray
    num_draft: np.ndarray
    temperatures: np.ndarray
    tokens: np.ndarray
    uniforms: np.ndarray
    residual: np.ndarray


def flatten(inp: Inputs, order: Optional[Sequence[int]] = None) -> FlatInputs:
    """Pack the rows each request uses, requests in `order` (default: ascending)."""
    w = inp.workload
    B = w.B
    order = list(range(B)) if order is None else list(order)
    ks = np.array([inp.k_of(b) for b in range(B)], dtype=np.int32)
    taus = (inp.temperatures.astype(np.float32) if inp.temperatures is not None else
            np.array([w.temperature_of(b) for b in range(B)], dtype=np.float32))
    ts = np.zeros(B, np.int32)
    ds = np.zeros(B, np.int32)
    nt = nd = 0
    for b in order:
        ts[b], nt = nt, nt + ks[b] + 1
        ds[b] = nd
        if taus[b] > 0:
            nd += ks[b]
    target = np.empty((nt, w.V), dtype=inp.target.dtype)
    draft = np.empty((nd, w.V), dtype=inp.target.dtype) if nd > 0 else None
    for b in order:
        target[ts[b]:ts[b] + ks[b] + 1] = inp.target[b, :ks[b] + 1]
        if taus[b] > 0 and ks[b] > 0:
            draft[ds[b]:ds[b] + ks[b]] = inp.draft[b, :ks[b]]
    return FlatInputs(w, target, draft, ts, ds, ks, taus, inp.tokens, inp.uniforms,
                      inp.residual)


def schedule_confidences(B: int, K: int, seed: int = 1007) -> np.ndarray:
    """Synthetic per-position draft confidences [B, K] float32 for the prefix scheduler: request
    b draws from default_rng(SeedSequence([seed, b])) one difficulty level and then a Beta
    sample per position around it, falling with the position (the pages' per-position
    acceptance of about 0.9 at the first draft that later positions lower), with occasional
    exact 1s (confident runs)."""
    out = np.empty((B, K), dtype=np.float32)
    for b in range(B):
        rng = np.random.default_rng(np.random.SeedSequence([seed, b]))
        level = rng.uniform(0.55, 0.97)
        mean = np.clip(level - 0.02 * np.arange(K), 0.05, 0.99)
        c = rng.beta(20.0 * mean, 20.0 * (1.0 - mean)).astype(np.float32)
        c[rng.random(K) < 0.03] = 1.0
        out[b] = c
    return out


def markov_factors(V: int, R: int, seed: int = 1008, sigma: float = 0.25):
    """Synthetic low-rank Markov-head factors [V, R] as bf16 bits (left: row = previous token,
    right: row = candidate token), N(0, sigma^2) entries: with R = 256 and sigma = 0.25 the
    bias sum_j L[p, j] * Rf[v, j] has a standard deviation of about 1, the scale of the base
    logits' noise. The trained factors are not available; these stand in for them."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, V, R]))
    left = to_bf16_bits(rng.normal(0.0, sigma, size=(V, R)).astype(np.float32))
    right = to_bf16_bits(rng.normal(0.0, sigma, size=(V, R)).astype(np.float32))
    return left, right


def markov_base(B: int, K: int, V: int, dtype: str = "bf16", seed: int = 1009,
                lead: float = 6.0) -> np.ndarray:
    """Synthetic base logits [B, K, V] of a parallel drafter, stored as `dtype` (bf16 bits or
    float32): N(0, 2^2) noise plus one favoured token per position at +lead. lead = 6 gives a
    clear leader that the Markov bias (standard deviation about 1 with markov_factors) overturns
    now and then; lead = 14 a draft distribution as a sampling drafter meets it, the favoured
    token holding about half the mass at the Qwen3 vocabulary (most at smaller ones) and the rest
    spread over the tail."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, B, K, V]))
    z = rng.normal(0.0, 2.0, size=(B, K, V)).astype(np.float32)
    top = rng.integers(0, V, size=(B, K))
    np.put_along_axis(z, top[..., None], np.take_along_axis(z, top[..., None], 2) + lead, 2)
    return _stored(z, dtype)


def markov_sampling(B: int, K: int, seed: int = 1010, greedy_share: float = 0.0,
                    temperatures=(1.0,)):
    """Per-request temperatures [B] float32 and per-position uniforms [B, K] float32 in [0, 1)
    for the sampled Markov head: each request takes one of `temperatures` (1.0 is the pages'
    evaluation setting), and a `greedy_share` of the requests temperature 0 (greedy)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, B, K]))
    tau = rng.choice(np.asarray(temperatures, dtype=np.float32), size=B).astype(np.float32)
    tau[rng.random(B) < greedy_share] = 0.0
    u = rng.random((B, K), dtype=np.float32)
    return tau, u

"""Plain, slow fp64 CPU oracle for batched lossless draft verification.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg import this module. The GPU library never calls it, and it shares no code with the GPU path.

What it computes, per request (the acceptance rule of "From draft-then-verify to DSpark",
section "How speculative decoding works"):
  * the target distribution p_i at each of the k+1 scored slots and the draft distribution q_i
    at each of the k draft slots are softmaxes of the stored logits over the full vocabulary
    ("Bringing DSpark to vLLM Metal", "Making the draft cheaper": the target verifies against
    its full vocabulary), after dividing the logits by one temperature tau;
  * draft token x_i is kept with probability min(1, p_i(x_i) / q_i(x_i));
  * the verifier keeps the longest run of kept drafts (the Commit row of the
    propose-verify-commit table in "Accelerating Large-Model Inference: Engineering Practice from
    Hidden-State Extraction to DSpark Speculative Decoding", section 1);
  * at the first rejected slot it draws a replacement from max(0, p - q) renormalised;
  * when every draft is kept it draws one more token from the target row after the last draft,
    the "+1" counted in the acceptance length (same article, section 1 causal chain and
    section 4).
Greedy mode ("Bringing DSpark to vLLM Metal": greedy-only serving whose output ids must equal
target-only greedy decoding) keeps drafts while they equal the target row's argmax and then
commits the target's argmax.

Readings taken where the pages leave a step open:
  * a uniform u in [0, 1) accepts iff u < t (strict), so P(accept) = t and p == q always accepts;
  * t = min(1, a / c) with a = p(x), c = q(x); c == 0 < a gives t = 1; a == c == 0 gives t = 0
    (a token with no draft mass is treated as not proposed: rejected);
  * a draft token outside [0, V) has p(x) = q(x) = 0, hence is rejected;
  * one residual uniform r per request drives either the residual draw or the bonus draw;
  * the uniform-to-token map is the inverse CDF in ascending vocabulary order: y is the smallest
    v with C_v > r * Z, C_v = sum_{j <= v} w_j, Z = C_{V-1}; if no such v exists (rounding),
    y is the largest v with w_v > 0; if Z == 0 (rounding only), w falls back to p at that slot;
  * per-request draft counts k_b in [0, K]: only slots < k_b are verified, the bonus comes from
    target row k_b, rows past k_b are never read, masked outputs are -1 / 0;
  * greedy argmax ties go to the lowest vocabulary index, compared on the stored values;
  * a flattened batch packs each request's used rows (k_b+1 target, k_b draft) at a start index
    of its own; a request with temperature 0 in a mixed batch is a greedy request and any other
    request samples at its own temperature; a request whose rows fall outside the flat arrays,
    whose k_b is outside [0, K] or whose temperature is negative, not finite or below TAU_MIN is
    reported invalid (RAGGED_INVALID) without reading anything;
  * bf16 logits are decoded exactly from their bit patterns; all arithmetic is fp64.

The parity harness also needs to know which requests are too close to a decision threshold for
a float32 kernel to be expected to agree: margins are reported for every decided slot and for the
final draw, and a request is ambiguous when any margin is below AMBIGUOUS_MARGIN.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

AMBIGUOUS_MARGIN = 1e-6


# ---------------------------------------------------------------------------------------------
# Stored logits -> fp64


def decode_logits(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> exact float64 values.

    dtype "f32": float32 values widen exactly. dtype "bf16": each uint16 holds the upper half of
    an IEEE float32 (sign, 8 exponent bits, 7 mantissa bits); shifting it into the top of a
    32-bit word gives that float32 exactly.
    """
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        words = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return words.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------------------------
# The steps of the acceptance rule ("From draft-then-verify to DSpark", "How speculative
# decoding works").


def softmax_fp64(logits: np.ndarray, tau: float) -> np.ndarray:
    """Full-vocabulary distribution softmax(logits / tau) in fp64.

    -inf logits get probability 0. The subtraction of the maximum only avoids overflow; the
    sum uses numpy's pairwise summation.
    """
    z = np.asarray(logits, dtype=np.float64) / float(tau)
    m = np.max(z)
    e = np.exp(z - m)
    return e / np.sum(e)


def accept_threshold(a: float, c: float) -> float:
    """t = min(1, a / c): the probability of keeping a draft with target mass a, draft mass c."""
    if c > 0.0:
        return min(1.0, a / c)
    return 1.0 if a > 0.0 else 0.0


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p - q) at the first rejected slot."""
    return np.maximum(0.0, p - q)


def inverse_cdf(w: np.ndarray, r: float):
    """Draw from w / sum(w) with the uniform r by inverse CDF in ascending index order.

    Returns (y, margin): y = min{v : C_v > r * Z}, and margin = distance of r * Z to the nearer
    end of y's CDF interval, divided by Z (how far r is from drawing a neighbouring token).
    """
    c = np.cumsum(w)
    z = float(c[-1])
    target = float(r) * z
    above = np.nonzero(c > target)[0]
    if above.size:
        y = int(above[0])
    else:  # only through rounding: the last token that has mass
        y = int(np.nonzero(w > 0.0)[0][-1])
    lo = float(c[y - 1]) if y > 0 else 0.0
    hi = float(c[y])
    margin = min(abs(target - lo), abs(target - hi)) / z if z > 0.0 else 0.0
    return y, margin


@dataclasses.dataclass
class RequestResult:
    n: int  # accepted drafts (0..k)
    committed: List[int]  # length K+1: x_0..x_{n-1}, y, then -1
    target_prob: List[float]  # length K: p_i(x_i) for i < k, else 0
    draft_prob: List[float]  # length K: q_i(x_i) for i < k, else 0
    thresholds: List[float]  # t_i for i < k
    slot_margins: List[float]  # |u_i - t_i| for every decided slot
    sample_margin: float  # margin of the final draw
    residual_mass: float  # Z of the final draw (1 for a bonus draw)
    bonus: bool  # True when every draft was kept

    @property
    def min_margin(self) -> float:
        return min(self.slot_margins + [self.sample_margin])

    @property
    def ambiguous(self) -> bool:
        return self.min_margin < AMBIGUOUS_MARGIN


def verify_request(target_rows: np.ndarray, draft_rows: np.ndarray, dtype: str,
                   tokens: np.ndarray, uniforms: np.ndarray, r: float, tau: float,
                   k: int, K: Optional[int] = None) -> RequestResult:
    """Sampling-mode verification of one request.

    target_rows: stored logits [>= k+1, V]; draft_rows: [>= k, V]; tokens, uniforms: [>= k].
    Only target rows 0..k and draft rows 0..k-1 are read. K (default: len(tokens)) sets the
    length of the padded outputs.
    """
    K = len(tokens) if K is None else K
    if not 0 <= k <= K:
        raise ValueError("k outside [0, K]")
    V = target_rows.shape[-1]
    p_rows = [softmax_fp64(decode_logits(target_rows[i], dtype), tau) for i in range(k + 1)]
    q_rows = [softmax_fp64(decode_logits(draft_rows[i], dtype), tau) for i in range(k)]

    target_prob = [0.0] * K
    draft_prob = [0.0] * K
    thresholds = []
    slot_margins = []
    n = k
    for i in range(k):
        x = int(tokens[i])
        a = float(p_rows[i][x]) if 0 <= x < V else 0.0
        c = float(q_rows[i][x]) if 0 <= x < V else 0.0
        target_prob[i], draft_prob[i] = a, c
        t = accept_threshold(a, c)
        thresholds.append(t)
    for i in range(k):
        u = float(uniforms[i])
        slot_margins.append(abs(u - thresholds[i]))
        if not u < thresholds[i]:
            n = i
            break

    if n < k:
        w = residual_weights(p_rows[n], q_rows[n])
        if not np.sum(w) > 0.0:
            w = p_rows[n]
    else:
        w = p_rows[k]
    y, sample_margin = inverse_cdf(w, r)
    committed = [int(tokens[i]) for i in range(n)] + [y] + [-1] * (K - n)
    return RequestResult(n=n, committed=committed, target_prob=target_prob,
                         draft_prob=draft_prob, thresholds=thresholds,
                         slot_margins=slot_margins, sample_margin=sample_margin,
                         residual_mass=float(np.sum(w)), bonus=(n == k))


def argmax_lowest(values: np.ndarray) -> int:
    """Index of the largest value; the lowest index among equal maxima."""
    best = int(np.argmax(values))  # numpy returns the first occurrence
    return best


def verify_greedy_request(target_rows: np.ndarray, dtype: str, tokens: np.ndarray, k: int,
                          K: Optional[int] = None):
    """Greedy-mode verification of one request: returns (n, committed[K+1])."""
    K = len(tokens) if K is None else K
    if not 0 <= k <= K:
        raise ValueError("k outside [0, K]")
    g = [argmax_lowest(decode_logits(target_rows[i], dtype)) for i in range(k + 1)]
    n = k
    for i in range(k):
        if int(tokens[i]) != g[i]:
            n = i
            break
    committed = [int(tokens[i]) for i in range(n)] + [g[n]] + [-1] * (K - n)
    return n, committed


# ---------------------------------------------------------------------------------------------
# Batch drivers over the host arrays of a workload (plain loops over requests).


@dataclasses.dataclass
class BatchResult:
    accepted_len: np.ndarray  # [B] int32
    committed: np.ndarray  # [B, K+1] int32
    target_prob: np.ndarray  # [B, K] float64
    draft_prob: Optional[np.ndarray]  # [B, K] float64 (sampling mode)
    requests: list  # per-request RequestResult (sampling) or None (greedy)

    @property
    def ambiguous(self) -> np.ndarray:
        return np.array([r is not None and r.ambiguous for r in self.requests], dtype=bool)


def _k_of(num_draft, b: int, K: int) -> int:
    return K if num_draft is None else int(num_draft[b])


def verify_batch(target: np.ndarray, draft: np.ndarray, dtype: str, tokens: np.ndarray,
                 uniforms: np.ndarray, residual: np.ndarray, tau: float,
                 num_draft: Optional[np.ndarray] = None,
                 requests: Optional[list] = None) -> BatchResult:
    """Sampling-mode verification of a batch ([B, K+1, V] target, [B, K, V] draft).

    `requests` restricts the work to a subset of request indices (rows of the outputs for other
    requests are left at -1 / 0).
    """
    B, K = tokens.shape
    idx = range(B) if requests is None else requests
    acc = np.full(B, -1, dtype=np.int32)
    com = np.full((B, K + 1), -1, dtype=np.int32)
    tp = np.zeros((B, K))
    dp = np.zeros((B, K))
    res = [None] * B
    for b in idx:
        k = _k_of(num_draft, b, K)
        rr = verify_request(target[b], draft[b], dtype, tokens[b], uniforms[b],
                            float(residual[b]), tau, k, K)
        acc[b], com[b], tp[b], dp[b], res[b] = rr.n, rr.committed, rr.target_prob, \
            rr.draft_prob, rr
    return BatchResult(acc, com, tp, dp, res)


def verify_greedy(target: np.ndarray, dtype: str, tokens: np.ndarray,
                  num_draft: Optional[np.ndarray] = None,
                  requests: Optional[list] = None) -> BatchResult:
    """Greedy-mode verification of a batch ([B, K+1, V] target logits)."""
    B, K = tokens.shape
    idx = range(B) if requests is None else requests
    acc = np.full(B, -1, dtype=np.int32)
    com = np.full((B, K + 1), -1, dtype=np.int32)
    for b in idx:
        k = _k_of(num_draft, b, K)
        n, c = verify_greedy_request(target[b], dtype, tokens[b], k, K)
        acc[b], com[b] = n, c
    return BatchResult(acc, com, np.zeros((B, K)), None, [None] * B)


# ---------------------------------------------------------------------------------------------
# Flattened, mixed batches: the per-request verify lengths of one batch packed without padding,
# each request's rows found through its start index ("flatten every token and track its request
# ID", the DSpark paper review, 4.2.2), and greedy and sampling requests in one batch (the vLLM
# Metal article's greedy-only path, with sampled verification listed as still in flight).

RAGGED_INVALID = -3  # accepted_len of a request whose rows, k_b or temperature are invalid
# Smallest positive temperature a sampling request may have: the scale log2(e) / tau of the
# logits must not exceed 2^21.
TAU_MIN = 1.4426950408889634 / 2.0 ** 21


def ragged_request_valid(k: int, K: int, tau: float, ts: int, ds: int, n_target_rows: int,
                         n_draft_rows: int) -> bool:
    """A request of a flattened batch is valid when 0 <= k <= K, its temperature is 0 (greedy)
    or in [TAU_MIN, inf), its k+1 target rows lie inside the flat target array and, when it
    samples and k > 0, its k draft rows lie inside the flat draft array."""
    if not 0 <= k <= K:
        return False
    if not (tau == 0.0 or (TAU_MIN <= tau < float("inf"))):
        return False
    if ts < 0 or ts + k + 1 > n_target_rows:
        return False
    if tau != 0.0 and k > 0 and (ds < 0 or ds + k > n_draft_rows):
        return False
    return True


def verify_ragged(target_flat: np.ndarray, draft_flat: Optional[np.ndarray], dtype: str,
                  tokens: np.ndarray, uniforms: np.ndarray, residual: np.ndarray,
                  temperatures: np.ndarray, num_draft: np.ndarray, target_row_start: np.ndarray,
                  draft_row_start: np.ndarray, requests: Optional[list] = None) -> BatchResult:
    """Verification of a flattened, mixed batch.

    target_flat [rows_t, V] and draft_flat [rows_d, V] hold the stored logit rows of all
    requests; request b's target rows are target_flat[target_row_start[b] + i] for i = 0..k_b and
    its draft rows draft_flat[draft_row_start[b] + i] for i < k_b. tokens and uniforms are
    [B, K] (entries past k_b unused), residual [B]. temperatures[b] == 0 makes request b a
    greedy request (its draft rows, uniforms and residual are not used; its probabilities are
    reported as 0); otherwise it is a sampling request at temperature temperatures[b]. Each
    request is then exactly verify_greedy_request or verify_request on its own rows. An invalid
    request (see ragged_request_valid) gets accepted_len RAGGED_INVALID, committed all -1 and
    probabilities 0, and none of its rows is read.
    """
    B, K = tokens.shape
    rows_t = target_flat.shape[0]
    rows_d = 0 if draft_flat is None else draft_flat.shape[0]
    idx = range(B) if requests is None else requests
    acc = np.full(B, -1, dtype=np.int32)
    com = np.full((B, K + 1), -1, dtype=np.int32)
    tp = np.zeros((B, K))
    dp = np.zeros((B, K))
    res = [None] * B
    for b in idx:
        k = int(num_draft[b])
        tau = float(temperatures[b])
        ts, ds = int(target_row_start[b]), int(draft_row_start[b])
        if not ragged_request_valid(k, K, tau, ts, ds, rows_t, rows_d):
            acc[b] = RAGGED_INVALID
            continue
        t_rows = target_flat[ts:ts + k + 1]
        if tau == 0.0:
            acc[b], com[b] = verify_greedy_request(t_rows, dtype, tokens[b], k, K)
            continue
        d_rows = draft_flat[ds:ds + k] if k > 0 else target_flat[ts:ts]
        rr = verify_request(t_rows, d_rows, dtype, tokens[b], uniforms[b], float(residual[b]),
                            tau, k, K)
        acc[b], com[b], tp[b], dp[b], res[b] = rr.n, rr.committed, rr.target_prob, \
            rr.draft_prob, rr
    return BatchResult(acc, com, tp, dp, res)

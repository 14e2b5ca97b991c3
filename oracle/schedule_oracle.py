"""Plain CPU oracle for confidence-scheduled prefix selection.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg import this module; the GPU library never calls it and shares no code with it.

What it computes (the DSpark paper review, 4.2.1 "Confidence Head" and 4.2.2 "Hardware-Aware
Prefix Scheduler"; the prefix-scheduler row of the DSpark table in "Accelerating Large-Model
Inference ...", section 1):
  * every draft token k of request b has a confidence c[b, k], the chance that it is accepted
    when every token before it was; its prefix survival is s[b, k] = c[b, 0] * ... * c[b, k],
    which never increases along the block;
  * threshold scheduler: a request keeps its drafts up to the first one whose confidence is
    below the threshold (that token and everything after it are cut);
  * hardware-aware scheduler: all draft tokens of all requests are ranked by survival and taken
    one at a time; taking the first N gives an expected B + sum of their survivals accepted
    tokens per target step (every request also commits the target's own token) for a step that
    verifies B + N tokens, whose time comes from a table measured beforehand; the whole table
    is searched (step times rise in jumps, so the first drop need not be the peak) and the N
    with the largest expected tokens per unit time is kept. Because survival never increases
    along a block, the first N ranked tokens of a request always form a prefix.

Readings taken where the pages leave a step open:
  * confidences are clamped to [0, 1], NaN counts as 0;
  * survivals are products in float32, left to right (the GPU path forms the same products,
    and the ranking is a decision taken on them);
  * ranking ties (equal survivals) go to the earlier position, then to the lower request index;
  * the expected token sums are fp64 running sums in ranked order;
  * among equal throughputs the smallest N wins;
  * step_time[n] is the time of a target step that verifies n tokens, for n = 0 .. T-1; a step
    time that is not finite or not positive makes that N unusable.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def clamp_confidence(c) -> np.ndarray:
    """float32 confidences clamped to [0, 1]; NaN becomes 0."""
    c = np.asarray(c, dtype=np.float32)
    c = np.where(np.isnan(c), np.float32(0.0), c)
    return np.clip(c, np.float32(0.0), np.float32(1.0)).astype(np.float32)


def prefix_survival(confidence) -> np.ndarray:
    """s[b, k] = c[b, 0] * ... * c[b, k], float32 products taken left to right."""
    c = clamp_confidence(confidence)
    B, K = c.shape
    s = np.empty((B, K), dtype=np.float32)
    for b in range(B):
        acc = np.float32(1.0)
        for k in range(K):
            acc = np.float32(acc * c[b, k])
            s[b, k] = acc
    return s


def schedule_threshold(confidence, threshold: float) -> np.ndarray:
    """num_draft[b]: drafts kept up to the first confidence below the threshold."""
    c = clamp_confidence(confidence)
    B, K = c.shape
    out = np.full(B, K, dtype=np.int32)
    for b in range(B):
        for k in range(K):
            if c[b, k] < np.float32(threshold):
                out[b] = k
                break
    return out


def rank_tokens(survival: np.ndarray) -> List[Tuple[int, int]]:
    """(b, k) of every draft token, highest survival first; ties: earlier k, then lower b."""
    B, K = survival.shape
    items = [(-float(survival[b, k]), k, b) for b in range(B) for k in range(K)]
    items.sort()
    return [(b, k) for _, k, b in items]


def schedule_hardware_aware(confidence, step_time):
    """num_draft[b], the chosen number of draft tokens N, and the expected accepted tokens per
    unit time at that N (see the module docstring)."""
    s = prefix_survival(confidence)
    B, K = s.shape
    t = np.asarray(step_time, dtype=np.float64)
    if t.shape[0] < B + B * K + 1:
        raise ValueError("the step-time table must cover B + B*K verified tokens")
    order = rank_tokens(s)
    best_n, best_rate = -1, -np.inf
    expected = float(B)  # every request commits the target's own token
    for n in range(0, B * K + 1):
        if n > 0:
            b, k = order[n - 1]
            expected += float(s[b, k])
        tn = t[B + n]
        if np.isfinite(tn) and tn > 0:
            rate = expected / tn
            if rate > best_rate:
                best_n, best_rate = n, rate
    num = np.zeros(B, dtype=np.int32)
    if best_n < 0:  # no usable step time: verify no drafts
        return num, 0, 0.0
    for b, k in order[:best_n]:
        num[b] += 1
    return num, best_n, best_rate


def row_starts(num_draft) -> Tuple[np.ndarray, np.ndarray]:
    """Flattened row starts for a verify call: request b's k_b + 1 target rows and k_b draft
    rows follow those of requests 0 .. b-1."""
    k = np.asarray(num_draft, dtype=np.int64)
    ts = np.concatenate([[0], np.cumsum(k + 1)[:-1]]).astype(np.int32)
    ds = np.concatenate([[0], np.cumsum(k)[:-1]]).astype(np.int32)
    return ts, ds

"""Plain CPU oracle for the Markov-head correction of a parallel draft block.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg import this module; the GPU library never calls it and shares no code with it.

What it computes ("Accelerating Large-Model Inference ...", section 3, DSpark drafting engine
table row 2 and the Markov Head paragraph; the DSpark paper review, 4.1 Semi-autoregressive
generation): a parallel backbone has produced base logits U_k for every draft position k of a
block; a low-rank head then walks the block left to right, adding to position k's logits a bias
set by the token already chosen at position k-1, and chooses position k's token from the
corrected logits. The head is a token-to-token affinity matrix kept as two factors of rank R
(default 256): bias_k[v] = sum_j L[prev, j] * Rf[v, j], prev = the token chosen at k-1.

Top-K variant ("Bringing DSpark to vLLM Metal", Making the draft cheaper): the candidates of a
position are chosen from its base logits first, and the sequential correction is applied to those
rows only; the token is the best corrected candidate. With kc = V it is the full head.

Readings taken where the pages leave a step open:
  * position 0 is corrected by the anchor token (the last committed token the block continues);
    anchor -1 (or any value outside [0, V)) means no bias at position 0; a chosen token is always
    inside [0, V);
  * the token chosen at each position is the argmax of the corrected logits (lowest index on
    ties): the drafter's proposal rule here, so proposals are deterministic;
  * the corrected logits of every position are the block's draft logits (the q rows the verifier
    reads);
  * top-K candidates: the kc largest stored base logits of the position (NaN below every number,
    -inf included; ties to the lower index), kept in ascending vocabulary order; the token is
    the candidate with the largest corrected logit, the lowest vocabulary index on ties; the
    corrected logits of the candidates are the block's draft output;
  * factors are bf16; logits fp32 or bf16; all arithmetic fp64. A position is ambiguous when its
    two largest corrected logits are closer than AMBIGUOUS_GAP (a float32 kernel's sum of R
    products may then order them the other way).
"""
from __future__ import annotations

import numpy as np

from .sv_oracle import argmax_lowest, decode_logits

AMBIGUOUS_GAP = 1e-4


def bf16_factor(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [V, R] -> fp64 values."""
    return decode_logits(np.asarray(bits, dtype=np.uint16), "bf16")


def markov_draft_request(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray,
                         anchor: int):
    """One request: base [K, V] stored logits; left, right [V, R] bf16 bits.

    Returns (tokens [K], corrected logits [K, V] fp64, top-2 gaps [K])."""
    K, V = base.shape
    L = bf16_factor(left)
    Rf = bf16_factor(right)
    tokens = np.zeros(K, dtype=np.int32)
    corrected = np.zeros((K, V))
    gaps = np.zeros(K)
    prev = int(anchor)
    for k in range(K):
        z = decode_logits(base[k], dtype).copy()
        if 0 <= prev < V:
            z = z + Rf @ L[prev]
        corrected[k] = z
        y = argmax_lowest(z)
        tokens[k] = y
        rest = np.delete(z, y)
        gaps[k] = z[y] - (np.max(rest) if rest.size else -np.inf)
        prev = y
    return tokens, corrected, gaps


def markov_draft(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray,
                 anchors=None):
    """Batch [B, K, V]: tokens [B, K], corrected logits [B, K, V] fp64, ambiguous [B] bool."""
    B, K, V = base.shape
    tokens = np.zeros((B, K), dtype=np.int32)
    corrected = np.zeros((B, K, V))
    amb = np.zeros(B, dtype=bool)
    for b in range(B):
        a = -1 if anchors is None else int(anchors[b])
        t, c, g = markov_draft_request(base[b], dtype, left, right, a)
        tokens[b], corrected[b] = t, c
        amb[b] = bool(np.any(g < AMBIGUOUS_GAP))
    return tokens, corrected, amb


def topk_candidates(z: np.ndarray, kc: int) -> np.ndarray:
    """Indices of the kc largest entries of a base-logit row (NaN below every number, ties to the
    lower index), in ascending vocabulary order."""
    z = np.asarray(z, dtype=np.float64)
    if not 1 <= kc <= z.shape[0]:
        raise ValueError("kc outside [1, V]")
    nan = np.isnan(z)
    # lexsort orders by its last key first: numbers before NaN, larger values first, then index
    order = np.lexsort((np.arange(z.shape[0]), -np.where(nan, 0.0, z), nan))
    return np.sort(order[:kc])


def markov_topk_request(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray,
                        anchor: int, kc: int):
    """Top-K Markov drafting of one request: base [K, V] stored logits; left, right [V, R] bf16
    bits. Per position the candidates are the kc largest base logits, the bias is added to those
    rows only, and the token is the best corrected candidate.

    Returns (tokens [K], candidates [K, kc], corrected logits of the candidates [K, kc] fp64,
    top-2 gaps among the candidates [K])."""
    K, V = base.shape
    L = bf16_factor(left)
    Rf = bf16_factor(right)
    tokens = np.zeros(K, dtype=np.int32)
    cands = np.zeros((K, kc), dtype=np.int64)
    corrected = np.zeros((K, kc))
    gaps = np.zeros(K)
    prev = int(anchor)
    for k in range(K):
        z = decode_logits(base[k], dtype)
        cand = topk_candidates(z, kc)
        zc = z[cand].copy()
        if 0 <= prev < V:
            zc = zc + Rf[cand] @ L[prev]
        j = argmax_lowest(zc)  # candidates ascend, so the lowest position is the lowest index
        cands[k], corrected[k] = cand, zc
        tokens[k] = int(cand[j])
        rest = np.delete(zc, j)
        gaps[k] = zc[j] - (np.max(rest) if rest.size else -np.inf)
        prev = int(cand[j])
    return tokens, cands, corrected, gaps


def markov_topk(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray, kc: int,
                anchors=None):
    """Batch [B, K, V]: tokens [B, K], candidates [B, K, kc], corrected [B, K, kc] fp64,
    ambiguous [B] bool."""
    B, K, V = base.shape
    tokens = np.zeros((B, K), dtype=np.int32)
    cands = np.zeros((B, K, kc), dtype=np.int64)
    corrected = np.zeros((B, K, kc))
    amb = np.zeros(B, dtype=bool)
    for b in range(B):
        a = -1 if anchors is None else int(anchors[b])
        t, c, z, g = markov_topk_request(base[b], dtype, left, right, a, kc)
        tokens[b], cands[b], corrected[b] = t, c, z
        amb[b] = bool(np.any(g < AMBIGUOUS_GAP))
    return tokens, cands, corrected, amb

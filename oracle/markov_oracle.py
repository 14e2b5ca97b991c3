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

Readings taken where the pages leave a step open:
  * position 0 is corrected by the anchor token (the last committed token the block continues);
    anchor -1 (or any value outside [0, V)) means no bias at position 0; a chosen token is always
    inside [0, V);
  * the token chosen at each position is the argmax of the corrected logits (lowest index on
    ties): the drafter's proposal rule here, so proposals are deterministic;
  * the corrected logits of every position are the block's draft logits (the q rows the verifier
    reads);
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

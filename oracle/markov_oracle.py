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
  * markov_draft: the token chosen at each position is the argmax of the corrected logits
    (lowest index on ties), the proposal rule of greedy serving;
  * markov_sampled: the pages' head samples each position and biases the next position with the
    sample. The draw is from softmax(stored / tau), stored = the corrected logits as the draft
    rows hold them (the rows the verifier turns into q), by inverse CDF in ascending vocabulary
    order with one uniform per position passed in (the verifier's bonus-draw rule); tau == 0 is
    markov_draft; a temperature that is negative, not finite or in (0, TAU_MIN) makes every
    token of the request MARKOV_INVALID (its later positions then get no bias);
  * the corrected logits of every position are the block's draft logits (the q rows the verifier
    reads);
  * top-K candidates: the kc largest stored base logits of the position (NaN below every number,
    -inf included; ties to the lower index), kept in ascending vocabulary order; the token is
    the candidate with the largest corrected logit, the lowest vocabulary index on ties (the
    article's serving path is greedy); the corrected logits of the candidates are the block's
    draft output;
  * factors are bf16; logits fp32 or bf16; all arithmetic fp64. A position is ambiguous when its
    two largest corrected logits are closer than AMBIGUOUS_GAP (a float32 kernel's sum of R
    products may then order them the other way). A draw is ambiguous when its uniform lies closer
    to a CDF boundary than SAMPLE_EPS plus what the kernel's corrected-logit error (at most
    KERNEL_LOGIT_ABS + KERNEL_LOGIT_REL |z|) can move the stored row's CDF (stored_uncertainty).
    At an ambiguous position every token inside the band is a correct result (valid_tokens);
    markov_sampled_request can follow a given one of them down the rest of the block.
"""
from __future__ import annotations

import numpy as np

from .sv_oracle import TAU_MIN, argmax_lowest, decode_logits, inverse_cdf

AMBIGUOUS_GAP = 1e-4


def bf16_factor(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [V, R] -> fp64 values."""
    return decode_logits(np.asarray(bits, dtype=np.uint16), "bf16")


def correct_row(base_row: np.ndarray, dtype: str, L: np.ndarray, Rf: np.ndarray,
                prev: int) -> np.ndarray:
    """One position's corrected logits: its base logits plus Rf @ L[prev] when the previous token
    lies inside the vocabulary (no bias otherwise)."""
    z = decode_logits(base_row, dtype).copy()
    if 0 <= prev < z.shape[0]:
        z = z + Rf @ L[prev]
    return z


def argmax_with_gap(z: np.ndarray):
    """(argmax, lowest index on ties; its lead over the best other entry)."""
    y = argmax_lowest(z)
    rest = np.delete(z, y)
    return y, z[y] - (np.max(rest) if rest.size else -np.inf)


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
        z = correct_row(base[k], dtype, L, Rf, prev)
        corrected[k] = z
        y, gaps[k] = argmax_with_gap(z)
        tokens[k] = y
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


# ---------------------------------------------------------------------------------------------
# Sampled proposals. The pages' head samples each position's token from its corrected
# distribution and feeds the sample to the next position (DSpark paper review, 4.1
# Semi-autoregressive generation; "From draft-then-verify to DSpark", Recovering sequential
# dependencies); the
# DSpark article's comparison runs at temperature 1.0 (section 3, evaluation setup).

# A float32 kernel's error in one draw, relative to the row's mass: the weights 2^((y - m) c)
# carry about 3 roundings of an exponent of at most ~30 (<= 4e-6 of the mass they weigh, at the
# flattest rows) and the sums of the weights at most ~36 roundings in sequence (<= 2.2e-6); a
# factor of 2 over the sum.
SAMPLE_EPS = 1e-5
# Bound on a float32 kernel's corrected-logit error, abs + rel * |z|: R bf16 products are exact in
# float32 and only their accumulation rounds (measured at most 1.34e-6 at R = 256 over the
# Qwen3 vocabulary; the GPU tests hold every float32 output to this bound).
KERNEL_LOGIT_ABS = 4e-6
KERNEL_LOGIT_REL = 1e-7
MARKOV_INVALID = -3   # token of every position of a request whose temperature is invalid


def round_stored(z: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values -> the values a draft-logit row of `dtype` holds (round to nearest even), as
    fp64. bf16 keeps 8 significant bits; the logits here are far from bf16's range limits."""
    z = np.asarray(z, dtype=np.float64)
    if dtype == "f32":
        return z.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    out = z.copy()
    fin = np.isfinite(z) & (z != 0.0)
    mant, expo = np.frexp(z[fin])  # z = mant * 2^expo, 0.5 <= |mant| < 1
    out[fin] = np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)
    return out


def sample_weights(y: np.ndarray, tau: float) -> np.ndarray:
    """Unnormalised softmax(y / tau) of a stored row: exp((y_v - M) / tau) with M the row's
    largest value. NaN and -inf entries weigh 0; when M is +inf, the +inf entries weigh 1 and all
    others 0; a row without a number above -inf weighs 0 everywhere."""
    y = np.asarray(y, dtype=np.float64)
    valid = ~np.isnan(y) & (y > -np.inf)
    if not valid.any():
        return np.zeros_like(y)
    m = float(np.max(y[valid]))
    if m == np.inf:
        return (y == np.inf).astype(np.float64)
    return np.where(valid, np.exp((np.where(valid, y, m) - m) / tau), 0.0)


def clamp_uniform(u: float) -> float:
    """A draw's uniform as used: NaN and values below 0 read as 0, values above 1 as 1."""
    return 0.0 if not u > 0.0 else min(float(u), 1.0)


def sample_stored_row(y: np.ndarray, tau: float, u: float):
    """One draw from softmax(y / tau) by inverse CDF in ascending vocabulary order with the
    uniform u (NaN and u < 0 read as 0, u >= 1 as 1: the last entry with mass). A row without
    mass gives token 0. Returns (token, margin): the margin as inverse_cdf's (inf without mass)."""
    w = sample_weights(y, tau)
    if not np.any(w > 0.0):
        return 0, np.inf
    return inverse_cdf(w, clamp_uniform(u))


def draw_valid_tokens(y: np.ndarray, tau: float, u: float, band: float) -> np.ndarray:
    """Tokens with mass whose CDF interval (relative to the row's mass, ascending order) meets
    [r - band, r + band], r the clamped uniform: every token a draw that errs by at most `band`
    could return. With band 0 it holds the draw alone (or, on a boundary, both neighbours)."""
    w = sample_weights(y, tau)
    if not np.any(w > 0.0):
        return np.array([0])
    r = clamp_uniform(u)
    c = np.cumsum(w) / float(np.sum(w))
    lo = np.concatenate(([0.0], c[:-1]))
    hit = (w > 0.0) & (c >= r - band) & (lo <= r + band)
    if r >= 1.0:
        hit |= np.arange(len(w)) == np.nonzero(w > 0.0)[0][-1]
    return np.nonzero(hit)[0]


def argmax_valid_tokens(z: np.ndarray) -> np.ndarray:
    """Entries within AMBIGUOUS_GAP of the largest corrected logit."""
    z = np.asarray(z, dtype=np.float64)
    return np.nonzero(z >= z[argmax_lowest(z)] - AMBIGUOUS_GAP)[0]


def stored_uncertainty(z: np.ndarray, dtype: str, tau: float) -> float:
    """How far (relative to the row's mass) the CDF of softmax(stored / tau) can move when the
    kernel's float32 corrected logits lie within KERNEL_LOGIT_ABS + KERNEL_LOGIT_REL |z| of the
    fp64 ones: each entry can then be stored as either rounding of the ends of that interval."""
    z = np.asarray(z, dtype=np.float64)
    tol = KERNEL_LOGIT_ABS + KERNEL_LOGIT_REL * np.abs(np.where(np.isfinite(z), z, 0.0))
    lo = round_stored(z - tol, dtype)
    hi = round_stored(z + tol, dtype)
    mid = round_stored(z, dtype)
    w_mid = sample_weights(mid, tau)
    total = float(np.sum(w_mid))
    if not total > 0.0:
        return 0.0
    valid = ~np.isnan(mid) & (mid > -np.inf)
    m = float(np.max(mid[valid]))
    if not np.isfinite(m):
        return 0.0
    spread = np.where(valid & np.isfinite(z),
                      np.abs(np.exp((hi - m) / tau) - np.exp((lo - m) / tau)), 0.0)
    return 2.0 * float(np.sum(spread)) / total


def markov_sampled_request(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray,
                           anchor: int, tau: float, uniforms: np.ndarray, choose=None):
    """One request of the sampled head: base [K, V] stored logits; left, right [V, R] bf16 bits;
    tau the request's temperature; uniforms [K] one per position.

    tau == 0: exactly markov_draft_request (argmax of the fp64 corrected logits).
    tau in [TAU_MIN, inf): position k's token is drawn from softmax(stored_k / tau), stored_k
      the corrected logits as the draft-logit rows hold them (dtype rounding), by inverse CDF
      with uniforms[k]; the drawn token sets the next position's bias.
    Any other tau: every token MARKOV_INVALID; positions after the first get no bias.

    Returns (tokens [K], corrected [K, V] fp64, ambiguous [K] bool): position k is ambiguous when
    a float32 kernel may decide it differently (argmax: top-2 gap below AMBIGUOUS_GAP; draw: the
    CDF margin below SAMPLE_EPS plus stored_uncertainty). choose [K] (optional): at an ambiguous
    position, when choose[k] is one of the tokens valid there (argmax_valid_tokens,
    draw_valid_tokens), that token is taken instead and biases the next position."""
    K, V = base.shape
    tau = float(tau)
    greedy = tau == 0.0
    valid = greedy or (TAU_MIN <= tau < np.inf)
    L = bf16_factor(left)
    Rf = bf16_factor(right)
    tokens = np.zeros(K, dtype=np.int32)
    corrected = np.zeros((K, V))
    amb = np.zeros(K, dtype=bool)
    prev = int(anchor)
    for k in range(K):
        z = correct_row(base[k], dtype, L, Rf, prev)
        corrected[k] = z
        if not valid:
            y = MARKOV_INVALID
        elif greedy:
            y, gap = argmax_with_gap(z)
            amb[k] = gap < AMBIGUOUS_GAP
            if amb[k] and choose is not None and int(choose[k]) in argmax_valid_tokens(z):
                y = int(choose[k])
        else:
            stored = round_stored(z, dtype)
            y, margin = sample_stored_row(stored, tau, float(uniforms[k]))
            band = SAMPLE_EPS + stored_uncertainty(z, dtype, tau)
            amb[k] = margin < band
            if amb[k] and choose is not None and \
                    int(choose[k]) in draw_valid_tokens(stored, tau, float(uniforms[k]), band):
                y = int(choose[k])
        tokens[k] = y
        prev = y
    return tokens, corrected, amb


def markov_sampled(base: np.ndarray, dtype: str, left: np.ndarray, right: np.ndarray,
                   temperatures: np.ndarray, uniforms: np.ndarray, anchors=None):
    """Batch [B, K, V], temperatures [B], uniforms [B, K]: tokens [B, K], corrected [B, K, V]
    fp64, first ambiguous position of each request [B] (K when none)."""
    B, K, V = base.shape
    tokens = np.zeros((B, K), dtype=np.int32)
    corrected = np.zeros((B, K, V))
    first = np.full(B, K, dtype=np.int64)
    for b in range(B):
        a = -1 if anchors is None else int(anchors[b])
        t, c, amb = markov_sampled_request(base[b], dtype, left, right, a,
                                           float(temperatures[b]), uniforms[b])
        tokens[b], corrected[b] = t, c
        if amb.any():
            first[b] = int(np.argmax(amb))
    return tokens, corrected, first


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

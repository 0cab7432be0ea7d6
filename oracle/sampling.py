"""Plain CPU oracle of drafting and verification at temperature 1.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU-baseline leg may import this module.
The HIP library never calls it and shares no code with it.

What is computed, and where it comes from
------------------------------------------
Page names as in ``dflash_ref``: [DF] is the DFlash paper-graph summary, [DDT] the DDTree one.

* [DF] §3.4.4 "Single forward pass prediction": at temperature 1 each block row's token is drawn from the
  softmax of that row's logits (the marginal q_i of [DDT] §3.4.2, over the full vocabulary).
* [DF] §3.4.4 "Integration with verification": the block is verified by standard speculative decoding
  (Leviathan et al., 2023).  The page's own steps for the stochastic mode are garbled (a draft is not kept
  merely because the target gives it non-zero probability), so the rule here is the published one of
  Leviathan, Kalman and Matias, "Fast Inference from Transformers via Speculative Decoding" (ICML 2023),
  §2.3 and Algorithm 1, which Chen et al., "Accelerating Large Language Model Decoding with Speculative
  Sampling" (2023) state as modified rejection sampling: keep draft y_j with probability
  min(1, p_j(y_j) / q_j(y_j)); at the first rejection draw the next token from the normalised residual
  max(0, p_j - q_j); if every draft is kept, draw the bonus token from the target's next distribution.  The
  output is then distributed exactly as the target's own samples (their Theorem 1), which the tests check
  by enumeration.
* [DF] §5 (temperature-1 rows of Table 1) and [DDT] §5: results at temperature 1 use this mode.

Readings (where the pages leave a step open):
  R1  Each block row is sampled independently: the pass is parallel, and no row's q depends on another
      row's sample ([DF] §5.2 notes that mask positions are predicted independently).
  R2  Sampler: the Gumbel-max identity (argmax_j of log p_j + G_j, with G_j independent standard Gumbel
      variables, is distributed as p; Gumbel 1954, and e.g. Maddison, Tarlow and Minka, "A* Sampling",
      NIPS 2014, §2).  It needs no normalisation and no prefix sum, so a row can be sampled in one pass
      over its logits.  Ties of the perturbed score go to the lowest id.
  R3  Random draws: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
      1, 2, 3", SC 2011), a counter-based generator, so that any element's draw can be made where it is
      needed.  The 32-bit word for (stream tag, row, index j) under a 64-bit seed is word j mod 4 of
      Philox4x32-10 at counter (j div 4, row, tag, 0) and key (seed mod 2^32, seed div 2^32).  A word c
      gives the uniform u = (c + 1/2) / 2^32 in (0, 1), and the Gumbel variable G = -ln(-ln(1 - u)).
      Tags: 1 = drafting (row = request * L + block row, j = vocabulary id); 2 = acceptance uniforms
      (row = request, j = draft position, from 0); 3 = residual or bonus sampling (row = request,
      j = vocabulary id).
  R4  Verification row j (0-based) of the target's logits is its distribution for the token after the
      block prefix that ends in draft j - 1 (the anchor for j = 0), and so pairs with draft j; row gamma is
      the bonus row.  The drafter's row for draft j is block row j + 1.
  R5  Draft j is kept iff ln u_j < ln p_j(y_j) - ln q_j(y_j) (the same test as u_j < min(1, p/q), since
      u_j < 1).  A draft id outside the vocabulary counts as rejected.
  R6  If the residual max(0, p - q) is zero everywhere (p equals q up to rounding), the next token is drawn
      from p.
  R7  tau = (number of kept drafts) + 1 counts the committed tokens, the next token included, as in the
      greedy mode.

Arithmetic is float64; the kernel works in float32, so the parity tests compare decisions only where the
margin of this oracle's decision exceeds float32 error, and report the rest.
"""
from __future__ import annotations

import itertools

import numpy as np

TAG_DRAFT, TAG_ACCEPT, TAG_RESAMPLE = 1, 2, 3

_M0, _M1 = 0xD2511F53, 0xCD9E8D57   # Philox4x32 multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85   # Philox key increments (Weyl sequence)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32-10 (Salmon et al. 2011, §4.2): ten rounds; each multiplies counter words 0 and 2 by the
    round multipliers into 64-bit products, and the new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by the Weyl constants between rounds.
    counter: [..., 4] unsigned 32-bit words, key: two words.  Returns [..., 4] uint32."""
    ctr = np.asarray(counter, dtype=np.uint64)
    c = [ctr[..., i] for i in range(4)]
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    for _ in range(10):
        p0 = np.uint64(_M0) * c[0]          # exact: 32 x 32 -> 64 bits
        p1 = np.uint64(_M1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _U32, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & _U32]
        k0 = (k0 + np.uint64(_W0)) & _U32
        k1 = (k1 + np.uint64(_W1)) & _U32
    return np.stack(c, axis=-1).astype(np.uint32)


def draw_bits(seed: int, tag: int, row: int, idx) -> np.ndarray:
    """The 32-bit words of stream (tag, row) at indices idx (R3)."""
    idx = np.asarray(idx, dtype=np.uint64)
    ctr = np.zeros(idx.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = idx >> np.uint64(2)
    ctr[..., 1] = np.uint64(row)
    ctr[..., 2] = np.uint64(tag)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    return np.take_along_axis(words, (idx & np.uint64(3)).astype(np.int64)[..., None], axis=-1)[..., 0]


def uniform(bits) -> np.ndarray:
    """u = (c + 1/2) / 2^32: the midpoint of the word's cell of (0, 1) (R3)."""
    return (np.asarray(bits, dtype=np.float64) + 0.5) / 4294967296.0


def gumbel(bits) -> np.ndarray:
    """G = -ln(-ln(1 - u)): inverse-CDF transform of the uniform (the standard Gumbel CDF is
    exp(-exp(-g)), and 1 - u is uniform as u is)."""
    u = uniform(bits)
    return -np.log(-np.log1p(-u))


def log_softmax(logits) -> np.ndarray:
    """ln q = logit - logsumexp over the row (the marginal of [DDT] §3.4.2, at temperature 1)."""
    lg = np.asarray(logits, dtype=np.float64)
    mx = lg.max(axis=-1, keepdims=True)
    return lg - (mx + np.log(np.exp(lg - mx).sum(axis=-1, keepdims=True)))


def _argmax_lowest(score: np.ndarray):
    """argmax with ties to the lowest index, and the gap to the runner-up (inf for a single finite entry)."""
    best = int(np.argmax(score))           # numpy returns the first maximum
    rest = np.delete(score, best)
    second = rest.max() if rest.size else -np.inf
    return best, float(score[best] - second)


def sample_rows(logits, seed: int, row0: int = 0):
    """Drafting at temperature 1 (R1, R2): row m (global row row0 + m) takes argmax_j of logit_mj + G_mj,
    with G from stream (TAG_DRAFT, row0 + m).  Returns (ids [M], margins [M]): the margin is the gap between
    the winning perturbed score and the runner-up, used to guard parity against float32 kernels."""
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    M, V = lg.shape
    ids = np.zeros(M, dtype=np.int64)
    margins = np.zeros(M)
    j = np.arange(V)
    for m in range(M):
        ids[m], margins[m] = _argmax_lowest(lg[m] + gumbel(draw_bits(seed, TAG_DRAFT, row0 + m, j)))
    return ids, margins


def accept_probability(p: np.ndarray, q: np.ndarray, y: int) -> float:
    """min(1, p(y) / q(y)) (Leviathan et al., Algorithm 1); 0 for an id outside the vocabulary (R5)."""
    if not 0 <= y < len(p):
        return 0.0
    if q[y] == 0.0:
        return 1.0
    return min(1.0, p[y] / q[y])


def residual(p: np.ndarray, q: np.ndarray):
    """The normalised residual max(0, p - q) / sum; None when it vanishes (R6)."""
    r = np.maximum(np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64), 0.0)
    s = r.sum()
    return None if s <= 0.0 else r / s


def speculative_verify(drafts, q_logits, p_logits, seed: int, row: int):
    """One verification of one request (R4-R7).

    drafts [gamma] ints; q_logits [gamma, V] (the drafter's rows of the drafts); p_logits [gamma + 1, V]
    (the target's rows).  Returns (tau, next_token, guard) where guard = the smallest decision margin:
    |ln u - (ln p - ln q)| over the acceptance tests taken, and the top-2 gap of the final sampling."""
    lq = log_softmax(q_logits) if len(drafts) else np.zeros((0, np.shape(p_logits)[-1]))
    lp = log_softmax(p_logits)
    gamma, V = len(drafts), lp.shape[-1]
    u = uniform(draw_bits(seed, TAG_ACCEPT, row, np.arange(gamma))) if gamma else np.zeros(0)
    guard = np.inf
    k = gamma
    for j in range(gamma):
        y = int(drafts[j])
        if not 0 <= y < V:
            k = j
            break
        d = np.log(u[j]) - (lp[j, y] - lq[j, y])
        guard = min(guard, abs(d))
        if not d < 0.0:
            k = j
            break
    g = gumbel(draw_bits(seed, TAG_RESAMPLE, row, np.arange(V)))
    if k < gamma:
        r = np.maximum(np.exp(lp[k]) - np.exp(lq[k]), 0.0)
        if r.max() > 0.0:
            with np.errstate(divide="ignore"):
                score = np.log(r) + g      # -inf where the residual is zero: never chosen
        else:
            score = lp[k] + g
    else:
        score = lp[gamma] + g
    nxt, gap = _argmax_lowest(score)
    return k + 1, nxt, min(guard, gap)


# ----------------------------------------------------------------------------------------------------
# exact distributions (tiny vocabularies), for the pins
# ----------------------------------------------------------------------------------------------------


def exact_cycle_outcomes(q: np.ndarray, target):
    """Exact distribution of one verification cycle's committed tokens, by enumerating every draft block.

    q [gamma, V]: drafter marginals (rows independent, R1).  target(prefix) -> probabilities [V] of the
    target's next token after the committed prefix (a tuple of token ids).  Each draft block y has
    probability prod_j q_j(y_j); the rule keeps y_1..y_k and commits the next token z from the residual
    (or the bonus row).  Returns {committed tokens tuple: probability}."""
    q = np.asarray(q, dtype=np.float64)
    gamma, V = q.shape
    out = {}
    for y in itertools.product(range(V), repeat=gamma):
        py = float(np.prod([q[j, y[j]] for j in range(gamma)]))
        if py == 0.0:
            continue
        reach = 1.0                      # probability that drafts 0..j-1 were all kept
        for j in range(gamma + 1):
            p = np.asarray(target(tuple(y[:j])), dtype=np.float64)
            if j == gamma:               # every draft kept: bonus token from the target
                for z in range(V):
                    key = tuple(y) + (z,)
                    out[key] = out.get(key, 0.0) + py * reach * p[z]
                break
            a = accept_probability(p, q[j], y[j])
            if a < 1.0:                  # rejected here: next token from the residual
                r = residual(p, q[j])
                if r is None:
                    r = p
                for z in range(V):
                    key = tuple(y[:j]) + (z,)
                    out[key] = out.get(key, 0.0) + py * reach * (1.0 - a) * r[z]
            reach *= a
            if reach == 0.0:
                break
    return out


def extend_with_target(outcomes: dict, target, length: int):
    """Continue every committed prefix with the target's own samples up to `length` tokens (what the next
    cycles would produce, by induction), giving a distribution over token sequences of that length."""
    out = {}
    stack = list(outcomes.items())
    while stack:
        seq, pr = stack.pop()
        if len(seq) >= length:
            out[seq[:length]] = out.get(seq[:length], 0.0) + pr
            continue
        p = np.asarray(target(seq), dtype=np.float64)
        for z in range(len(p)):
            if p[z] > 0.0:
                stack.append((seq + (z,), pr * p[z]))
    return out

"""Pins of the temperature-1 oracle (drafting by Gumbel-max sampling, verification by modified rejection
sampling) against what the published definitions and the mathematics fix:

* the generator against the Philox4x32-10 known-answer vectors;
* the Gumbel transform against the Gumbel law (Kolmogorov-Smirnov, mean = Euler's constant, variance pi^2/6);
* the sampler against the softmax it must draw from (chi-square over many independent streams);
* the acceptance rule by exact enumeration: one cycle followed by plain target sampling yields exactly the
  target's joint distribution (Leviathan et al. 2023, Theorem 1), on several tiny vocabularies;
* the Philox-driven verifier against that exact cycle distribution (chi-square over seeds);
* the degenerate cases (no drafts, p = q, disjoint supports, invalid ids)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# upper 99.9% quantiles of chi-square, by degrees of freedom (tables of the chi-square law)
_CHI2_999 = {3: 16.27, 4: 18.47, 5: 20.52, 7: 24.32, 8: 26.12, 10: 29.59, 12: 32.91, 15: 37.70, 20: 45.31,
             25: 52.62, 30: 59.70, 35: 66.62, 38: 70.70, 40: 73.40, 45: 80.08, 50: 86.66, 60: 99.61, 80: 124.84}


def _chi2_bound(dof):
    keys = sorted(_CHI2_999)
    for k in keys:
        if k >= dof:
            return _CHI2_999[k]
    # Wilson-Hilferty beyond the table
    z = 3.09
    return dof * (1 - 2 / (9 * dof) + z * math.sqrt(2 / (9 * dof))) ** 3


def _chi2(counts: dict, probs: dict, n: int):
    """Chi-square statistic over outcomes, pooling those with expected count < 5 into one cell."""
    stat, pool_o, pool_e, cells = 0.0, 0.0, 0.0, 0
    for key, p in probs.items():
        e = n * p
        o = counts.get(key, 0)
        if e < 5:
            pool_o += o
            pool_e += e
            continue
        stat += (o - e) ** 2 / e
        cells += 1
    extra = sum(v for k, v in counts.items() if k not in probs)
    pool_o += extra
    if pool_e >= 5:
        stat += (pool_o - pool_e) ** 2 / pool_e
        cells += 1
    else:
        assert pool_o <= max(10, 3 * pool_e), "outcomes of (near) zero probability occurred too often"
    return stat, cells - 1


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for c in kat["cases"]:
        ctr = np.array([[int(x, 16) for x in c["counter"]]], dtype=np.uint64)
        out = S.philox4x32_10(ctr, [int(x, 16) for x in c["key"]])[0]
        assert [f"{int(v):08x}" for v in out] == c["out"]


def test_streams_are_distinct_and_reproducible():
    a = S.draw_bits(7, S.TAG_DRAFT, 3, np.arange(64))
    assert np.array_equal(a, S.draw_bits(7, S.TAG_DRAFT, 3, np.arange(64)))
    for other in (S.draw_bits(8, S.TAG_DRAFT, 3, np.arange(64)), S.draw_bits(7, S.TAG_ACCEPT, 3, np.arange(64)),
                  S.draw_bits(7, S.TAG_DRAFT, 4, np.arange(64)), S.draw_bits(7 + (1 << 32), S.TAG_DRAFT, 3,
                                                                            np.arange(64))):
        assert np.mean(a == other) < 0.1
    # the index runs through four words per counter: all 64 words distinct
    assert len(set(a.tolist())) == 64


def test_gumbel_law():
    n = 1 << 16
    g = S.gumbel(S.draw_bits(12345, S.TAG_RESAMPLE, 0, np.arange(n)))
    gs = np.sort(g)
    cdf = np.exp(-np.exp(-gs))
    ecdf_hi = np.arange(1, n + 1) / n
    ks = max(np.max(ecdf_hi - cdf), np.max(cdf - (ecdf_hi - 1 / n)))
    assert ks < 1.95 / math.sqrt(n)                          # KS at the 0.1% level
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 4 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    u = S.uniform(np.array([0, 0xFFFFFFFF], dtype=np.uint64))
    assert 0 < u[0] < u[1] < 1


@pytest.mark.parametrize("logits", [[0.0, 1.0, 2.0, -1.0, 0.5], [3.0, 3.0, 3.0, 3.0], [-np.inf, 0.0, 2.0, -np.inf, 1.0]])
def test_gumbel_max_samples_the_softmax(logits):
    lg = np.array(logits, dtype=np.float64)
    n = 30000
    ids, _ = S.sample_rows(np.tile(lg, (n, 1)), seed=99, row0=0)
    p = np.exp(S.log_softmax(lg))
    counts = {int(k): int(v) for k, v in zip(*np.unique(ids, return_counts=True))}
    probs = {j: float(p[j]) for j in range(len(lg)) if p[j] > 0}
    assert set(counts) <= set(probs)                         # never a masked (-inf) id
    stat, dof = _chi2(counts, probs, n)
    assert stat < _chi2_bound(dof), (stat, dof)


def _random_target(rng, V, alpha, zeros=False):
    """A target model on a tiny vocabulary: its next-token distribution is a fixed random function of the
    committed prefix (memoised), optionally with zeros."""
    table = {}

    def target(prefix):
        if prefix not in table:
            p = rng.gamma(alpha, size=V)
            if zeros:
                p[rng.random(V) < 0.3] = 0.0
                if p.sum() == 0:
                    p[rng.integers(V)] = 1.0
            table[prefix] = p / p.sum()
        return table[prefix]
    return target


def _target_joint(target, V, length):
    out = {}
    for seq in itertools.product(range(V), repeat=length):
        pr = 1.0
        for i in range(length):
            pr *= target(seq[:i])[seq[i]]
        if pr > 0:
            out[seq] = pr
    return out


@pytest.mark.parametrize("seed,V,gamma,zeros", [(0, 3, 2, False), (1, 2, 3, False), (2, 4, 1, False),
                                                (3, 3, 3, False), (4, 3, 2, True), (5, 2, 4, True)])
def test_cycle_then_target_equals_target_joint(seed, V, gamma, zeros):
    """Theorem 1 of Leviathan et al. by enumeration: committing one cycle's tokens and then sampling the target
    gives the target's joint law of the first gamma + 1 tokens, whatever the drafter's marginals."""
    rng = np.random.default_rng(500 + seed)
    q = rng.gamma(0.7, size=(gamma, V))
    if zeros:
        q[rng.random((gamma, V)) < 0.3] = 0.0
        q[q.sum(axis=1) == 0, 0] = 1.0
    q /= q.sum(axis=1, keepdims=True)
    target = _random_target(rng, V, 0.7, zeros)
    out = S.exact_cycle_outcomes(q, target)
    assert sum(out.values()) == pytest.approx(1.0, abs=1e-12)
    got = S.extend_with_target(out, target, gamma + 1)
    want = _target_joint(target, V, gamma + 1)
    for key in set(got) | set(want):
        assert got.get(key, 0.0) == pytest.approx(want.get(key, 0.0), abs=1e-12), key


def test_expected_kept_drafts_closed_form():
    """With a single draft, the chance of keeping it is sum_x min(p(x), q(x)) (Leviathan et al., §3.1)."""
    rng = np.random.default_rng(77)
    V = 5
    q = rng.dirichlet(np.ones(V))[None, :]
    p = rng.dirichlet(np.ones(V))
    out = S.exact_cycle_outcomes(q, lambda prefix: p if len(prefix) == 0 else np.full(V, 1.0 / V))
    kept = sum(pr for seq, pr in out.items() if len(seq) == 2)
    assert kept == pytest.approx(np.minimum(p, q[0]).sum(), abs=1e-12)


def test_verifier_samples_the_exact_cycle_law():
    """The Philox-driven drafter sampler plus verifier, over many seeds, reproduces the exact outcome law."""
    rng = np.random.default_rng(4242)
    V, gamma = 3, 2
    q = rng.dirichlet(0.8 * np.ones(V), size=gamma)
    target = _random_target(rng, V, 0.8)
    exact = S.exact_cycle_outcomes(q, target)
    lq = np.log(q)
    n = 12000
    counts = {}
    for seed in range(n):
        y, _ = S.sample_rows(lq, seed, row0=0)
        p_logits = np.log(np.stack([target(tuple(int(t) for t in y[:j])) for j in range(gamma + 1)]))
        tau, nxt, _ = S.speculative_verify(y, lq, p_logits, seed, row=0)
        key = tuple(int(t) for t in y[:tau - 1]) + (int(nxt),)
        counts[key] = counts.get(key, 0) + 1
    stat, dof = _chi2(counts, exact, n)
    assert stat < _chi2_bound(dof), (stat, dof)


def test_verifier_degenerate_cases():
    rng = np.random.default_rng(3)
    V = 6
    lg = rng.normal(size=(4, V))
    # p == q: every draft is kept (ln u < 0 = ln p - ln q), the next token is the bonus
    for seed in range(20):
        y = rng.integers(V, size=3)
        tau, nxt, _ = S.speculative_verify(y, lg[:3], np.concatenate([lg[:3], lg[3:]]), seed, row=1)
        assert tau == 4 and 0 <= nxt < V
    # no drafts: tau = 1 and the next token is a sample of the bonus row; a one-hot row fixes it
    one = np.full((1, V), -np.inf)
    one[0, 4] = 0.0
    assert S.speculative_verify([], np.zeros((0, V)), one, 5, 0)[:2] == (1, 4)
    # disjoint supports: q is one-hot on 2, p is zero there -> rejected at once, next token from p's support
    q1 = np.full((1, V), -np.inf)
    q1[0, 2] = 0.0
    p1 = np.array([[0.0, 1.0, -np.inf, 0.5, -np.inf, -np.inf], [0.0] * V])
    for seed in range(20):
        tau, nxt, _ = S.speculative_verify([2], q1, p1, seed, row=0)
        assert tau == 1 and nxt in (0, 1, 3)
    # an id outside the vocabulary counts as a rejection at its position
    tau, nxt, _ = S.speculative_verify([0, V + 3], lg[:2], lg[:3], 1, row=0)
    assert tau in (1, 2)
    if tau == 2:
        assert 0 <= nxt < V

"""Pins of the DDTree oracle ([DDT] = "Accelerating Speculative Decoding with Block Diffusion Draft Trees"):
a hand-worked example, Proposition 1 by enumerating every continuation, Proposition 2 and Lemma 1 by brute
force over every prefix, the heap's structural invariants, and the verifier walk on a hand-drawn tree."""
import itertools

import numpy as np
import pytest

from oracle import ddtree as T


def _prefixes(nodes, vocab_ids):
    """Token prefixes of the tree's nodes, as tuples."""
    out = {}
    for i, (ranks, _, parent) in enumerate(nodes):
        tok = int(vocab_ids[len(ranks) - 1, ranks[-1]])
        out[i] = (out[parent] if parent >= 0 else ()) + (tok,)
    return set(out.values())


def test_hand_example():
    """q1 = (.6, .3, .1), q2 = (.5, .4, .1) over tokens (a, b, c) = (0, 1, 2), budget 4.  By hand the prefix
    probabilities are a .6, b .3, aa .3, ab .24, ba .15, ...; the top 4 are {a, aa, b, ab} with total 1.44."""
    q = np.array([[0.6, 0.3, 0.1], [0.5, 0.4, 0.1]])
    ids = np.array([[0, 1, 2], [0, 1, 2]])
    nodes = T.build_tree(np.log(q), 4)
    got = {p: None for p in _prefixes(nodes, ids)}
    assert set(got) == {(0,), (0, 0), (1,), (0, 1)}
    probs = sorted(np.exp([s for _, s, _ in nodes]), reverse=True)
    np.testing.assert_allclose(probs, [0.6, 0.3, 0.3, 0.24], rtol=1e-12)
    # Proposition 1 on this tree: E[alpha] by enumeration over all 9 continuations = 1.44
    assert T.expected_acceptance_enumerated(q, set(got)) == pytest.approx(1.44, rel=1e-12)


def _random_q(rng, D, V):
    q = rng.gamma(0.6, size=(D, V))
    return q / q.sum(axis=1, keepdims=True)


def _random_tree(rng, D, V, n):
    """A random prefix-closed set of n token prefixes."""
    tree = set()
    frontier = [()]
    while len(tree) < n:
        base = frontier[rng.integers(len(frontier))]
        if len(base) == D:
            continue
        child = base + (int(rng.integers(V)),)
        if child not in tree:
            tree.add(child)
            frontier.append(child)
    return tree


@pytest.mark.parametrize("seed", range(6))
def test_prop1_expected_acceptance_is_sum_of_node_probabilities(seed):
    rng = np.random.default_rng(100 + seed)
    D, V = 3, 3
    q = _random_q(rng, D, V)
    tree = _random_tree(rng, D, V, int(rng.integers(1, 12)))
    rhs = sum(float(np.prod([q[i, u[i]] for i in range(len(u))])) for u in tree)
    assert T.expected_acceptance_enumerated(q, tree) == pytest.approx(rhs, rel=1e-12)


@pytest.mark.parametrize("seed,D,V", [(0, 3, 4), (1, 2, 5), (2, 4, 3), (3, 3, 4), (4, 1, 6)])
def test_prop2_and_lemma1_heap_equals_brute_force(seed, D, V):
    """For every budget: the heap's pops are the B best prefixes over the whole vocabulary (Proposition 2),
    and restricting each depth to its top K = min(B, V) tokens changes nothing (Lemma 1)."""
    rng = np.random.default_rng(200 + seed)
    q = _random_q(rng, D, V)
    lq_full = np.log(q)
    order = np.argsort(-lq_full, axis=1, kind="stable")
    lq_sorted = np.take_along_axis(lq_full, order, axis=1)
    total = sum(V ** d for d in range(1, D + 1))
    for B in range(1, min(total, 40) + 1):
        brute = T.brute_force_top(lq_sorted, B)
        K = min(B, V)
        nodes = T.build_tree(lq_sorted[:, :K], B)
        assert len(nodes) == len(brute) == B
        np.testing.assert_allclose(sorted(s for _, s, _ in nodes), sorted(s for _, s in brute), rtol=0, atol=1e-12)
        # with continuous random q there are no ties: the sets themselves agree
        assert {r for r, _, _ in nodes} == {r for r, _ in brute}


@pytest.mark.parametrize("seed", range(4))
def test_heap_invariants(seed):
    """Pops are non-increasing in sigma, the tree is prefix-closed with consistent parent links, each
    node's sigma is the sum of its ranks' log-probabilities, and the size is min(budget, |S_K|)."""
    rng = np.random.default_rng(300 + seed)
    D, K = 4, 5
    lq = np.sort(np.log(_random_q(rng, D, 9)), axis=1)[:, ::-1][:, :K]
    for B in (1, 7, 50, 400, 10000):
        nodes = T.build_tree(lq, B)
        assert len(nodes) == min(B, sum(K ** d for d in range(1, D + 1)))
        sig = [s for _, s, _ in nodes]
        assert all(a >= b for a, b in zip(sig, sig[1:]))
        for i, (ranks, s, parent) in enumerate(nodes):
            assert s == pytest.approx(sum(lq[d, r] for d, r in enumerate(ranks)), abs=1e-12)
            if len(ranks) == 1:
                assert parent == -1
            else:
                assert 0 <= parent < i and nodes[parent][0] == ranks[:-1]


def test_verify_walk_hand_tree():
    """Tree over tokens: node 0 = a(5), node 1 = a b (5, 7), node 2 = c (9), node 3 = a b d (5, 7, 4).
    Target choices: after root 5, after node 0 7, after node 1 8 -> accept nodes 0, 1; bonus 8.
    A target that disagrees at the root accepts nothing and its choice is the bonus."""
    tok = [5, 7, 9, 4]
    par = [-1, 0, -1, 1]
    tgt = [5, 7, 8, 0, 0]
    assert T.verify_walk(tok, par, tgt) == ([0, 1], 8)
    assert T.verify_walk(tok, par, [3, 7, 8, 0, 0]) == ([], 3)
    assert T.verify_walk(tok, par, [5, 7, 4, 0, 6]) == ([0, 1, 3], 6)


def test_topk_logprobs_matches_sorting_and_softmax():
    rng = np.random.default_rng(7)
    lg = rng.normal(size=(3, 50))
    lg[1, [4, 9, 20]] = lg[1].max() + 1.0  # a three-way tie at the top: ids ascending
    ids, lp = T.topk_logprobs(lg, 6)
    for r in range(3):
        order = sorted(range(50), key=lambda j: (-lg[r, j], j))[:6]
        assert list(ids[r]) == order
        p = np.exp(lg[r] - lg[r].max())
        p /= p.sum()
        np.testing.assert_allclose(lp[r], np.log(p[order]), rtol=0, atol=1e-12)
    assert list(ids[1, :3]) == [4, 9, 20]

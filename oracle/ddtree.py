"""Plain CPU oracle of DDTree draft-tree construction and the greedy verifier walk.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU-baseline leg may import this module.
The HIP library never calls it and shares no code with it.

Source: "Accelerating Speculative Decoding with Block Diffusion Draft Trees" (paper-graph summary), cited
as [DDT]:
  * §3.4.2  the drafter's per-position marginals q_i = softmax of the block row's logits, and the factorised
            surrogate Q(y_1..y_L) = prod_i q_i(y_i);
  * §3.4.3  acceptance length alpha_T(y) = the longest prefix of y that is a node of the tree T (0 if no
            depth-1 node matches); Proposition 1: E_{Y~Q}[alpha_T(Y)] = sum over nodes u of q(u), with
            q(u) = prod over the node's positions of q_i(u_i); Proposition 2: the B most probable prefixes
            form a valid (prefix-closed) tree that maximises that sum among trees of at most B nodes;
  * §3.4.4  Lemma 1 (only the top K = min(B, |V|) tokens of each position can appear in the optimal tree),
            rank tuples, log-probability scores sigma, and Algorithm 1 (best-first heap: pop the best tuple,
            add its prefix to the tree, push its next sibling if its last rank is below K and its first
            child if its depth is below L);
  * §3.4.5  the greedy verifier walk: from the root, take the target's choice after the current prefix,
            move to the child holding that token if there is one, else stop; the stopping choice is the
            next bonus token.

Readings (where the page leaves a step open):
  * the depth-d distribution is the drafter's block row d (rows 1 .. block_len-1; row 0 holds the anchor),
    so a block of length L gives trees of depth at most L - 1;
  * ties in sigma pop in creation order (the sibling of a popped tuple is created before its child);
  * scores follow the page's update rules: the next sibling of a popped tuple scores sigma - log q_d(rank) +
    log q_d(rank + 1), the first child sigma + log q_{d+1}(rank 1).  A parity run against a float32 kernel
    that scores a node as its parent's score plus its own log-probability (the same quantity in exact
    arithmetic) can ask for that summation order (score="path_sum") together with dtype=np.float32, to take
    the kernel's float32 decisions; the fp64 default is the page's order;
  * the tree's node i is the i-th pop; its parent is the node index of its prefix without the last token
    (-1 for a depth-1 node, whose parent is the root = the bonus token).

Arithmetic is float64 in the page's order unless a caller asks otherwise.  Which prefixes enter the tree is
decided by comparisons of float sums: a parity test compares a float32 kernel with this fp64 pop order on
every pop whose fp64 margin exceeds float32 error (build_tree(..., with_gaps=True) reports the margins), and
may also replay the kernel's own float32 decisions (dtype=np.float32, score="path_sum").
"""
from __future__ import annotations

import heapq
import itertools

import numpy as np

from .dflash_ref import log_sum_exp, ranked_ids


def topk_logprobs(logits: np.ndarray, k: int):
    """The k best tokens of each row by (logit descending, id ascending) and their log-probabilities
    log softmax = logit - logsumexp over the full vocabulary ([DDT] §3.4.2; Lemma 1 for why k suffices)."""
    lg = np.asarray(logits, dtype=np.float64)
    ids = ranked_ids(lg, k)
    lse = log_sum_exp(lg)
    return ids, np.take_along_axis(lg, ids, axis=-1) - lse[..., None]


def build_tree(logp: np.ndarray, budget: int, dtype=np.float64, score: str = "incremental",
               with_gaps: bool = False):
    """Algorithm 1 of [DDT] §3.4.4 on sorted per-depth log-probabilities.

    logp: [D, K], row d-1 = log q_d of the depth-d ranks 1..K, each row non-increasing.
    Returns the pops in order as a list of (ranks, sigma, parent): ranks is a 0-based rank tuple (rank 0 is
    the page's rank 1), sigma its log-probability score, parent the node index of ranks[:-1] (-1: root).
    score="incremental" (default) scores a sibling by the page's update sigma - log q_d(rank) + log q_d(rank+1);
    score="path_sum" scores it as the parent's score + log q_d(rank+1) (see the module docstring).
    with_gaps=True also returns, per pop, the popped score minus the best score left in the heap (inf if
    none): how far that pop was from a different decision.
    """
    if score not in ("incremental", "path_sum"):
        raise ValueError(score)
    lq = np.asarray(logp, dtype=dtype)
    D, K = lq.shape
    nodes, gaps = [], []
    if budget < 1 or D < 1 or K < 1:
        return (nodes, gaps) if with_gaps else nodes
    seq = itertools.count()
    # heap entries: (-sigma, creation order, ranks, parent node index, parent sigma)
    zero = dtype(0)
    heap = [(-(zero + lq[0, 0]), next(seq), (0,), -1, zero)]
    while heap and len(nodes) < budget:
        neg, _, ranks, parent, psig = heapq.heappop(heap)
        sigma = -neg
        gaps.append(float(sigma) - float(-heap[0][0]) if heap else np.inf)
        me = len(nodes)
        nodes.append((ranks, sigma, parent))
        d, r = len(ranks), ranks[-1]
        if r + 1 < K:       # next sibling: same prefix, next rank at this depth
            if score == "incremental":
                s = dtype(dtype(sigma - lq[d - 1, r]) + lq[d - 1, r + 1])
            else:
                s = dtype(psig + lq[d - 1, r + 1])
            heapq.heappush(heap, (-s, next(seq), ranks[:-1] + (r + 1,), parent, psig))
        if d < D:           # first child: best token at the next depth
            s = dtype(sigma + lq[d, 0])
            heapq.heappush(heap, (-s, next(seq), ranks + (0,), me, sigma))
    return (nodes, gaps) if with_gaps else nodes


def tree_tokens(nodes, ids: np.ndarray):
    """Token of every node: ids[depth-1][last rank] ([DDT] §3.4.4: a rank tuple names one token per depth)."""
    return [int(ids[len(r) - 1, r[-1]]) for r, _, _ in nodes]


def brute_force_top(logp: np.ndarray, budget: int):
    """All rank tuples of depth 1..D over the K columns, scored by sum of log-probabilities, best `budget`
    of them (Proposition 2's definition, enumerated; tiny D and K only).  Returns (ranks, sigma) pairs."""
    lq = np.asarray(logp, dtype=np.float64)
    D, K = lq.shape
    allp = []
    for d in range(1, D + 1):
        for ranks in itertools.product(range(K), repeat=d):
            allp.append((ranks, float(sum(lq[i, r] for i, r in enumerate(ranks)))))
    allp.sort(key=lambda t: -t[1])
    return allp[:budget]


def acceptance_length(tree_prefixes: set, y) -> int:
    """alpha_T(y): the longest prefix of y that is a node of T ([DDT] §3.4.3)."""
    a = 0
    for d in range(1, len(y) + 1):
        if tuple(y[:d]) in tree_prefixes:
            a = d
        else:
            break
    return a


def expected_acceptance_enumerated(q: np.ndarray, tree_prefixes: set) -> float:
    """E_{Y~Q}[alpha_T(Y)] by enumerating every continuation Y of the factorised Q = prod_i q_i
    (q: [D, V] probabilities; tiny D and V only)."""
    D, V = q.shape
    e = 0.0
    for y in itertools.product(range(V), repeat=D):
        p = float(np.prod([q[i, y[i]] for i in range(D)]))
        e += p * acceptance_length(tree_prefixes, y)
    return e


def verify_walk(node_token, node_parent, target_next):
    """Greedy verifier walk ([DDT] §3.4.5).  target_next[0] is the target's choice after the root, and
    target_next[i + 1] its choice after node i's prefix.  Returns (accepted node indices, bonus token)."""
    children = {}
    for i, (t, p) in enumerate(zip(node_token, node_parent)):
        children.setdefault(p, {})[t] = i
    cur, path = -1, []
    while True:
        y = int(target_next[cur + 1])
        nxt = children.get(cur, {}).get(y)
        if nxt is None:
            return path, y
        path.append(nxt)
        cur = nxt

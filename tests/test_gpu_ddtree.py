"""DDTree kernels against the oracle ([DDT] = "Accelerating Speculative Decoding with Block Diffusion Draft
Trees"): the wide top-K (ids exact, log-probs to float32 rounding, ties by id), the best-first tree, the
verifier walk (exact), and the whole chain on a drafter pass.

The tree is checked against the fp64 oracle, which follows Algorithm 1's update rules ([DDT] §3.4.4):
node for node up to the first pop whose fp64 margin (popped score minus the best score left in the heap) is
within float32 error, and beyond it by what Proposition 2 fixes -- the same number of nodes, every node of
the fp64 top-B above the guard band present, no node below it, prefix-closed, distinct and popped in
non-increasing order.  As a secondary check the kernel's float32 decisions are replayed (float32 path sums)
and compared score bit for score bit."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import ddtree as T

pytestmark = pytest.mark.gpu


def _mods():
    import torch
    assert torch.cuda.is_available()
    from block_diffusion_drafter_forward_amd import dflash as D, session as S
    return torch, D, S


def _topk_gpu(torch, D, lg, k):
    rows, V = lg.shape
    x = torch.from_numpy(np.ascontiguousarray(lg.astype(np.float32))).cuda()
    ids = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    lp = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    nws = D.dflash_topk_logprobs_workspace_bytes(rows, V, k)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    D.check(D.dflash_topk_logprobs(rows, V, k, x.data_ptr(), V, ids.data_ptr(), lp.data_ptr(), ws.data_ptr(), nws,
                                   D._stream()), "topk")
    torch.cuda.synchronize()
    return ids.cpu().numpy(), lp.cpu().numpy()


@pytest.mark.parametrize("k", [1, 8, 100, 1000, 1024])
def test_topk_logprobs_matches_oracle(k):
    torch, D, S = _mods()
    rng = np.random.default_rng(500 + k)
    V = 5003
    lg = rng.normal(0.0, 2.0, size=(6, V)).astype(np.float32)
    lg[1] = np.round(lg[1] * 2) / 2          # heavy ties: half-integer levels
    lg[2] = 0.5                              # every logit equal
    lg[3, rng.choice(V, 40, replace=False)] = lg[3].max() + 1.0  # a 40-way tie at the top
    lg[4] = -lg[4]                           # negative keys dominate the order
    ids, lp = _topk_gpu(torch, D, lg, k)
    want_ids, want_lp = T.topk_logprobs(lg.astype(np.float64), k)
    np.testing.assert_array_equal(ids, want_ids)
    assert np.all(np.abs(lp - want_lp) <= 2e-5 + 2e-6 * np.abs(want_lp))


@pytest.mark.parametrize("rows,V,k", [(16, 151936, 1024), (16, 151936, 16), (1, 151936, 1000), (3, 65537, 257),
                                      (256, 5003, 64), (40, 2000, 1024)])
def test_topk_logprobs_split_rows_match_oracle(rows, V, k):
    """Row counts that split each row over many workgroups (few rows, the drafter's 16 block rows at the full
    vocabulary) and ones that do not (256 rows), with ties inside and across chunks: heavy ties (left to the
    merge's sort) and few-way ties (ordered by id in its counting sort)."""
    torch, D, S = _mods()
    rng = np.random.default_rng(rows * 7 + V + k)
    lg = rng.normal(0.0, 2.5, size=(rows, V)).astype(np.float32)
    lg[0] = np.round(lg[0] * 4) / 4                                  # ties everywhere, across chunk borders
    if rows > 1:
        lg[1] = -3.0                                                # one value: the smallest ids win
    if rows > 2:
        lg[2, rng.choice(V, min(V, 3 * k), replace=False)] = 30.0   # 3k-way tie at the top
    if rows > 3:
        lg[3] = np.round(lg[3] * 64) / 64                           # few-way ties (1/64 steps)
    ids, lp = _topk_gpu(torch, D, lg, k)
    want_ids, want_lp = T.topk_logprobs(lg.astype(np.float64), k)
    np.testing.assert_array_equal(ids, want_ids)
    assert np.all(np.abs(lp - want_lp) <= 2e-5 + 2e-6 * np.abs(want_lp))


def _sorted_logprobs(rng, batch, depth, K, V=3000):
    lg = rng.normal(0.0, 2.5, size=(batch * depth, V))
    ids, lp = T.topk_logprobs(lg, K)
    return ids.reshape(batch, depth, K).astype(np.int32), lp.reshape(batch, depth, K).astype(np.float32)


def _build_gpu(torch, D, ids, lp, budget):
    batch, depth, K = lp.shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    lpd, idd = dev(lp), dev(ids)
    tok = torch.empty((batch, budget), dtype=torch.int32, device="cuda")
    par = torch.empty_like(tok)
    dep = torch.empty_like(tok)
    lq = torch.empty((batch, budget), dtype=torch.float32, device="cuda")
    n = torch.empty(batch, dtype=torch.int32, device="cuda")
    D.check(D.dflash_ddtree_build(batch, depth, K, lpd.data_ptr(), idd.data_ptr(), depth * K, budget, tok.data_ptr(),
                                  par.data_ptr(), dep.data_ptr(), lq.data_ptr(), n.data_ptr(), D._stream()), "build")
    torch.cuda.synchronize()
    return tok.cpu().numpy(), par.cpu().numpy(), dep.cpu().numpy(), lq.cpu().numpy(), n.cpu().numpy()


def check_tree_fp64(tok, par, dep, n, ids, lp, budget):
    """The GPU tree of one request against the fp64 oracle on the same float32 log-probabilities.  Returns
    the number of leading pops compared node for node."""
    lp64 = lp.astype(np.float64)
    Dd, K = lp64.shape
    nodes, gaps = T.build_tree(lp64, budget, with_gaps=True)
    assert n == len(nodes)
    # rank tuples and exact scores of the GPU's nodes
    rank_of = [{int(t): r for r, t in enumerate(ids[d])} for d in range(Dd)]
    ranks, sig = [], np.empty(n)
    for i in range(n):
        p, d = int(par[i]), int(dep[i])
        assert -1 <= p < i and 1 <= d <= Dd and d == (1 if p < 0 else int(dep[p]) + 1)
        tup = (() if p < 0 else ranks[p]) + (rank_of[d - 1][int(tok[i])],)
        ranks.append(tup)
        sig[i] = sum(lp64[j, r] for j, r in enumerate(tup))
    # A float32 path sum of d <= Dd non-positive terms errs by at most d * 2^-24 |sigma| (every partial sum is
    # smaller in magnitude than the node's score); two compared scores together by twice that.  Scores of
    # the popped nodes and of the candidates they were compared with lie above the lowest one seen here
    # minus the largest single drop.
    low = min(sig.min(), min(s for _, s, _ in nodes)) - np.abs(lp64).max()
    eps = Dd * 2.0 ** -23 * (abs(low) + 1.0)
    want_tok = T.tree_tokens(nodes, ids)
    amb = [i for i, g in enumerate(gaps) if g <= eps]
    head = amb[0] + 1 if amb else n          # pops 0..amb[0] are decided before any ambiguous choice
    np.testing.assert_array_equal(tok[:head], want_tok[:head])
    np.testing.assert_array_equal(par[:head], [p for _, _, p in nodes[:head]])
    np.testing.assert_array_equal(dep[:head], [len(r) for r, _, _ in nodes[:head]])
    # Proposition 2: the B best prefixes, up to the guard band around the B-th score
    assert len(set(ranks)) == n
    assert np.all(np.diff(sig) <= eps)
    sig_b = float(nodes[-1][1])
    have = set(ranks)
    for r, s, _ in nodes:
        if s > sig_b + eps:
            assert r in have, (r, s, sig_b)
    assert sig.min() >= sig_b - eps
    return head


@pytest.mark.parametrize("depth,K,budget", [(15, 64, 1), (15, 64, 16), (15, 256, 256), (15, 1024, 1000),
                                            (6, 512, 2047), (3, 3, 100), (1, 50, 64), (16, 8, 512)])
def test_ddtree_build_matches_oracle(depth, K, budget):
    torch, D, S = _mods()
    rng = np.random.default_rng(600 + depth * 7 + K + budget)
    batch = 3
    ids, lp = _sorted_logprobs(rng, batch, depth, K)
    tok, par, dep, lq, n = _build_gpu(torch, D, ids, lp, budget)
    for b in range(batch):
        head = check_tree_fp64(tok[b], par[b], dep[b], int(n[b]), ids[b], lp[b], budget)
        assert head >= min(int(n[b]), 8)
        # secondary: the kernel's own float32 decisions, replayed, score bit for score bit
        nodes = T.build_tree(lp[b], budget, dtype=np.float32, score="path_sum")
        assert n[b] == len(nodes) == min(budget, sum(K ** d for d in range(1, depth + 1)))
        np.testing.assert_array_equal(tok[b, :n[b]], T.tree_tokens(nodes, ids[b]))
        np.testing.assert_array_equal(par[b, :n[b]], [p for _, _, p in nodes])
        np.testing.assert_array_equal(dep[b, :n[b]], [len(r) for r, _, _ in nodes])
        np.testing.assert_array_equal(lq[b, :n[b]].view(np.uint32), np.array([s for _, s, _ in nodes], np.float32).view(np.uint32))
        # pops non-increasing, prefix-closed
        assert np.all(np.diff(lq[b, :n[b]]) <= 0)
        assert np.all(par[b, :n[b]] < np.arange(n[b]))


def _tie_logprobs(rng, kind, batch, depth, K):
    """Sorted per-depth log-probabilities with exact float32 score ties: rounded to 2^-10 (short runs of equal
    scores), to 2^-3 (long runs), all equal, or one dominant token per depth."""
    if kind == "peaked":
        lg = rng.normal(0.0, 1.0, size=(batch * depth, 3000))
        lg[:, 0] += 9.0
        ids, lp = T.topk_logprobs(lg, K)
        return ids.reshape(batch, depth, K).astype(np.int32), lp.reshape(batch, depth, K).astype(np.float32)
    ids, lp = _sorted_logprobs(rng, batch, depth, K)
    if kind == "q10":
        lp = (np.round(lp.astype(np.float64) * 1024) / 1024).astype(np.float32)
    elif kind == "q3":
        lp = (np.round(lp.astype(np.float64) * 8) / 8).astype(np.float32)
    elif kind == "const":
        lp = np.full_like(lp, -np.log(K))
    return ids, lp


def _check_f32(tok, par, dep, lq, n, ids, lp, budget):
    nodes = T.build_tree(lp, budget, dtype=np.float32, score="path_sum")
    assert n == len(nodes)
    np.testing.assert_array_equal(tok[:n], T.tree_tokens(nodes, ids))
    np.testing.assert_array_equal(par[:n], [p for _, _, p in nodes])
    np.testing.assert_array_equal(dep[:n], [len(r) for r, _, _ in nodes])
    np.testing.assert_array_equal(lq[:n].view(np.uint32), np.array([s for _, s, _ in nodes], np.float32).view(np.uint32))


@pytest.mark.parametrize("kind", ["q10", "q3", "const", "peaked"])
@pytest.mark.parametrize("depth,K,budget", [(15, 1024, 1024), (6, 512, 2047), (16, 8, 512), (3, 3, 100)])
def test_ddtree_build_with_score_ties(kind, depth, K, budget):
    """Exact float32 score ties: equal scores pop in creation order ([DDT] §3.4.4), whichever way the tree is
    built (the parallel selection orders short runs itself and hands long ones to the heap)."""
    torch, D, S = _mods()
    rng = np.random.default_rng(900 + depth + K + budget + len(kind))
    ids, lp = _tie_logprobs(rng, kind, 2, depth, K)
    tok, par, dep, lq, n = _build_gpu(torch, D, ids, lp, budget)
    for b in range(2):
        _check_f32(tok[b], par[b], dep[b], lq[b], int(n[b]), ids[b], lp[b], budget)


def _select_gpu(torch, D, ids, lp, budget):
    batch, depth, K = lp.shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    lpd, idd = dev(lp), dev(ids)
    tok = torch.empty((batch, budget), dtype=torch.int32, device="cuda")
    par, dep = torch.empty_like(tok), torch.empty_like(tok)
    lq = torch.empty((batch, budget), dtype=torch.float32, device="cuda")
    n = torch.empty(batch, dtype=torch.int32, device="cuda")
    D.check(D.dflash_ddtree_select(batch, depth, K, lpd.data_ptr(), idd.data_ptr(), depth * K, budget,
                                   tok.data_ptr(), par.data_ptr(), dep.data_ptr(), lq.data_ptr(), n.data_ptr(),
                                   D._stream()), "select")
    torch.cuda.synchronize()
    return tok.cpu().numpy(), par.cpu().numpy(), dep.cpu().numpy(), lq.cpu().numpy(), n.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "q10", "peaked", "q3", "const"])
@pytest.mark.parametrize("depth,K,budget", [(15, 1024, 1024), (15, 64, 16), (6, 512, 2047), (16, 8, 512),
                                            (1, 50, 64), (2, 1, 5), (15, 32, 2047)])
def test_ddtree_select_decides_and_matches(kind, depth, K, budget):
    """The parallel selection alone: it must decide every request with continuous scores or short runs of
    equal scores, and whatever it decides is Algorithm 1's pop order, score bit for score bit."""
    torch, D, S = _mods()
    rng = np.random.default_rng(1000 + depth * 3 + K + budget + len(kind))
    if kind == "normal":
        ids, lp = _sorted_logprobs(rng, 3, depth, K)
    else:
        ids, lp = _tie_logprobs(rng, kind, 3, depth, K)
    tok, par, dep, lq, n = _select_gpu(torch, D, ids, lp, budget)
    for b in range(3):
        if kind in ("normal", "q10", "peaked"):
            assert n[b] != -1
        if n[b] != -1:
            _check_f32(tok[b], par[b], dep[b], lq[b], int(n[b]), ids[b], lp[b], budget)


def test_ddtree_select_declines_unsorted_rows():
    """Rows that are not non-increasing log-probabilities are left to the heap (n_nodes = -1), and the full
    build still returns the heap's pops."""
    torch, D, S = _mods()
    rng = np.random.default_rng(77)
    ids, lp = _sorted_logprobs(rng, 2, 5, 64)
    lp[0, 2, 10], lp[0, 2, 11] = lp[0, 2, 11], lp[0, 2, 10] - 0.5   # request 0: one row out of order
    lp[1, 0, 0] = 0.25                                              # request 1: a log-probability above 0
    tok, par, dep, lq, n = _select_gpu(torch, D, ids, lp, 200)
    assert list(n) == [-1, -1]
    tok, par, dep, lq, n = _build_gpu(torch, D, ids, lp, 200)
    for b in range(2):
        nodes = T.build_tree(lp[b], 200, dtype=np.float32, score="path_sum")
        assert n[b] == len(nodes)
        np.testing.assert_array_equal(par[b, :n[b]], [p for _, _, p in nodes])
        np.testing.assert_array_equal(tok[b, :n[b]], T.tree_tokens(nodes, ids[b]))


@pytest.mark.parametrize("seed", range(4))
def test_ddtree_walk_matches_oracle(seed):
    torch, D, S = _mods()
    rng = np.random.default_rng(700 + seed)
    batch, depth, K, budget = 4, 12, 32, 300
    ids, lp = _sorted_logprobs(rng, batch, depth, K)
    tok, par, dep, lq, n = _build_gpu(torch, D, ids, lp, budget)
    # target choices: follow the tree's first child with probability 0.8, else a token outside the tree
    tgt = rng.integers(0, 3000, size=(batch, budget + 1)).astype(np.int32)
    for b in range(batch):
        first_child = {}
        for i in range(n[b]):
            first_child.setdefault(int(par[b, i]), int(tok[b, i]))
        for node in range(-1, n[b]):
            if node in first_child and rng.random() < 0.8:
                tgt[b, node + 1] = first_child[node]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    alen = torch.empty(batch, dtype=torch.int32, device="cuda")
    anodes = torch.full((batch, depth), -1, dtype=torch.int32, device="cuda")
    bonus = torch.empty(batch, dtype=torch.int32, device="cuda")
    keep = [dev(a) for a in (tok, par, n, tgt)]  # held until the kernel has run
    D.check(D.dflash_ddtree_walk(batch, budget, depth, keep[0].data_ptr(), keep[1].data_ptr(), keep[2].data_ptr(),
                                 keep[3].data_ptr(), alen.data_ptr(), anodes.data_ptr(), bonus.data_ptr(),
                                 D._stream()), "walk")
    torch.cuda.synchronize()
    alen, anodes, bonus = alen.cpu().numpy(), anodes.cpu().numpy(), bonus.cpu().numpy()
    for b in range(batch):
        path, y = T.verify_walk(tok[b, :n[b]].tolist(), par[b, :n[b]].tolist(), tgt[b])
        assert alen[b] == len(path) and list(anodes[b, :alen[b]]) == path and bonus[b] == y


def test_ddtree_chain_on_a_drafter_pass():
    """Drafter pass -> full logits -> per-depth top-K -> tree, checked against the oracle on the same logits."""
    torch, D, S = _mods()
    wl = W.by_name("small-bf16-paged-b2")
    s = wl.shape
    g = S.GpuWorkload(wl)
    g.prefill()
    B, L, V = wl.batch, s.block_len, s.vocab
    logits = torch.zeros((B, L, V), dtype=torch.float32, device="cuda")
    g.draft(logits=logits)
    torch.cuda.synchronize()
    budget = 128
    K = min(budget, V)
    ids = torch.empty((B, L, K), dtype=torch.int32, device="cuda")
    lp = torch.empty((B, L, K), dtype=torch.float32, device="cuda")
    nws = D.dflash_topk_logprobs_workspace_bytes(B * L, V, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    D.check(D.dflash_topk_logprobs(B * L, V, K, logits.data_ptr(), V, ids.data_ptr(), lp.data_ptr(), ws.data_ptr(),
                                   nws, D._stream()), "topk")
    tok = torch.empty((B, budget), dtype=torch.int32, device="cuda")
    par, dep = torch.empty_like(tok), torch.empty_like(tok)
    lq = torch.empty((B, budget), dtype=torch.float32, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    # depth d reads block row d (rows 1 .. L-1): start one row in, request stride L * K
    D.check(D.dflash_ddtree_build(B, L - 1, K, lp.data_ptr() + 4 * K, ids.data_ptr() + 4 * K, L * K, budget,
                                  tok.data_ptr(), par.data_ptr(), dep.data_ptr(), lq.data_ptr(), n.data_ptr(),
                                  D._stream()), "build")
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    for b in range(B):
        want_ids, want_lp = T.topk_logprobs(lg[b], K)
        np.testing.assert_array_equal(ids[b].cpu().numpy(), want_ids)
        lpb = lp[b, 1:].cpu().numpy()
        check_tree_fp64(tok[b].cpu().numpy(), par[b].cpu().numpy(), dep[b].cpu().numpy(), int(n[b].item()),
                        want_ids[1:], lpb, budget)
        nodes = T.build_tree(lpb, budget, dtype=np.float32, score="path_sum")
        assert n[b].item() == len(nodes)
        np.testing.assert_array_equal(tok[b, :len(nodes)].cpu().numpy(), T.tree_tokens(nodes, want_ids[1:]))
        np.testing.assert_array_equal(par[b, :len(nodes)].cpu().numpy(), [p for _, _, p in nodes])

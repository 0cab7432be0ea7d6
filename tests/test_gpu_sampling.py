"""GPU parity of the temperature-1 path (drafting by Gumbel-max sampling, verification by modified rejection
sampling) against the oracle of ``oracle/sampling.py``, through the C ABI.

Criteria:
* drafting: the sampled tokens equal the oracle's Gumbel-max samples on the oracle's fp64 logits wherever
  the oracle's gap between the best and second-best perturbed score exceeds 1e-2 (as for greedy tokens), and
  equal the oracle's samples on the kernel's own logits wherever that gap exceeds 1e-4 (float32 rounding of
  the noise); logits and top-k outputs are bit-identical to the greedy pass's;
* verification: tau and the next token equal the oracle's wherever every decision the oracle took has a
  margin above 1e-3 (acceptance tests |ln u - (ln p - ln q)| and the final sample's top-2 gap); the rest are
  counted and must be rare;
* distribution: over many independent requests of one call, the committed tokens follow the exact law of a
  cycle (chi-square), which the oracle's enumeration ties to the target's own law.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import sampling as S

pytestmark = pytest.mark.gpu

MARGIN = 1e-2
VERIFY_MARGIN = 1e-3


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


# ------------------------------------------------------------------------------------------------------
# drafting at temperature 1
# ------------------------------------------------------------------------------------------------------
CASES = {}


@pytest.fixture(scope="module", params=["small-bf16-b1", "small-bf16-paged-b2", "small-gqa8-b3", "small-fp32-b2",
                                        "small-bf16-l10-b3", "small-bf16-serve9"])
def drafted(request):
    """Greedy pass with logits, and the oracle's fp64 logits, for one small workload."""
    torch = _torch()
    from block_diffusion_drafter_forward_amd import session
    if request.param not in CASES:
        CASES.clear()
        wl = W.by_name(request.param)
        s = wl.shape
        weights = wl.weights()
        print(f"[sampling] {wl.name}: prefill and greedy pass", flush=True)
        g = session.GpuWorkload(wl, weights=weights)
        g.prefill()
        B, L, V = wl.batch, s.block_len, s.vocab
        logits = torch.zeros((B, L, V), dtype=torch.float32, device="cuda")
        g.draft(logits=logits)
        torch.cuda.synchronize()
        greedy = dict(logits=logits.cpu().numpy(), topk_ids=g.topk_ids.cpu().numpy(), topk_lp=g.topk_lp.cpu().numpy())
        kv = [O.inject(weights, s, wl.features(r, int(g.ctx[r])), 0) for r in range(B)]
        ref = O.draft_block(weights, s, kv, wl.block_tokens(), wl.top_k)
        CASES[request.param] = (wl, g, greedy, ref)
    return CASES[request.param]


@pytest.mark.parametrize("seed", [12345, (7 << 32) + 99])
def test_draft_sample_matches_oracle(drafted, seed):
    torch = _torch()
    wl, g, greedy, ref = drafted
    s = wl.shape
    B, L, V = wl.batch, s.block_len, s.vocab
    logits = torch.full((B, L, V), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[sampling] {wl.name}: sampled pass, seed {seed:#x}", flush=True)
    g.draft_sample(seed, logits=logits)
    torch.cuda.synchronize()
    assert g.error_word() == 0
    lg = logits.cpu().numpy()
    tok = g.tokens.cpu().numpy().reshape(-1)
    # the sampled pass computes exactly what the greedy pass computes, and only the choice differs
    assert np.array_equal(lg, greedy["logits"])
    assert np.array_equal(g.topk_ids.cpu().numpy(), greedy["topk_ids"])
    assert np.array_equal(g.topk_lp.cpu().numpy(), greedy["topk_lp"])
    # against the oracle's fp64 logits
    ids, gap = S.sample_rows(ref["logits"].reshape(B * L, V), seed)
    ok = gap > MARGIN
    print(f"[sampling] rows checked {ok.sum()}/{ok.size}, mismatched {(tok[ok] != ids[ok]).sum()}", flush=True)
    assert ok.mean() > 0.8
    np.testing.assert_array_equal(tok[ok], ids[ok])
    # against the kernel's own logits: only float32 rounding of the noise separates the two
    ids2, gap2 = S.sample_rows(lg.reshape(B * L, V).astype(np.float64), seed)
    ok2 = gap2 > 1e-4
    assert ok2.mean() > 0.95
    np.testing.assert_array_equal(tok[ok2], ids2[ok2])


def test_draft_sample_is_deterministic_and_seeded(drafted):
    torch = _torch()
    wl, g, greedy, ref = drafted
    runs = []
    for seed in (5, 5, 6, 5 + (1 << 32)):
        g.draft_sample(seed)
        torch.cuda.synchronize()
        runs.append(g.tokens.cpu().numpy().copy())
    assert np.array_equal(runs[0], runs[1])
    assert not np.array_equal(runs[0], runs[2]) or runs[0].size < 4
    assert not np.array_equal(runs[0], runs[3]) or runs[0].size < 4   # the seed's high word keys the stream


# ------------------------------------------------------------------------------------------------------
# verification at temperature 1
# ------------------------------------------------------------------------------------------------------


def _verify_gpu(drafts, q, p, seed):
    torch = _torch()
    from block_diffusion_drafter_forward_amd import dflash as D
    B, n = drafts.shape
    V = p.shape[-1]
    dd = torch.as_tensor(np.ascontiguousarray(drafts, dtype=np.int32), device="cuda")
    qd = torch.as_tensor(np.ascontiguousarray(q, dtype=np.float32), device="cuda") if n else \
        torch.zeros((B, 0, V), dtype=torch.float32, device="cuda")
    pd = torch.as_tensor(np.ascontiguousarray(p, dtype=np.float32), device="cuda")
    tau = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(D.verify_sample_workspace_bytes(B, n, V) + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    D.verify_sample(dd, qd, pd, seed, tau, nxt, ws[off:])
    torch.cuda.synchronize()
    return tau.cpu().numpy(), nxt.cpu().numpy()


def _synthetic(rng, B, n, V, spread, corr, scale=2.0):
    """Drafter logits q, target logits p = q + independent noise (corr controls agreement), drafts drawn from
    softmax(q) on the host, and a few out-of-vocabulary drafts."""
    q = rng.normal(0, scale, size=(B, max(n, 1), V))[:, :n]
    p = np.concatenate([q, rng.normal(0, scale, size=(B, 1, V))], axis=1) + rng.normal(0, spread, size=(B, n + 1, V))
    p = corr * p + (1 - corr) * rng.normal(0, scale, size=p.shape)
    q = q.astype(np.float32).astype(np.float64)
    p = p.astype(np.float32).astype(np.float64)
    drafts = np.zeros((B, n), dtype=np.int64)
    for b in range(B):
        for j in range(n):
            pr = np.exp(S.log_softmax(q[b, j]))
            drafts[b, j] = rng.choice(V, p=pr / pr.sum())
    return drafts, q, p


@pytest.mark.parametrize("B,n,V,spread,corr", [
    (4, 15, 1000, 0.3, 1.0), (3, 7, 5003, 1.0, 1.0), (8, 1, 4096, 0.5, 0.8), (2, 15, 151936, 0.2, 1.0),
    (5, 0, 777, 0.0, 1.0), (2, 63, 300, 0.05, 1.0), (16, 15, 9000, 2.0, 0.5),
])
def test_verify_sample_matches_oracle(B, n, V, spread, corr):
    rng = np.random.default_rng(1000 + B * 131 + n * 7 + V)
    drafts, q, p = _synthetic(rng, B, n, V, spread, corr)
    if n >= 2:
        drafts[0, n // 2] = -1            # out of the vocabulary: a rejection at that position
        if B > 1:
            drafts[1, 0] = V + 5
    checked = 0
    taus = []
    for seed in (3, 2 ** 40 + 17):
        print(f"[verify] B={B} n={n} V={V} seed={seed:#x}", flush=True)
        tau, nxt = _verify_gpu(drafts, q, p, seed)
        for b in range(B):
            t_ref, n_ref, guard = S.speculative_verify(drafts[b], q[b], p[b], seed, b)
            taus.append(int(tau[b]))
            if guard <= VERIFY_MARGIN:
                continue
            checked += 1
            assert (tau[b], nxt[b]) == (t_ref, n_ref), (b, tau[b], nxt[b], t_ref, n_ref, guard)
    assert checked >= 0.9 * 2 * B
    assert all(1 <= t <= n + 1 for t in taus)


def test_verify_sample_identical_rows_keep_everything():
    """p == q: every acceptance test passes (ln u < 0), so tau = n + 1 and the next token is the bonus
    sample of the target's last row."""
    rng = np.random.default_rng(9)
    B, n, V = 6, 15, 2000
    q = rng.normal(0, 2, size=(B, n, V)).astype(np.float32).astype(np.float64)
    p = np.concatenate([q, rng.normal(0, 2, size=(B, 1, V)).astype(np.float32)], axis=1)
    drafts = rng.integers(0, V, size=(B, n))
    tau, nxt = _verify_gpu(drafts, q, p, 11)
    assert np.all(tau == n + 1)
    for b in range(B):
        t_ref, n_ref, guard = S.speculative_verify(drafts[b], q[b], p[b], 11, b)
        assert t_ref == n + 1
        if guard > VERIFY_MARGIN:
            assert nxt[b] == n_ref


def test_verify_sample_output_law():
    """The committed tokens of many independent requests (one call, one Philox stream per request) follow the
    exact law of one cycle, which the oracle pins to the target's own law by enumeration."""
    rng = np.random.default_rng(2024)
    V, n, B = 4, 2, 40000
    qprob = rng.dirichlet(0.8 * np.ones(V), size=n)
    table = {}

    def target(prefix):
        if prefix not in table:
            table[prefix] = rng.dirichlet(0.8 * np.ones(V))
        return table[prefix]

    exact = S.exact_cycle_outcomes(qprob, target)
    drafts = np.stack([rng.choice(V, size=B, p=qprob[j]) for j in range(n)], axis=1)
    q = np.broadcast_to(np.log(qprob), (B, n, V))
    p = np.stack([np.log(np.stack([target(tuple(int(t) for t in drafts[b, :j])) for j in range(n + 1)]))
                  for b in range(B)])
    tau, nxt = _verify_gpu(drafts, q, p, 77)
    counts = {}
    for b in range(B):
        key = tuple(int(t) for t in drafts[b, :tau[b] - 1]) + (int(nxt[b]),)
        counts[key] = counts.get(key, 0) + 1
    stat, cells = 0.0, 0
    for key, pr in exact.items():
        e = B * pr
        if e >= 5:
            stat += (counts.get(key, 0) - e) ** 2 / e
            cells += 1
    assert set(counts) <= set(exact)
    dof = cells - 1
    bound = dof * (1 - 2 / (9 * dof) + 3.09 * math.sqrt(2 / (9 * dof))) ** 3   # chi-square 99.9% quantile
    assert stat < bound, (stat, dof)

"""GPU parity of the tree-attention kernels against the dense masked oracle (``oracle/tree_attention.py``),
through the C ABI.

Criterion: every output element within |err| <= 1e-2 |ref| + 2^-8 max|v|.  The oracle computes in fp64 and
rounds the output to bfloat16; the kernel rounds the rotated q / k to bfloat16 from float32 (a float32 and
an fp64 rotation can round to neighbouring bfloat16 values), carries the context probabilities into the
MFMA as bfloat16 (relative error 2^-9 per weight, so at most 2^-9 max|v| on the output), and rounds its
float32 output to bfloat16 (one step, 2^-8 relative, inside the 1e-2 |ref| term).  A wrong mask, position
or head is far outside: the cases with little or no context make the tree part dominate, and one extra or
missing key among a few dozen moves the output by a sizeable fraction of rms(v) (~1, while 2^-8 max|v| is
below 0.02).
"""
import numpy as np
import pytest

import oracle as O
from oracle import ddtree as DT
from oracle import tree_attention as TA

pytestmark = pytest.mark.gpu

THETA = 1e6


def _bits(x):
    """bfloat16 bit patterns of values that are already bfloat16 (fp64 in)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16(rng, shape, scale=1.0):
    return O.bf16_round(rng.normal(0, scale, size=shape))


def _random_parents(rng, T, max_depth=15):
    parent = np.full(T, -1)
    depth = np.zeros(T, dtype=int)
    for i in range(1, T):
        while True:
            p = int(rng.integers(0, i))
            if depth[p] < max_depth:
                break
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def _ddtree_parents(rng, budget, depth=15):
    """Parents of the flattened tree that Algorithm 1 pops for random drafter marginals (token 0 = root)."""
    K = min(budget, 64)
    lq = np.log(rng.dirichlet(0.3 * np.ones(400), size=depth))
    lq = np.sort(lq, axis=1)[:, ::-1][:, :K]
    nodes = DT.build_tree(lq, budget)
    return np.array([-1] + [p + 1 for _, _, p in nodes])


def _to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def _run(rng, n_tokens, parents, ctx, nq, nkv, theta=THETA, qscale=1.5, max_tokens=None, oracle=True,
         bad_page=None):
    """Build the synthetic layer, run the kernel, return (gpu out [B, T, nq, d] fp64, oracle outs, max |v|, err)."""
    import torch
    from block_diffusion_drafter_forward_amd import dflash as D
    B = len(n_tokens)
    T = max_tokens or max(n_tokens)
    d = 128
    q = _bf16(rng, (B, T, nq, d), qscale)
    k = _bf16(rng, (B, T, nkv, d), qscale)
    v = _bf16(rng, (B, T, nkv, d))
    par = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        par[b, :n_tokens[b]] = parents[b][:n_tokens[b]]
        par[b, n_tokens[b]:] = 12345       # never read
    max_ctx = max(ctx) if max(ctx) > 0 else 0
    max_pages = max(1, (max_ctx + 15) // 16)
    n_pages = B * max_pages + 3
    perm = rng.permutation(n_pages)
    pt = perm[: B * max_pages].reshape(B, max_pages).astype(np.int32)
    kpool = np.zeros((n_pages, nkv, 16, d))
    vpool = np.zeros((n_pages, nkv, d, 16))
    kctx, vctx = [], []
    for b in range(B):
        kc = _bf16(rng, (ctx[b], nkv, d), qscale)
        vc = _bf16(rng, (ctx[b], nkv, d))
        kctx.append(kc)
        vctx.append(vc)
        for p in range(ctx[b]):
            kpool[pt[b, p // 16], :, p % 16, :] = kc[p]
            vpool[pt[b, p // 16], :, :, p % 16] = vc[p]
    if bad_page is not None:  # (request, page slot): an id past the pool
        pt[bad_page] = n_pages + 7
    out = torch.zeros((B, T, nq, d), dtype=torch.bfloat16, device="cuda")
    nbytes = D.dflash_tree_attention_workspace_bytes(B, T, nq, nkv, d, max_ctx)
    assert nbytes > 0
    ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:]
    print(f"[tree] B={B} T={T} n={list(n_tokens)} ctx={list(ctx)} nq={nq} nkv={nkv} theta={theta}", flush=True)
    D.tree_attention(_to_dev(np.asarray(n_tokens, dtype=np.int32)), _to_dev(par), _to_dev(_bits(q), "bf16"),
                     _to_dev(_bits(k), "bf16"), _to_dev(_bits(v), "bf16"), _to_dev(_bits(kpool), "bf16"),
                     _to_dev(_bits(vpool), "bf16"), _to_dev(pt), _to_dev(np.asarray(ctx, dtype=np.int32)), max_ctx,
                     theta, out, ws)
    torch.cuda.synchronize()
    err = int(ws[:4].view(torch.int32).item()) & 0xFFFFFFFF
    got = out.float().cpu().numpy().astype(np.float64)
    refs = []
    for b in range(B if oracle else 0):
        n = n_tokens[b]
        pb = np.asarray(par[b, :n]).copy()
        pb[0] = -1
        o, _ = TA.tree_attention(q[b, :n], k[b, :n], v[b, :n], pb, kctx[b], vctx[b], theta)
        refs.append(o)
    vmax = max([float(np.abs(v).max())] + [float(np.abs(vc).max()) for vc in vctx if vc.size])
    return got, refs, vmax, err


def _check(got, refs, vmax, n_tokens):
    worst = 0.0
    for b, ref in enumerate(refs):
        n = n_tokens[b]
        diff = np.abs(got[b, :n] - ref)
        bound = 1e-2 * np.abs(ref) + 2.0 ** -8 * vmax
        worst = max(worst, float((diff / bound).max()))
        assert np.all(diff <= bound), (b, float(diff.max()), np.unravel_index(np.argmax(diff - bound), diff.shape))
    print(f"[tree] worst error / bound = {worst:.3f}", flush=True)


@pytest.mark.parametrize("case", [
    dict(n=[17], ctx=[0], nq=32, nkv=8, tree="chain"),
    dict(n=[100, 57], ctx=[1, 37], nq=32, nkv=8, tree="random"),
    dict(n=[300, 1, 129], ctx=[500, 0, 2048], nq=32, nkv=8, tree="random"),
    dict(n=[1025], ctx=[4096], nq=32, nkv=8, tree="ddtree"),
    dict(n=[257, 65], ctx=[20, 3000], nq=32, nkv=8, tree="ddtree"),
    dict(n=[64, 50], ctx=[300, 77], nq=16, nkv=16, tree="random"),
    dict(n=[64, 50], ctx=[300, 77], nq=16, nkv=8, tree="random"),
    dict(n=[40, 33], ctx=[130, 0], nq=64, nkv=8, tree="random"),
    dict(n=[2048], ctx=[16], nq=32, nkv=8, tree="random"),
    # streamed context splits in which a workgroup's rounds run from one request's last token tiles into the
    # next request's first, with ragged contexts
    dict(n=[321, 200, 290], ctx=[1024, 700, 1000], nq=32, nkv=8, tree="ddtree"),
    dict(n=[129, 100, 64], ctx=[4096, 4000, 1500], nq=32, nkv=8, tree="random"),
    dict(n=[513], ctx=[1024], nq=64, nkv=8, tree="ddtree"),                              # streamed, 8 heads per KV head
    dict(n=[257, 180, 97], ctx=[1536, 900, 1400], nq=16, nkv=16, tree="random"),      # streamed across requests, MHA
])
def test_tree_attention_matches_oracle(case):
    rng = np.random.default_rng(sum(case["n"]) * 7 + sum(case["ctx"]) + case["nq"])
    parents = []
    for n in case["n"]:
        if case["tree"] == "chain":
            parents.append(np.arange(n) - 1)
        elif case["tree"] == "ddtree":
            parents.append(_ddtree_parents(rng, n - 1))
        else:
            parents.append(_random_parents(rng, n))
    got, refs, vmax, err = _run(rng, case["n"], parents, case["ctx"], case["nq"], case["nkv"])
    assert err == 0
    _check(got, refs, vmax, case["n"])


def test_tree_attention_rope_off_and_deep_chain():
    rng = np.random.default_rng(77)
    n = [63]
    got, refs, vmax, err = _run(rng, n, [np.arange(63) - 1], [40], 32, 8, theta=0.0)
    assert err == 0
    _check(got, refs, vmax, n)


def test_tree_attention_rows_past_n_tokens_untouched():
    """Rows at or past n_tokens are not written (the output buffer keeps its zeros)."""
    rng = np.random.default_rng(5)
    got, refs, vmax, err = _run(rng, [10, 3], [_random_parents(rng, 10), _random_parents(rng, 3)], [50, 20], 32, 8,
                                max_tokens=40)
    assert err == 0
    _check(got, refs, vmax, [10, 3])
    assert np.all(got[0, 10:] == 0) and np.all(got[1, 3:] == 0)


def test_tree_attention_flags_bad_page_ids():
    """A page id past the pool, in the last workgroup's rounds of a long context, is flagged in the device error
    word (its keys are read from page 0 instead)."""
    from block_diffusion_drafter_forward_amd import dflash as D
    rng = np.random.default_rng(8)
    n = [300, 90]
    par = [_random_parents(rng, 300), _random_parents(rng, 90)]
    _, _, _, err = _run(rng, n, par, [4096, 2500], 32, 8, oracle=False, bad_page=(1, 150))
    assert err == D.DEVERR_PAGE


def test_tree_attention_flags_bad_parent_links():
    """A parent link that does not point to an earlier token is flagged in the device error word; the kernel
    still reads only inside the tree (the link is cut at the root)."""
    from block_diffusion_drafter_forward_amd import dflash as D
    rng = np.random.default_rng(6)
    par = _random_parents(rng, 30)
    par[12] = 12
    _, _, _, err = _run(rng, [30], [par], [40], 32, 8, oracle=False)
    assert err == D.DEVERR_TREE

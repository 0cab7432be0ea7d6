"""Pins of the tree-attention oracle ([DDT] = "Accelerating Speculative Decoding with Block Diffusion Draft
Trees", §3.4.5) against what the page and the mathematics fix:

* a chain tree is ordinary causal attention over [context ; chain] (torch scaled_dot_product_attention with a
  causal-with-prefix mask, rotary embedding by complex multiplication);
* every token's output equals plain attention over [context ; its own root-to-token path] (brute force per
  token, no mask at all);
* the flattening order does not matter (any parents-first relabelling permutes the outputs);
* tokens on other branches are invisible (perturbing them changes nothing, bit for bit);
* position ids are depths: a path gives the same outputs wherever it sits in a larger tree;
* the degenerate trees (root only; no context)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle import tree_attention as TA

THETA = 1e6


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


def _rope_complex(x, pos, theta):
    """Rotary embedding as multiplication of the pairs (x_i, x_{i+d/2}) by e^{i angle} (complex numbers)."""
    d = x.shape[-1]
    ang = O.rope_angles(np.asarray(pos), d, theta)[:, None, :]
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def _case(rng, T, C, n_q=4, n_kv=2, d=16, scale=1.0):
    q = _bf16(rng, (T, n_q, d), scale)
    k = _bf16(rng, (T, n_kv, d), scale)
    v = _bf16(rng, (T, n_kv, d))
    kc = _bf16(rng, (C, n_kv, d), scale)
    vc = _bf16(rng, (C, n_kv, d))
    return q, k, v, kc, vc


def _close(a, b):
    """Equal up to one bfloat16 rounding step (the two sides sum in different orders before rounding)."""
    return np.all(np.abs(a - b) <= 2.0 ** -8 * np.abs(b) + 1e-12)


@pytest.mark.parametrize("T,C", [(1, 5), (6, 0), (9, 13)])
def test_chain_tree_is_causal_attention(T, C):
    rng = np.random.default_rng(10 * T + C)
    q, k, v, kc, vc = _case(rng, T, C)
    parent = np.arange(T) - 1
    o, _ = TA.tree_attention(q, k, v, parent, kc, vc, THETA)
    pos = C + np.arange(T)
    qr = O.bf16_round(_rope_complex(q, pos, THETA))
    kr = O.bf16_round(_rope_complex(k, pos, THETA))
    keys = np.concatenate([kc, kr])
    vals = np.concatenate([vc, v])
    n_q, n_kv = q.shape[1], k.shape[1]
    mask = np.concatenate([np.ones((T, C), bool), np.tril(np.ones((T, T), bool))], axis=1)
    qt = torch.tensor(qr.transpose(1, 0, 2))                                     # [n_q, T, d]
    kt = torch.tensor(keys.transpose(1, 0, 2)).repeat_interleave(n_q // n_kv, 0)
    vt = torch.tensor(vals.transpose(1, 0, 2)).repeat_interleave(n_q // n_kv, 0)
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.tensor(mask)).numpy().transpose(1, 0, 2)
    assert _close(o, O.bf16_round(ref))


@pytest.mark.parametrize("seed,T,C", [(0, 40, 7), (1, 17, 0), (2, 64, 30)])
def test_each_token_sees_exactly_its_path(seed, T, C):
    rng = np.random.default_rng(seed)
    q, k, v, kc, vc = _case(rng, T, C, scale=1.5)
    parent = _random_parents(rng, T)
    o, _ = TA.tree_attention(q, k, v, parent, kc, vc, THETA)
    d = q.shape[-1]
    group = q.shape[1] // k.shape[1]
    for i in range(T):
        path = [i]
        while path[-1] != 0:
            path.append(parent[path[-1]])
        path = path[::-1]
        depth = len(path) - 1
        pos = np.full(len(path), 0) + C + np.arange(len(path))   # the path's tokens sit at depths 0..depth
        qi = O.bf16_round(_rope_complex(q[i:i + 1], [C + depth], THETA))[0]
        kp = O.bf16_round(_rope_complex(k[path], pos, THETA))
        for h in range(q.shape[1]):
            g = h // group
            keys = np.concatenate([kc[:, g], kp[:, g]])
            vals = np.concatenate([vc[:, g], v[path, g]])
            s = keys @ qi[h] / math.sqrt(d)
            w = np.exp(s - s.max())
            ref = (w / w.sum()) @ vals
            assert _close(o[i, h], O.bf16_round(ref)), (i, h)


def test_flattening_order_does_not_matter():
    rng = np.random.default_rng(5)
    T, C = 50, 11
    q, k, v, kc, vc = _case(rng, T, C)
    parent = _random_parents(rng, T)
    o, _ = TA.tree_attention(q, k, v, parent, kc, vc, THETA)
    # a random parents-first relabelling: repeatedly emit a random token whose parent is already placed
    placed, order = {0: 0}, [0]
    frontier = [i for i in range(1, T) if parent[i] == 0]
    while frontier:
        i = frontier.pop(int(rng.integers(len(frontier))))
        placed[i] = len(order)
        order.append(i)
        frontier += [j for j in range(1, T) if parent[j] == i]
    order = np.array(order)
    new_parent = np.array([-1] + [placed[parent[i]] for i in order[1:]])
    o2, _ = TA.tree_attention(q[order], k[order], v[order], new_parent, kc, vc, THETA)
    assert _close(o2, o[order])


def test_other_branches_are_invisible():
    rng = np.random.default_rng(6)
    T, C = 30, 5
    q, k, v, kc, vc = _case(rng, T, C)
    parent = _random_parents(rng, T)
    o, _ = TA.tree_attention(q, k, v, parent, kc, vc, THETA)
    mask = TA.tree_mask(parent)
    for i in (3, 17, 29):
        others = np.where(~mask[i])[0]
        k2, v2 = k.copy(), v.copy()
        k2[others] = _bf16(rng, k2[others].shape, 3.0)
        v2[others] = _bf16(rng, v2[others].shape, 3.0)
        o2, _ = TA.tree_attention(q, k2, v2, parent, kc, vc, THETA)
        assert np.array_equal(o2[i], o[i])
    # and an ancestor does matter
    i = 29
    anc = TA.ancestors_or_self(parent, i)[:-1]
    v3 = v.copy()
    v3[anc] += 1.0
    o3, _ = TA.tree_attention(q, k, v3, parent, kc, vc, THETA)
    assert not np.array_equal(o3[i], o[i])


def test_position_is_depth():
    """The chain 0 -> a -> b keeps its outputs when other branches are inserted before b's position in the
    flattening: each token's position comes from its depth, not its index."""
    rng = np.random.default_rng(8)
    C = 9
    q, k, v, kc, vc = _case(rng, 3, C)
    o_small, _ = TA.tree_attention(q, k, v, np.array([-1, 0, 1]), kc, vc, THETA)
    extra_q, extra_k, extra_v, _, _ = _case(rng, 4, 0)
    # big tree: root, a, x1 (child of root), x2 (child of a), x3, b (child of a), x4
    idx = [0, 1, None, None, None, 2, None]
    parent = np.array([-1, 0, 0, 1, 2, 1, 3])
    qs, ks, vs, e = [], [], [], 0
    for j in idx:
        if j is None:
            qs.append(extra_q[e]); ks.append(extra_k[e]); vs.append(extra_v[e]); e += 1
        else:
            qs.append(q[j]); ks.append(k[j]); vs.append(v[j])
    o_big, _ = TA.tree_attention(np.stack(qs), np.stack(ks), np.stack(vs), parent, kc, vc, THETA)
    assert _close(o_big[[0, 1, 5]], o_small)
    assert list(TA.tree_depths(parent)) == [0, 1, 1, 2, 2, 2, 3]


def test_degenerate_trees():
    rng = np.random.default_rng(9)
    # root only: attends to the context and itself
    q, k, v, kc, vc = _case(rng, 1, 4)
    o, p = TA.tree_attention(q, k, v, np.array([-1]), kc, vc, THETA)
    assert p.shape == (1, 5) and np.all(p > 0)
    # no context: the root attends to itself alone, so its output is its own value (per KV group)
    o0, p0 = TA.tree_attention(q, k, v, np.array([-1]), kc[:0], vc[:0], THETA)
    assert np.allclose(p0, 1.0)
    group = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        assert np.array_equal(o0[0, h], O.bf16_round(v[0, h // group]))

"""Plain CPU oracle of tree attention for DDTree verification.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU-baseline leg may import this module.
The HIP library never calls it and shares no code with it.

Source: "Accelerating Speculative Decoding with Block Diffusion Draft Trees" ([DDT]), §3.4.5 "Verification:
Tree Attention and the Verifier Walk":
  * flattening: the tree's tokens form one sequence; any order works as long as the mask encodes the tree;
  * position ids: every token's position id is its depth in the tree (the root, the bonus token, has 0);
  * tree (ancestor-only) attention: a token attends to the whole past context through the KV cache, to the
    root, to its ancestors and to itself, and to nothing on another branch;
  * one target-model forward pass over the flattened tokens computes every node's output at once.

Readings (where the page leaves a step open):
  T1  Order: token 0 is the root; every other token's parent precedes it (parent[i] < i), which any
      breadth-first or depth-first flattening, and the pop order of the tree builder, satisfies.
  T2  Positions: the position id is an offset after the committed context, so a token at depth d sits at
      absolute position C + d, where C is the request's cached context length (the root takes the position
      the bonus token has in a plain decode step).
  T3  Numerics of the synthetic target layer: the tree tokens' q, k, v arrive as bfloat16 projections
      before the rotary embedding; q and k are rotated at C + depth with the drafter's rotary convention
      (rotate-half pairs, float32 angle) and rounded to bfloat16, as a bfloat16 target keeps them for its
      attention; the cached context K/V are bfloat16 and already rotated at their own positions.
  T4  Attention: scale 1/sqrt(d), softmax over the visible keys, grouped-query heads as in the drafter
      (query head h reads KV head h // (n_q / n_kv)); the output is rounded to bfloat16.

The computation is the definition written out: a dense boolean mask over [context ; tree] keys and one
masked softmax per query row (fp64).
"""
from __future__ import annotations

import math

import numpy as np

from .dflash_ref import bf16_round, rope, softmax_rows, to_f64


def tree_depths(parent) -> np.ndarray:
    """Depth of every token (root 0): one more than its parent's (T1 guarantees parents come first)."""
    parent = np.asarray(parent)
    depth = np.zeros(len(parent), dtype=np.int64)
    for i in range(1, len(parent)):
        assert 0 <= parent[i] < i, "parent links must point to an earlier token"
        depth[i] = depth[parent[i]] + 1
    return depth


def ancestors_or_self(parent, i: int):
    """Tokens on the path from the root to token i, both included, root first."""
    path = [i]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
    return path[::-1]


def tree_mask(parent) -> np.ndarray:
    """mask[i, j] = token i may attend to tree token j: j is an ancestor of i or i itself ([DDT] §3.4.5)."""
    T = len(parent)
    m = np.zeros((T, T), dtype=bool)
    for i in range(T):
        m[i, ancestors_or_self(parent, i)] = True
    return m


def tree_attention(q, k_tree, v_tree, parent, k_ctx, v_ctx, theta: float):
    """Ancestor-only attention of the flattened tree over [cached context ; tree tokens].

    q [T, n_q, d], k_tree / v_tree [T, n_kv, d]: the tree tokens' projections (bfloat16 bit patterns or
    floats), q and k before RoPE.  parent [T] (parent[0] ignored).  k_ctx / v_ctx [C, n_kv, d]: the cached
    context (already rotated).  Returns (o [T, n_q, d] fp64 holding bfloat16 values, probabilities of the
    last head [T, C + T] for inspection)."""
    q, k_tree, v_tree = to_f64(q), to_f64(k_tree), to_f64(v_tree)
    k_ctx, v_ctx = to_f64(k_ctx), to_f64(v_ctx)
    T, n_q, d = q.shape
    C, n_kv = k_ctx.shape[0], k_tree.shape[1]
    group = n_q // n_kv
    pos = C + tree_depths(parent)                                  # T2
    qr = bf16_round(rope(q, pos, theta))                           # T3
    kr = bf16_round(rope(k_tree, pos, theta))
    keys = np.concatenate([k_ctx, kr], axis=0)                     # [C + T, n_kv, d]
    vals = np.concatenate([v_ctx, v_tree], axis=0)
    visible = np.concatenate([np.ones((T, C), dtype=bool), tree_mask(parent)], axis=1)
    o = np.empty((T, n_q, d))
    p = None
    for h in range(n_q):
        g = h // group
        s = (qr[:, h, :] @ keys[:, g, :].T) / math.sqrt(d)
        s = np.where(visible, s, -np.inf)
        p = softmax_rows(s)
        o[:, h, :] = p @ vals[:, g, :]
    return bf16_round(o), p

"""Plain fp64 CPU oracle of the DFlash drafter pass. TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU-baseline leg may import this
module.  The HIP library never calls it, and it shares no code with the HIP library.

What is computed, and where it comes from
------------------------------------------
Page names used below:
  [DF]   "DFlash: Block Diffusion for Flash Speculative Decoding" (paper-graph summary of arXiv 2602.06036)
  [DDT]  "Accelerating Speculative Decoding with Block Diffusion Draft Trees" (paper-graph summary)
  [EXP]  the DFlash explainer at romaanj.github.io (paper-viz)
  [REV]  "DFlash: Block Diffusion for Flash Speculative Decoding Review" (dimensionstp.github.io)

1. fuse          [DF] §3.4.3 "Feature fusion": the target hidden states of several layers are concatenated
                 and mapped by one learned linear projection to the fused context feature.
2. inject        [DF] §3.4.3 "What KV injection means operationally" and [REV] §3) "KV injection": per
                 drafter layer, the fused feature is projected by that layer's own U_K, U_V and stored in the
                 layer's KV cache, where the block sees it as extra key/value pairs.
3. block input   [DF] §3.4.4 "Input structure": one anchor token followed by mask tokens.
4. layers        [DF] §3.2 item 3 (a few transformer layers).  The layer internals are not fixed by the
                 pages; this oracle uses the standard Qwen3 / LLaMA-3.1-style pre-norm block: RMSNorm,
                 grouped-query attention with rotary position embedding, SwiGLU FFN.
5. attention     [DF] §3.4.4 "Attention pattern", [EXP] (bidirectional inside the block), [REV] §4):
                 every block row attends to all context keys and to all block keys, with no mask.
6. head          [DF] §3.4.4 "Single forward pass prediction" and [REV] §7): the target's frozen LM head
                 turns each row into logits; greedy drafting takes the argmax.  [DDT] §3.4.2: the per-
                 position marginals are softmax of those logits; we return top-k log-probabilities.
7. accept        [DF] §3.4.1 (bonus-token bookkeeping under Eq. 1), [DF] §3.4.4 "Integration with
                 verification", [EXP] (the verification paragraph): accept drafts up to the first mismatch;
                 the cycle commits that many tokens plus the target's bonus token.

Readings where the pages are silent or disagree are listed in the design notes and restated next to
the function that applies them.  Numerics: every floating-point step is fp64.  The pages fix no precision;
the reading here is that a bfloat16 drafter keeps its weights, its input features and its KV cache in
bfloat16, and nothing else: the cached K/V (the one activation tensor that persists across calls) is
rounded to bfloat16 (round to nearest, ties to even), while every transient activation (fused feature,
normalised inputs, q/k/v, attention output, SwiGLU output, final state, residual, logits) is carried at
full precision.  For float32 drafters nothing is rounded.

Weights are passed as numpy arrays: bfloat16 as uint16 bit patterns, or float32/float64.  They are
converted to fp64 one matrix (or one row block) at a time, so the oracle never holds a whole drafter in
fp64.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------------------


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a bfloat16 (uint16 bit pattern), float32 or float64 array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even (result returned as fp64).

    bfloat16 keeps 8 significant bits and float32's exponent range.  For normal results the fp64
    significand is cut to 8 bits; below 2^-126 the spacing is fixed at 2^-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    ax = np.abs(x)
    small = ax < 2.0 ** -126
    # normal range: round the 52-bit fraction to 7 bits
    bits = x.view(np.uint64)
    drop = np.uint64(45)
    half_minus = np.uint64((1 << 44) - 1)
    lsb = (bits >> drop) & np.uint64(1)
    r = (bits + half_minus + lsb) & ~np.uint64((1 << 45) - 1)
    out[...] = r.view(np.float64)
    # subnormal range of bfloat16: multiples of 2^-133, ties to even (np.round is half-to-even)
    q = 2.0 ** -133
    out[small] = np.round(x[small] / q) * q
    # overflow beyond the largest finite bfloat16 goes to infinity
    big = np.abs(out) > _BF16_MAX
    out[big] = np.copysign(np.inf, x[big])
    nan = np.isnan(x)
    out[nan] = np.nan
    return out


def _rounder(bf16: bool):
    """Rounding applied to values stored in the KV cache."""
    return bf16_round if bf16 else (lambda v: np.asarray(v, dtype=np.float64))


def matmul_wT(x: np.ndarray, w: np.ndarray, rows_per_chunk: int = 8192) -> np.ndarray:
    """x @ W^T in fp64 for W stored [out, in]; W converted to fp64 a row block at a time."""
    x = np.asarray(x, dtype=np.float64)
    n_out = w.shape[0]
    y = np.empty(x.shape[:-1] + (n_out,), dtype=np.float64)
    for r0 in range(0, n_out, rows_per_chunk):
        wb = to_f64(w[r0: r0 + rows_per_chunk])
        y[..., r0: r0 + wb.shape[0]] = x @ wb.T
    return y


# ----------------------------------------------------------------------------------------------------
# layer pieces
# ----------------------------------------------------------------------------------------------------


def rms_norm(h: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: h / sqrt(mean(h^2) + eps) * gain."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * to_f64(gain)


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Per-pair rotary frequency theta^(-2i/d), i < d/2, rounded to float32 (returned as fp64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-(2.0 * i) / head_dim)  # rounded by the caller


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Rotation angle per (position, pair): float32(float32(pos) * float32(inv_freq)), as fp64.

    Reading: the angle is formed in float32, the common rotary convention; the product of two float32
    numbers is exact in fp64, so rounding it to float32 gives the float32 product.
    """
    inv = rope_inv_freq(head_dim, theta).astype(np.float32).astype(np.float64)
    p = np.asarray(pos, dtype=np.float32).astype(np.float64)
    return (p[..., None] * inv).astype(np.float32).astype(np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding on x [n, heads, d] at positions pos [n], rotate-half pairing (i, i + d/2).

    theta == 0 turns the rotation off (identity), a switch used by the permutation tests.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)[:, None, :]          # [n, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def block_attention(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, k_blk: np.ndarray,
                    v_blk: np.ndarray, return_probs: bool = False):
    """Non-causal attention of the block over [context keys ; block keys].

    q [L, n_q, d]; k_ctx, v_ctx [C, n_kv, d]; k_blk, v_blk [L, n_kv, d].  Query head h reads KV head
    h // (n_q / n_kv) (grouped-query attention).  Scores are scaled by 1/sqrt(d); no mask: the context
    is fully visible and the block is bidirectional ([DF] §3.4.4 "Attention pattern"; reading: the
    anchor row also sees the masks, as the explainer and the review state).
    Returns o [L, n_q, d] (and the probabilities [n_q, L, C+L] if asked).
    """
    L, n_q, d = q.shape
    n_kv = k_blk.shape[1]
    group = n_q // n_kv
    keys = np.concatenate([k_ctx, k_blk], axis=0)          # [C+L, n_kv, d]
    vals = np.concatenate([v_ctx, v_blk], axis=0)
    o = np.empty((L, n_q, d), dtype=np.float64)
    probs = np.empty((n_q, L, keys.shape[0]), dtype=np.float64) if return_probs else None
    for h in range(n_q):
        g = h // group
        s = (q[:, h, :] @ keys[:, g, :].T) / math.sqrt(d)
        p = softmax_rows(s)
        o[:, h, :] = p @ vals[:, g, :]
        if return_probs:
            probs[h] = p
    return (o, probs) if return_probs else o


# ----------------------------------------------------------------------------------------------------
# 1-2: context feature fusion and KV injection
# ----------------------------------------------------------------------------------------------------


def fuse(feats: np.ndarray, fc_w: np.ndarray, fc_b: Optional[np.ndarray], bf16: bool) -> np.ndarray:
    """f_j = W_fc x_j (+ b) for each context token ([DF] §3.4.3 "Feature fusion").

    Reading: the fused width equals the drafter hidden size and no norm is applied to f (the pages
    show only the projection of the concatenation).  f is transient (only the K/V made from it are
    cached), so it is not rounded.
    """
    f = matmul_wT(to_f64(feats), fc_w)
    if fc_b is not None:
        f = f + to_f64(fc_b)
    return f


def inject_layer(f: np.ndarray, uk: np.ndarray, uv: np.ndarray, positions: np.ndarray, n_kv: int,
                 head_dim: int, theta: float, bf16: bool):
    """Context K/V of one drafter layer ([DF] §3.4.3 KV injection; [REV] §3)).

    K_j = RoPE(U_K f_j) at the token's own position j, V_j = U_V f_j, one row per context token.
    Reading: the context enters as extra key/value pairs appended in the cache (not as an additive
    bias on the block's keys), so each context key carries the rotary phase of its own position.  These are
    the cached values, rounded to bfloat16 on the bfloat16 path.
    Returns (K [n, n_kv, d], V [n, n_kv, d]).
    """
    rnd = _rounder(bf16)
    n = f.shape[0]
    k = matmul_wT(f, uk).reshape(n, n_kv, head_dim)
    v = matmul_wT(f, uv).reshape(n, n_kv, head_dim)
    return rnd(rope(k, positions, theta)), rnd(v)


def inject(w: Dict[str, np.ndarray], cfg, feats: np.ndarray, start_pos: int, fc_b=None,
           chunk: int = 4096):
    """Fuse the features of tokens start_pos.. and project them into every layer's context K/V.

    Returns a list over layers of (K, V), each [n_new, n_kv, d].  Rows are processed in chunks to
    bound memory; every row is independent, so chunking does not change any value.
    """
    n_new = feats.shape[0]
    ks = [[] for _ in range(cfg.n_layers)]
    vs = [[] for _ in range(cfg.n_layers)]
    for r0 in range(0, n_new, chunk):
        f = fuse(feats[r0: r0 + chunk], w["fc_w"], fc_b, cfg.bf16)
        pos = np.arange(start_pos + r0, start_pos + r0 + f.shape[0])
        for l in range(cfg.n_layers):
            k, v = inject_layer(f, w[f"l{l}.uk"], w[f"l{l}.uv"], pos, cfg.n_kv_heads, cfg.head_dim,
                                cfg.rope_theta, cfg.bf16)
            ks[l].append(k)
            vs[l].append(v)
    d, nkv = cfg.head_dim, cfg.n_kv_heads
    return [(np.concatenate(ks[l]) if ks[l] else np.zeros((0, nkv, d)),
             np.concatenate(vs[l]) if vs[l] else np.zeros((0, nkv, d))) for l in range(cfg.n_layers)]


# ----------------------------------------------------------------------------------------------------
# 3-6: the drafter pass over one block
# ----------------------------------------------------------------------------------------------------


def drafter_hidden(w: Dict[str, np.ndarray], cfg, ctx_kv_per_req: List[Sequence], block_tokens: np.ndarray,
                   return_taps: bool = False):
    """Residual stream of the block rows of a batch of requests.

    block_tokens [B, L]: the anchor then mask ids ([DF] §3.4.4 "Input structure").  ctx_kv_per_req[r]:
    per layer (K_ctx, V_ctx) of request r, C_r rows each.  Block row i of request r sits at position
    C_r + i (the anchor at C_r: the anchor is the newest token, not yet in the context, [DDT] §3.4.1).
    Row-wise steps (norms, projections) run on all B*L rows at once; attention runs per request.
    Returns the final residual h [B, L, H] (and taps [B, n_layers + 1, L, H] if asked).
    """
    B, L = block_tokens.shape
    d, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    ctx = [ctx_kv_per_req[r][0][0].shape[0] for r in range(B)]
    pos = np.concatenate([np.arange(c, c + L) for c in ctx])          # [B*L]
    h = to_f64(w["embed"][block_tokens.reshape(-1)])                   # shared frozen embedding ([REV] §7)
    taps = [h.copy()]
    for l in range(cfg.n_layers):
        p = f"l{l}."
        u = rms_norm(h, w[p + "attn_norm"], cfg.rms_eps)
        q = rope(matmul_wT(u, w[p + "wq"]).reshape(B * L, nq, d), pos, cfg.rope_theta)
        k = rope(matmul_wT(u, w[p + "wk"]).reshape(B * L, nkv, d), pos, cfg.rope_theta)
        v = matmul_wT(u, w[p + "wv"]).reshape(B * L, nkv, d)
        o = np.empty((B * L, nq, d))
        for r in range(B):
            rows = slice(r * L, (r + 1) * L)
            k_ctx, v_ctx = ctx_kv_per_req[r][l]
            o[rows] = block_attention(q[rows], k_ctx, v_ctx, k[rows], v[rows])
        o = o.reshape(B * L, nq * d)
        h = h + matmul_wT(o, w[p + "wo"])
        u2 = rms_norm(h, w[p + "ffn_norm"], cfg.rms_eps)
        a = silu(matmul_wT(u2, w[p + "w_gate"])) * matmul_wT(u2, w[p + "w_up"])
        h = h + matmul_wT(a, w[p + "w_down"])
        taps.append(h.copy())
    h = h.reshape(B, L, -1)
    if return_taps:
        return h, np.stack(taps).reshape(cfg.n_layers + 1, B, L, -1).transpose(1, 0, 2, 3)
    return h


def lm_head_logits(w: Dict[str, np.ndarray], cfg, h: np.ndarray) -> np.ndarray:
    """Final RMSNorm, then the shared LM head: logits [L, V] (never rounded)."""
    z = rms_norm(h, w["final_norm"], cfg.rms_eps)
    return matmul_wT(z, w["lm_head"], rows_per_chunk=16384)


def log_sum_exp(logits: np.ndarray) -> np.ndarray:
    m = np.max(logits, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(logits - m), axis=-1, keepdims=True)))[..., 0]


def ranked_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k best logits per row, ordered by (logit descending, id ascending).

    Reading: ties go to the smaller token id, which makes greedy argmax and top-k deterministic.
    """
    out = np.empty(logits.shape[:-1] + (k,), dtype=np.int64)
    flat = logits.reshape(-1, logits.shape[-1])
    ids = np.arange(flat.shape[1])
    for r in range(flat.shape[0]):
        order = np.lexsort((ids, -flat[r]))             # primary: -logit, secondary: id
        out.reshape(-1, k)[r] = order[:k]
    return out


def head_outputs(logits: np.ndarray, top_k: int) -> dict:
    """Greedy tokens, top-k ids and top-k log-probs (natural log, temperature 1, full vocabulary)."""
    kk = max(top_k, 1)
    ids = ranked_ids(logits, kk)
    lse = log_sum_exp(logits)
    lp = np.take_along_axis(logits, ids, axis=-1) - lse[..., None]
    return {"tokens": ids[..., 0].astype(np.int64), "topk_ids": ids[..., :top_k],
            "topk_logprobs": lp[..., :top_k], "lse": lse}


def sorted_margins(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between consecutive sorted logits among the top k+1, per row.

    A row whose margin exceeds a tolerance has a top-k set and order that no error below half of that
    tolerance can change; argmax uses k = 1 (the top-2 gap).
    """
    part = -np.sort(-logits, axis=-1)[..., : k + 1]
    return np.min(part[..., :-1] - part[..., 1:], axis=-1)


def draft_block(w: Dict[str, np.ndarray], cfg, ctx_kv_per_req: List[Sequence], block_tokens: np.ndarray,
                top_k: int, return_taps: bool = False) -> dict:
    """The whole drafter pass for a batch: each request's block in one parallel pass ([DF] Eq. 3).

    Returns logits [B, L, V] and the head outputs (tokens, topk_ids, topk_logprobs, lse)."""
    res = drafter_hidden(w, cfg, ctx_kv_per_req, block_tokens, return_taps)
    h = res[0] if return_taps else res
    logits = lm_head_logits(w, cfg, h)
    out = head_outputs(logits, top_k)
    out["logits"] = logits
    if return_taps:
        out["taps"] = res[1]
    return out


# ----------------------------------------------------------------------------------------------------
# 7: greedy acceptance
# ----------------------------------------------------------------------------------------------------


def accept_len(draft: np.ndarray, target: np.ndarray) -> np.ndarray:
    """tau = 1 + the number of leading draft tokens equal to the target's tokens.

    draft [B, n] (the predictions at block rows 1..n); target [B, >= n] (the target's token at each of
    those positions; a further bonus slot is never compared).  tau counts the accepted drafts plus the
    bonus token, so tau lies in [1, n + 1] ([DF] §3.4.1 bonus-token bookkeeping; [EXP] tau >= 1).
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, n = draft.shape
    tau = np.ones(B, dtype=np.int64)
    for r in range(B):
        k = 0
        while k < n and draft[r, k] == target[r, k]:
            k += 1
        tau[r] = k + 1
    return tau


def per_token_latency(t_draft: float, t_verify: float, tau: float) -> float:
    """L = (T_draft + T_verify) / tau ([DF] Eq. 1)."""
    return (t_draft + t_verify) / tau


def speedup(l_target: float, t_draft: float, t_verify: float, tau: float) -> float:
    """eta = L_target / L ([DF] Eq. 1)."""
    return l_target / per_token_latency(t_draft, t_verify, tau)

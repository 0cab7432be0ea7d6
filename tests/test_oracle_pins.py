"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: a value printed on the pages, a closed
form, an invariant, a library routine, or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


class Cfg:
    """Minimal shape record for oracle calls."""

    def __init__(self, **kw):
        self.rms_eps = 1e-6
        self.bf16 = False
        self.__dict__.update(kw)


def _rand_weights(cfg, rng, scale=0.05):
    H, d, nq, nkv, Fd = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.ffn
    w = {"fc_w": rng.normal(0, scale, (H, cfg.feat_dim)), "embed": rng.normal(0, 1.0, (cfg.vocab, H)),
         "final_norm": 1 + 0.1 * rng.normal(size=H), "lm_head": rng.normal(0, scale, (cfg.vocab, H))}
    for l in range(cfg.n_layers):
        p = f"l{l}."
        w[p + "attn_norm"] = 1 + 0.1 * rng.normal(size=H)
        w[p + "ffn_norm"] = 1 + 0.1 * rng.normal(size=H)
        w[p + "wq"] = rng.normal(0, scale, (nq * d, H))
        w[p + "wk"] = rng.normal(0, scale, (nkv * d, H))
        w[p + "wv"] = rng.normal(0, scale, (nkv * d, H))
        w[p + "wo"] = rng.normal(0, scale, (H, nq * d))
        w[p + "uk"] = rng.normal(0, scale, (nkv * d, H))
        w[p + "uv"] = rng.normal(0, scale, (nkv * d, H))
        w[p + "w_gate"] = rng.normal(0, scale, (Fd, H))
        w[p + "w_up"] = rng.normal(0, scale, (Fd, H))
        w[p + "w_down"] = rng.normal(0, scale, (H, Fd))
    return w


def _tiny_cfg(**kw):
    base = dict(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=50,
                feat_dim=24, rope_theta=1e4)
    base.update(kw)
    return Cfg(**base)


# ----------------------------------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------------------------------


def test_philox_known_answers():
    kat = _load("philox4x32_10_kat.json")
    for c in kat["cases"]:
        out = W.philox_block([int(x, 16) for x in c["counter"]], [int(x, 16) for x in c["key"]])
        assert [f"{x:08x}" for x in out] == c["out"]


def test_generator_offsets_and_moments():
    a = W.normal(11, 3, (4001,), 1.0, False)
    b = W.normal(11, 3, (3000,), 1.0, False, start=1001)
    assert np.array_equal(a[1001:], b)
    big = W.normal(12, 4, (400_000,), 0.02, False).astype(np.float64)
    assert abs(big.mean()) < 0.02 * 5 / math.sqrt(4e5)
    assert abs(big.std() / 0.02 - 1) < 0.01


# ----------------------------------------------------------------------------------------------------
# number format
# ----------------------------------------------------------------------------------------------------


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(100_000) * np.exp(rng.uniform(-30, 30, 100_000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x32.astype(np.float64)), ref)


def test_to_f64_decodes_every_bfloat16_pattern_like_torch():
    """to_f64 reads every bfloat16 value the parity tests compare: all 65536 bit patterns against torch's own
    bfloat16 decoding (NaN patterns as NaN, both zeros with their signs, subnormals, infinities)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.to_f64(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert got.dtype == np.float64
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 * 127
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x0001] == 2.0 ** -133
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf


def test_bf16_round_ties_and_direct_rounding():
    one = 1.0
    assert O.bf16_round(np.array([one + 2.0 ** -8]))[0] == 1.0                     # tie -> even
    assert O.bf16_round(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6     # tie -> even (up)
    # just above a tie: a value that float32 cannot hold must still round up (no double rounding)
    assert O.bf16_round(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert O.bf16_round(np.array([-(one + 2.0 ** -8 + 2.0 ** -40)]))[0] == -(1.0 + 2.0 ** -7)
    assert O.bf16_round(np.array([3.5e38]))[0] == np.inf
    assert O.bf16_round(np.array([0.0]))[0] == 0.0


# ----------------------------------------------------------------------------------------------------
# RMSNorm, SwiGLU, RoPE
# ----------------------------------------------------------------------------------------------------


def test_rms_norm_closed_form():
    rng = np.random.default_rng(1)
    h = rng.normal(0, 3, (7, 64))
    y = O.rms_norm(h, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-12)
    assert np.allclose(O.rms_norm(5.0 * h, np.ones(64), 0.0), y, atol=1e-12)   # scale invariance
    g = rng.normal(size=64)
    ref = F.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(O.rms_norm(h, g, 1e-6), ref, atol=1e-12)


def test_silu_matches_torch():
    x = np.linspace(-20, 20, 1001)
    assert np.allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), atol=1e-14)


def test_rope_is_a_rotation_by_position_angle():
    rng = np.random.default_rng(2)
    d, theta = 16, 1e4
    x = rng.normal(size=(5, 3, d))
    pos = np.array([0, 1, 7, 100, 32768])
    y = O.rope(x, pos, theta)
    # complex formulation: (x_i + i x_{i+d/2}) * exp(i * pos * w_i), w_i = theta^(-2i/d)
    w = (theta ** (-np.arange(d // 2) * 2.0 / d)).astype(np.float32).astype(np.float64)
    ang = (pos.astype(np.float32)[:, None].astype(np.float64) * w).astype(np.float32).astype(np.float64)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)[:, None, :]
    assert np.allclose(y, np.concatenate([z.real, z.imag], axis=-1), atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.array_equal(O.rope(x, np.zeros(5, int), theta), x)                 # position 0: identity
    assert np.array_equal(O.rope(x, pos, 0.0), x)                                 # RoPE off


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(3)
    d, theta = 32, 1e4
    q = rng.normal(size=(1, 1, d))
    k = rng.normal(size=(1, 1, d))
    base = (O.rope(q, np.array([10]), theta) * O.rope(k, np.array([3]), theta)).sum()
    for t in (1, 50, 1000):
        s = (O.rope(q, np.array([10 + t]), theta) * O.rope(k, np.array([3 + t]), theta)).sum()
        assert abs(s - base) < 1e-4 * (1 + t / 100)      # float32 angle quantisation only


# ----------------------------------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------------------------------


def _attn_inputs(rng, L=5, C=9, nq=4, nkv=2, d=8, scale=1.0):
    return (rng.normal(0, scale, (L, nq, d)), rng.normal(0, scale, (C, nkv, d)),
            rng.normal(0, scale, (C, nkv, d)), rng.normal(0, scale, (L, nkv, d)),
            rng.normal(0, scale, (L, nkv, d)))


def test_attention_probabilities_sum_to_one():
    rng = np.random.default_rng(4)
    q, kc, vc, kb, vb = _attn_inputs(rng, scale=2.0)
    _, p = O.block_attention(q, kc, vc, kb, vb, return_probs=True)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-12)
    assert (p > 0).all()                             # every key visible: no mask inside the block


def test_zero_context_features_give_uniform_context_weight():
    """Zero fused features and zero bias give K_ctx = V_ctx = 0: each context key gets weight
    1 / (C + sum_j exp(s_ij)) and o_i = sum_blk exp(s_ij) v_j / (C + sum_blk exp(s_ij))."""
    rng = np.random.default_rng(5)
    cfg = _tiny_cfg()
    w = _rand_weights(cfg, rng)
    C = 13
    feats = np.zeros((C, cfg.feat_dim))
    kv = O.inject(w, cfg, feats, 0)
    assert all(np.all(k == 0) and np.all(v == 0) for k, v in kv)
    L, nq, nkv, d = 6, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q, _, _, kb, vb = _attn_inputs(rng, L=L, C=0, nq=nq, nkv=nkv, d=d)
    o, p = O.block_attention(q, kv[0][0], kv[0][1], kb, vb, return_probs=True)
    for h in range(nq):
        g = h // (nq // nkv)
        e = np.exp(q[:, h] @ kb[:, g].T / math.sqrt(d))
        denom = C + e.sum(-1, keepdims=True)
        assert np.allclose(p[h][:, :C], 1.0 / denom, atol=1e-13)
        assert np.allclose(o[:, h], (e @ vb[:, g]) / denom, atol=1e-12)


def test_attention_without_context_is_plain_bidirectional_sdpa():
    rng = np.random.default_rng(6)
    q, _, _, kb, vb = _attn_inputs(rng, L=7, C=0, nq=6, nkv=2, d=16)
    o = O.block_attention(q, np.zeros((0, 2, 16)), np.zeros((0, 2, 16)), kb, vb)
    qt = torch.from_numpy(q).permute(1, 0, 2)                                   # [heads, L, d]
    kt = torch.from_numpy(kb).permute(1, 0, 2).repeat_interleave(3, dim=0)
    vt = torch.from_numpy(vb).permute(1, 0, 2).repeat_interleave(3, dim=0)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=False).permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_with_context_equals_sdpa_over_concatenated_keys():
    rng = np.random.default_rng(7)
    q, kc, vc, kb, vb = _attn_inputs(rng, L=4, C=11, nq=8, nkv=2, d=8)
    o = O.block_attention(q, kc, vc, kb, vb)
    keys = torch.from_numpy(np.concatenate([kc, kb])).permute(1, 0, 2).repeat_interleave(4, dim=0)
    vals = torch.from_numpy(np.concatenate([vc, vb])).permute(1, 0, 2).repeat_interleave(4, dim=0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2), keys, vals)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_split_merge_identity():
    """Softmax over [ctx ; blk] equals the log-sum-exp merge of the two partial attentions."""
    rng = np.random.default_rng(8)
    q, kc, vc, kb, vb = _attn_inputs(rng, L=3, C=20, nq=2, nkv=1, d=8, scale=1.5)
    o = O.block_attention(q, kc, vc, kb, vb)
    parts = []
    for k, v in ((kc, vc), (kb, vb)):
        s = np.einsum("lhd,cd->hlc", q, k[:, 0]) / math.sqrt(8)
        m = s.max(-1)
        e = np.exp(s - m[..., None])
        parts.append((m, e.sum(-1), np.einsum("hlc,cd->lhd", e, v[:, 0])))
    m = np.maximum(parts[0][0], parts[1][0])
    num = sum(np.exp(pm - m).T[..., None] * po for pm, _, po in parts)
    den = sum(np.exp(pm - m) * pl for pm, pl, _ in parts).T[..., None]
    assert np.allclose(o, num / den, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    q, kc, vc, kb, vb = _attn_inputs(rng, L=5, C=6, nq=6, nkv=3, d=8)
    o = O.block_attention(q, kc, vc, kb, vb)
    rep = lambda a: np.repeat(a, 2, axis=1)
    o_mha = O.block_attention(q, rep(kc), rep(vc), rep(kb), rep(vb))
    assert np.allclose(o, o_mha, atol=1e-14)


# ----------------------------------------------------------------------------------------------------
# fuse / inject
# ----------------------------------------------------------------------------------------------------


def test_fuse_and_inject_are_linear_maps_of_the_features():
    rng = np.random.default_rng(10)
    cfg = _tiny_cfg(rope_theta=0.0)
    w = _rand_weights(cfg, rng)
    for j in (0, 5, cfg.feat_dim - 1):
        e = np.zeros((1, cfg.feat_dim))
        e[0, j] = 1.0
        f = O.fuse(e, w["fc_w"], None, False)
        assert np.allclose(f[0], w["fc_w"][:, j], atol=1e-15)
        kv = O.inject(w, cfg, e, 0)
        assert np.allclose(kv[1][0][0].reshape(-1), w["l1.uk"] @ w["fc_w"][:, j], atol=1e-14)
        assert np.allclose(kv[0][1][0].reshape(-1), w["l0.uv"] @ w["fc_w"][:, j], atol=1e-14)
    b = rng.normal(size=cfg.hidden)
    assert np.allclose(O.fuse(np.zeros((2, cfg.feat_dim)), w["fc_w"], b, False), b)
    # the bias enters f, before U_K / U_V: zero features give every context token K = U_K b, V = U_V b
    # (RoPE off), and features and bias add
    kv0 = O.inject(w, cfg, np.zeros((3, cfg.feat_dim)), 0, fc_b=b)
    for l in range(cfg.n_layers):
        for j in range(3):
            assert np.allclose(kv0[l][0][j].reshape(-1), w[f"l{l}.uk"] @ b, atol=1e-14)
            assert np.allclose(kv0[l][1][j].reshape(-1), w[f"l{l}.uv"] @ b, atol=1e-14)
    e = np.zeros((1, cfg.feat_dim))
    e[0, 7] = 1.0
    kvb = O.inject(w, cfg, e, 0, fc_b=b)
    assert np.allclose(kvb[1][1][0].reshape(-1), w["l1.uv"] @ (w["fc_w"][:, 7] + b), atol=1e-14)
    # the fused feature is transient: not rounded even on the bfloat16 path; the cached K/V are
    x = rng.normal(size=(3, cfg.feat_dim))
    assert np.allclose(O.fuse(x, w["fc_w"], None, True), x @ w["fc_w"].T, atol=1e-14)
    cfg16 = _tiny_cfg(rope_theta=0.0, bf16=True)
    kv = O.inject(w, cfg16, x, 0)
    assert np.array_equal(kv[0][0].reshape(3, -1), O.bf16_round(x @ w["fc_w"].T @ w["l0.uk"].T))
    assert np.array_equal(kv[1][1].reshape(3, -1), O.bf16_round(x @ w["fc_w"].T @ w["l1.uv"].T))


def test_inject_keys_carry_their_own_positions():
    rng = np.random.default_rng(11)
    cfg = _tiny_cfg()
    w = _rand_weights(cfg, rng)
    feats = rng.normal(size=(9, cfg.feat_dim))
    whole = O.inject(w, cfg, feats, 0)
    tail = O.inject(w, cfg, feats[4:], 4)          # appending later tokens reproduces the same rows
    for l in range(cfg.n_layers):
        assert np.allclose(whole[l][0][4:], tail[l][0], atol=1e-14)
        assert np.allclose(whole[l][1][4:], tail[l][1], atol=1e-14)


# ----------------------------------------------------------------------------------------------------
# drafter pass
# ----------------------------------------------------------------------------------------------------


def _torch_drafter(w, cfg, ctx_kv, tokens):
    """The same pass composed from torch library routines (fp64, one request, float32 drafter)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    L = tokens.shape[0]
    C = ctx_kv[0][0].shape[0]
    d, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    pos = torch.arange(C, C + L, dtype=torch.float32)
    inv = torch.tensor(cfg.rope_theta, dtype=torch.float64) ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = (pos[:, None] * inv.float()[None, :]).double()
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]

    def rope(x):  # x [L, heads, d]; rotate-half pairs as complex numbers
        z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    h = t(w["embed"])[torch.from_numpy(tokens.astype(np.int64))]
    for l in range(cfg.n_layers):
        p = f"l{l}."
        u = F.rms_norm(h, (cfg.hidden,), t(w[p + "attn_norm"]), eps=cfg.rms_eps)
        q = rope(F.linear(u, t(w[p + "wq"])).view(L, nq, d))
        k = rope(F.linear(u, t(w[p + "wk"])).view(L, nkv, d))
        v = F.linear(u, t(w[p + "wv"])).view(L, nkv, d)
        keys = torch.cat([t(ctx_kv[l][0]), k]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        vals = torch.cat([t(ctx_kv[l][1]), v]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2), keys, vals).permute(1, 0, 2).reshape(L, -1)
        h = h + F.linear(o, t(w[p + "wo"]))
        u2 = F.rms_norm(h, (cfg.hidden,), t(w[p + "ffn_norm"]), eps=cfg.rms_eps)
        h = h + F.linear(F.silu(F.linear(u2, t(w[p + "w_gate"]))) * F.linear(u2, t(w[p + "w_up"])),
                         t(w[p + "w_down"]))
    z = F.rms_norm(h, (cfg.hidden,), t(w["final_norm"]), eps=cfg.rms_eps)
    return F.linear(z, t(w["lm_head"])).numpy()


@pytest.mark.parametrize("C", [0, 1, 23])
def test_drafter_pass_matches_torch_composition(C):
    rng = np.random.default_rng(12 + C)
    cfg = _tiny_cfg()
    w = _rand_weights(cfg, rng)
    feats = rng.normal(size=(C, cfg.feat_dim))
    kv = O.inject(w, cfg, feats, 0)
    tokens = np.array([[3, 49, 49, 49, 49, 49]])
    out = O.draft_block(w, cfg, [kv], tokens, top_k=3)
    ref = _torch_drafter(w, cfg, kv, tokens[0])
    assert np.allclose(out["logits"][0], ref, atol=1e-10)


def test_block_rows_are_permutation_equivariant_without_rope():
    """With RoPE off the block attention has no positional signal and no mask, so permuting the block
    tokens permutes every row's output; the mask rows (identical inputs) give identical logits."""
    rng = np.random.default_rng(13)
    cfg = _tiny_cfg(rope_theta=0.0)
    w = _rand_weights(cfg, rng)
    kv = O.inject(w, cfg, rng.normal(size=(10, cfg.feat_dim)), 0)
    tok = np.array([[7, 3, 11, 11, 42, 0]])
    perm = np.array([4, 2, 0, 5, 1, 3])
    a = O.draft_block(w, cfg, [kv], tok, top_k=2)["logits"][0]
    b = O.draft_block(w, cfg, [kv], tok[:, perm], top_k=2)["logits"][0]
    assert np.allclose(a[perm], b, atol=1e-12)
    assert np.allclose(a[2], a[3], atol=1e-14)
    # with RoPE on the mask rows differ (positions differ)
    cfg_r = _tiny_cfg(rope_theta=1e4)
    c = O.draft_block(w, cfg_r, [O.inject(w, cfg_r, rng.normal(size=(10, cfg.feat_dim)), 0)], tok, 2)
    assert not np.allclose(c["logits"][0][2], c["logits"][0][3])


def test_requests_in_a_batch_are_independent():
    rng = np.random.default_rng(14)
    cfg = _tiny_cfg()
    w = _rand_weights(cfg, rng)
    kvs = [O.inject(w, cfg, rng.normal(size=(c, cfg.feat_dim)), 0) for c in (0, 5, 17)]
    tok = np.array([[1, 49, 49, 49], [2, 49, 49, 49], [3, 49, 49, 49]])
    together = O.draft_block(w, cfg, kvs, tok, top_k=4)["logits"]
    for r in range(3):
        alone = O.draft_block(w, cfg, [kvs[r]], tok[r: r + 1], top_k=4)["logits"][0]
        assert np.allclose(together[r], alone, atol=1e-12)


# ----------------------------------------------------------------------------------------------------
# head: argmax, top-k, log-probs
# ----------------------------------------------------------------------------------------------------


def test_topk_matches_brute_force_sort_and_logprobs_normalise():
    rng = np.random.default_rng(15)
    logits = rng.normal(0, 2, (6, 4096))
    logits[1, 100] = logits[1, 7] = logits[1].max() + 1.0          # exact tie at the top
    out = O.head_outputs(logits, 8)
    for r in range(6):
        order = sorted(range(4096), key=lambda i: (-logits[r, i], i))[:8]
        assert list(out["topk_ids"][r]) == order
        assert out["tokens"][r] == int(np.argmax(logits[r]))
    assert out["tokens"][1] == 7                                      # tie goes to the smaller id
    assert np.allclose(np.exp(logits - out["lse"][:, None]).sum(-1), 1.0)
    assert (out["topk_logprobs"] <= 0).all()
    assert (np.diff(out["topk_logprobs"], axis=-1) <= 0).all()
    ref_lse = torch.logsumexp(torch.from_numpy(logits), -1).numpy()
    assert np.allclose(out["lse"], ref_lse, atol=1e-12)


def test_margins():
    lg = np.array([[5.0, 4.0, 3.5, 0.0], [1.0, 1.0, 0.0, -1.0]])
    assert np.allclose(O.sorted_margins(lg, 1), [1.0, 0.0])
    assert np.allclose(O.sorted_margins(lg, 2), [0.5, 0.0])


# ----------------------------------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------------------------------


def test_acceptance_bookkeeping_examples():
    g = _load("acceptance_bookkeeping.json")
    for c in g["cases"]:
        n = c["gamma"]
        draft = np.arange(n)[None, :] + 10
        target = np.concatenate([draft, [[999]]], axis=1)
        if c["first_mismatch"] is not None:
            target[0, c["first_mismatch"]] = -1
        assert O.accept_len(draft, target)[0] == c["tau"]


def test_acceptance_brute_force_small_vocab():
    """All draft/target pairs over V = 3, three drafts: tau = 1 + length of the common prefix."""
    import itertools
    seqs = list(itertools.product(range(3), repeat=3))
    draft = np.array([s for s in seqs for _ in seqs])
    target = np.array([t + (0,) for _ in seqs for t in seqs])
    tau = O.accept_len(draft, target)
    eq = (draft == target[:, :3]).astype(int)
    prefix = np.cumprod(eq, axis=1).sum(axis=1)
    assert np.array_equal(tau, 1 + prefix)
    assert tau.min() == 1 and tau.max() == 4


@pytest.mark.parametrize("p,L,expect", [(0.8, 8, 4.16), (0.85, 16, 6.17), (0.8, 16, 4.86)])
def test_expected_acceptance_length_of_the_synthetic_target(p, L, expect):
    """With target slot = draft w.p. p (else uniform over V), E[tau] = (1 - q^L) / (1 - q),
    q = p + (1 - p) / V."""
    V, n = 4096, 20000
    q = p + (1 - p) / V
    closed = (1 - q ** L) / (1 - q)
    assert abs(closed - expect) < 0.01
    key = W.seed_key(999)
    u = W.uniform01(key, 1, n * L).reshape(n, L)
    rand = W.uniform_int(key, 2, n * L, 0, V - 1).reshape(n, L)
    greedy = W.uniform_int(key, 3, n * L, 0, V - 1).reshape(n, L)
    y = W.make_target(greedy, u < p, rand)
    tau = O.accept_len(greedy[:, 1:], y)
    se = tau.std() / math.sqrt(n)
    assert abs(tau.mean() - closed) < 4 * se


def test_eq1_worked_examples():
    g = _load("eq1_worked_examples.json")
    for c in g["latency_cases"]:
        assert math.isclose(O.per_token_latency(c["t_draft_ms"], c["t_verify_ms"], c["tau"]), c["per_token_ms"])
        assert math.isclose(O.speedup(c["l_target_ms"], c["t_draft_ms"], c["t_verify_ms"], c["tau"]), c["speedup"])
    for c in g["cycle_cases"]:
        assert math.isclose(O.per_token_latency(c["t_draft_ms"], c["t_verify_ms"], 1.0), c["cycle_ms"])


def test_inject_rotates_keys_only():
    rng = np.random.default_rng(16)
    cfg = _tiny_cfg(rope_theta=1e4)
    w = _rand_weights(cfg, rng)
    j, start = 3, 37
    e = np.zeros((2, cfg.feat_dim))
    e[:, j] = 1.0
    kv = O.inject(w, cfg, e, start)
    d = cfg.head_dim
    inv = (1e4 ** (-np.arange(d // 2) * 2.0 / d)).astype(np.float32).astype(np.float64)
    for r, pos in enumerate((start, start + 1)):
        raw = (w["l0.uk"] @ w["fc_w"][:, j]).reshape(cfg.n_kv_heads, d)
        ang = np.float64(np.float32(np.float32(pos) * inv.astype(np.float32)))
        z = (raw[:, : d // 2] + 1j * raw[:, d // 2:]) * np.exp(1j * ang)
        assert np.allclose(kv[0][0][r], np.concatenate([z.real, z.imag], -1), atol=1e-13)
        assert np.allclose(kv[0][1][r].reshape(-1), w["l0.uv"] @ w["fc_w"][:, j], atol=1e-14)


def test_bf16_drafter_rounds_only_the_cache():
    """On the bfloat16 path only the cached K/V are rounded: the block pass itself equals the float32-path
    pass on the same (rounded) cache, while rounding the block's activations as well would move the logits
    by far more."""
    rng = np.random.default_rng(17)
    cfg = _tiny_cfg(hidden=64, head_dim=16, ffn=96, bf16=True)
    cfg32 = _tiny_cfg(hidden=64, head_dim=16, ffn=96, bf16=False)
    w = {k: O.bf16_round(v) for k, v in _rand_weights(cfg, rng).items()}
    feats = O.bf16_round(rng.normal(size=(12, cfg.feat_dim)))
    kv16 = O.inject(w, cfg, feats, 0)
    kv32 = O.inject(w, cfg32, feats, 0)
    assert all(np.array_equal(a[0], O.bf16_round(b[0])) and np.array_equal(a[1], O.bf16_round(b[1]))
               for a, b in zip(kv16, kv32))
    tok = np.array([[5, 49, 49, 49, 49]])
    got = O.draft_block(w, cfg, [kv16], tok, top_k=1)["logits"][0]
    same = O.draft_block(w, cfg32, [kv16], tok, top_k=1)["logits"][0]
    assert np.array_equal(got, same)
    ref = _torch_drafter(w, cfg32, kv16, tok[0])
    assert np.abs(got - ref).max() < 1e-10

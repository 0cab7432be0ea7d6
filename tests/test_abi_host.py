"""The C ABI library loads, exports every symbol of include/dflash.h, and rejects bad arguments before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def D():
    from block_diffusion_drafter_forward_amd import dflash
    if not os.path.exists(dflash.LIB_PATH):
        from block_diffusion_drafter_forward_amd.build import build
        build()
    dflash.lib()
    return dflash


def _declared():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(D):
    names = _declared()
    assert "dflash_draft_block" in names and "dflash_inject_ctx" in names and "dflash_accept_len" in names
    lib = D.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(D.EXPORTS)


def _shape(**kw):
    import workloads as W
    s = dict(W.SMALL_BF16.__dict__)
    s.update(kw)
    return W.DrafterShape(**s)


def _fake_weights(shape, bad=None):
    """Non-null dummy pointers (never dereferenced: creation makes no HIP call)."""
    names = ["fc_w", "embed", "final_norm", "lm_head"]
    for l in range(shape.n_layers):
        names += [f"l{l}.{f}" for f in D_LAYER]
    return {n: (None if n == bad else _Fake(0x1000 + 0x100 * i)) for i, n in enumerate(names)}


D_LAYER = ["attn_norm", "wq", "wk", "wv", "wo", "uk", "uv", "ffn_norm", "w_gate", "w_up", "w_down"]


class _Fake:
    def __init__(self, p):
        self.p = p

    def data_ptr(self):
        return self.p


def _create(D, shape, bad=None):
    return D.DraftModel(shape, _fake_weights(shape, bad), pack=False)


def test_create_accepts_supported_shapes(D):
    import workloads as W
    for s in (W.TINY, W.QWEN3_8B, W.LLAMA31_8B, W.SMALL_FP32, W.SMALL_GQA8, W.SMALL_BF16_D64, W.SMALL_GQA8_D64,
              W.SMALL_MHA_D64):
        m = _create(D, s)
        assert m.handle
        m.close()


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -4),  # bfloat16 kernels: head_dim 64 or 128
    (dict(head_dim=32), -4),
    (dict(n_q_heads=7), -2),
    (dict(n_q_heads=32, n_kv_heads=2), -4),
    (dict(block_len=17), -4),
    (dict(block_len=1), -4),
    (dict(hidden=500), -4),
    (dict(page_size=32), -4),
    (dict(n_layers=0), -1),
    (dict(vocab=0), -1),
])
def test_create_rejects_bad_configs(D, kw, code):
    with pytest.raises(D.DFlashError) as e:
        _create(D, _shape(**kw))
    assert e.value.code == code


def test_create_rejects_null_weights(D):
    with pytest.raises(D.DFlashError) as e:
        _create(D, _shape(), bad="l1.w_down")
    assert e.value.code == D.DFLASH_E_ARG and "layer 1" in str(e.value)


def _draft(D, h, **over):
    a = dict(batch=1, block_tokens=0x10, ctx_len=0x20, page_table=0x30, max_pages=8, kv=D.dflash_kv(0x40, 0x50, 8),
             max_ctx=100, top_k=8, tokens=0x60, topk_ids=0x70, topk_lp=0x80, dbg=None, ws=0x100000, ws_bytes=1 << 40,
             stream=None)
    a.update(over)
    return D.dflash_draft_block(h, a["batch"], a["block_tokens"], a["ctx_len"], a["page_table"], a["max_pages"],
                                a["kv"], a["max_ctx"], a["top_k"], a["tokens"], a["topk_ids"], a["topk_lp"], a["dbg"],
                                a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), -1),
    (dict(block_tokens=None), -1),
    (dict(tokens=None), -1),
    (dict(top_k=9), -4),
    (dict(topk_ids=None), -1),
    (dict(max_ctx=-1), -1),
    (dict(max_ctx=129), -3),          # beyond max_pages * 16
    (dict(page_table=None), -1),
    (dict(kv=None), -1),
    (dict(ws_bytes=100), -3),
    (dict(ws=0x100010), -1),          # misaligned workspace
])
def test_draft_block_validation(D, over, code):
    m = _create(D, _shape())
    try:
        assert _draft(D, m.handle, **over) == code
        assert D.dflash_last_error()
    finally:
        m.close()


def test_float32_drafter_limits_block_rows(D):
    import workloads as W
    m = _create(D, W.SMALL_FP32)                      # block_len 5: 7 requests = 35 rows > 32
    try:
        assert _draft(D, m.handle, batch=7, max_ctx=40) == D.DFLASH_E_UNSUPPORTED
    finally:
        m.close()


def test_draft_block_null_handle(D):
    assert _draft(D, None) == D.DFLASH_E_ARG


def test_workspace_sizes(D):
    m = _create(D, _shape())
    try:
        a = D.dflash_draft_workspace_bytes(m.handle, 1, 100)
        b = D.dflash_draft_workspace_bytes(m.handle, 2, 4096)
        assert 0 < a < b and a % 256 == 0
        assert D.dflash_draft_workspace_bytes(m.handle, 0, 100) == 0
        assert D.dflash_inject_workspace_bytes(m.handle, 7) > 0
        assert D.dflash_inject_workspace_bytes(m.handle, 0) == 0
    finally:
        m.close()


def test_inject_validation(D):
    m = _create(D, _shape())
    kv = D.dflash_kv(0x40, 0x50, 8)
    try:
        call = lambda **o: D.dflash_inject_ctx(m.handle, o.get("batch", 1), o.get("n_rows", 4), o.get("feats", 0x10),
                                               o.get("stride", 1536), 0x20, 0x30, 0x40, 8, o.get("kv", kv), 0x100000,
                                               o.get("ws_bytes", 1 << 40), None)
        assert call(batch=0) == -1
        assert call(feats=None) == -1
        assert call(stride=100) == -1
        assert call(stride=1540) == -1          # rows not 16-byte aligned
        assert call(ws_bytes=10) == -3
        assert call(kv=D.dflash_kv(0, 0x50, 8)) == -1
    finally:
        m.close()


def test_accept_and_linear_validation(D):
    assert D.dflash_accept_len(0, 15, 0x10, 16, 0x20, 16, 0x30, None) == -1
    assert D.dflash_accept_len(1, 15, None, 16, 0x20, 16, 0x30, None) == -1
    assert D.dflash_accept_len(1, 15, 0x10, 8, 0x20, 16, 0x30, None) == -1
    assert D.dflash_linear(1, 16, 64, 100, 0x10, 100, 0x20, 0x30, 0x40, 1 << 30, None) == -4
    assert D.dflash_linear(2, 16, 64, 256, 0x10, 256, 0x20, 0x30, 0x40, 1 << 30, None) == -1
    assert D.dflash_linear(1, 16, 64, 256, 0x10, 256, 0x20, 0x30, 0x40, 16, None) == -3
    assert D.dflash_linear_workspace_bytes(1, 16, 4096, 4096) > 0
    assert D.dflash_copy(0x10, 0x20, 17, None) == -1


def _packed_elems(n, k):
    """Rows padded to whole 64-row groups (four 16-row fragment tiles)."""
    return -(-n // 64) * 64 * k


def test_packed_weight_store_size(D):
    """The packed store holds every projection matrix once; matrices one GEMM stacks ([wq; wk; wv], [w_gate;
    w_up], the layers' [uk; uv]) are packed as one matrix, each padded to whole 64-row groups."""
    import workloads as W
    for s in (W.QWEN3_8B, W.SMALL_BF16, W.SMALL_GQA8):
        m = _create(D, s)
        qd, kvd, H, F = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim, s.hidden, s.ffn
        per_layer = (_packed_elems(qd + 2 * kvd, H) + _packed_elems(2 * kvd, H) + _packed_elems(H, qd)
                     + _packed_elems(2 * F, H) + _packed_elems(H, F))
        want = 2 * (s.n_layers * per_layer + _packed_elems(H, s.feat_dim) + _packed_elems(s.vocab, H))
        assert D.dflash_packed_weight_bytes(m.handle) == want
        m.close()
    m = _create(D, W.SMALL_FP32)
    assert D.dflash_packed_weight_bytes(m.handle) == 0
    assert D.dflash_pack_weights(m.handle, None, 0, None) == 0  # float32: nothing to pack, no HIP call
    m.close()


@pytest.mark.parametrize("dst,nbytes,code", [
    (None, 1 << 40, -1),
    (0x100010, 1 << 40, -1),   # misaligned
    (0x100000, 1024, -3),      # too small
])
def test_pack_weights_validation(D, dst, nbytes, code):
    m = _create(D, _shape())
    try:
        assert D.dflash_pack_weights(m.handle, dst, nbytes, None) == code
        assert D.dflash_last_error()
    finally:
        m.close()


def test_unpacked_bf16_handle_refuses_to_run(D):
    m = _create(D, _shape())
    try:
        assert _draft(D, m.handle) == D.DFLASH_E_ARG
        assert "packed" in D.dflash_last_error()
        kv = D.dflash_kv(0x40, 0x50, 8)
        rc = D.dflash_inject_ctx(m.handle, 1, 4, 0x10, m.shape.feat_dim, 0x20, 0x30, 0x40, 8, kv, 0x100000, 1 << 40,
                                 None)
        assert rc == D.DFLASH_E_ARG and "packed" in D.dflash_last_error()
    finally:
        m.close()


@pytest.mark.parametrize("args,code", [
    (dict(rows=0), -1), (dict(k=0), -1), (dict(k=6000), -1), (dict(k=1025, vocab=4096), -4),
    (dict(row_stride=10), -1), (dict(logits=None), -1),
    (dict(ws=None), -1), (dict(ws_bytes=100), -1), (dict(ws=0x8008), -1),
])
def test_topk_logprobs_validation(D, args, code):
    a = dict(rows=2, vocab=5003, k=8, logits=0x1000, row_stride=5003, ids=0x2000, lp=0x3000, ws=0x8000,
             ws_bytes=1 << 30)
    a.update(args)
    assert D.dflash_topk_logprobs(a["rows"], a["vocab"], a["k"], a["logits"], a["row_stride"], a["ids"], a["lp"],
                                  a["ws"], a["ws_bytes"], None) == code
    assert D.dflash_last_error()


def test_topk_logprobs_workspace_size(D):
    """Few rows split over chunks: a 16-byte partial per chunk plus (key, id) slots for its candidates (twice its
    share kt = ceil(1.5 K / C) + 8, plus 32); a batch that fills the chip with one workgroup per row needs
    none."""
    # 16 rows of 151936: 16 chunks of 9496
    assert D.dflash_topk_logprobs_workspace_bytes(16, 151936, 1024) == 16 * 16 * (16 + (2 * (96 + 8) + 32) * 8)
    assert D.dflash_topk_logprobs_workspace_bytes(16, 151936, 16) == 16 * 16 * (16 + (2 * (2 + 8) + 32) * 8)
    assert D.dflash_topk_logprobs_workspace_bytes(256, 151936, 1024) == 0
    assert D.dflash_topk_logprobs_workspace_bytes(16, 151936, 1025) == 0   # refused by the call itself
    # a short row: chunks shorter than k keep every entry
    n = D.dflash_topk_logprobs_workspace_bytes(1, 5003, 1000)
    assert n > 0 and n % 16 == 0


@pytest.mark.parametrize("args,code", [
    (dict(batch=0), -1), (dict(depth=0), -1), (dict(depth=17), -4), (dict(k=1025), -4),
    (dict(budget=2048), -4), (dict(budget=0), -1), (dict(req_stride=7), -1), (dict(n_nodes=None), -1),
])
@pytest.mark.parametrize("entry", ["dflash_ddtree_build", "dflash_ddtree_select"])
def test_ddtree_build_validation(D, args, code, entry):
    a = dict(batch=1, depth=15, k=64, lp=0x1000, ids=0x2000, req_stride=15 * 64, budget=256, tok=0x3000,
             par=0x4000, dep=0x5000, lq=0x6000, n_nodes=0x7000)
    a.update(args)
    assert getattr(D, entry)(a["batch"], a["depth"], a["k"], a["lp"], a["ids"], a["req_stride"], a["budget"],
                             a["tok"], a["par"], a["dep"], a["lq"], a["n_nodes"], None) == code
    assert D.dflash_last_error()


@pytest.mark.parametrize("args,code", [
    (dict(batch=0), -1), (dict(budget=2048), -4), (dict(max_accept=0), -1), (dict(target=None), -1),
])
def test_ddtree_walk_validation(D, args, code):
    a = dict(batch=1, budget=256, max_accept=15, tok=0x1000, par=0x2000, n=0x3000, target=0x4000, alen=0x5000,
             anodes=0x6000, bonus=0x7000)
    a.update(args)
    assert D.dflash_ddtree_walk(a["batch"], a["budget"], a["max_accept"], a["tok"], a["par"], a["n"], a["target"],
                                a["alen"], a["anodes"], a["bonus"], None) == code
    assert D.dflash_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), -1), (dict(tokens=None), -1), (dict(top_k=9), -4), (dict(ws_bytes=100), -3),
    (dict(max_ctx=129), -3), (dict(ws=0x100010), -1),
])
def test_draft_block_sample_validation(D, over, code):
    """The temperature-1 pass shares the greedy pass's checks (same shapes, same workspace)."""
    m = _create(D, _shape())
    a = dict(batch=1, max_ctx=100, top_k=8, tokens=0x60, ws=0x100000, ws_bytes=1 << 40)
    a.update(over)
    try:
        assert D.dflash_draft_block_sample(m.handle, a["batch"], 0x10, 0x20, 0x30, 8, D.dflash_kv(0x40, 0x50, 8),
                                           a["max_ctx"], a["top_k"], 12345, a["tokens"], 0x70, 0x80, 0x90, a["ws"],
                                           a["ws_bytes"], None) == code
        assert D.dflash_last_error()
    finally:
        m.close()


def test_verify_sample_workspace_size(D):
    a = D.dflash_verify_sample_workspace_bytes(1, 15, 151936)
    assert a >= 31 * 38 * 8 + 38 * 16 + 4 and a % 256 == 0
    assert D.dflash_verify_sample_workspace_bytes(16, 15, 151936) > a
    assert D.dflash_verify_sample_workspace_bytes(1, 0, 10) > 0
    assert D.dflash_verify_sample_workspace_bytes(0, 15, 100) == 0
    assert D.dflash_verify_sample_workspace_bytes(1, 64, 100) == 0
    assert D.dflash_verify_sample_workspace_bytes(1, 15, 0) == 0


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), -1), (dict(batch=65536), -1), (dict(n_draft=64), -4), (dict(n_draft=-1), -4),
    (dict(vocab=0), -1), (dict(p=None), -1), (dict(tau=None), -1), (dict(nxt=None), -1), (dict(ws=None), -1),
    (dict(draft=None), -1), (dict(q=None), -1), (dict(dstride=14), -1), (dict(p_req=15 * 1000), -1),
    (dict(q_req=14 * 1000), -1), (dict(ws_bytes=100), -3), (dict(ws=0x100010), -1),
])
def test_verify_sample_validation(D, over, code):
    a = dict(batch=2, n_draft=15, vocab=1000, draft=0x10, dstride=16, q=0x20, q_req=16 * 1000, p=0x30,
             p_req=16 * 1000, tau=0x40, nxt=0x50, ws=0x100000, ws_bytes=1 << 30)
    a.update(over)
    assert D.dflash_verify_sample(a["batch"], a["n_draft"], a["vocab"], a["draft"], a["dstride"], a["q"], a["q_req"],
                                  a["p"], a["p_req"], 7, a["tau"], a["nxt"], a["ws"], a["ws_bytes"], None) == code
    assert D.dflash_last_error()


def test_tree_attention_workspace_size(D):
    a = D.dflash_tree_attention_workspace_bytes(1, 1025, 32, 8, 128, 4096)
    assert a > 1025 * 40 * 128 * 2 and a % 256 == 0
    assert D.dflash_tree_attention_workspace_bytes(1, 1025, 32, 8, 128, 0) < a
    assert D.dflash_tree_attention_workspace_bytes(1, 2049, 32, 8, 128, 100) == 0
    assert D.dflash_tree_attention_workspace_bytes(1, 16, 32, 8, 64, 100) == 0
    assert D.dflash_tree_attention_workspace_bytes(1, 16, 24, 8, 128, 100) == 0
    assert D.dflash_tree_attention_workspace_bytes(0, 16, 32, 8, 128, 100) == 0
    # the context rounds of every (request, token tile) are indexed in 32 bits
    assert D.dflash_tree_attention_workspace_bytes(1, 2048, 32, 8, 128, 1 << 20) > 0
    assert D.dflash_tree_attention_workspace_bytes(65535, 2048, 32, 8, 128, 1 << 20) == 0


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), -1), (dict(T=0), -1), (dict(T=2049), -1), (dict(d=64), -4), (dict(nq=24), -4), (dict(nq=20), -1),
    (dict(nq=48, nkv=3), -4), (dict(max_ctx=-1), -1), (dict(n_tok=None), -1), (dict(parent=None), -1),
    (dict(q=None), -1), (dict(out=None), -1), (dict(kp=None), -1), (dict(pt=None), -1), (dict(max_pages=0), -1),
    (dict(max_ctx=8 * 16 + 1), -3), (dict(theta=-1.0), -1), (dict(q=0x1008), -1), (dict(ws_bytes=100), -3),
    (dict(ws=0x100010), -1),
])
def test_tree_attention_validation(D, over, code):
    a = dict(batch=1, T=64, n_tok=0x10, parent=0x20, nq=32, nkv=8, d=128, q=0x1000, k=0x2000, v=0x3000,
             kp=0x4000, vp=0x5000, n_pages=8, pt=0x6000, max_pages=8, ctx=0x7000, max_ctx=100, theta=1e6,
             out=0x8000, ws=0x100000, ws_bytes=1 << 30)
    a.update(over)
    assert D.dflash_tree_attention(a["batch"], a["T"], a["n_tok"], a["parent"], a["nq"], a["nkv"], a["d"], a["q"],
                                   a["k"], a["v"], a["kp"], a["vp"], a["n_pages"], a["pt"], a["max_pages"], a["ctx"],
                                   a["max_ctx"], a["theta"], a["out"], a["ws"], a["ws_bytes"], None) == code
    assert D.dflash_last_error()


def test_inject_workspace_covers_every_chunk(D):
    """A call of n rows runs chunks of 4096 rows and a shorter last chunk, and a short chunk may be split
    further along K than a long one.  The size dflash_inject_workspace_bytes(h, n) reports must pass the call's
    own capacity check for every row count up to n (here up to two whole chunks).  The call then stops at the
    missing weight store (-1, "packed"), which proves the capacity check passed."""
    import workloads as W
    kv = D.dflash_kv(0x40, 0x50, 8)
    for s in (W.QWEN3_8B, W.QWEN3_4B, W.SMALL_BF16):
        m = _create(D, s)
        try:
            prev = 0
            sizes = {}
            for n in list(range(1, 65)) + list(range(100, 2 * 4096 + 1, 37)) + [4095, 4096, 4097, 5096, 8192]:
                ws = D.dflash_inject_workspace_bytes(m.handle, n)
                sizes[n] = ws
                rc = D.dflash_inject_ctx(m.handle, 1, n, 0x10, s.feat_dim, 0x20, 0x30, 0x40, 8, kv, 0x100000, ws,
                                         None)
                assert rc == D.DFLASH_E_ARG and "packed" in D.dflash_last_error(), (s, n, rc)
            for n in sorted(sizes):
                assert sizes[n] >= prev, (s, n)   # a bound for every call of at most n rows
                prev = sizes[n]
            assert sizes[8192] == sizes[4096]         # chunks never exceed 4096 rows
        finally:
            m.close()


def test_no_context_ignores_page_table(D):
    """max_ctx = 0: no page table or pool is read, so NULL is accepted whatever max_pages says (the call then
    stops at the missing weight store, after every shape check)."""
    m = _create(D, _shape())
    try:
        rc = _draft(D, m.handle, max_ctx=0, page_table=None, max_pages=8, kv=None)
        assert rc == D.DFLASH_E_ARG and "packed" in D.dflash_last_error()
        rc = _draft(D, m.handle, max_ctx=0, page_table=None, max_pages=0, kv=None)
        assert rc == D.DFLASH_E_ARG and "packed" in D.dflash_last_error()
    finally:
        m.close()


def _min_inject_ws(D, m, n, kv):
    """Smallest workspace (multiple of 256) that passes the capacity check of an n-row call."""
    lo, hi = 0, D.dflash_inject_workspace_bytes(m.handle, n) // 256
    while lo < hi:
        mid = (lo + hi) // 2
        rc = D.dflash_inject_ctx(m.handle, 1, n, 0x10, m.shape.feat_dim, 0x20, 0x30, 0x40, 8, kv, 0x100000, mid * 256,
                                 None)
        if rc == D.DFLASH_E_CAPACITY:
            lo = mid + 1
        else:
            hi = mid
    return lo * 256


def test_inject_short_last_chunk_needs_its_own_split_partials(D):
    """4096 + t rows: the t-row tail chunk has its own GEMM plans, and a tail whose fusion or KV GEMM splits K
    further than a whole chunk's writes more float32 partials than a whole 4096-row chunk.  Some of the tried
    tails must do so (the plan weighs generations of workgroups against partial traffic, so which ones
    depends on it), and for each of them a workspace sized for one whole chunk must be refused instead of
    being overrun."""
    import workloads as W
    kv = D.dflash_kv(0x40, 0x50, 8)
    m = _create(D, W.QWEN3_8B)
    try:
        one_chunk = _min_inject_ws(D, m, 4096, kv)
        larger = [t for t in (1000, 2500, 3500) if _min_inject_ws(D, m, 4096 + t, kv) > one_chunk]
        assert larger
        for t in larger:
            rc = D.dflash_inject_ctx(m.handle, 1, 4096 + t, 0x10, m.shape.feat_dim, 0x20, 0x30, 0x40, 8, kv,
                                     0x100000, one_chunk, None)
            assert rc == D.DFLASH_E_CAPACITY
            assert D.dflash_inject_workspace_bytes(m.handle, 4096 + t) >= _min_inject_ws(D, m, 4096 + t, kv)
    finally:
        m.close()


def test_noalloc_pass_validates_before_touching_the_gpu(D):
    """dflash_draft_block_noalloc shares the pass's argument checks and refuses, before any HIP call, a pass
    whose workspace would exceed its static scratch (DFLASH_NOALLOC_SCRATCH_BYTES = 32 MiB)."""
    import workloads as W
    m = _create(D, W.QWEN3_8B)
    kv = D.dflash_kv(0x40, 0x50, 8192)
    call = lambda **o: D.dflash_draft_block_noalloc(m.handle, o.get("batch", 1), 0x10, 0x20, 0x30,
                                                    o.get("max_pages", 512), kv, o.get("max_ctx", 4096), 8, 0x60,
                                                    0x70, 0x80, None, None)
    try:
        assert D.dflash_draft_workspace_bytes(m.handle, 16, 8192) > 32 << 20
        assert call(batch=16, max_ctx=8192) == D.DFLASH_E_CAPACITY
        assert "allocation-free" in D.dflash_last_error()
        assert call(batch=0) == D.DFLASH_E_ARG
        assert call(max_ctx=8193) == D.DFLASH_E_CAPACITY        # beyond max_pages * 16
        # batch 1 at any context fits: the call gets as far as the missing weight store
        for ctx in (0, 4096, 8192):
            assert D.dflash_draft_workspace_bytes(m.handle, 1, ctx) <= 32 << 20
            assert call(max_ctx=ctx) == D.DFLASH_E_ARG and "packed" in D.dflash_last_error()
    finally:
        m.close()

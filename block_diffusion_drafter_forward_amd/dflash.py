"""Thin Python binding of libdflash.so (include/dflash.h): argument marshalling only.

Every function of the C ABI is exposed under its own name.  ``DraftModel`` is a convenience holder that
keeps torch device tensors (weights, KV pool, workspaces) alive and turns them into the pointers and
structs the ABI takes; all computation happens in the HIP kernels of the library.  Importing this module
raises if the library is not built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdflash.so")

DFLASH_OK = 0
DFLASH_E_ARG = -1
DFLASH_E_SHAPE = -2
DFLASH_E_CAPACITY = -3
DFLASH_E_UNSUPPORTED = -4
DFLASH_E_HIP = -5
DFLASH_F32 = 0
DFLASH_BF16 = 1
DEVERR_PAGE, DEVERR_POS, DEVERR_TOKEN, DEVERR_ROWS, DEVERR_TREE = 1, 2, 4, 8, 16


class dflash_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("feat_dim", ctypes.c_int), ("block_len", ctypes.c_int),
                ("page_size", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("dtype", ctypes.c_int)]


_LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "uk", "uv", "ffn_norm", "w_gate", "w_up", "w_down"]


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _LAYER_FIELDS]


class dflash_weights(ctypes.Structure):
    _fields_ = [("fc_w", ctypes.c_void_p), ("fc_b", ctypes.c_void_p), ("embed", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(dflash_layer_weights))]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_pages", ctypes.c_int)]


class dflash_debug(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("hidden", ctypes.c_void_p)]


class dflash_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


_lib = None

_SIGS = {
    "dflash_create": (ctypes.c_int, [ctypes.POINTER(dflash_config), ctypes.POINTER(dflash_weights),
                                     ctypes.POINTER(ctypes.c_void_p)]),
    "dflash_destroy": (None, [ctypes.c_void_p]),
    "dflash_packed_weight_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "dflash_pack_weights": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_draft_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]),
    "dflash_inject_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int]),
    "dflash_inject_ctx": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.POINTER(dflash_kv), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_draft_block": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(dflash_kv), ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.POINTER(dflash_debug), ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]),
    "dflash_draft_block_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(dflash_kv),
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.POINTER(dflash_debug), ctypes.c_void_p]),
    "dflash_accept_len": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "dflash_draft_block_sample": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(dflash_kv),
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_verify_sample_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dflash_verify_sample": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_last_error": (ctypes.c_char_p, []),
    "dflash_topk_logprobs_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dflash_topk_logprobs": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "dflash_ddtree_build": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dflash_ddtree_select": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dflash_ddtree_walk": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "dflash_tree_attention_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "dflash_tree_attention": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_linear_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dflash_linear": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dflash_profile_enable": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "dflash_profile_collect": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(dflash_kernel_stat), ctypes.c_int]),
}

EXPORTS = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded library; raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class DFlashError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().dflash_last_error().decode()
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


def check(code: int, where: str) -> None:
    if code != DFLASH_OK:
        raise DFlashError(code, where)


# ---- the ABI functions, same names -------------------------------------------------------------------------

def dflash_create(cfg: dflash_config, w: dflash_weights) -> int:
    h = ctypes.c_void_p()
    check(lib().dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)), "dflash_create")
    return h.value


def dflash_destroy(h: int) -> None:
    lib().dflash_destroy(h)


def dflash_topk_logprobs_workspace_bytes(rows, vocab, k) -> int:
    return lib().dflash_topk_logprobs_workspace_bytes(rows, vocab, k)


def dflash_topk_logprobs(rows, vocab, k, logits, row_stride, ids, logprobs, workspace, workspace_bytes,
                         stream) -> int:
    return lib().dflash_topk_logprobs(rows, vocab, k, logits, row_stride, ids, logprobs, workspace, workspace_bytes,
                                      stream)


def dflash_ddtree_build(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent, node_depth,
                        node_logq, n_nodes, stream) -> int:
    return lib().dflash_ddtree_build(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent,
                                     node_depth, node_logq, n_nodes, stream)


def dflash_ddtree_select(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent, node_depth,
                         node_logq, n_nodes, stream) -> int:
    return lib().dflash_ddtree_select(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent,
                                      node_depth, node_logq, n_nodes, stream)


def dflash_ddtree_walk(batch, budget, max_accept, node_token, node_parent, n_nodes, target_next, accept_len,
                       accept_nodes, bonus, stream) -> int:
    return lib().dflash_ddtree_walk(batch, budget, max_accept, node_token, node_parent, n_nodes, target_next,
                                    accept_len, accept_nodes, bonus, stream)


def dflash_packed_weight_bytes(h: int) -> int:
    return lib().dflash_packed_weight_bytes(h)


def dflash_pack_weights(h: int, dst, dst_bytes: int, stream) -> int:
    return lib().dflash_pack_weights(h, dst, dst_bytes, stream)


def dflash_draft_workspace_bytes(h: int, max_batch: int, max_ctx: int) -> int:
    return lib().dflash_draft_workspace_bytes(h, max_batch, max_ctx)


def dflash_inject_workspace_bytes(h: int, max_rows: int) -> int:
    return lib().dflash_inject_workspace_bytes(h, max_rows)


def dflash_inject_ctx(h, batch, n_rows, feats, feat_row_stride, row_offsets, start_pos, page_table, max_pages,
                      kv: dflash_kv, ws, ws_bytes, stream) -> int:
    return lib().dflash_inject_ctx(h, batch, n_rows, feats, feat_row_stride, row_offsets, start_pos, page_table,
                                   max_pages, ctypes.byref(kv), ws, ws_bytes, stream)


def dflash_draft_block(h, batch, block_tokens, ctx_len, page_table, max_pages, kv: Optional[dflash_kv], max_ctx,
                       top_k, tokens, topk_ids, topk_logprobs, dbg: Optional[dflash_debug], ws, ws_bytes,
                       stream) -> int:
    return lib().dflash_draft_block(h, batch, block_tokens, ctx_len, page_table, max_pages,
                                    ctypes.byref(kv) if kv is not None else None, max_ctx, top_k, tokens, topk_ids,
                                    topk_logprobs, ctypes.byref(dbg) if dbg is not None else None, ws, ws_bytes,
                                    stream)


def dflash_draft_block_noalloc(h, batch, block_tokens, ctx_len, page_table, max_pages, kv: Optional[dflash_kv],
                               max_ctx, top_k, tokens, topk_ids, topk_logprobs, dbg: Optional[dflash_debug],
                               stream) -> int:
    return lib().dflash_draft_block_noalloc(h, batch, block_tokens, ctx_len, page_table, max_pages,
                                            ctypes.byref(kv) if kv is not None else None, max_ctx, top_k, tokens,
                                            topk_ids, topk_logprobs, ctypes.byref(dbg) if dbg is not None else None,
                                            stream)


def dflash_accept_len(batch, n_draft, draft, draft_stride, target, target_stride, tau, stream) -> int:
    return lib().dflash_accept_len(batch, n_draft, draft, draft_stride, target, target_stride, tau, stream)


def dflash_draft_block_sample(h, batch, block_tokens, ctx_len, page_table, max_pages, kv: Optional[dflash_kv],
                              max_ctx, top_k, seed, tokens, topk_ids, topk_logprobs, logits, ws, ws_bytes,
                              stream) -> int:
    return lib().dflash_draft_block_sample(h, batch, block_tokens, ctx_len, page_table, max_pages,
                                           ctypes.byref(kv) if kv is not None else None, max_ctx, top_k, seed,
                                           tokens, topk_ids, topk_logprobs, logits, ws, ws_bytes, stream)


def dflash_verify_sample_workspace_bytes(batch, n_draft, vocab) -> int:
    return lib().dflash_verify_sample_workspace_bytes(batch, n_draft, vocab)


def dflash_verify_sample(batch, n_draft, vocab, draft, draft_stride, q_logits, q_req_stride, p_logits, p_req_stride,
                         seed, tau, next_token, ws, ws_bytes, stream) -> int:
    return lib().dflash_verify_sample(batch, n_draft, vocab, draft, draft_stride, q_logits, q_req_stride, p_logits,
                                      p_req_stride, seed, tau, next_token, ws, ws_bytes, stream)


def dflash_last_error() -> str:
    return lib().dflash_last_error().decode()


def dflash_linear_workspace_bytes(dtype, M, N, K) -> int:
    return lib().dflash_linear_workspace_bytes(dtype, M, N, K)


def dflash_linear(dtype, M, N, K, x, ldx, w, y, ws, ws_bytes, stream) -> int:
    return lib().dflash_linear(dtype, M, N, K, x, ldx, w, y, ws, ws_bytes, stream)


def dflash_copy(dst, src, n_bytes, stream) -> int:
    return lib().dflash_copy(dst, src, n_bytes, stream)


def dflash_profile_enable(h, on) -> int:
    return lib().dflash_profile_enable(h, on)


def dflash_profile_collect(h, max_entries: int = 64):
    arr = (dflash_kernel_stat * max_entries)()
    n = lib().dflash_profile_collect(h, arr, max_entries)
    if n < 0:
        raise DFlashError(n, "dflash_profile_collect")
    return [(arr[i].name.decode(), arr[i].launches, arr[i].total_ms) for i in range(n)]


# ---- torch marshalling helper ------------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class DraftModel:
    """Device-resident drafter: weights, config and a handle of the library.

    weights: dict name -> torch tensor on the GPU, names as in the header (fc_w, fc_b, embed, final_norm,
    lm_head, and per layer "l{i}.attn_norm", "l{i}.wq", ...).  bfloat16 tensors may be given as int16/uint16
    bit patterns or torch.bfloat16; float32 as torch.float32.  pack=False skips the packed weight store
    (argument-validation tests without a GPU; such a bfloat16 handle cannot run a pass).
    """

    def __init__(self, shape, weights: Dict[str, "object"], pack: bool = True):
        self.shape = shape
        self.weights = weights
        s = shape
        self.cfg = dflash_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                                 s.feat_dim, s.block_len, s.page_size, s.rms_eps, s.rope_theta,
                                 DFLASH_BF16 if s.bf16 else DFLASH_F32)
        self._layers = (dflash_layer_weights * s.n_layers)()
        for l in range(s.n_layers):
            for f in _LAYER_FIELDS:
                setattr(self._layers[l], f, _ptr(weights[f"l{l}.{f}"]))
        self.w = dflash_weights(_ptr(weights["fc_w"]), _ptr(weights.get("fc_b")), _ptr(weights["embed"]),
                                _ptr(weights["final_norm"]), _ptr(weights["lm_head"]), self._layers)
        self.handle = dflash_create(self.cfg, self.w)
        # bfloat16 drafters stream a fragment-ordered copy of the projection matrices (made once, on device)
        self.packed = None
        n = dflash_packed_weight_bytes(self.handle)
        if n and pack:
            import torch
            self.packed = torch.empty(n, dtype=torch.uint8, device="cuda")
            check(dflash_pack_weights(self.handle, self.packed.data_ptr(), n, _stream()), "dflash_pack_weights")

    def close(self):
        if self.handle:
            dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # workspaces -------------------------------------------------------------------------------------------
    def draft_workspace(self, max_batch: int, max_ctx: int):
        import torch
        n = dflash_draft_workspace_bytes(self.handle, max_batch, max_ctx)
        return torch.empty(n, dtype=torch.uint8, device="cuda")

    def inject_workspace(self, max_rows: int):
        import torch
        n = dflash_inject_workspace_bytes(self.handle, max_rows)
        return torch.empty(n, dtype=torch.uint8, device="cuda")

    # calls ------------------------------------------------------------------------------------------------
    def inject(self, feats, row_offsets, start_pos, page_table, kv: dflash_kv, ws, stream=None) -> None:
        batch = row_offsets.numel() - 1
        check(dflash_inject_ctx(self.handle, batch, feats.shape[0], feats.data_ptr(), feats.stride(0),
                                row_offsets.data_ptr(), start_pos.data_ptr(), page_table.data_ptr(),
                                page_table.shape[1], kv, ws.data_ptr(), ws.numel(), _stream(stream)),
              "dflash_inject_ctx")

    def draft(self, block_tokens, ctx_len, page_table, kv: Optional[dflash_kv], max_ctx: int, top_k: int, tokens,
              topk_ids=None, topk_logprobs=None, ws=None, logits=None, hidden=None, stream=None) -> None:
        dbg = dflash_debug(_ptr(logits), _ptr(hidden)) if (logits is not None or hidden is not None) else None
        batch = block_tokens.shape[0]
        check(dflash_draft_block(self.handle, batch, block_tokens.data_ptr(), ctx_len.data_ptr(),
                                 _ptr(page_table), page_table.shape[1] if page_table is not None else 0, kv,
                                 max_ctx, top_k, tokens.data_ptr(), _ptr(topk_ids), _ptr(topk_logprobs), dbg,
                                 ws.data_ptr(), ws.numel(), _stream(stream)), "dflash_draft_block")

    def draft_sample(self, block_tokens, ctx_len, page_table, kv: Optional[dflash_kv], max_ctx: int, top_k: int,
                     seed: int, tokens, topk_ids=None, topk_logprobs=None, ws=None, logits=None, stream=None) -> None:
        """Temperature-1 drafting: tokens are Gumbel-max samples keyed by `seed`; logits (optional) receives
        the full [batch][L][V] float32 logits that verify_sample reads."""
        batch = block_tokens.shape[0]
        check(dflash_draft_block_sample(self.handle, batch, block_tokens.data_ptr(), ctx_len.data_ptr(),
                                        _ptr(page_table), page_table.shape[1] if page_table is not None else 0, kv,
                                        max_ctx, top_k, seed, tokens.data_ptr(), _ptr(topk_ids), _ptr(topk_logprobs),
                                        _ptr(logits), ws.data_ptr(), ws.numel(), _stream(stream)),
              "dflash_draft_block_sample")


def accept_len(draft, target, tau, stream=None) -> None:
    """tau[r] = 1 + common-prefix length of draft[r] and target[r] (int32 CUDA tensors, row-major)."""
    check(dflash_accept_len(draft.shape[0], draft.shape[1], draft.data_ptr(), draft.stride(0), target.data_ptr(),
                            target.stride(0), tau.data_ptr(), _stream(stream)), "dflash_accept_len")


def verify_sample_workspace_bytes(batch: int, n_draft: int, vocab: int) -> int:
    return dflash_verify_sample_workspace_bytes(batch, n_draft, vocab)


def verify_sample(draft, q_logits, p_logits, seed: int, tau, next_token, ws, stream=None) -> None:
    """Temperature-1 verification.  draft: int32 [B, n] (any row stride); q_logits: float32 [B, n, V] view
    (rows contiguous, any request stride); p_logits: float32 [B, n + 1, V] likewise; tau, next_token: int32 [B];
    ws: a 256-byte-aligned tensor of at least verify_sample_workspace_bytes(B, n, V) bytes."""
    B, n = draft.shape
    V = p_logits.shape[-1]
    if p_logits.stride(-1) != 1 or p_logits.stride(1) != V or (n and (q_logits.stride(-1) != 1 or
                                                                     q_logits.stride(1) != V)):
        raise ValueError("logit rows must be contiguous with stride V")
    check(dflash_verify_sample(B, n, V, draft.data_ptr(), draft.stride(0), _ptr(q_logits) if n else None,
                               q_logits.stride(0) if n else 0, p_logits.data_ptr(), p_logits.stride(0), seed,
                               tau.data_ptr(), next_token.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                               _stream(stream)), "dflash_verify_sample")


def dflash_tree_attention_workspace_bytes(batch, max_tokens, n_q_heads, n_kv_heads, head_dim, max_ctx) -> int:
    return lib().dflash_tree_attention_workspace_bytes(batch, max_tokens, n_q_heads, n_kv_heads, head_dim, max_ctx)


def dflash_tree_attention(batch, max_tokens, n_tokens, parent, n_q_heads, n_kv_heads, head_dim, q, k, v, k_pages,
                          v_pages, n_pages, page_table, max_pages, ctx_len, max_ctx, rope_theta, out, ws, ws_bytes,
                          stream) -> int:
    return lib().dflash_tree_attention(batch, max_tokens, n_tokens, parent, n_q_heads, n_kv_heads, head_dim, q, k,
                                       v, k_pages, v_pages, n_pages, page_table, max_pages, ctx_len, max_ctx,
                                       rope_theta, out, ws, ws_bytes, stream)


def tree_attention(n_tokens, parent, q, k, v, k_pages, v_pages, page_table, ctx_len, max_ctx: int,
                   rope_theta: float, out, ws, stream=None) -> None:
    """Tree attention over CUDA tensors: n_tokens int32 [B], parent int32 [B, T], q bf16 [B, T, n_q, 128],
    k / v bf16 [B, T, n_kv, 128], k_pages bf16 [P, n_kv, 16, 128], v_pages bf16 [P, n_kv, 128, 16], page_table
    int32 [B, max_pages], ctx_len int32 [B], out bf16 [B, T, n_q, 128], ws a 256-byte-aligned uint8 tensor."""
    B, T, nq, d = q.shape
    nkv = k.shape[2]
    check(dflash_tree_attention(B, T, n_tokens.data_ptr(), parent.data_ptr(), nq, nkv, d, q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), _ptr(k_pages), _ptr(v_pages),
                                k_pages.shape[0] if k_pages is not None else 0, _ptr(page_table),
                                page_table.shape[1] if page_table is not None else 0, ctx_len.data_ptr(), max_ctx,
                                rope_theta, out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
          "dflash_tree_attention")


def make_kv(kpool, vpool, n_pages: int) -> dflash_kv:
    return dflash_kv(kpool.data_ptr(), vpool.data_ptr(), n_pages)

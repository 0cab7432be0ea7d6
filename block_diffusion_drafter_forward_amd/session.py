"""Device-side setup of a seeded workload: uploads the generated weights, features, page tables and block
tokens, owns the paged KV pool and the workspaces, and calls the library.  Data movement only: every step
of the drafter runs in libdflash's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dflash as D


def to_device(a: np.ndarray) -> torch.Tensor:
    """numpy -> CUDA tensor; bfloat16 bit patterns (uint16) travel as int16."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class GpuWorkload:
    """A Workload (see the ``workloads`` package) materialised on the GPU.

    extra_tokens reserves page-table room beyond each request's context (for appending in steady state).
    """

    def __init__(self, wl, weights=None, extra_tokens: int = 0, max_ctx=None):
        self.wl = wl
        s = wl.shape
        self.shape = s
        host_w = weights if weights is not None else wl.weights()
        self.weights = {k: to_device(v) for k, v in host_w.items()}
        self.model = D.DraftModel(s, self.weights)
        self.ctx = wl.ctx_lens().astype(np.int32)
        pt, n_pages = wl.page_table(extra_tokens)
        self.page_table_np = pt
        self.n_pages = n_pages
        self.page_table = to_device(pt)
        dt = torch.int16 if s.bf16 else torch.float32
        pool = (s.n_layers, n_pages, s.n_kv_heads, s.page_size, s.head_dim)
        self.kpool = torch.zeros(pool, dtype=dt, device="cuda")
        self.vpool = torch.zeros(pool, dtype=dt, device="cuda")
        self.kv = D.make_kv(self.kpool, self.vpool, n_pages)
        self.block_tokens = to_device(wl.block_tokens())
        self.ctx_len = to_device(self.ctx)
        self.max_ctx = int(self.ctx.max()) if max_ctx is None else int(max_ctx)
        B, L = wl.batch, s.block_len
        self.tokens = torch.zeros((B, L), dtype=torch.int32, device="cuda")
        k = max(wl.top_k, 1)
        self.topk_ids = torch.zeros((B, L, k), dtype=torch.int32, device="cuda")
        self.topk_lp = torch.zeros((B, L, k), dtype=torch.float32, device="cuda")
        self.draft_ws = self.model.draft_workspace(B, self.max_ctx)
        self.tau = torch.zeros(B, dtype=torch.int32, device="cuda")

    # ---- context injection -------------------------------------------------------------------------------
    def inject_rows(self, feats_per_req, start_pos, ws=None):
        """Inject feature rows: feats_per_req[r] is a host array [n_r, feat_dim] placed at start_pos[r]."""
        rows = [np.asarray(f) for f in feats_per_req]
        offs = np.zeros(len(rows) + 1, dtype=np.int32)
        offs[1:] = np.cumsum([f.shape[0] for f in rows])
        n = int(offs[-1])
        if n == 0:
            return
        feats = to_device(np.concatenate(rows, axis=0))
        if ws is None:
            ws = self.model.inject_workspace(n)
        self.model.inject(feats, to_device(offs), to_device(np.asarray(start_pos, dtype=np.int32)),
                          self.page_table, self.kv, ws)

    def prefill(self, rows_per_call: int = 16384):
        """Inject every request's full context, in calls of at most rows_per_call rows."""
        B = self.wl.batch
        done = [0] * B
        ws = None
        while any(done[r] < self.ctx[r] for r in range(B)):
            feats, starts, budget = [], [], rows_per_call
            for r in range(B):
                take = int(min(self.ctx[r] - done[r], budget))
                feats.append(self.wl.features(r, take, row0=done[r]) if take > 0
                             else np.zeros((0, self.shape.feat_dim), dtype=np.uint16 if self.shape.bf16 else np.float32))
                starts.append(done[r])
                done[r] += take
                budget -= take
            if ws is None:
                ws = self.model.inject_workspace(rows_per_call)
            self.inject_rows(feats, starts, ws)

    # ---- drafting ----------------------------------------------------------------------------------------
    def draft(self, top_k=None, logits=None, hidden=None, stream=None):
        k = self.wl.top_k if top_k is None else top_k
        self.model.draft(self.block_tokens, self.ctx_len, self.page_table, self.kv, self.max_ctx, k, self.tokens,
                         self.topk_ids if k > 0 else None, self.topk_lp if k > 0 else None, self.draft_ws,
                         logits=logits, hidden=hidden, stream=stream)

    def draft_sample(self, seed: int, top_k=None, logits=None, stream=None):
        """Temperature-1 pass: tokens are Gumbel-max samples keyed by seed; logits (optional) gets the full
        float32 logits."""
        k = self.wl.top_k if top_k is None else top_k
        self.model.draft_sample(self.block_tokens, self.ctx_len, self.page_table, self.kv, self.max_ctx, k, seed,
                                self.tokens, self.topk_ids if k > 0 else None, self.topk_lp if k > 0 else None,
                                self.draft_ws, logits=logits, stream=stream)

    def accept(self, target: torch.Tensor, stream=None):
        L = self.shape.block_len
        D.check(D.dflash_accept_len(self.wl.batch, L - 1, self.tokens.data_ptr() + 4, L, target.data_ptr(),
                                    target.stride(0), self.tau.data_ptr(), D._stream(stream)), "dflash_accept_len")

    def error_word(self, ws=None) -> int:
        w = self.draft_ws if ws is None else ws
        return int(w[:4].view(torch.int32).item()) & 0xFFFFFFFF

    def cache_rows(self, r: int, layer: int, positions):
        """Read back (K, V) of request r at the given positions as host arrays [n, n_kv, d] (bit patterns or
        float32): a gather by the documented page layout."""
        pos = np.asarray(positions)
        pages = self.page_table_np[r, pos // 16]
        slots = pos % 16
        k = self.kpool[layer][torch.as_tensor(pages, device="cuda"), :, torch.as_tensor(slots, device="cuda"), :]
        vt = self.vpool[layer].view(self.n_pages, self.shape.n_kv_heads, self.shape.head_dim, 16)
        v = vt[torch.as_tensor(pages, device="cuda"), :, :, torch.as_tensor(slots, device="cuda")]
        k, v = k.cpu().numpy(), v.cpu().numpy()
        if self.shape.bf16:
            k, v = k.view(np.uint16), v.view(np.uint16)
        return k, v

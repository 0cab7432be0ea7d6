"""The allocation-free drafter pass (dflash_draft_block_noalloc, for callers that cannot allocate) against
the workspace pass (dflash_draft_block), both called through the C ABI on the same inputs.  The two run the
same kernels with the same launch plan, so every output must be bit-identical: tokens, top-k ids and
log-probs, the full logits and the residual-stream taps.  Two workloads run back to back, the second smaller
than the first (fewer requests, shorter context, another handle), so the second call finds the static
scratch holding the first call's values; it must not read them.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _run(g, noalloc):
    import torch
    from block_diffusion_drafter_forward_amd import dflash as D
    wl, s = g.wl, g.shape
    B, L, V, k = wl.batch, s.block_len, s.vocab, wl.top_k
    out = dict(tokens=torch.full((B, L), -7, dtype=torch.int32, device="cuda"),
               ids=torch.full((B, L, k), -7, dtype=torch.int32, device="cuda"),
               lp=torch.full((B, L, k), float("nan"), dtype=torch.float32, device="cuda"),
               logits=torch.full((B, L, V), float("nan"), dtype=torch.float32, device="cuda"),
               hidden=torch.full((s.n_layers + 1, B * L, s.hidden), float("nan"), dtype=torch.float32,
                                 device="cuda"))
    dbg = D.dflash_debug(out["logits"].data_ptr(), out["hidden"].data_ptr())
    args = (g.model.handle, B, g.block_tokens.data_ptr(), g.ctx_len.data_ptr(), g.page_table.data_ptr(),
            g.page_table.shape[1], g.kv, g.max_ctx, k, out["tokens"].data_ptr(), out["ids"].data_ptr(),
            out["lp"].data_ptr(), dbg)
    if noalloc:
        rc = D.dflash_draft_block_noalloc(*args, D._stream())
    else:
        rc = D.dflash_draft_block(*args, g.draft_ws.data_ptr(), g.draft_ws.numel(), D._stream())
    D.check(rc, "noalloc pass" if noalloc else "workspace pass")
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in out.items()}


def test_noalloc_pass_equals_workspace_pass_on_two_calls():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_diffusion_drafter_forward_amd import session as S
    seen = []
    for name in ("small-bf16-serve9", "small-bf16-b1"):     # the second call is smaller
        wl = W.by_name(name)
        print(f"[noalloc] {name}: B={wl.batch}", flush=True)
        g = S.GpuWorkload(wl)
        g.prefill()
        seen.append(g.draft_ws.numel())
        a = _run(g, noalloc=True)
        b = _run(g, noalloc=False)
        assert g.error_word() == 0
        for n in a:
            np.testing.assert_array_equal(a[n], b[n], err_msg=f"{name}: {n}")
        assert not np.isnan(a["logits"]).any() and (a["tokens"] >= 0).all()
    assert seen[1] < seen[0]


def test_noalloc_pass_at_the_full_qwen3_8b_shape():
    """The headline shape (batch 1, 4096 cached tokens: 16 MB of scratch), twice in a row."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_diffusion_drafter_forward_amd import session as S
    wl = W.by_name("qwen3-8b-shape")
    print(f"[noalloc] {wl.name}", flush=True)
    g = S.GpuWorkload(wl)
    g.prefill()
    for _ in range(2):
        a = _run(g, noalloc=True)
        b = _run(g, noalloc=False)
        for n in a:
            np.testing.assert_array_equal(a[n], b[n], err_msg=n)

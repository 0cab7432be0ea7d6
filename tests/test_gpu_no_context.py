"""A drafter pass with no cached context at all: max_ctx = 0, no page table and no K/V pool (the C ABI allows
NULL for both then).  The block attends only to itself.  The HIP path is compared with the fp64 oracle on an
empty context, to the same criteria as the parity tests, and must leave the device error word clear.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

MARGIN = 1e-2


@pytest.mark.parametrize("name", ["small-bf16-paged-b2", "small-gqa8-b3", "small-fp32-b2"])
def test_draft_without_context(name):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_diffusion_drafter_forward_amd import session as S

    wl = W.by_name(name)
    s = wl.shape
    weights = wl.weights()
    g = S.GpuWorkload(wl, weights=weights)
    B, L, V, k = wl.batch, s.block_len, s.vocab, wl.top_k
    ctx0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.zeros((B, L, V), dtype=torch.float32, device="cuda")
    print(f"[no-context draft] {name}: B={B} L={L} V={V}", flush=True)
    g.model.draft(g.block_tokens, ctx0, None, None, 0, k, g.tokens, g.topk_ids, g.topk_lp, g.draft_ws,
                  logits=logits)
    torch.cuda.synchronize()
    assert g.error_word() == 0

    kv = [O.inject(weights, s, wl.features(r, 0), 0) for r in range(B)]
    ref = O.draft_block(weights, s, kv, wl.block_tokens(), k, return_taps=True)
    got = logits.cpu().numpy()
    tol = (3e-2 + 2e-2 * np.abs(ref["logits"])) if s.bf16 else (1e-4 + 1e-4 * np.abs(ref["logits"]))
    err = np.abs(got - ref["logits"])
    assert np.all(err <= tol), err.max()
    margin = O.sorted_margins(ref["logits"], 1)
    ok = margin > MARGIN
    assert ok.mean() > 0.5
    np.testing.assert_array_equal(g.tokens.cpu().numpy()[ok], ref["tokens"][ok])
    margin_k = O.sorted_margins(ref["logits"], k)
    ok_k = margin_k > MARGIN
    np.testing.assert_array_equal(g.topk_ids.cpu().numpy()[..., :k][ok_k], ref["topk_ids"][ok_k])

"""LM-head reductions under exact ties.  The vocabulary rows of the LM head repeat with a short period, so
whole classes of logits are exactly equal (bit for bit on the GPU, where equal weight rows go through the
same arithmetic).  The greedy token and the top-k ids must then follow the (logit descending, id ascending)
order exactly, and the log-probabilities must match the log-sum-exp of the same logits.  Checked against
the oracle's ranking applied to the GPU's own logits (so the check does not depend on how close the class
logits are to the fp64 ones), at a vocabulary where the tied candidates fit the merge kernel's buffer and
at one where they overflow it (its fallback tree)."""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("vocab,period", [(2048, 7), (20032, 7), (20032, 1)])
def test_tied_logits_rank_by_id(vocab, period):
    import torch
    from block_diffusion_drafter_forward_amd import session as S
    base = W.by_name("small-bf16-b1")
    shape = dataclasses.replace(base.shape, vocab=vocab)
    wl = dataclasses.replace(base, shape=shape)
    w = wl.weights()
    w["lm_head"] = np.ascontiguousarray(w["lm_head"][np.arange(vocab) % period])
    g = S.GpuWorkload(wl, weights=w)
    g.prefill()
    logits = torch.zeros((wl.batch, shape.block_len, vocab), dtype=torch.float32, device="cuda")
    g.draft(logits=logits)
    torch.cuda.synchronize()
    assert g.error_word() == 0
    lg = logits.cpu().numpy().astype(np.float64)
    # the ties are exact: every row's logits take at most `period` distinct values
    for row in lg.reshape(-1, vocab):
        assert len(np.unique(row)) <= period
    want = O.head_outputs(lg, wl.top_k)
    np.testing.assert_array_equal(g.tokens.cpu().numpy(), want["tokens"])
    np.testing.assert_array_equal(g.topk_ids.cpu().numpy(), want["topk_ids"])
    lp = g.topk_lp.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lp - want["topk_logprobs"]) <= 1e-4 + 1e-5 * np.abs(want["topk_logprobs"]))

"""Per-kernel GPU checks through the C ABI: the GEMM kernels against the oracle's fp64 product (with a
rigorous float32-accumulation bound), acceptance on random inputs, determinism, and the device error word."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _mods():
    import torch
    assert torch.cuda.is_available()
    from block_diffusion_drafter_forward_amd import dflash as D, session as S
    return torch, D, S


@pytest.mark.parametrize("M,N,K,bf16", [
    (16, 4096, 4096, True),      # skinny, one m-tile
    (1, 1000, 512, True),        # a single row, ragged N
    (7, 336, 256, True),         # ragged N (multiple of 16, not of 64)
    (32, 2048, 1024, True),      # two m-tiles
    (20, 300, 768, True),        # ragged M and N
    (16, 5003, 2560, True),      # vocabulary-like ragged N, K not a multiple of 1024
    (256, 640, 512, True),       # tiled kernel
    (130, 200, 256, True),       # tiled, ragged M and N
    (4096, 256, 2048, True),     # tiled, prefill-like
    (300, 2048, 768, True),      # tiled 192 wide, ragged M and last column tile; four splits of six 32-deep
                                 # k-tiles (the four-stage loop ends two tiles into its second pass)
    (200, 1536, 1792, True),     # tiled: ten splits, nine of six k-tiles and a last one of two
    (8, 4096, 256, False),       # float32
    (10, 777, 128, False),
])
def test_linear_matches_fp64_product(M, N, K, bf16):
    torch, D, S = _mods()
    key = W.seed_key(7000 + M + N + K)
    x = W.normal(key, 1, (M, K), 1.0, bf16)
    w = W.normal(key, 2, (N, K), 0.02, bf16)
    ref = O.matmul_wT(O.to_f64(x), w)
    bound = np.abs(O.to_f64(x)) @ np.abs(O.to_f64(w)).T
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    dt = D.DFLASH_BF16 if bf16 else D.DFLASH_F32
    xd, wd = S.to_device(x), S.to_device(w)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(D.dflash_linear_workspace_bytes(dt, M, N, K), dtype=torch.uint8, device="cuda")
    D.check(D.dflash_linear(dt, M, N, K, xd.data_ptr(), K, wd.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                            D._stream()), "dflash_linear")
    got = y.cpu().numpy().astype(np.float64)
    # float32 accumulation over K terms plus the split reduction and the final rounding
    assert np.all(np.abs(got - ref) <= 2 * gamma * bound + 2.0 ** -24 * np.abs(ref) + 1e-30)


def test_accept_kernel_random():
    torch, D, S = _mods()
    key = W.seed_key(7100)
    B, n = 300, 15
    draft = W.uniform_int(key, 1, B * n, 0, 3).reshape(B, n).astype(np.int32)
    target = np.concatenate([draft, np.zeros((B, 1), np.int32)], axis=1)
    flip = W.uniform01(key, 2, B * n).reshape(B, n) < 0.15
    target[:, :n][flip] = (target[:, :n][flip] + 1) % 4
    tau = torch.zeros(B, dtype=torch.int32, device="cuda")
    dd, td = S.to_device(draft), S.to_device(target)
    D.check(D.dflash_accept_len(B, n, dd.data_ptr(), n, td.data_ptr(), n + 1, tau.data_ptr(), D._stream()), "accept")
    np.testing.assert_array_equal(tau.cpu().numpy(), O.accept_len(draft, target))
    assert tau.min().item() >= 1 and tau.max().item() <= n + 1


def test_draft_is_deterministic_and_mask_rows_agree_without_rope():
    """Two runs are bit-identical; with RoPE off every mask row has identical input and no positional
    signal, so all mask rows produce bit-identical logits (non-causal block)."""
    import dataclasses
    torch, D, S = _mods()
    shape = dataclasses.replace(W.SMALL_BF16, rope_theta=0.0)
    wl = dataclasses.replace(W.by_name("small-bf16-b1"), shape=shape)
    g = S.GpuWorkload(wl)
    g.prefill()
    outs = []
    for _ in range(2):
        lg = torch.zeros((1, shape.block_len, shape.vocab), dtype=torch.float32, device="cuda")
        g.draft(logits=lg)
        torch.cuda.synchronize()
        outs.append((g.tokens.cpu().numpy().copy(), lg.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    lg = outs[0][1][0]
    for i in range(2, shape.block_len):
        assert np.array_equal(lg[1].view(np.uint32), lg[i].view(np.uint32))


def test_device_error_word_flags_bad_pages_positions_and_tokens():
    torch, D, S = _mods()
    wl = W.by_name("small-bf16-paged-b2")
    g = S.GpuWorkload(wl)
    g.prefill()
    g.draft()
    torch.cuda.synchronize()
    assert g.error_word() == 0
    # a page id outside the pool: the kernels skip it and flag it
    bad = g.page_table.clone()
    bad[0, 0] = g.n_pages + 5
    good = g.page_table
    g.page_table = bad
    g.draft()
    torch.cuda.synchronize()
    assert g.error_word() & D.DEVERR_PAGE
    g.page_table = good
    # a context length beyond max_ctx
    g.ctx_len[1] = g.max_ctx + 1
    g.draft()
    torch.cuda.synchronize()
    assert g.error_word() & D.DEVERR_POS
    g.ctx_len.copy_(S.to_device(g.ctx))
    # a token id outside the vocabulary
    g.block_tokens[0, 0] = wl.shape.vocab + 3
    g.draft()
    torch.cuda.synchronize()
    assert g.error_word() & D.DEVERR_TOKEN
    # and a clean call clears the word again
    g.block_tokens.copy_(S.to_device(wl.block_tokens()))
    g.draft()
    torch.cuda.synchronize()
    assert g.error_word() == 0


def test_graph_replay_matches_eager():
    """The drafter pass captured as a HIP graph and replayed several times, with eager calls and
    synchronisations in between, reproduces the eager outputs bit for bit every time."""
    torch, D, S = _mods()
    wl = W.by_name("small-bf16-paged-b2")
    g = S.GpuWorkload(wl)
    g.prefill()
    lg = torch.zeros((wl.batch, wl.shape.block_len, wl.shape.vocab), dtype=torch.float32, device="cuda")
    g.draft(logits=lg)
    torch.cuda.synchronize()
    ref_tok, ref_lg, ref_lp = g.tokens.clone(), lg.clone(), g.topk_lp.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            g.draft(logits=lg, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    other = g.block_tokens.clone()
    for it in range(3):
        g.tokens.zero_()
        lg.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g.tokens, ref_tok), it
        assert torch.equal(lg.view(torch.int32), ref_lg.view(torch.int32)), it
        assert torch.equal(g.topk_lp.view(torch.int32), ref_lp.view(torch.int32)), it
        # eager work between replays: a pass on different anchors, then restore
        g.block_tokens[:, 0] = (other[:, 0] + 7 + it) % wl.shape.vocab
        g.draft()
        torch.cuda.synchronize()
        g.block_tokens.copy_(other)

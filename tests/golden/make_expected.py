"""Write the oracle's expected outputs for the full-size workloads (tests/golden/expected_<name>.npz).

Only the CPU oracle and the seeded input generator are used: the files hold what the fp64 oracle computes
for each workload, so the GPU parity tests at full size need no heavy CPU work where they run.

Stored per workload:
  tokens [B, L], topk_ids [B, L, 8], topk_logprobs [B, L, 8], lse [B, L], margin1 / margin8 [B, L]
  (the top-2 and top-9 gaps), target [B, L] and tau [B] (the generator's target built from the oracle's
  greedy tokens), sampled logits (ids [B, L, 48] = the top 16 plus 32 seeded random ids, and their values),
  and sampled cached K/V rows (positions [B, 8] and, per layer, K/V as float32 [n_layers, B, 8, n_kv, d]).

Usage: python tests/golden/make_expected.py [workload names...]   (default: every full-size workload)
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

N_TOP_LOGITS = 16
N_RAND_LOGITS = 32
N_KV_SAMPLES = 8


def sample_positions(wl, r, C):
    key = W.seed_key(50_000 + wl.cfg_id)
    pos = W.uniform_int(key, 100 + r, N_KV_SAMPLES, 0, max(C - 1, 0))
    return np.sort(pos)


def make(wl):
    t0 = time.time()
    s = wl.shape
    weights = wl.weights()
    ctx = wl.ctx_lens()
    kv = []
    for r in range(wl.batch):
        kv.append(O.inject(weights, s, wl.features(r, int(ctx[r])), 0, fc_b=weights.get("fc_b")))
        print(f"  {wl.name}: inject request {r} ({ctx[r]} tokens) done at {time.time() - t0:.0f} s", flush=True)
    out = O.draft_block(weights, s, kv, wl.block_tokens(), 8)
    logits = out["logits"]
    B, L, V = logits.shape
    key = W.seed_key(60_000 + wl.cfg_id)
    rand_ids = W.uniform_int(key, 1, B * L * N_RAND_LOGITS, 0, V - 1).reshape(B, L, N_RAND_LOGITS)
    top_ids = O.ranked_ids(logits, N_TOP_LOGITS)
    ids = np.concatenate([top_ids, rand_ids], axis=-1)
    bern, rand = wl.target_draws()
    target = W.make_target(out["tokens"], bern, rand)
    pos = np.stack([sample_positions(wl, r, int(ctx[r])) for r in range(B)])
    kvk = np.stack([np.stack([kv[r][l][0][pos[r]] for r in range(B)]) for l in range(s.n_layers)])
    kvv = np.stack([np.stack([kv[r][l][1][pos[r]] for r in range(B)]) for l in range(s.n_layers)])
    res = dict(
        tokens=out["tokens"].astype(np.int32),
        topk_ids=out["topk_ids"].astype(np.int32),
        topk_logprobs=out["topk_logprobs"].astype(np.float64),
        lse=out["lse"].astype(np.float64),
        margin1=O.sorted_margins(logits, 1),
        margin8=O.sorted_margins(logits, 8),
        target=target,
        tau=O.accept_len(out["tokens"][:, 1:], target).astype(np.int32),
        logit_ids=ids.astype(np.int32),
        logit_vals=np.take_along_axis(logits, ids, axis=-1),
        kv_pos=pos.astype(np.int32),
        kv_k=kvk.astype(np.float32),
        kv_v=kvv.astype(np.float32),
    )
    path = os.path.join(HERE, f"expected_{wl.name}.npz")
    np.savez_compressed(path, **res)
    print(f"{wl.name}: wrote {path} in {time.time() - t0:.0f} s", flush=True)


def main():
    names = sys.argv[1:] or [w.name for w in W.CONFIGS + W.FULL_EXTRA]
    for n in names:
        make(W.by_name(n))


if __name__ == "__main__":
    main()

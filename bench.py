"""Benchmark of the DFlash drafter hot path on one MI355X.

A step is one steady-state speculative cycle of the library on one batch of synthetic input:
  dflash_inject_ctx  (fuse + inject the target features of the tokens verified in the previous cycle),
  dflash_draft_block (one parallel drafter pass over [anchor, mask x 15] per request),
  dflash_accept_len  (greedy acceptance against the target's tokens).
The default workload is the Qwen3-8B-shaped drafter at batch 1, block 16, 4096-token context.  The step
re-injects the last N_NEW context positions each time, so the context length stays fixed across steps.

Output: one JSON line (metric, value = blocks/s of whole steps, roofline of the dominant kernel measured
with HIP events on the library's stream, and the CPU oracle timed on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafter block fwd µs & blocks/s (Qwen3-8B-shape, B=1, L=16); HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
N_NEW = 7  # tokens committed per cycle: the pages report mean acceptance of about 6.5-7.8 for Qwen3-8B


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="qwen3-8b-shape")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-s", type=float, default=30.0, help="cap on CPU oracle work (seconds)")
    return p.parse_args()


def algorithmic_bytes(s, batch, ctx_total, n_new):
    """Bytes one step must move at least once, per kernel family (weights read once, context K/V read once,
    activations counted where they are read or written)."""
    E = 2 if s.bf16 else 4
    H, qd, kvd, F, V = s.hidden, s.q_dim, s.kv_dim, s.ffn, s.vocab
    M = batch * s.block_len
    per = {}
    gemm = 0
    # inject: fc over n_new rows, then all layers' U_K / U_V
    gemm += H * s.feat_dim * E + n_new * s.feat_dim * E + n_new * H * 4
    gemm += s.n_layers * 2 * kvd * H * E + n_new * H * E + n_new * s.n_layers * 2 * kvd * 4
    for _ in range(s.n_layers):
        gemm += (qd + 2 * kvd) * H * E + M * H * E + M * (qd + 2 * kvd) * 4     # QKV
        gemm += H * qd * E + M * qd * E + M * H * 4                               # O
        gemm += 2 * F * H * E + M * H * E + M * 2 * F * 4                         # gate/up
        gemm += H * F * E + M * F * E + M * H * 4                                 # down
    per["gemm"] = gemm
    per["attn"] = s.n_layers * (ctx_total * 2 * kvd * E + M * (qd + 2 * kvd) * E + M * qd * 4)
    per["lm_head"] = V * H * E + M * H * E
    per["total"] = sum(per.values())
    return per


def cpu_baseline(wl, weights, n_new, cap_s):
    """The oracle (fp64 NumPy) on the host: one steady-state cycle on the same workload.  The oracle's own
    prefill of the context is done first and not timed; the timed sample is inject(n_new) + draft + accept."""
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    s = wl.shape
    kv = []
    for r in range(wl.batch):
        C = int(wl.ctx_lens()[r])
        kv.append(O.inject(weights, s, wl.features(r, C - n_new), 0))
    t0 = time.perf_counter()
    for r in range(wl.batch):
        C = int(wl.ctx_lens()[r])
        tail = O.inject(weights, s, wl.features(r, n_new, row0=C - n_new), C - n_new)
        kv[r] = [(np.concatenate([kv[r][l][0], tail[l][0]]), np.concatenate([kv[r][l][1], tail[l][1]]))
                 for l in range(s.n_layers)]
    out = O.draft_block(weights, s, kv, wl.block_tokens(), wl.top_k)
    bern, rand = wl.target_draws()
    O.accept_len(out["tokens"][:, 1:], W.make_target(out["tokens"], bern, rand))
    dt = time.perf_counter() - t0
    return {"value": wl.batch / dt, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one full cycle of {wl.name} (inject {n_new} tokens x {wl.batch} request(s) + drafter pass "
                      f"+ acceptance), fp64 NumPy, after an untimed oracle prefill of the context; "
                      f"{dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    from block_diffusion_drafter_forward_amd import dflash as D
    from block_diffusion_drafter_forward_amd import session as S

    if not os.path.exists(D.LIB_PATH):
        from block_diffusion_drafter_forward_amd.build import build
        build()
    torch.cuda.set_device(0)
    wl = W.by_name(args.workload)
    s = wl.shape
    t_setup = time.perf_counter()
    weights = wl.weights()
    g = S.GpuWorkload(wl, weights=weights)
    ctx = g.ctx.astype(np.int64)
    n_new = min(N_NEW, int(ctx.min()))
    # prefill everything except the last n_new tokens of each request; the step injects those
    full_ctx = g.ctx.copy()
    g.ctx = (full_ctx - n_new).astype(np.int32)
    g.prefill()
    g.ctx = full_ctx
    feats = [wl.features(r, n_new, row0=int(ctx[r]) - n_new) for r in range(wl.batch)]
    offs = np.arange(wl.batch + 1, dtype=np.int32) * n_new
    feats_d = S.to_device(np.concatenate(feats, axis=0))
    offs_d = S.to_device(offs)
    start_d = S.to_device((ctx - n_new).astype(np.int32))
    inj_ws = g.model.inject_workspace(feats_d.shape[0])
    stream = torch.cuda.current_stream()

    def inject():
        g.model.inject(feats_d, offs_d, start_d, g.page_table, g.kv, inj_ws, stream=stream)

    # target tokens: the drafter's own greedy tokens from an untimed pass, kept with probability p,
    # else a uniform token (the acceptance kernel's cost does not depend on the values)
    inject()
    g.draft(stream=stream)
    torch.cuda.synchronize()
    bern, rand = wl.target_draws()
    target = S.to_device(W.make_target(g.tokens.cpu().numpy(), bern, rand))
    setup_s = time.perf_counter() - t_setup

    def step():
        inject()
        g.draft(stream=stream)
        g.accept(target, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # the drafter pass alone
    for _ in range(3):
        g.draft(stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        g.draft(stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_draft = e0.elapsed_time(e1) / args.steps
    assert g.error_word() == 0, "device error word set"

    # per-kernel HIP-event timing over a few steps (separate from the timed region)
    prof_steps = 5
    D.check(D.dflash_profile_enable(g.model.handle, 1), "profile_enable")
    for _ in range(prof_steps):
        step()
    torch.cuda.synchronize()
    stats = D.dflash_profile_collect(g.model.handle)
    D.check(D.dflash_profile_enable(g.model.handle, 0), "profile_disable")
    kernels = {n: {"launches_per_step": c / prof_steps, "avg_us": 1e3 * t / c, "total_us_per_step": 1e3 * t / prof_steps}
               for n, c, t in stats}

    ab = algorithmic_bytes(s, wl.batch, int(ctx.sum()), n_new)
    fam = {"gemm": [n for n in kernels if n.startswith("gemm_")],
           "attn": [n for n in kernels if n.startswith("attn_bf16") or n == "attn_f32"],
           "lm_head": [n for n in kernels if n.startswith("lm_head")]}
    fam_time = {f: sum(kernels[n]["total_us_per_step"] for n in ns) for f, ns in fam.items()}
    dom = max(fam_time, key=fam_time.get)
    launches = sum(kernels[n]["launches_per_step"] for n in fam[dom])
    bytes_per_launch = ab[dom] / launches
    avg_us = fam_time[dom] / launches
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": ",".join(sorted({n.split(" ")[0] for n in fam[dom]})), "bytes_per_launch": int(bytes_per_launch),
                "avg_launch_us": round(avg_us, 2)}

    blocks_per_s = wl.batch * 1e3 / ms_step
    out = {
        "metric": METRIC,
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "block_len": s.block_len,
                   "ctx_len": int(ctx.max()), "n_new_per_step": n_new, "layers": s.n_layers, "hidden": s.hidden,
                   "vocab": s.vocab, "top_k": wl.top_k},
        "us_per_step": round(ms_step * 1e3, 1),
        "draft_block_us": round(ms_draft * 1e3, 1),
        "step_algorithmic_bytes": int(ab["total"]),
        "step_hbm_gbs": round(ab["total"] / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(ab["total"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roofline,
        "kernels": {n: {k: round(v, 2) for k, v in d.items()} for n, d in kernels.items()},
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, weights, n_new, args.cpu_sample_s)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the KV-correction hot path on one MI355X.

One step = the whole correction of one Llama-3-8B-shaped segment cache
(32 layers x 8 KV heads x 4096 tokens x head_dim 128, bf16): L2 scores of K
and V at check layer 1, top-b selection (b = 615 = ceil(0.15 * 4096)), the
per-layer probe mean with fresh scatter, and the fused apply (rotary
re-alignment + clipped-weight mean + rank-4 state) of both planes.  Inputs
are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line: corrected-KV GB/s of algorithmic bytes (each reused
byte read once, each output byte written once, fresh bytes only for probe
rows, plus states, scores and indices), the apply kernel's roofline from
events recorded around its launches, and the CPU oracle timed on a bounded
sample of the same workload.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
COUNTERS = os.path.join(ROOT, "profiles", "apply_c2_counters.json")
KERNEL_SOURCES = ["cross_context_kv_amd/csrc/correct.hip", "cross_context_kv_amd/csrc/common.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def alg_bytes(cfg):
    """Algorithmic bytes of one step, split by kernel."""
    L, S, H, n, hd, b, r = (cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens,
                            cfg.head_dim, cfg.b, cfg.rank)
    row = hd * 2
    words = (n + 31) // 32
    score = 2 * (2 * S * H * n * row + S * n * 4)                  # fresh + reuse at the check layer
    select = 2 * (S * n * 4 + S * b * 4 + S * words * 4)
    fit = 2 * (L * S * H * b * (3 * row + r * 4) + L * S * H * (r * hd * 4 + hd * 4) + S * b * 4)
    apply_one = (L * S * H * (n - b) * (2 * row + r * 4) + L * S * H * (r * hd * 4 + hd * 4)
                 + S * n * 4 + S * words * 4)
    return {"score": score, "select": select, "fit_mean": fit, "apply": 2 * apply_one,
            "apply_per_launch": apply_one, "apply_units_per_launch": L * S * H * (n - b),
            "total": score + select + fit + 2 * apply_one}


def build_inputs(cfg, torch, kv):
    """Seeded synthetic C2 inputs, generated on the GPU."""
    from synthetic import draw_correction
    raw = draw_correction(cfg, "cuda")
    delta = raw["delta"].to("cuda")
    t = {"delta": delta}
    # stored keys: the aligned content rotated back to the old position
    xk = raw["x_k"].to(torch.bfloat16)
    reuse_k = torch.empty_like(xk)
    kv.kvfix_rope_shift(kv.Plane.dense(xk), kv.Plane.dense(reuse_k), -delta, cfg.theta)
    t["reuse_k"], t["reuse_v"] = reuse_k, raw["x_v"].to(torch.bfloat16)
    t["fresh_k"], t["fresh_v"] = raw["fresh_k"].contiguous(), raw["fresh_v"].contiguous()
    t["A_k"], t["B_k"], t["A_v"], t["B_v"] = raw["a_k"], raw["b_k"], raw["a_v"], raw["b_v"]
    S, n, b, L, H, hd = cfg.n_segs, cfg.n_tokens, cfg.b, cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    t["scores"] = torch.empty(2, S, n, dtype=torch.float32, device="cuda")
    t["idx"] = torch.empty(2, S, b, dtype=torch.int32, device="cuda")
    t["mask"] = torch.empty(2, S, (n + 31) // 32, dtype=torch.int32, device="cuda")
    t["mu"] = torch.empty(2, L, S, H, hd, dtype=torch.float32, device="cuda")
    t["out_k"] = torch.empty_like(reuse_k)
    t["out_v"] = torch.empty_like(t["reuse_v"])
    del raw, xk
    torch.cuda.synchronize()
    return t


def make_step(cfg, t, kv, events=None):
    P = kv.Plane.dense
    planes = {p: (P(t["fresh_" + p]), P(t["reuse_" + p]), P(t["out_" + p])) for p in ("k", "v")}
    S, n, b = cfg.n_segs, cfg.n_tokens, cfg.b
    c = cfg.check_layer
    sc2, idx2, mask2 = t["scores"].view(2 * S, n), t["idx"].view(2 * S, b), t["mask"].view(2 * S, -1)

    def step():
        kv.kvfix_score(planes["k"][0], c, planes["k"][1], c, t["scores"][0], t["delta"], cfg.theta)
        kv.kvfix_score(planes["v"][0], c, planes["v"][1], c, t["scores"][1])
        kv.kvfix_select_topb(sc2, b, idx2, mask2)
        for i, p in enumerate(("k", "v")):
            fresh, reuse, out = planes[p]
            d = t["delta"] if p == "k" else None
            kv.kvfix_fit_mean(fresh, reuse, out, t["idx"][i], b, t["mu"][i], d, cfg.theta,
                              A=t["A_" + p], B=t["B_" + p])
        for i, p in enumerate(("k", "v")):
            fresh, reuse, out = planes[p]
            d = t["delta"] if p == "k" else None
            if events is not None:
                events.append(kv_event_pair_start())
            kv.kvfix_apply(reuse, out, t["mask"][i], t["mu"][i], t["scores"][i], cfg.w_lo,
                           cfg.w_hi, d, cfg.theta, A=t["A_" + p], B=t["B_" + p])
            if events is not None:
                kv_event_pair_end(events[-1])
    return step


def kv_event_pair_start():
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()          # torch's current stream: the stream every kvfix call here uses
    return (s, e)


def kv_event_pair_end(pair):
    pair[1].record()


def cpu_baseline(cfg, t, torch, n_layers_sample=None, repeats=3):
    """The oracle (as it stands, one thread) on the same input bytes.

    Sample: the whole step (scores, selection, mean fit and apply of K and V)
    over the first n_layers_sample layers (default: all), repeated `repeats`
    times; the rate uses the median time."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    from oracle import kvref as K
    Ls = cfg.n_layers if not n_layers_sample else max(n_layers_sample, cfg.check_layer + 1)

    def host(x):
        x = x[:Ls].detach().cpu()
        if x.dtype == torch.bfloat16:
            return x.contiguous().view(torch.int16).numpy().view(np.uint16)
        return x.contiguous().numpy()

    data = {k: host(t[k]) for k in ("reuse_k", "reuse_v", "fresh_k", "fresh_v", "A_k", "B_k",
                                     "A_v", "B_v")}
    deltas = [int(v) for v in t["delta"].tolist()]
    sub = cfg.replace(n_layers=Ls)

    def run():
        c = cfg.check_layer
        sk = K.score_l2(data["fresh_k"], data["reuse_k"], "bf16", c, deltas, cfg.theta)
        sv = K.score_l2(data["fresh_v"], data["reuse_v"], "bf16", c)
        for p, s in (("k", sk), ("v", sv)):
            idx, mask = K.select_topb(s, cfg.b)
            K.correct(data["fresh_" + p], data["reuse_" + p], "bf16", idx, mask, s, cfg.w_lo,
                      cfg.w_hi, data["A_" + p], data["B_" + p],
                      deltas if p == "k" else None, cfg.theta)

    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        if threadpool_limits:
            with threadpool_limits(limits=1):
                run()
        else:
            run()
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    nbytes = alg_bytes(sub)["total"]
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole step on layers 0..{Ls - 1} of the same input bytes "
                      f"({Ls} of {cfg.n_layers} layers, {nbytes / 1e6:.1f} MB algorithmic), "
                      f"median of {repeats} runs of {dt:.1f} s, numpy fp64, one thread"}


def read_traffic(per_launch_units: int):
    """HBM traffic of the apply kernel from the committed counter summary, or None
    when the kernel source has changed since the counters were taken."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_hash") != kernel_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=0, help="oracle sample layers (0 = all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the correction path is sharded by segment/layer/head without exchange; "
              "see DESIGN.md for the multi-GPU design)", file=sys.stderr)
        sys.exit(2)

    import torch
    import cross_context_kv_amd.kvfix as kv
    from synthetic import CONFIGS
    kv.lib()                          # fails loudly without the built library
    cfg = CONFIGS["c2"]
    t = build_inputs(cfg, torch, kv)
    step = make_step(cfg, t, kv)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = []
    timed = make_step(cfg, t, kv, events)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        timed()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    apply_ms = sum(s.elapsed_time(e) for s, e in events) / len(events)

    # Measured copy ceiling: a plain device-to-device copy of a known size
    # (also the calibration kernel for the HBM byte counters).
    n_copy = 256 << 20
    src_c = torch.empty(n_copy, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst_c = torch.empty_like(src_c)
    dst_c.copy_(src_c)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(5):
        dst_c.copy_(src_c)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src_c.numel() * 2 / (c0.elapsed_time(c1) / 5 * 1e-3) / 1e9
    del src_c, dst_c

    ab = alg_bytes(cfg)
    gbs = ab["total"] / (ms * 1e-3) / 1e9
    apply_gbs = ab["apply_per_launch"] / (apply_ms * 1e-3) / 1e9
    traffic = read_traffic(ab["apply_units_per_launch"])
    line = {
        "metric": "corrected-KV GB/s (read+write) and % of HBM peak; segment-layers/s at 8B shape",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "c2_llama3_8b: one segment, 32 layers x 8 KV heads x 4096 tokens x hd 128 "
                        "bf16; L2 probes at check layer 1, b=615 (r=0.15), w=clip(d,0,2), "
                        "rank-4 state, theta 5e5",
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "segment_layers_per_s": round(cfg.n_segs * cfg.n_layers / (ms * 1e-3), 1),
            "alg_bytes_per_step": ab["total"],
            "copy_ceiling_GBs": round(copy_gbs, 1),
            "pct_copy_ceiling": round(100 * gbs / copy_gbs, 2),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kvfix apply_kernel<bf16, fp32, hd128, rotate-half, rank 4>",
            "achieved": round(apply_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(apply_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": ab["apply_per_launch"],
            "avg_launch_ms": round(apply_ms, 5),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, t, torch, args.cpu_layers)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the KV-correction hot path on one MI355X.

Default workload (c2): the whole correction of one Llama-3-8B-shaped segment
cache (32 layers x 8 KV heads x 4096 tokens x head_dim 128, bf16): L2 scores
of K and V at check layer 1, top-b selection (b = 615 = ceil(0.15 * 4096)),
the per-layer probe mean with fresh scatter, and the fused apply (rotary
re-alignment + clipped-weight mean + rank-4 state) of both planes.

Other workloads (--workload), one step each:
  c3  collective round: 16 agents x 32 layers x 8192 tokens, block-sparse diff
      encode against the master, then the fused restore of all 16 caches;
  c4  Qwen2.5-14B-shaped draft repair: 48 layers, 40/8 heads, 32768 tokens,
      draft attention mass -> top 10 % -> mean fit and apply of K and V;
  c5  Llama-3-70B-shaped paged batch: 80 layers x 32 segments x 4096 tokens,
      scores at check layer 1 -> top 10 % -> mean + rank-2 fit and apply, in
      place through the page tables.

Inputs are synthetic, seeded, and resident in HBM before timing starts.
Prints one JSON line: corrected-KV GB/s of algorithmic bytes (each reused
byte read once, each output byte written once, fresh bytes only for probe
rows, plus states, scores and indices), the dominant kernel's roofline from
events recorded around its launches, and the CPU oracle timed on a bounded
sample of the same workload.

  c4 takes --layout: rows (top b), chunk (BCR-chunk: 64-token chunks by mean
  draft mass), coin (the same budget in random chunks, no draft) or grow
  (BCR-grow spans, tau 0.25).  c3 takes --layout: dense (default), paged
  (restore into a paged pool through a slot mapping) or plan (the reuse plan
  first: deviation scores of every agent and the master selection).  c2 takes
  --layout anchor: the same segment corrected through an anchor pool of 10
  anchors at rank 32 (reliability gate, token weights, blended delta apply).

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload c2]
                  [--layout rows] [--no-cpu-baseline]
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
METRIC = "corrected-KV GB/s (read+write) and % of HBM peak; segment-layers/s at 8B shape"
# Sources each roofline kernel is built from: a counter summary stays valid
# while these files are unchanged.
KERNEL_SOURCES = {
    "apply": ["cross_context_kv_amd/csrc/correct.hip", "cross_context_kv_amd/csrc/common.h"],
    "diff_decode": ["cross_context_kv_amd/csrc/diff.hip", "cross_context_kv_amd/csrc/common.h"],
    "anchor_match": ["cross_context_kv_amd/csrc/anchor.hip", "cross_context_kv_amd/csrc/common.h"],
}


def kernel_hash(kernel_tag: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel_tag]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(W) -> str:
    return os.path.join(ROOT, "profiles", f"{W.kernel_tag}_{W.counter_name}_counters.json")


def read_traffic(W):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary, or None when the kernel sources changed since it was taken."""
    p = counters_path(W)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("kernel_hash") != kernel_hash(W.kernel_tag):
        return None
    return c.get("traffic_bytes_per_launch")


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


class Timed:
    """Events around the roofline kernel's launches (torch's current stream,
    the stream every kvfix call here is issued on)."""

    def __init__(self, torch):
        self.torch, self.pairs, self.on = torch, [], False

    def __enter__(self):
        if self.on:
            s, e = _events(self.torch)
            s.record()
            self.pairs.append((s, e))
        return self

    def __exit__(self, *a):
        if self.on:
            self.pairs[-1][1].record()

    def avg_ms(self):
        return sum(s.elapsed_time(e) for s, e in self.pairs) / len(self.pairs)


def host(t, torch, np):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def timed_oracle(fn, repeats):
    """Median wall time of the oracle on one thread (BLAS pinned to one thread)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        if threadpool_limits:
            with threadpool_limits(limits=1):
                fn()
        else:
            fn()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2]


def host_info():
    """The host the oracle ran on: CPU model, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": aff}


def widen(np, a, dtype):
    """Plane values as float64 (bf16 bit patterns widened exactly)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def max_rel_err(np, g, o, dtype="f32"):
    """max |g - o| / (|o| + 1e-3): the parity metric of the tests."""
    gv, ov = widen(np, g, dtype), widen(np, o, dtype)
    return float(np.max(np.abs(gv - ov) / (np.abs(ov) + 1e-3))) if gv.size else 0.0


def index_mismatches(np, g, o):
    """Indices in one selection and not the other, summed over rows."""
    return int(sum(len(set(a.tolist()) ^ set(b.tolist())) for a, b in zip(g, o)))


PARITY_BAR = {"bf16 values": 8e-3, "fp32 values and means": 1e-5, "indices and masks": "exact"}


class Workload:
    ALL = {}
    kernel_tag = "apply"
    extra_timed = {}
    # roofline of the dominant kernel: bound, unit, published peak, unit scale
    roof = ("hbm", "GB/s", HBM_PEAK_GBS, 1e9)

    @property
    def counter_name(self):
        return self.name

    def __init__(self, cfg, torch, kv):
        self.cfg, self.torch, self.kv = cfg, torch, kv
        self.timed = Timed(torch)              # the roofline kernel's launches
        self.timed_v = Timed(torch)            # the value-plane apply, where there is one
        self.extra_timed = {}
        self.parity = None


# ----------------------------------------------------------------------------
# correction chains: c2 (dense, L2 at a check layer), c5 (paged, in place)
# ----------------------------------------------------------------------------


class Correction(Workload):
    kernel_tag = "apply"
    paged = False

    def alg_bytes(self):
        """Algorithmic bytes of one step, split by kernel."""
        c = self.cfg
        L, S, H, n, hd, b, r = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_tokens, c.head_dim,
                                c.b, c.rank)
        row = hd * 2
        words = (n + 31) // 32
        wbytes = S * n * 4 if c.weight == "clip" else 0
        score = 2 * (2 * S * H * n * row + S * n * 4)        # fresh + reuse at the check layer
        select = 2 * (S * n * 4 + S * b * 4 + S * words * 4)
        state = L * S * H * (r * hd * 4) if r else 0
        fit = 2 * (L * S * H * b * (3 * row + r * 4) + state + L * S * H * hd * 4 + S * b * 4)
        apply_one = (L * S * H * (n - b) * (2 * row + r * 4) + state + L * S * H * hd * 4
                     + wbytes + S * words * 4)
        return {"score": score, "select": select, "fit_mean": fit, "apply": 2 * apply_one,
                "roofline_per_launch": apply_one, "roofline_units": L * S * H * (n - b),
                "total": score + select + fit + 2 * apply_one}

    def _prep(self, i, p):
        """Score, select and fit of one plane (on the current stream)."""
        kv, t, c = self.kv, self.t, self.cfg
        R = self.reuse_planes
        d = t["delta"] if p == "k" else None
        kv.kvfix_score(self.fresh_check_planes[p], self.fresh_check_layer, R[p], c.check_layer,
                       t["scores"][i], d, c.theta)
        kv.kvfix_select_topb(t["scores"][i], c.b, t["idx"][i], t["mask"][i])
        kv.kvfix_fit_mean(self.fit_fresh_planes[p], R[p], self.out_planes[p], t["idx"][i], c.b,
                          t["mu"][i], d, c.theta, A=t["A_" + p], B=t["B_" + p],
                          fresh_by_slot=self.paged, ws=t["ws_fit_" + p])

    def step(self):
        """The K and V chains are independent: the V plane's score, selection
        and fit run on a second stream while the K plane's run and its apply
        streams; the V apply follows the K apply on the main stream."""
        kv, t, c, torch = self.kv, self.t, self.cfg, self.torch
        main = torch.cuda.current_stream()
        self.ev_fork.record(main)
        self.side.wait_event(self.ev_fork)
        with torch.cuda.stream(self.side):
            self._prep(1, "v")
            self.ev_join.record(self.side)
        self._prep(0, "k")
        for i, p in enumerate("kv"):
            if p == "v":
                main.wait_event(self.ev_join)
            d = t["delta"] if p == "k" else None
            sc = t["scores"][i] if c.weight == "clip" else None
            with (self.timed if p == "k" else self.timed_v):
                kv.kvfix_apply(self.reuse_planes[p], self.out_planes[p], t["mask"][i], t["mu"][i],
                               sc, c.w_lo, c.w_hi, d, c.theta, A=t["A_" + p], B=t["B_" + p])


class C2(Correction):
    name = "c2"

    def workload_text(self):
        return ("c2_llama3_8b: one segment, 32 layers x 8 KV heads x 4096 tokens x hd 128 "
                "bf16; L2 probes at check layer 1, b=615 (r=0.15), w=clip(d,0,2), "
                "rank-4 state, theta 5e5")

    def build(self):
        torch, kv, c = self.torch, self.kv, self.cfg
        from synthetic import draw_correction
        raw = draw_correction(c, "cuda")
        delta = raw["delta"].to("cuda")
        t = {"delta": delta}
        # stored keys: the aligned content rotated back to the old position
        xk = raw["x_k"].to(torch.bfloat16)
        reuse_k = torch.empty_like(xk)
        kv.kvfix_rope_shift(kv.Plane.dense(xk), kv.Plane.dense(reuse_k), -delta, c.theta)
        t["reuse_k"], t["reuse_v"] = reuse_k, raw["x_v"].to(torch.bfloat16)
        t["fresh_k"], t["fresh_v"] = raw["fresh_k"].contiguous(), raw["fresh_v"].contiguous()
        for p in "kv":
            t["A_" + p], t["B_" + p] = raw["a_" + p], raw["b_" + p]
        self._alloc_step_buffers(t)
        t["out_k"] = torch.empty_like(reuse_k)
        t["out_v"] = torch.empty_like(t["reuse_v"])
        del raw, xk
        P = kv.Plane.dense
        self.reuse_planes = {p: P(t["reuse_" + p]) for p in "kv"}
        self.out_planes = {p: P(t["out_" + p]) for p in "kv"}
        self.fit_fresh_planes = {p: P(t["fresh_" + p]) for p in "kv"}
        self.fresh_check_planes = self.fit_fresh_planes
        self.fresh_check_layer = c.check_layer
        self.t = t
        torch.cuda.synchronize()

    def _alloc_step_buffers(self, t):
        torch, kv, c = self.torch, self.kv, self.cfg
        S, n, b, L, H, hd = c.n_segs, c.n_tokens, c.b, c.n_layers, c.n_kv_heads, c.head_dim
        t["scores"] = torch.empty(2, S, n, dtype=torch.float32, device="cuda")
        t["idx"] = torch.empty(2, S, b, dtype=torch.int32, device="cuda")
        t["mask"] = torch.empty(2, S, (n + 31) // 32, dtype=torch.int32, device="cuda")
        t["mu"] = torch.empty(2, L, S, H, hd, dtype=torch.float32, device="cuda")
        ws = kv.kvfix_fit_mean_workspace(L, S, H, hd, b)
        for p in "kv":             # one workspace per plane: the two chains run concurrently
            t["ws_fit_" + p] = torch.empty(max(ws, 16), dtype=torch.uint8, device="cuda")
        self.side = torch.cuda.Stream()
        self.ev_fork, self.ev_join = torch.cuda.Event(), torch.cuda.Event()

    def cpu_baseline(self, np):
        """The oracle (as it stands, one thread) on the same input bytes: the
        whole step over all 32 layers, median of 3 runs.  Its results are
        compared with the GPU's last step (parity)."""
        torch, c, t = self.torch, self.cfg, self.t
        from oracle import kvref as K
        data = {k: host(t[k], torch, np) for k in ("reuse_k", "reuse_v", "fresh_k", "fresh_v",
                                                   "A_k", "B_k", "A_v", "B_v")}
        deltas = [int(v) for v in t["delta"].tolist()]
        box = {}

        def run():
            ck = c.check_layer
            sk = K.score_l2(data["fresh_k"], data["reuse_k"], "bf16", ck, deltas, c.theta)
            sv = K.score_l2(data["fresh_v"], data["reuse_v"], "bf16", ck)
            for p, s in (("k", sk), ("v", sv)):
                idx, mask = K.select_topb(s, c.b)
                out, mu = K.correct(data["fresh_" + p], data["reuse_" + p], "bf16", idx, mask, s,
                                    c.w_lo, c.w_hi, data["A_" + p], data["B_" + p],
                                    deltas if p == "k" else None, c.theta)
                box[p] = (s, idx, mask, out, mu)

        dt = timed_oracle(run, 3)
        par = {"scope": f"the whole step, all {c.n_layers} layers, both planes, against the "
                        "GPU's last timed step", "bar": PARITY_BAR, "max_rel_err": {},
               "index_mismatches": {}, "mask_word_mismatches": {}}
        for i, p in enumerate("kv"):
            s, idx, mask, out, mu = box[p]
            par["max_rel_err"]["scores_" + p] = max_rel_err(np, host(t["scores"][i], torch, np), s)
            par["max_rel_err"]["mu_" + p] = max_rel_err(np, host(t["mu"][i], torch, np), mu)
            par["max_rel_err"]["out_" + p] = max_rel_err(np, host(t["out_" + p], torch, np), out,
                                                         "bf16")
            par["index_mismatches"][p] = index_mismatches(np, host(t["idx"][i], torch, np), idx)
            par["mask_word_mismatches"][p] = int(np.sum(
                host(t["mask"][i], torch, np).view(np.uint32) != mask))
        self.parity = par
        nbytes = self.alg_bytes()["total"]
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole step on all {c.n_layers} layers of the same input bytes "
                          f"({nbytes / 1e6:.1f} MB algorithmic), median of 3 runs of {dt:.1f} s, "
                          f"numpy fp64, one thread"}


class C5(Correction):
    name = "c5"
    paged = True

    def workload_text(self):
        return ("c5_llama3_70b_paged: 32 segments x 80 layers x 8 KV heads x 4096 tokens x hd 128 "
                "bf16 in a paged pool (page 16, seeded permutation of 8192 pages); L2 probes at "
                "check layer 1, b=410 (r=0.1), w=1, rank-2 state, in place, theta 5e5")

    def build(self):
        torch, kv, c = self.torch, self.kv, self.cfg
        from synthetic import draw_correction, draw_deltas, draw_page_table
        L, S, H, n, hd, ps, NP, b = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_tokens, c.head_dim,
                                     c.page_size, c.n_pages, c.b)
        t = {"delta": draw_deltas(c).to("cuda")}
        pt = draw_page_table(c, "cuda")
        t["pt"] = pt
        neg = -t["delta"]
        for p in "kv":
            t["pool_" + p] = torch.empty(L, NP, ps, H, hd, dtype=torch.bfloat16, device="cuda")
            t["A_" + p] = torch.empty(L, S, H, n, c.rank, dtype=torch.float32, device="cuda")
            t["B_" + p] = torch.empty(L, S, H, c.rank, hd, dtype=torch.float32, device="cuda")
            # fresh rows by probe slot, for every layer; filled with each layer's
            # fresh rows of a fixed seeded slot set (the probe set itself is only
            # known inside the step; the bytes moved are the same)
            t["fslot_" + p] = torch.empty(L, S, H, b, hd, dtype=torch.bfloat16, device="cuda")
        g = torch.Generator(device="cpu")
        g.manual_seed(c.seed)
        slots = torch.sort(torch.randperm(n, generator=g)[:b]).values.to("cuda")
        tmp = torch.empty(1, S, H, n, hd, dtype=torch.bfloat16, device="cuda")
        for l in range(L):
            raw = draw_correction(c, "cuda", layers=[l])
            for p in "kv":
                x = raw["x_" + p].to(torch.bfloat16)
                if p == "k":
                    kv.kvfix_rope_shift(kv.Plane.dense(x), kv.Plane.dense(tmp), neg, c.theta)
                    x = tmp
                pool_l = t["pool_" + p][l]
                pool_l[pt.long()] = x[0].permute(0, 2, 1, 3).reshape(S, pt.shape[1], ps, H, hd)
                t["A_" + p][l] = raw["a_" + p][0]
                t["B_" + p][l] = raw["b_" + p][0]
                t["fslot_" + p][l] = raw["fresh_" + p][0][:, :, slots]
                if l == c.check_layer:
                    t["fcheck_" + p] = raw["fresh_" + p].contiguous()
            del raw
        del tmp
        self._alloc_step_buffers(t)
        P = kv.Plane
        self.reuse_planes = {p: P.paged(t["pool_" + p], pt, ps, n) for p in "kv"}
        self.out_planes = self.reuse_planes                       # in place
        self.fit_fresh_planes = {p: P.dense(t["fslot_" + p]) for p in "kv"}
        self.fresh_check_planes = {p: P.dense(t["fcheck_" + p]) for p in "kv"}
        self.fresh_check_layer = 0
        self.t = t
        torch.cuda.synchronize()

    _alloc_step_buffers = C2._alloc_step_buffers

    def cpu_baseline(self, np):
        """The oracle on a bounded sample: scores at the check layer for all 32
        segments, selection, and fit + apply of K and V on layers 0 and 1.
        The step corrects the pool in place, so parity takes layers 0-1 of
        the pool before and after one more GPU step and runs the oracle on
        the former."""
        torch, c, t = self.torch, self.cfg, self.t
        from oracle import kvref as K
        L2 = 2
        S, H, n, hd, ps = c.n_segs, c.n_kv_heads, c.n_tokens, c.head_dim, c.page_size
        pt = t["pt"].long()

        def logical(pool):
            return torch.stack([pool[l][pt].reshape(S, n, H, hd).permute(0, 2, 1, 3)
                                for l in range(L2)])

        data = {}
        for p in "kv":
            data["reuse_" + p] = host(logical(t["pool_" + p]), torch, np)
            data["fslot_" + p] = host(t["fslot_" + p][:L2], torch, np)
            data["fcheck_" + p] = host(t["fcheck_" + p], torch, np)
            data["A_" + p] = host(t["A_" + p][:L2], torch, np)
            data["B_" + p] = host(t["B_" + p][:L2], torch, np)
        self.step()                                   # one more step: the pool after it
        torch.cuda.synchronize()
        after = {p: host(logical(t["pool_" + p]), torch, np) for p in "kv"}
        g_idx = host(t["idx"], torch, np)
        g_mask = host(t["mask"], torch, np).view(np.uint32)
        deltas = [int(v) for v in t["delta"].tolist()]
        ck = c.check_layer
        box = {}

        def run():
            for p in "kv":
                d = deltas if p == "k" else None
                s = K.score_l2(data["fcheck_" + p], data["reuse_" + p][ck:ck + 1], "bf16", 0, d,
                               c.theta)
                idx, mask = K.select_topb(s, c.b)
                out, _ = K.correct(data["fslot_" + p], data["reuse_" + p], "bf16", idx, mask,
                                   None, 0.0, 1.0, data["A_" + p], data["B_" + p], d, c.theta,
                                   "half", True)
                box[p] = (idx, mask, out)

        dt = timed_oracle(run, 1)
        par = {"scope": f"selection of all {S} segments and corrected layers 0-1 (2 of "
                        f"{c.n_layers}) of the in-place pool, one GPU step against the oracle on "
                        "the same pool bytes", "bar": PARITY_BAR, "max_rel_err": {},
               "index_mismatches": {}, "mask_word_mismatches": {}}
        for i, p in enumerate("kv"):
            idx, mask, out = box[p]
            par["max_rel_err"]["out_" + p + " layers 0-1"] = max_rel_err(np, after[p], out, "bf16")
            par["index_mismatches"][p] = index_mismatches(np, g_idx[i], idx)
            par["mask_word_mismatches"][p] = int(np.sum(g_mask[i] != mask))
        self.parity = par
        sub = c.replace(n_layers=L2)
        ab = Correction.alg_bytes(type("X", (), {"cfg": sub})())
        nbytes = ab["total"]
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"scores at the check layer, selection, and fit + apply of K and V on "
                          f"layers 0-1 (2 of {c.n_layers}) for all {S} segments "
                          f"({nbytes / 1e6:.1f} MB algorithmic), one run of {dt:.1f} s, numpy "
                          f"fp64, one thread"}


# ----------------------------------------------------------------------------
# c4: draft-selected repair
# ----------------------------------------------------------------------------


class C4(Workload):
    name = "c4"
    kernel_tag = "apply"
    # probe layout: top-b rows, whole 64-token chunks (BCR-chunk), chunks by
    # coin at the same budget (no draft), or grown spans (BCR-grow)
    layout = "rows"
    CHUNK, TAU, RHO = 64, 0.25, (1, 10)
    LAYOUT_TEXT = {
        "rows": "top b=3277 rows (r=0.1) of the draft mass",
        "chunk": "BCR-chunk: 64-token chunks by mean draft mass, round(0.1 n / 64) = 51 chunks",
        "coin": "coin control: 51 random 64-token chunks (no draft)",
        "grow": "BCR-grow: b=3277 rows in spans grown while a neighbour scores >= 0.25 x seed",
    }

    def workload_text(self):
        return ("c4_qwen25_14b_draft: 48 layers x 8 KV heads (40 query heads) x 32768 tokens x "
                "hd 128 bf16; draft mass of 2 query tokens over layers 1-47; probes: "
                f"{self.LAYOUT_TEXT[self.layout]}, for both planes; w=1, no rank state, theta 1e6")

    def n_chunks(self):
        return -(-self.cfg.n_tokens // self.CHUNK)

    def chunk_budget(self):
        """Chunks repaired (BCR App. B Algorithm 1), from the library's own rule."""
        return self.kv.kvfix_chunk_budget(self.cfg.n_tokens, self.CHUNK, *self.RHO,
                                          self.kv.BUDGET_SKIP)

    def probe_rows(self):
        """Probe rows per segment of the layout (whole chunks: c * 64 here,
        the segment length being a multiple of 64)."""
        if self.layout in ("chunk", "coin"):
            return min(self.chunk_budget() * self.CHUNK, self.cfg.n_tokens)
        return self.cfg.b

    def alg_bytes(self):
        c = self.cfg
        L, S, H, Hq, T, n, hd = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_q_heads, c.n_draft,
                                 c.n_tokens, c.head_dim)
        b = self.probe_rows()
        row = hd * 2
        words = (n + 31) // 32
        draft = 0 if self.layout == "coin" else (
            (L - c.first_layer) * S * H * n * row + L * Hq * T * row * S + S * n * 4)
        if self.layout in ("chunk", "coin"):
            nc, ch = self.n_chunks(), self.chunk_budget()
            select = (S * n * 4 if self.layout == "chunk" else 0) + 2 * S * nc * 4 + \
                S * ch * 4 + S * (nc + 31) // 32 * 4 + S * (ch * self.CHUNK * 4 + words * 4 + 4)
        else:
            select = S * n * 4 + S * b * 4 + S * words * 4
        fit = 2 * (L * S * H * b * 3 * row + L * S * H * hd * 4 + S * b * 4)
        apply_one = L * S * H * (n - b) * 2 * row + L * S * H * hd * 4 + S * words * 4
        return {"draft": draft, "select": select, "fit_mean": fit, "apply": 2 * apply_one,
                "roofline_per_launch": apply_one, "roofline_units": L * S * H * (n - b),
                "total": draft + select + fit + 2 * apply_one}

    def build(self):
        torch, kv, c = self.torch, self.kv, self.cfg
        from synthetic import draw_correction, draw_deltas, draw_draft_queries
        from synthetic.workloads import draw_coin_keys
        L, S, H, Hq, T, n, hd = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_q_heads, c.n_draft,
                                 c.n_tokens, c.head_dim)
        b = self.probe_rows()
        t = {"delta": draw_deltas(c).to("cuda")}
        for p in "kv":
            t["reuse_" + p] = torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device="cuda")
            t["fresh_" + p] = torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device="cuda")
            t["out_" + p] = torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device="cuda")
        for l in range(L):
            raw = draw_correction(c, "cuda", layers=[l])
            xk = raw["x_k"].to(torch.bfloat16)
            kv.kvfix_rope_shift(kv.Plane.dense(xk), kv.Plane.dense(t["reuse_k"][l:l + 1]),
                                -t["delta"], c.theta)
            t["reuse_v"][l] = raw["x_v"][0].to(torch.bfloat16)
            t["fresh_k"][l], t["fresh_v"][l] = raw["fresh_k"][0], raw["fresh_v"][0]
            del raw, xk
        t["q"] = draw_draft_queries(c, "cuda")[None].contiguous()
        t["ws_draft"] = torch.empty(kv.kvfix_score_draft_workspace(S, L, c.first_layer, Hq, T, n)
                                    // 4 + 64, dtype=torch.float32, device="cuda")
        t["scores"] = torch.empty(S, n, dtype=torch.float32, device="cuda")
        t["idx"] = torch.empty(S, b, dtype=torch.int32, device="cuda")
        t["mask"] = torch.empty(S, (n + 31) // 32, dtype=torch.int32, device="cuda")
        if self.layout in ("chunk", "coin"):
            nc, ch = self.n_chunks(), self.chunk_budget()
            t["means"] = torch.empty(S, nc, dtype=torch.float32, device="cuda")
            t["cidx"] = torch.empty(S, ch, dtype=torch.int32, device="cuda")
            t["cmask"] = torch.empty(S, (nc + 31) // 32, dtype=torch.int32, device="cuda")
            t["counts"] = torch.empty(S, dtype=torch.int32, device="cuda")
            t["idx"] = torch.empty(S, ch * self.CHUNK, dtype=torch.int32, device="cuda")
            t["keys"] = draw_coin_keys(c.seed, S, nc, "cuda")
        t["mu"] = torch.empty(2, L, S, H, hd, dtype=torch.float32, device="cuda")
        for p in "kv":             # one workspace per plane: the two fits run concurrently
            t["ws_fit_" + p] = torch.empty(
                kv.kvfix_fit_mean_workspace(L, S, H, hd, t["idx"].shape[1]), dtype=torch.uint8,
                device="cuda")
        self.side = torch.cuda.Stream()
        self.ev_fork, self.ev_join = torch.cuda.Event(), torch.cuda.Event()
        P = kv.Plane.dense
        self.planes = {k: P(t[k]) for k in ("reuse_k", "reuse_v", "fresh_k", "fresh_v", "out_k",
                                            "out_v")}
        self.t = t
        torch.cuda.synchronize()

    def select(self):
        kv, t, c = self.kv, self.t, self.cfg
        if self.layout == "rows":
            kv.kvfix_select_topb(t["scores"], c.b, t["idx"], t["mask"])
        elif self.layout == "grow":
            kv.kvfix_select_grow(t["scores"], c.b, self.TAU, t["idx"], t["mask"])
        else:
            if self.layout == "chunk":
                kv.kvfix_chunk_means(t["scores"], self.CHUNK, t["means"])
            keys = t["means"] if self.layout == "chunk" else t["keys"]
            kv.kvfix_select_topb(keys, t["cidx"].shape[1], t["cidx"], t["cmask"])
            kv.kvfix_expand_chunks(t["cidx"], c.n_tokens, self.CHUNK, t["idx"], t["counts"],
                                   t["mask"])

    def step(self):
        kv, t, c, P = self.kv, self.t, self.cfg, self.planes
        if self.layout != "coin":
            kv.kvfix_score_draft(t["q"], P["reuse_k"], c.first_layer, t["delta"], c.theta,
                                 t["scores"], t["ws_draft"])
        self.select()
        width = t["idx"].shape[1]
        torch = self.torch
        main = torch.cuda.current_stream()

        def fit(i, p):
            d = t["delta"] if p == "k" else None
            kv.kvfix_fit_mean(P["fresh_" + p], P["reuse_" + p], P["out_" + p], t["idx"], width,
                              t["mu"][i], d, c.theta, ws=t["ws_fit_" + p])

        # the V fit runs on a second stream beside the K fit and apply
        self.ev_fork.record(main)
        self.side.wait_event(self.ev_fork)
        with torch.cuda.stream(self.side):
            fit(1, "v")
            self.ev_join.record(self.side)
        fit(0, "k")
        for i, p in enumerate("kv"):
            if p == "v":
                main.wait_event(self.ev_join)
            d = t["delta"] if p == "k" else None
            with (self.timed if p == "k" else self.timed_v):
                kv.kvfix_apply(P["reuse_" + p], P["out_" + p], t["mask"], t["mu"][i], None, 0.0,
                               1.0, d, c.theta)

    def cpu_baseline(self, np):
        """The oracle on a bounded sample: the draft mass over layers 1-3, the
        same probe layout, and fit + apply of K and V on layers 0-3."""
        torch, c, t = self.torch, self.cfg, self.t
        from oracle import kvref as K
        L4 = 4
        data = {k: host(t[k][:L4], torch, np) for k in ("reuse_k", "reuse_v", "fresh_k",
                                                       "fresh_v")}
        q = host(t["q"][0, :L4], torch, np)
        deltas = [int(v) for v in t["delta"].tolist()]
        keys = host(t["keys"], torch, np) if "keys" in t else None

        def run():
            s = None if self.layout == "coin" else K.score_draft(q, data["reuse_k"], deltas,
                                                                  c.theta, c.first_layer)
            if self.layout == "rows":
                idx, mask = K.select_topb(s, c.b)
            elif self.layout == "grow":
                idx, mask = K.select_grow(s, c.b, self.TAU)
            else:
                ks = K.chunk_means(s, self.CHUNK) if self.layout == "chunk" else keys
                nch = K.chunk_budget(c.n_tokens, self.CHUNK, *self.RHO, "alg1")
                idx, _, mask = K.expand_chunks(K.select_topb(ks, nch)[0], c.n_tokens, self.CHUNK)
            for p in "kv":
                K.correct(data["fresh_" + p], data["reuse_" + p], "bf16", idx, mask, None, 0.0,
                          1.0, None, None, deltas if p == "k" else None, c.theta)

        dt = timed_oracle(run, 1)
        # parity: the GPU's selection of its own scores (the sample's draft
        # mass covers layers 1-3 only, so its selection is not the step's),
        # and layers 0-3 of the step's corrected planes against the oracle
        # run on the GPU's probe set
        g_idx = host(t["idx"], torch, np)
        g_mask = host(t["mask"], torch, np).view(np.uint32)
        par = {"scope": "the GPU's probe selection on its own draft scores, and corrected "
                        f"layers 0-3 (4 of {c.n_layers}) of both planes with that selection",
               "bar": PARITY_BAR, "max_rel_err": {}, "index_mismatches": {}}
        if self.layout in ("rows", "grow"):
            g_sc = host(t["scores"], torch, np)
            o_idx, _ = (K.select_topb(g_sc, c.b) if self.layout == "rows"
                        else K.select_grow(g_sc, c.b, self.TAU))
            par["index_mismatches"]["selection on the GPU scores"] = index_mismatches(
                np, g_idx, o_idx)
        for i, p in enumerate("kv"):
            out, mu = K.correct(data["fresh_" + p], data["reuse_" + p], "bf16", g_idx, g_mask,
                                None, 0.0, 1.0, None, None, deltas if p == "k" else None, c.theta)
            par["max_rel_err"]["mu_" + p] = max_rel_err(np, host(t["mu"][i][:L4], torch, np), mu)
            par["max_rel_err"]["out_" + p] = max_rel_err(np, host(t["out_" + p][:L4], torch, np),
                                                         out, "bf16")
        self.parity = par
        sub = C4.__new__(C4)
        sub.cfg, sub.layout, sub.kv = c.replace(n_layers=L4), self.layout, self.kv
        nbytes = sub.alg_bytes()["total"]
        draft = "no draft; " if self.layout == "coin" else "draft mass over layers 1-3; "
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the whole step on layers 0-3 (4 of {c.n_layers}; {draft}the same "
                          f"probe layout) of the same input bytes ({nbytes / 1e6:.1f} MB "
                          f"algorithmic), one run of {dt:.1f} s, numpy fp64, one thread"}


# ----------------------------------------------------------------------------
# c3: collective round (diff encode + fused restore)
# ----------------------------------------------------------------------------


class C3(Workload):
    name = "c3"
    kernel_tag = "diff_decode"
    # restore into dense planes, into a paged pool through a slot mapping
    # (page 16, seeded permutation), or with the reuse plan first (deviation
    # score of every agent against the shared blocks at check layer 1, then
    # the master selection)
    layout = "dense"
    LAYOUT_TEXT = {"dense": "restore of all 16 caches into dense planes",
                   "paged": "restore of all 16 caches into a paged pool (16-token pages, seeded "
                            "slot mapping)",
                   "plan": "reuse plan first (every agent's check-layer deviation from the shared "
                           "blocks, master = lowest total), then restore into dense planes"}
    CHECK = 1

    def workload_text(self):
        return ("c3_collective: 16 agents x 32 layers x 8 KV heads x 8192 tokens x hd 128 bf16 at "
                "distinct offsets in [0,16384]; 16-token blocks, 3-9 % planted, eps 0.0625; "
                f"diff encode against the master, then {self.LAYOUT_TEXT[self.layout]}, theta 5e5")

    def alg_bytes(self, total_blocks=None):
        c = self.cfg
        L, A, H, n, hd, bt = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_tokens, c.head_dim,
                              c.block_tokens)
        nb = -(-n // bt)
        plane = L * H * n * hd * 2
        blk = H * bt * hd * 2
        tot = self.total if total_blocks is None else total_blocks
        meta = A * L * (-(-nb // 32)) * 4 + (A * L + 1) * 8 + tot * 4
        encode = 2 * A * plane + 2 * plane + 2 * tot * blk + meta
        decode = 2 * plane + 2 * tot * blk + meta + 2 * A * plane
        if self.layout == "paged":
            decode += A * (-(-n // 16)) * 4                  # the slot mapping
        plan = 0
        if self.layout == "plan":                            # one layer of K, agents and shared
            layer = H * n * hd * 2
            plan = 2 * A * layer + A * n * 4 + A * n * 4 + A * 8 + 4
        return {"plan": plan, "encode": encode, "decode": decode, "roofline_per_launch": decode,
                "roofline_units": A * L * H * n, "total": plan + encode + decode}

    def build(self):
        torch, kv, c = self.torch, self.kv, self.cfg
        from synthetic import draw_collective
        L, A, H, n, hd, bt = (c.n_layers, c.n_segs, c.n_kv_heads, c.n_tokens, c.head_dim,
                              c.block_tokens)
        t = {}
        pps = -(-n // 16)
        for p in "kv":
            t["m_" + p] = torch.empty(L, 1, H, n, hd, dtype=torch.bfloat16, device="cuda")
            t["s_" + p] = torch.empty(L, A, H, n, hd, dtype=torch.bfloat16, device="cuda")
            if self.layout == "paged":
                t["o_" + p] = torch.empty(L, A * pps, 16, H, hd, dtype=torch.bfloat16,
                                          device="cuda")
            else:
                t["o_" + p] = torch.empty(L, A, H, n, hd, dtype=torch.bfloat16, device="cuda")
        if self.layout == "paged":
            from synthetic.workloads import make_gen
            g = make_gen("cpu", c.seed, "restore_pages")
            t["pt"] = torch.randperm(A * pps, generator=g).to(torch.int32).reshape(A, pps).to(
                "cuda")
        planted = offs = None
        for l in range(L):
            raw = draw_collective(c, "cuda", layers=[l])
            planted, offs = raw["planted"], raw["offsets"].to("cuda")
            t["m_k"][l], t["m_v"][l] = raw["master_k"][0], raw["master_v"][0]
            kv.kvfix_rope_shift(kv.Plane.dense(raw["y_k"]), kv.Plane.dense(t["s_k"][l:l + 1]),
                                offs, c.theta)
            t["s_v"][l] = raw["y_v"][0]
            del raw
        t["to_m"], t["from_m"] = -offs, offs
        self.total = int(planted.sum()) * L
        self.diff = kv.Diff(A, L, n, H, hd, bt, self.total + 64, dtype=torch.bfloat16)
        t["status"] = torch.zeros(1, dtype=torch.int32, device="cuda")
        t["ws_e"] = torch.empty(kv.kvfix_diff_encode_workspace(A, L, n, bt) + 256,
                                dtype=torch.uint8, device="cuda")
        t["ws_d"] = torch.empty(kv.kvfix_diff_decode_workspace(A, hd) + 256, dtype=torch.uint8,
                                device="cuda")
        P = kv.Plane.dense
        self.planes = {k: P(t[k]) for k in ("m_k", "m_v", "s_k", "s_v")}
        for k in ("o_k", "o_v"):
            self.planes[k] = (kv.Plane.paged(t[k], t["pt"], 16, n) if self.layout == "paged"
                              else P(t[k]))
        if self.layout == "plan":
            self.planes["shared_k"] = P(t["m_k"].expand(-1, A, -1, -1, -1))
            t["dev"] = torch.empty(A, n, dtype=torch.float32, device="cuda")
            t["totals"] = torch.empty(A, dtype=torch.float64, device="cuda")
            t["master"] = torch.empty(1, dtype=torch.int32, device="cuda")
        self.t = t
        torch.cuda.synchronize()

    def step(self):
        kv, t, c, P = self.kv, self.t, self.cfg, self.planes
        if self.layout == "plan":
            kv.kvfix_score(P["s_k"], self.CHECK, P["shared_k"], self.CHECK, t["dev"],
                           t["from_m"], c.theta)
            kv.kvfix_select_master(t["dev"], t["totals"], t["master"])
        kv.kvfix_diff_encode(P["m_k"], P["m_v"], P["s_k"], P["s_v"], t["to_m"], c.theta, c.eps,
                             self.diff, t["status"], t["ws_e"])
        with self.timed:
            kv.kvfix_diff_decode(P["m_k"], P["m_v"], self.diff, t["from_m"], c.theta, P["o_k"],
                                 P["o_v"], t["ws_d"])

    def storage_report(self):
        """The group's storage under the master-mirror layout, from the blocks
        the encode listed (TD §6.4): every mirror's compression R = full
        cache / its diff, and the round's full caches over master + diffs."""
        np_ = __import__("numpy")
        c = self.cfg
        A, L = c.n_segs, c.n_layers
        nb = -(-c.n_tokens // c.block_tokens)
        off = host(self.diff.offsets, self.torch, np_)
        per_agent = np_.array([off[(a + 1) * L] - off[a * L] for a in range(A)], dtype=np_.float64)
        full_blocks = L * nb                     # one cache, in blocks (K and V alike)
        return {"diff_blocks_listed": int(off[-1]),
                "mirror_compression_mean": round(float(np_.mean(full_blocks / per_agent)), 2),
                "mirror_compression_min_max": [round(float(full_blocks / per_agent.max()), 2),
                                               round(float(full_blocks / per_agent.min()), 2)],
                "group_full_over_master_plus_diffs": round(
                    float(A * full_blocks / (full_blocks + per_agent.sum())), 2)}

    def cpu_baseline(self, np):
        """The oracle on a bounded sample: encode and restore of layer 0 for all
        16 agents."""
        torch, c, t = self.torch, self.cfg, self.t
        from oracle import kvref as K
        d = {k: host(t[k][:1], torch, np) for k in ("m_k", "m_v", "s_k", "s_v")}
        offs = [int(v) for v in t["from_m"].tolist()]
        plan = self.layout == "plan"
        if plan:
            ck = {k: host(t[k][self.CHECK:self.CHECK + 1], torch, np) for k in ("m_k", "s_k")}
        box = {}

        def run():
            if plan:
                A = c.n_segs
                dev = K.score_l2(ck["s_k"], np.repeat(ck["m_k"], A, axis=1), "bf16", 0, offs,
                                 c.theta)
                K.select_master(dev)
            o = K.diff_encode(d["m_k"], d["m_v"], d["s_k"], d["s_v"], [-x for x in offs],
                              c.theta, c.eps, c.block_tokens)
            ok, ov = K.diff_decode(d["m_k"], d["m_v"], o, offs, c.theta, c.n_segs, c.block_tokens)
            box["total"] = o["total"]
            box["o"], box["ok"], box["ov"] = o, ok, ov

        dt = timed_oracle(run, 1)
        # parity on layer 0: the listed blocks (bit-exact), their packed values
        # and the restored caches against the oracle's encode and decode
        A, L = c.n_segs, c.n_layers
        o = box["o"]
        g_mask = host(self.diff.mask, torch, np).view(np.uint32)
        g_off = host(self.diff.offsets, torch, np)
        slots = np.concatenate([np.arange(g_off[a * L], g_off[a * L + 1]) for a in range(A)])
        par = {"scope": f"layer 0 (1 of {L}) of all {A} agents: the listed blocks, the packed "
                        "values and the restored caches", "bar": PARITY_BAR, "max_rel_err": {},
               "mismatches": {}}
        par["mismatches"]["block mask words"] = int(np.sum(g_mask[:, 0:1] != o["mask"]))
        g_bi = host(self.diff.block_idx, torch, np)[slots]
        par["mismatches"]["block indices"] = (int(np.sum(g_bi != o["block_idx"]))
                                              if len(g_bi) == len(o["block_idx"]) else -1)
        if len(g_bi) == len(o["block_idx"]):
            par["max_rel_err"]["packed K"] = max_rel_err(
                np, host(self.diff.vals_k, torch, np)[slots], o["vals_k"], "bf16")
            par["mismatches"]["packed V elements"] = int(np.sum(
                host(self.diff.vals_v, torch, np)[slots] != o["vals_v"]))
        if self.layout != "paged":
            g_ok, g_ov = host(t["o_k"][:1], torch, np), host(t["o_v"][:1], torch, np)
        else:
            # layer 0 gathered from the pool through the slot mapping:
            # pool [L][page][16][H][hd] -> [1][A][H][n][hd]
            tok = np.arange(c.n_tokens)
            pt = host(t["pt"], torch, np)
            g_ok, g_ov = ((host(t[k][:1], torch, np)[:, pt[:, tok // 16], tok % 16]
                           .transpose(0, 1, 3, 2, 4)) for k in ("o_k", "o_v"))
        par["max_rel_err"]["restored K"] = max_rel_err(np, g_ok, box["ok"], "bf16")
        par["mismatches"]["restored V elements"] = int(np.sum(g_ov != box["ov"]))
        self.parity = par
        sub = C3.__new__(C3)
        sub.cfg, sub.total, sub.layout = c.replace(n_layers=1), box["total"], self.layout
        nbytes = sub.alg_bytes()["total"]
        what = "the reuse plan (check layer) and " if plan else ""
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{what}encode + restore of layer 0 (1 of {c.n_layers}) for all "
                          f"{c.n_segs} agents ({nbytes / 1e6:.1f} MB algorithmic), one run of "
                          f"{dt:.1f} s, numpy fp64, one thread"}


class C2Anchor(Workload):
    """The c2 segment corrected through an anchor pool (KVCMAS eq. 8-11, App.
    A.3): match (gate + token weights of K and V) and the blended apply."""
    name = "c2"
    counter_name = "c2_anchor"
    kernel_tag = "anchor_match"
    V, RANK, SRC_OFF, TAU = 10, 32, 2048, 0.5
    # The match call (three kernels) dominates and is bound by vector ALU work: one absolute
    # add per element and anchor on the key plane, an absolute add and a
    # fused multiply-add on the value plane (4 flops per element and anchor
    # over both planes), against the fp32 vector peak of 157.3 TFLOP/s.
    roof = ("alu", "TFLOP/s", 157.3, 1e12)

    def workload_text(self):
        return ("c2_llama3_8b segment (32 layers x 8 KV heads x 4096 tokens x hd 128 bf16) "
                f"corrected through an anchor pool: V={self.V} anchors, rank {self.RANK}, "
                "gate over the whole segment, token weights of K and V, blended delta apply "
                "with re-alignment, theta 5e5")

    def mfma_flops(self):
        c = self.cfg
        D = c.n_kv_heads * c.head_dim
        return 2 * (self.V * c.n_layers * 2 * c.n_tokens * D * self.RANK * 2)

    def alg_bytes(self):
        c = self.cfg
        L, H, n, hd, V, r = c.n_layers, c.n_kv_heads, c.n_tokens, c.head_dim, self.V, self.RANK
        plane = L * H * n * hd * 2
        a = V * L * 2 * n * r * 2
        bt = V * L * 2 * H * hd * r * 2
        wts = L * 2 * n * V * 4
        parts = L * -(-n // 128) * V * 8
        match = 2 * plane + a + bt + wts + parts
        apply = 4 * plane + a + bt + wts
        match_flops = L * n * H * hd * V * 4
        return {"match": match, "apply": apply, "roofline_per_launch": match_flops,
                "roofline_units": 2 * L * H * n, "total": match + apply}

    def build(self):
        torch, kv, c = self.torch, self.kv, self.cfg
        from synthetic import draw_anchor_pool, draw_deltas
        L, n, V = c.n_layers, c.n_tokens, self.V
        raw = draw_anchor_pool(c, V, "cuda", rank=self.RANK)
        t = {k: raw[k] for k in ("a_base", "bt_base", "a_delta", "bt_delta")}
        self.tgt_off = self.SRC_OFF + int(draw_deltas(c)[0])
        # keys stored at positions SRC_OFF + j: the canonical content rotated forward
        canon = raw["src_k"].to(torch.bfloat16)
        t["src_k"] = torch.empty_like(canon)
        off = torch.full((1,), self.SRC_OFF, dtype=torch.int64, device="cuda")
        kv.kvfix_rope_shift(kv.Plane.dense(canon), kv.Plane.dense(t["src_k"]), off, c.theta)
        t["src_v"] = raw["src_v"].to(torch.bfloat16)
        del raw, canon
        t["out_k"], t["out_v"] = torch.empty_like(t["src_k"]), torch.empty_like(t["src_v"])
        t["w"] = torch.empty(L, 2, V, n, dtype=torch.float32, device="cuda")
        t["gate"] = torch.empty(V + 1, dtype=torch.float64, device="cuda")
        t["accept"] = torch.empty(1, dtype=torch.int32, device="cuda")
        t["ws"] = torch.empty(kv.kvfix_anchor_match_workspace(L, c.n_kv_heads, n, V),
                              dtype=torch.uint8, device="cuda")
        lengths = [n] * V
        self.base = kv.AnchorPool(t["a_base"], t["bt_base"], lengths)
        self.delta = kv.AnchorPool(t["a_delta"], t["bt_delta"], lengths)
        self.planes = {k: kv.Plane.dense(t[k]) for k in ("src_k", "src_v", "out_k", "out_v")}
        self.extra_timed = {"anchor_apply_kernel": Timed(torch)}
        self.t = t
        torch.cuda.synchronize()

    def step(self):
        kv, t, c, P = self.kv, self.t, self.cfg, self.planes
        with self.timed:
            kv.kvfix_anchor_match(P["src_k"], P["src_v"], 0, self.base, self.SRC_OFF, c.theta,
                                  c.n_tokens, self.TAU, t["w"], t["gate"], t["accept"], t["ws"])
        with self.extra_timed["anchor_apply_kernel"]:
            kv.kvfix_anchor_apply(P["src_k"], P["src_v"], 0, self.delta, t["w"], self.SRC_OFF,
                                  self.tgt_off, c.theta, P["out_k"], P["out_v"])

    def cpu_baseline(self, np):
        """The oracle on a bounded sample: gate, token weights and apply of K
        and V on layers 0-3 of the same input bytes (all tokens, all anchors)."""
        torch, c, t = self.torch, self.cfg, self.t
        from oracle import kvref as K
        LS = 4
        d = {k: host(t[k][:LS], torch, np) for k in ("src_k", "src_v")}
        d.update({k: host(t[k][:, :LS], torch, np) for k in ("a_base", "bt_base", "a_delta",
                                                             "bt_delta")})
        lengths = [c.n_tokens] * self.V

        def run():
            K.anchor_gate(d["src_v"], d["a_base"], d["bt_base"], lengths, c.n_tokens, self.TAU,
                          "bf16")
            w = K.anchor_weights(d["src_k"], d["src_v"], d["a_base"], d["bt_base"], lengths,
                                 self.SRC_OFF, c.theta, "half", "bf16")
            for p, key in ((0, "src_k"), (1, "src_v")):
                K.anchor_apply(d[key], p, d["a_delta"], d["bt_delta"], w, lengths, self.SRC_OFF,
                               self.tgt_off, c.theta, "half", "bf16")

        dt = timed_oracle(run, 1)
        nbytes = self.alg_bytes()["total"] * LS // c.n_layers
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"gate, weights and apply of layers 0-{LS - 1} ({LS} of {c.n_layers}), "
                          f"all {c.n_tokens} tokens and {self.V} anchors ({nbytes / 1e6:.1f} MB "
                          f"algorithmic), one run of {dt:.1f} s, numpy fp64, one thread"}


Workload.ALL = {"c2": C2, "c3": C3, "c4": C4, "c5": C5}
# workload variants chosen by --layout
VARIANTS = {("c2", "anchor"): C2Anchor}

ROOFLINE_KERNEL = {
    "c2": "kvfix apply_kernel<bf16, fp32, hd128, rotate-half, rank 4>",
    "c3": "kvfix diff_decode_kernel<bf16, hd128, rotate-half> (with its rotary-table pre-kernel)",
    "c4": "kvfix apply_kernel<bf16, fp32, hd128, rotate-half, rank 0>",
    "c5": "kvfix apply_kernel<bf16, fp32, hd128, rotate-half, rank 2, paged>",
    "c2_anchor": "kvfix_anchor_match: anchor_match_kernel<rotate-half> + anchor_finish_kernel + "
                 "anchor_gate_kernel (V=10, rank 32, K and V planes)",
}


def copy_ceiling(torch):
    """Measured copy ceiling: a plain device-to-device bf16 copy of 512 MiB."""
    n_copy = 256 << 20
    src = torch.empty(n_copy, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = _events(torch)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    return 2 * src.numel() * 2 / (c0.elapsed_time(c1) / 5 * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", choices=sorted(Workload.ALL))
    ap.add_argument("--layout", default=None,
                    help="c4: probe layout rows|chunk|coin|grow (BCR layouts and the coin "
                         "control); c3: restore target dense|paged, or plan (reuse plan first); "
                         "c2: anchor (the segment corrected through an anchor pool)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    W = Workload.ALL[args.workload]
    if (args.workload, args.layout) in VARIANTS:
        W = VARIANTS[(args.workload, args.layout)]
    elif args.layout is not None and args.layout not in getattr(W, "LAYOUT_TEXT", {}):
        print(f"--layout {args.layout} does not apply to {args.workload}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the correction path is sharded by segment/layer/head without exchange; "
              "see DESIGN.md for the multi-GPU design)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import cross_context_kv_amd.kvfix as kv
    from synthetic import CONFIGS
    kv.lib()                          # fails loudly without the built library
    w = W(CONFIGS[args.workload], torch, kv)
    if args.layout is not None and W is Workload.ALL[args.workload]:
        w.layout = args.layout
    w.build()
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()

    # The step time comes from a timed region without per-launch events (an
    # event pair costs a few microseconds of stream time); a second timed
    # region of the same steps records events around the roofline kernel.
    start, end = _events(torch)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        w.step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    w.timed.on = True
    w.timed_v.on = True
    for tm in w.extra_timed.values():
        tm.on = True
    torch.cuda.synchronize()
    for _ in range(args.steps):
        w.step()
    torch.cuda.synchronize()
    roof_ms = w.timed.avg_ms()
    copy_gbs = copy_ceiling(torch)

    ab = w.alg_bytes()
    gbs = ab["total"] / (ms * 1e-3) / 1e9
    bound, roof_unit, roof_peak, roof_scale = w.roof
    roof_val = ab["roofline_per_launch"] / (roof_ms * 1e-3) / roof_scale
    c = w.cfg
    line = {
        "metric": METRIC,
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
            "workload": w.workload_text(),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "segment_layers_per_s": round(c.n_segs * c.n_layers / (ms * 1e-3), 1),
            "alg_bytes_per_step": ab["total"],
            "copy_ceiling_GBs": round(copy_gbs, 1),
            "pct_copy_ceiling": round(100 * gbs / copy_gbs, 2),
            "seed": c.seed,
        },
        "roofline": {
            "bound": bound,
            "kernel": ROOFLINE_KERNEL[w.counter_name],
            "achieved": round(roof_val, 2),
            "peak": roof_peak,
            "unit": roof_unit,
            "frac": round(roof_val / roof_peak, 4),
            "traffic": read_traffic(w),
            ("alg_bytes_per_launch" if roof_unit == "GB/s" else "alg_flops_per_launch"):
                ab["roofline_per_launch"],
            "avg_launch_ms": round(roof_ms, 5),
        },
        "cpu_baseline": None,
    }
    for label, tm in w.extra_timed.items():
        line["config"][f"avg_ms {label}"] = round(tm.avg_ms(), 5)
    if w.timed_v.pairs:
        # the value-plane apply, timed apart from the roofline (key-plane) kernel
        v_ms = w.timed_v.avg_ms()
        line["config"]["avg_ms apply_kernel value plane"] = round(v_ms, 5)
        line["config"]["value plane apply GB/s"] = round(
            ab["roofline_per_launch"] / (v_ms * 1e-3) / 1e9, 2)
    if hasattr(w, "mfma_flops"):
        line["config"]["mfma_TFLOPs"] = round(w.mfma_flops() / (ms * 1e-3) / 1e12, 1)
    if hasattr(w, "storage_report"):
        line["config"].update(w.storage_report())
    if not args.no_cpu_baseline:
        cb = w.cpu_baseline(np)
        cb.update(host_info())
        line["cpu_baseline"] = cb
        line["parity"] = w.parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

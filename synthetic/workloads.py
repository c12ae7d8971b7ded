"""Workload shapes and seeded random draws for the five correction workloads.

Every number drawn here is either a raw random draw or a plain sum of raw
draws that defines the synthetic residual model of a workload (the "fresh"
cache is the aligned reuse content plus an offset, a low-rank term and noise).
Turning the aligned reuse content into a stored cache at its old position needs
a rotary rotation; that step is left to the caller, because rotation is part of
the method under test.

Distributions follow the workload descriptions; N(m, s) always means mean m
and STANDARD DEVIATION s.  All draws use torch generators seeded from a stable
hash of (workload seed, stream name, layer), so any subset of layers can be
redrawn on its own, on the CPU or on the GPU.  A CPU generator and a GPU
generator with the same seed give different (equally valid) numbers.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Iterable, Optional

import torch


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    n_segs: int
    dtype: str                     # "f32" or "bf16" storage
    theta: float
    seed: int
    ratio: float = 0.0             # probe ratio r
    b: int = 0                     # stated probe budget ceil(r*n)
    check_layer: int = 0
    weight: str = "one"            # "one" (w = 1) or "clip" (w = clip(d, lo, hi))
    w_lo: float = 0.0
    w_hi: float = 2.0
    rank: int = 0
    mu_std: float = 0.5
    noise_std: float = 0.05
    w_std: float = 0.1             # std of the low-rank right factor
    n_outliers: int = 0
    outlier_std: float = 2.0
    delta_lo: int = 0
    delta_hi: int = 0
    delta_fixed: Optional[int] = None
    per_segment_delta: bool = False
    # draft scoring
    n_q_heads: int = 0
    n_draft: int = 0
    first_layer: int = 1
    # paged layout
    page_size: int = 0
    n_pages: int = 0
    # collective diff
    block_tokens: int = 16
    frac_lo: float = 0.0
    frac_hi: float = 0.0
    perturb_std: float = 0.0
    eps: float = 0.0
    offset_hi: int = 0
    in_place: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def row_bytes(self) -> int:
        return self.head_dim * (4 if self.dtype == "f32" else 2)

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, WorkloadConfig] = {
    # Tiny fp32 case, mean-only correction with L2-chosen probes.
    "c1": WorkloadConfig(
        name="c1_tiny_fp32", n_layers=1, n_kv_heads=2, head_dim=64, n_tokens=256, n_segs=1,
        dtype="f32", theta=1.0e4, seed=1000, ratio=0.1, b=26, check_layer=0, weight="one",
        rank=0, mu_std=0.5, noise_std=0.05, n_outliers=8, outlier_std=2.0, delta_fixed=37),
    # Llama-3-8B-shaped cache: mean + rank-4 + clipped weights.
    "c2": WorkloadConfig(
        name="c2_llama3_8b", n_layers=32, n_kv_heads=8, head_dim=128, n_tokens=4096, n_segs=1,
        dtype="bf16", theta=5.0e5, seed=2000, ratio=0.15, b=615, check_layer=1, weight="clip",
        w_lo=0.0, w_hi=2.0, rank=4, mu_std=0.5, noise_std=0.02, w_std=0.1,
        delta_lo=1, delta_hi=8192),
    # Collective round: 16 agents, one 8192-token segment, block-sparse diffs.
    "c3": WorkloadConfig(
        name="c3_collective_16x8192", n_layers=32, n_kv_heads=8, head_dim=128, n_tokens=8192,
        n_segs=16, dtype="bf16", theta=5.0e5, seed=3000, block_tokens=16, frac_lo=0.03,
        frac_hi=0.09, perturb_std=0.1, eps=0.0625, offset_hi=16384),
    # Qwen2.5-14B-shaped draft-selected repair.
    "c4": WorkloadConfig(
        name="c4_qwen25_14b_draft", n_layers=48, n_kv_heads=8, head_dim=128, n_tokens=32768,
        n_segs=1, dtype="bf16", theta=1.0e6, seed=4000, ratio=0.1, b=3277, weight="one",
        rank=0, mu_std=0.5, noise_std=0.05, delta_lo=1, delta_hi=32768, n_q_heads=40,
        n_draft=2, first_layer=1),
    # Llama-3-70B-shaped paged batch of 32 segments, corrected in place.
    "c5": WorkloadConfig(
        name="c5_llama3_70b_paged", n_layers=80, n_kv_heads=8, head_dim=128, n_tokens=4096,
        n_segs=32, dtype="bf16", theta=5.0e5, seed=5000, ratio=0.1, b=410, check_layer=1,
        weight="one", rank=2, mu_std=0.5, noise_std=0.02, w_std=0.1, delta_lo=1,
        delta_hi=32768, per_segment_delta=True, page_size=16, n_pages=8192, in_place=True),
}


def make_gen(device, *keys) -> torch.Generator:
    """A torch generator on `device`, seeded from a stable hash of `keys`."""
    h = hashlib.sha256(repr(keys).encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def _normal(shape, std, device, *keys) -> torch.Tensor:
    g = make_gen(device, *keys)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def draw_deltas(cfg: WorkloadConfig) -> torch.Tensor:
    """Position shift per segment (int64, host tensor)."""
    S = cfg.n_segs
    if cfg.delta_fixed is not None:
        return torch.full((S,), cfg.delta_fixed, dtype=torch.int64)
    g = make_gen("cpu", cfg.seed, "delta")
    if cfg.offset_hi:   # collective: distinct offsets in [0, offset_hi]
        return torch.randperm(cfg.offset_hi + 1, generator=g)[:S].to(torch.int64)
    n_draw = S if cfg.per_segment_delta else 1
    d = torch.randint(cfg.delta_lo, cfg.delta_hi + 1, (n_draw,), generator=g, dtype=torch.int64)
    return d.expand(S).clone() if n_draw == 1 else d


def draw_correction(cfg: WorkloadConfig, device="cpu", layers: Optional[Iterable[int]] = None,
                    segs: Optional[Iterable[int]] = None) -> dict:
    """Raw draws of a correction workload for the chosen layers (default: all).

    Returns float32 tensors shaped [len(layers), len(segs), H, n, hd]:
      x_k, x_v      aligned reuse content, N(0, 1)
      fresh_k/_v    x + 1 mu^T + U W + noise (+ outlier rows), in the storage dtype
    plus the rank state (a_k, b_k, a_v, b_v: U [.., n, r] and W [.., r, hd], float32)
    and the true offsets mu_k, mu_v [.., H, hd].
    """
    L = list(range(cfg.n_layers)) if layers is None else list(layers)
    S = list(range(cfg.n_segs)) if segs is None else list(segs)
    H, n, hd, r = cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, cfg.rank
    out = {}
    for plane in ("k", "v"):
        xs, fr, As, Bs, mus = [], [], [], [], []
        for l in L:
            xl, fl, al, bl, ml = [], [], [], [], []
            for s in S:
                key = (cfg.seed, plane, l, s)
                x = _normal((H, n, hd), 1.0, device, *key, "x")
                mu = _normal((H, hd), cfg.mu_std, device, *key, "mu")
                f = x + mu[:, None, :] + _normal((H, n, hd), cfg.noise_std, device, *key, "xi")
                if r > 0:
                    U = _normal((H, n, r), 1.0, device, *key, "U")
                    W = _normal((H, r, hd), cfg.w_std, device, *key, "W")
                    f = f + torch.bmm(U, W)
                    al.append(U)
                    bl.append(W)
                if cfg.n_outliers:
                    g = make_gen("cpu", *key, "outlier_rows")
                    rows = torch.randperm(n, generator=g)[: cfg.n_outliers].to(device)
                    f[:, rows, :] += _normal((H, cfg.n_outliers, hd), cfg.outlier_std, device,
                                             *key, "outlier_vals")
                xl.append(x)
                fl.append(f.to(cfg.torch_dtype))
                ml.append(mu)
            xs.append(torch.stack(xl))
            fr.append(torch.stack(fl))
            mus.append(torch.stack(ml))
            if r > 0:
                As.append(torch.stack(al))
                Bs.append(torch.stack(bl))
        out["x_" + plane] = torch.stack(xs)
        out["fresh_" + plane] = torch.stack(fr)
        out["mu_" + plane] = torch.stack(mus)
        out["a_" + plane] = torch.stack(As) if r > 0 else None
        out["b_" + plane] = torch.stack(Bs) if r > 0 else None
    out["delta"] = draw_deltas(cfg)[S]
    return out


def draw_draft_queries(cfg: WorkloadConfig, device="cpu") -> torch.Tensor:
    """Draft query rows, N(0, 1) in bf16, shaped [L, Hq, n_draft, hd]."""
    q = _normal((cfg.n_layers, cfg.n_q_heads, cfg.n_draft, cfg.head_dim), 1.0, device,
                cfg.seed, "draft_q")
    return q.to(torch.bfloat16)


def draw_coin_keys(seed: int, rows: int, n_chunks: int, device="cpu", draw: int = 0) -> torch.Tensor:
    """Uniform [0, 1) float32 keys [rows, n_chunks], one per chunk, for the
    coin control (the chunks holding the largest keys form a uniformly random
    subset of any fixed size).  `draw` tells repeated coins apart."""
    g = make_gen(device, seed, "coin", draw)
    return torch.rand(rows, n_chunks, generator=g, device=device, dtype=torch.float32)


def draw_page_table(cfg: WorkloadConfig, device="cpu") -> torch.Tensor:
    """Seeded permutation of the page pool, int32 [n_segs, n_tokens / page_size]."""
    per_seg = -(-cfg.n_tokens // cfg.page_size)
    g = make_gen("cpu", cfg.seed, "pages")
    perm = torch.randperm(cfg.n_pages, generator=g)[: cfg.n_segs * per_seg]
    return perm.to(torch.int32).reshape(cfg.n_segs, per_seg).to(device)


def draw_collective(cfg: WorkloadConfig, device="cpu", layers: Optional[Iterable[int]] = None,
                    agents: Optional[Iterable[int]] = None) -> dict:
    """Raw draws of a collective round.

    master_k / master_v : bf16 [len(layers), 1, H, n, hd], N(0, 1)
    y_k / y_v           : bf16 [len(layers), len(agents), H, n, hd] — the master with
                          N(0, perturb_std) added on each agent's planted blocks
    planted             : bool [n_agents, n_blocks] (same token blocks at every layer)
    offsets             : int64 [n_agents] distinct positions in [0, offset_hi]
    An agent's stored K cache is y_k rotated to its offset (done by the caller).
    """
    L = list(range(cfg.n_layers)) if layers is None else list(layers)
    A = list(range(cfg.n_segs)) if agents is None else list(agents)
    H, n, hd, bt = cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, cfg.block_tokens
    nb = -(-n // bt)
    planted = torch.zeros(cfg.n_segs, nb, dtype=torch.bool)
    for a in range(cfg.n_segs):
        g = make_gen("cpu", cfg.seed, "frac", a)
        f = cfg.frac_lo + (cfg.frac_hi - cfg.frac_lo) * torch.rand((), generator=g).item()
        k = max(1, int(round(f * nb)))
        planted[a, torch.randperm(nb, generator=g)[:k]] = True
    out = {"planted": planted, "offsets": draw_deltas(cfg)}
    for plane in ("k", "v"):
        ms, ys = [], []
        for l in L:
            m = _normal((H, n, hd), 1.0, device, cfg.seed, plane, l, "master").to(torch.bfloat16)
            ms.append(m[None])
            yl = []
            for a in A:
                rows = planted[a].repeat_interleave(bt)[:n].to(device)
                y = m.float()
                noise = _normal((H, n, hd), cfg.perturb_std, device, cfg.seed, plane, l, a, "dy")
                y = torch.where(rows[None, :, None], y + noise, y)
                yl.append(y.to(torch.bfloat16))
            ys.append(torch.stack(yl))
        out["master_" + plane] = torch.stack(ms)
        out["y_" + plane] = torch.stack(ys)
    return out


def draw_anchor_pool(cfg: WorkloadConfig, n_anchors: int, device="cpu",
                     layers: Optional[Iterable[int]] = None, n_max: Optional[int] = None,
                     rank: int = 32, spread: float = 0.25, delta_std: float = 0.1) -> dict:
    """Raw draws of an anchor pool and of a source segment that resembles it.

    Per (layer, plane): shared factors A0 [n_max, rank] ~ N(0, 1) and
    B0 [D, rank] ~ N(0, 1/sqrt(rank)) (D = H * hd); anchor v's base factors
    are A0 + s_v N(0, 1) and B0 + s_v N(0, 1/sqrt(rank)) with s_v = spread *
    (v + 1) / V, so the anchors sit at graded distances from the shared
    structure; the source content is A_s B_s^T + N(0, noise_std) with its
    own perturbation of strength spread / 2.  Delta factors are independent:
    A ~ N(0, delta_std), B ~ N(0, 1/sqrt(rank)).

    Returns
      src_k, src_v         float32 [len(layers), 1, H, n, hd]: the source
                           content in canonical (segment-relative) positions
                           (storing keys at an offset needs a rotation, left to
                           the caller)
      a_base, bt_base      bf16 [V, len(layers), 2, n_max, rank] and
      a_delta, bt_delta    bf16 [V, len(layers), 2, D, rank] (B transposed)
    """
    L = list(range(cfg.n_layers)) if layers is None else list(layers)
    H, n, hd, V = cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, n_anchors
    n_max = n if n_max is None else n_max
    D = H * hd
    bs = 1.0 / rank ** 0.5
    out = {k: torch.empty(shape, dtype=torch.bfloat16, device=device) for k, shape in (
        ("a_base", (V, len(L), 2, n_max, rank)), ("bt_base", (V, len(L), 2, D, rank)),
        ("a_delta", (V, len(L), 2, n_max, rank)), ("bt_delta", (V, len(L), 2, D, rank)))}
    src = {p: torch.empty((len(L), 1, H, n, hd), dtype=torch.float32, device=device)
           for p in ("k", "v")}
    for li, l in enumerate(L):
        for pi, plane in enumerate(("k", "v")):
            key = (cfg.seed, "anchor", plane, l)
            A0 = _normal((max(n, n_max), rank), 1.0, device, *key, "A0")
            B0 = _normal((D, rank), bs, device, *key, "B0")
            for v in range(V):
                s_v = spread * (v + 1) / V
                out["a_base"][v, li, pi] = A0[:n_max] + _normal((n_max, rank), s_v, device, *key, v, "A")
                out["bt_base"][v, li, pi] = B0 + _normal((D, rank), s_v * bs, device, *key, v, "B")
                out["a_delta"][v, li, pi] = _normal((n_max, rank), delta_std, device, *key, v, "dA")
                out["bt_delta"][v, li, pi] = _normal((D, rank), bs, device, *key, v, "dB")
            As = A0[:n] + _normal((n, rank), spread / 2, device, *key, "As")
            Bs = B0 + _normal((D, rank), spread / 2 * bs, device, *key, "Bs")
            x = As @ Bs.T + _normal((n, D), cfg.noise_std, device, *key, "xs")
            src[plane][li, 0] = x.reshape(n, H, hd).transpose(0, 1)
    out["src_k"], out["src_v"] = src["k"], src["v"]
    return out

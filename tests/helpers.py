"""Shared test utilities: input assembly, dtype views, tolerance metric.

Inputs come from `synthetic` (seeded raw draws).  The stored cache of a
segment at its old position is the aligned content rotated back by the
segment's shift; tests build it with the oracle's rotation (test
infrastructure), never with the library under test.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from oracle import kvref as K

# Parity bar: max |g - o| / (|o| + 1e-3) <= 8e-3 for bf16 values, <= 1e-5 for fp32.
TOL = {"bf16": 8e-3, "f32": 1e-5}


def log(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device or host tensor -> numpy in the oracle's storage format."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def from_np(a: np.ndarray, device="cpu") -> torch.Tensor:
    """Oracle storage format -> torch (uint16 bits -> bfloat16)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def rel_err(g: np.ndarray, o: np.ndarray, dtype: str) -> float:
    """max |g - o| / (|o| + 1e-3) over all elements, values as float64."""
    gv = K.to_f64(g, dtype) if dtype in ("bf16", "f32") else g.astype(np.float64)
    ov = K.to_f64(o, dtype) if dtype in ("bf16", "f32") else o.astype(np.float64)
    if gv.size == 0:
        return 0.0
    return float(np.max(np.abs(gv - ov) / (np.abs(ov) + 1e-3)))


def assert_values(g: np.ndarray, o: np.ndarray, dtype: str, what: str = "") -> float:
    e = rel_err(g, o, dtype)
    assert e <= TOL[dtype], f"{what}: max rel err {e:.3g} > {TOL[dtype]}"
    return e


def mask_from_idx(idx: np.ndarray, n: int) -> np.ndarray:
    rows, b = idx.shape
    m = np.zeros((rows, (n + 31) // 32), dtype=np.uint32)
    for r in range(rows):
        for j in idx[r]:
            m[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return m


def correction_case(cfg, device="cpu", style="half"):
    """Assemble one correction workload (small sizes: drawn on the CPU).

    Returns numpy arrays in oracle format (reuse_k/v, fresh_k/v, A/B per
    plane, deltas) and the config.  reuse_k is the aligned content rotated
    back by -delta and rounded once; reuse_v is the content itself.
    """
    from synthetic import draw_correction
    raw = draw_correction(cfg, device)
    deltas = [int(d) for d in raw["delta"].tolist()]
    xk = raw["x_k"].double().cpu().numpy()
    xv = raw["x_v"].double().cpu().numpy()
    case = {
        "deltas": deltas,
        "reuse_k": K.store(K.align_plane_f64(xk, [-d for d in deltas], cfg.theta, style), cfg.dtype),
        "reuse_v": K.store(xv, cfg.dtype),
        "fresh_k": to_np(raw["fresh_k"]),
        "fresh_v": to_np(raw["fresh_v"]),
        "A_k": None if raw["a_k"] is None else raw["a_k"].cpu().numpy(),
        "B_k": None if raw["b_k"] is None else raw["b_k"].cpu().numpy(),
        "A_v": None if raw["a_v"] is None else raw["a_v"].cpu().numpy(),
        "B_v": None if raw["b_v"] is None else raw["b_v"].cpu().numpy(),
    }
    return case


def torch_rotate(x: torch.Tensor, deltas, theta: float, style: str = "half") -> torch.Tensor:
    """Rotary rotation by deltas[s] positions in fp64 with plain torch ops (test
    infrastructure for building stored caches on the GPU; the library under
    test is not involved).  x: [..., S, H, n, hd]; returns float64."""
    hd = x.shape[-1]
    dev = x.device
    i = torch.arange(hd // 2, dtype=torch.float64, device=dev)
    inv_freq = torch.pow(torch.tensor(theta, dtype=torch.float64, device=dev), -2.0 * i / hd)
    d = torch.as_tensor(list(deltas), dtype=torch.float64, device=dev)
    phi = d[:, None] * inv_freq[None, :]                       # [S][hd/2]
    c = torch.cos(phi)[:, None, None, :]
    s = torch.sin(phi)[:, None, None, :]
    x = x.double()
    if style == "half":
        a, b = x[..., : hd // 2], x[..., hd // 2:]
        return torch.cat([a * c - b * s, b * c + a * s], dim=-1)
    a, b = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def correction_case_gpu(cfg, style: str = "half"):
    """The full-size correction workload drawn on the GPU (same recipe as
    correction_case, different random numbers); numpy arrays in oracle format.
    Stored keys are rotated back by -delta with torch_rotate, layer by layer."""
    from synthetic import draw_correction
    raw = draw_correction(cfg, "cuda")
    deltas = [int(d) for d in raw["delta"].tolist()]
    neg = [-d for d in deltas]
    xk = raw["x_k"]
    reuse_k = torch.empty(xk.shape, dtype=cfg.torch_dtype, device=xk.device)
    for l in range(xk.shape[0]):
        reuse_k[l] = torch_rotate(xk[l], neg, cfg.theta, style).to(cfg.torch_dtype)
    case = {
        "deltas": deltas,
        "reuse_k": to_np(reuse_k),
        "reuse_v": to_np(raw["x_v"].to(cfg.torch_dtype)),
        "fresh_k": to_np(raw["fresh_k"]),
        "fresh_v": to_np(raw["fresh_v"]),
    }
    for p in ("k", "v"):
        case["A_" + p] = None if raw["a_" + p] is None else raw["a_" + p].cpu().numpy()
        case["B_" + p] = None if raw["b_" + p] is None else raw["b_" + p].cpu().numpy()
    del raw, xk, reuse_k
    torch.cuda.empty_cache()
    return case

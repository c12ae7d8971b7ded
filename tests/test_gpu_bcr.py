"""GPU parity of the BCR probe layouts against the CPU oracle: chunk means,
the rows of whole chunks, the coin control, grown spans, and the probe mean
and correction over padded index lists.

Chunk means are bit-exact (the same fp64 sums in token order, one rounding);
indices, counts and masks are bit-exact; corrected values are within
max |g - o| / (|o| + 1e-3) <= 8e-3 (bf16) or 1e-5 (fp32)."""
import numpy as np
import pytest
import torch

from helpers import assert_values, correction_case, from_np, log, rel_err, to_np
from oracle import kvref as K
from synthetic import CONFIGS
from synthetic.workloads import draw_coin_keys

import cross_context_kv_amd.kvfix as kv
from cross_context_kv_amd.kvfix import Plane

pytestmark = pytest.mark.gpu
DEV = "cuda"


def draw_scores(seed, rows, n, kind):
    """Score rows of three shapes: peaky (log-normal), flat (1 +- 5 %), ties
    (small integers, signed zeros included)."""
    rng = np.random.default_rng(seed)
    if kind == "peaky":
        a = np.exp(3.0 * rng.standard_normal((rows, n)))
    elif kind == "flat":
        a = 1.0 + 0.05 * rng.standard_normal((rows, n))
    else:
        a = np.round(rng.random((rows, n)) * 6.0)
        a[rng.random((rows, n)) < 0.1] = -0.0
    return a.astype(np.float32)


def gpu_means(x, B):
    t = torch.from_numpy(x).to(DEV)
    nc = -(-x.shape[1] // B)
    m = torch.full((x.shape[0], nc), float("nan"), dtype=torch.float32, device=DEV)
    kv.kvfix_chunk_means(t, B, m)
    return m


def gpu_topb(keys, c):
    rows, n = keys.shape
    idx = torch.full((rows, c), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((rows, (n + 31) // 32), -1, dtype=torch.int32, device=DEV)
    kv.kvfix_select_topb(keys, c, idx, mask)
    return idx


def gpu_expand(cidx, n, B):
    rows, c = cidx.shape
    idx = torch.full((rows, c * B), -7, dtype=torch.int32, device=DEV)
    counts = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((rows, (n + 31) // 32), -1, dtype=torch.int32, device=DEV)
    kv.kvfix_expand_chunks(cidx, n, B, idx, counts, mask)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), counts.cpu().numpy(), mask.cpu().numpy().view(np.uint32)


def gpu_grow(x, b, tau):
    t = torch.from_numpy(x).to(DEV)
    rows, n = x.shape
    idx = torch.full((rows, b), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((rows, (n + 31) // 32), -1, dtype=torch.int32, device=DEV)
    kv.kvfix_select_grow(t, b, tau, idx, mask)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), mask.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n,B", [(1000, 64), (4096, 64), (300, 16), (777, 1), (2048, 1024),
                                 (100, 128), (33000, 64)])
def test_chunk_means_bit_exact(n, B):
    x = draw_scores(n + B, 3, n, "peaky")
    log("chunk means", n, B)
    g = gpu_means(x, B).cpu().numpy()
    o = K.chunk_means(x, B)
    assert np.array_equal(g.view(np.uint32), o.view(np.uint32))


@pytest.mark.parametrize("n,B,rho,rule", [(1000, 64, (1, 5), kv.BUDGET_SKIP),
                                          (2048, 64, (1, 5), kv.BUDGET_SKIP),
                                          (4097, 64, (1, 10), kv.BUDGET_SKIP),
                                          (100, 64, (1, 1), kv.BUDGET_AT_LEAST_ONE),
                                          (300, 16, (1, 5), kv.BUDGET_AT_LEAST_ONE),
                                          (2048, 1024, (1, 5), kv.BUDGET_AT_LEAST_ONE),
                                          (127, 64, (1, 5), kv.BUDGET_SKIP)])
def test_chunk_layout_matches_oracle(n, B, rho, rule):
    rows = 4
    x = draw_scores(7 * n + B, rows, n, "peaky")
    c = kv.kvfix_chunk_budget(n, B, rho[0], rho[1], rule)
    assert c == K.chunk_budget(n, B, rho[0], rho[1], "alg1" if rule == kv.BUDGET_SKIP else "table8")
    log("chunk layout", n, B, rho, rule, "chunks", c)
    m = gpu_means(x, B)
    cidx = gpu_topb(m, c)
    g_idx, g_counts, g_mask = gpu_expand(cidx, n, B)
    o_cidx, _ = K.select_topb(K.chunk_means(x, B), c)
    assert np.array_equal(cidx.cpu().numpy(), o_cidx)
    o_idx, o_counts, o_mask = K.expand_chunks(o_cidx, n, B)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_counts, o_counts)
    assert np.array_equal(g_mask, o_mask)


def test_expand_lists_in_order_and_skips_ids_out_of_range():
    n, B = 1000, 64                                      # 16 chunks, the last one 40 rows
    ids = np.array([[15, 3, -1, 0, 16], [7, 7, 15, 99, 2], [-5, -5, -5, -5, -5]], np.int32)
    log("expand", ids.tolist())
    g = gpu_expand(torch.from_numpy(ids).to(DEV), n, B)
    o = K.expand_chunks(ids, n, B)
    for a, b in zip(g, o):
        assert np.array_equal(a, b)
    # no chunks at all: counts 0, masks cleared
    g_idx, g_counts, g_mask = gpu_expand(torch.zeros((2, 0), dtype=torch.int32, device=DEV), n, B)
    assert g_idx.shape == (2, 0) and not g_counts.any() and not g_mask.any()


def test_coin_control_matches_oracle():
    n, B, rows = 4096, 64, 5
    c = kv.kvfix_chunk_budget(n, B, 1, 5, kv.BUDGET_SKIP)
    keys = draw_coin_keys(11, rows, -(-n // B), DEV)
    log("coin", n, B, c)
    cidx = gpu_topb(keys, c)
    g = gpu_expand(cidx, n, B)
    o_cidx, _ = K.select_topb(keys.cpu().numpy(), c)
    o = K.expand_chunks(o_cidx, n, B)
    for a, b in zip(g, o):
        assert np.array_equal(a, b)


GROW_CASES = [(1000, 100, 0.25), (5000, 500, 0.25), (3000, 3000, 0.25), (2048, 410, 0.0),
              (4096, 615, 1.5), (700, 1, 0.25), (700, 0, 0.25), (20000, 2000, 0.5),
              (32768, 3277, 0.25), (40000, 4000, 0.25)]


@pytest.mark.parametrize("kind", ["peaky", "flat", "ties"])
@pytest.mark.parametrize("n,b,tau", GROW_CASES)
def test_select_grow_matches_oracle(kind, n, b, tau):
    rows = 3
    x = draw_scores(n + b, rows, n, kind)
    log("grow", kind, n, b, tau)
    g_idx, g_mask = gpu_grow(x, b, tau)
    o_idx, o_mask = K.select_grow(x, b, tau)
    assert np.array_equal(g_idx, o_idx)
    assert np.array_equal(g_mask, o_mask)


def test_select_grow_nan_never_chosen_while_numbers_remain():
    n, b = 2000, 300
    x = draw_scores(5, 2, n, "peaky")
    x[:, ::7] = np.nan
    log("grow with NaN", n, b)
    g_idx, g_mask = gpu_grow(x, b, 0.25)
    # NaN ranks lowest and never joins a span: the oracle on -inf in its place
    o_idx, o_mask = K.select_grow(np.where(np.isnan(x), -np.inf, x).astype(np.float32), b, 0.25)
    assert np.array_equal(g_idx, o_idx) and np.array_equal(g_mask, o_mask)
    assert not np.isnan(x[0][g_idx[0]]).any()


def test_select_grow_deterministic():
    x = draw_scores(9, 4, 30000, "peaky")
    a = gpu_grow(x, 3000, 0.25)
    b = gpu_grow(x, 3000, 0.25)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_fit_mean_padding_matches_oracle():
    cfg = CONFIGS["c2"].replace(n_layers=2, n_kv_heads=2, n_tokens=100, b=0, rank=2)
    case = correction_case(cfg)
    n, B = cfg.n_tokens, 64                       # chunk 1 is short: 36 rows
    ids = np.array([[0, 1]], np.int32)
    idx, counts, mask = K.expand_chunks(ids, n, B)
    assert counts.tolist() == [100] and (idx == -1).sum() == 28
    t = {k: from_np(case[k], DEV) for k in ("reuse_k", "fresh_k")}
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV)
    A = torch.from_numpy(case["A_k"]).to(DEV)
    Bm = torch.from_numpy(case["B_k"]).to(DEV)
    out = torch.full_like(t["reuse_k"], float("nan"))
    mu = torch.full((cfg.n_layers, 1, cfg.n_kv_heads, cfg.head_dim), float("nan"),
                    dtype=torch.float32, device=DEV)
    g_idx = torch.from_numpy(idx).to(DEV)
    log("fit with padding")
    kv.kvfix_fit_mean(Plane.dense(t["fresh_k"]), Plane.dense(t["reuse_k"]), Plane.dense(out), g_idx,
                      idx.shape[1], mu, delta, cfg.theta, kv.ROPE_HALF, A, Bm)
    kv.kvfix_apply(Plane.dense(t["reuse_k"]), Plane.dense(out), torch.from_numpy(mask.view(np.int32)).to(DEV),
                   mu, None, 0.0, 1.0, delta, cfg.theta, kv.ROPE_HALF, A, Bm)
    torch.cuda.synchronize()
    o_mu = K.fit_mean(case["fresh_k"], case["reuse_k"], "bf16", idx, case["deltas"], cfg.theta,
                      "half", case["A_k"], case["B_k"])
    assert rel_err(mu.cpu().numpy(), o_mu, "f32") <= 1e-5
    # every row is a probe here: the output is the fresh plane, bit for bit
    assert np.array_equal(to_np(out), case["fresh_k"])
    # padding only: mu = 0
    pad = torch.full((1, 5), -1, dtype=torch.int32, device=DEV)
    kv.kvfix_fit_mean(Plane.dense(t["fresh_k"]), Plane.dense(t["reuse_k"]), None, pad, 5, mu, delta,
                      cfg.theta)
    torch.cuda.synchronize()
    assert not mu.cpu().numpy().any()


def test_chunk_layout_correction_end_to_end():
    """Chunk layout on the check-layer L2 scores of a small 8B-shaped case,
    then fit_mean over the padded rows and apply, against the oracle."""
    cfg = CONFIGS["c2"].replace(n_layers=3, n_kv_heads=2, n_tokens=1000, b=0)
    case = correction_case(cfg)
    L, S, H, n, hd = cfg.n_layers, 1, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim
    B = 64
    c = kv.kvfix_chunk_budget(n, B, 3, 20, kv.BUDGET_SKIP)        # r = 0.15 as in the 8B case
    t = {k: from_np(case[k], DEV) for k in ("reuse_k", "fresh_k")}
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV)
    A = torch.from_numpy(case["A_k"]).to(DEV)
    Bm = torch.from_numpy(case["B_k"]).to(DEV)
    scores = torch.empty(S, n, dtype=torch.float32, device=DEV)
    log("chunk correction", n, B, c)
    kv.kvfix_score(Plane.dense(t["fresh_k"]), cfg.check_layer, Plane.dense(t["reuse_k"]),
                   cfg.check_layer, scores, delta, cfg.theta)
    means = torch.empty(S, -(-n // B), dtype=torch.float32, device=DEV)
    kv.kvfix_chunk_means(scores, B, means)
    cidx = gpu_topb(means, c)
    idx = torch.empty(S, c * B, dtype=torch.int32, device=DEV)
    counts = torch.empty(S, dtype=torch.int32, device=DEV)
    mask = torch.empty(S, (n + 31) // 32, dtype=torch.int32, device=DEV)
    kv.kvfix_expand_chunks(cidx, n, B, idx, counts, mask)
    out = torch.empty_like(t["reuse_k"])
    mu = torch.empty(L, S, H, hd, dtype=torch.float32, device=DEV)
    kv.kvfix_fit_mean(Plane.dense(t["fresh_k"]), Plane.dense(t["reuse_k"]), Plane.dense(out), idx,
                      c * B, mu, delta, cfg.theta, kv.ROPE_HALF, A, Bm)
    kv.kvfix_apply(Plane.dense(t["reuse_k"]), Plane.dense(out), mask, mu, scores, cfg.w_lo, cfg.w_hi,
                   delta, cfg.theta, kv.ROPE_HALF, A, Bm)
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    o_idx, o_counts, o_mask = K.expand_chunks(K.select_topb(K.chunk_means(g_scores, B), c)[0], n, B)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), o_mask)
    o_out, _ = K.correct(case["fresh_k"], case["reuse_k"], "bf16", o_idx, o_mask, g_scores,
                         cfg.w_lo, cfg.w_hi, case["A_k"], case["B_k"], case["deltas"], cfg.theta)
    e = assert_values(to_np(out), o_out, "bf16", "chunk-layout correction")
    log("chunk correction rel err", e)

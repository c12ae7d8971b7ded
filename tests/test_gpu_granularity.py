"""GPU parity of the per-head probe sets and of the covered prefix (the _ex
calls) against the CPU oracle, plus the weight without scores.

Indices and masks bit-exact; scores within 2^-23 relative; values within
max |g - o| / (|o| + 1e-3) <= 8e-3 (bf16) or 1e-5 (fp32)."""
import numpy as np
import pytest
import torch

from helpers import assert_values, correction_case, from_np, log, rel_err, to_np
from oracle import kvref as K
from synthetic import CONFIGS

import cross_context_kv_amd.kvfix as kv
from cross_context_kv_amd.kvfix import Plane

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(**kw):
    base = dict(n_layers=3, n_kv_heads=4, n_tokens=300, n_segs=2, per_segment_delta=True)
    base.update(kw)
    base.setdefault("b", K.probe_budget(CONFIGS["c2"].ratio, base["n_tokens"]))
    return CONFIGS["c2"].replace(**base)


def ab(case, p):
    if case["A_" + p] is None:
        return None, None
    return torch.from_numpy(case["A_" + p]).to(DEV), torch.from_numpy(case["B_" + p]).to(DEV)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_head_chain_matches_oracle(dtype):
    cfg = small(dtype=dtype)
    case = correction_case(cfg)
    L, S, H, n, hd, b = cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, cfg.b
    words = (n + 31) // 32
    t = {k: from_np(case[k], DEV) for k in ("reuse_k", "reuse_v", "fresh_k", "fresh_v")}
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV)
    c = cfg.check_layer
    scores = torch.full((2, S, H, n), float("nan"), dtype=torch.float32, device=DEV)
    log("per-head score", dtype)
    kv.kvfix_score(Plane.dense(t["fresh_k"]), c, Plane.dense(t["reuse_k"]), c, scores[0], delta,
                   cfg.theta, per_head=True)
    kv.kvfix_score(Plane.dense(t["fresh_v"]), c, Plane.dense(t["reuse_v"]), c, scores[1],
                   per_head=True)
    idx = torch.full((2, S, H, b), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((2, S, H, words), -1, dtype=torch.int32, device=DEV)
    kv.kvfix_select_topb(scores.view(2 * S * H, n), b, idx.view(2 * S * H, b),
                         mask.view(2 * S * H, words))
    mu = torch.full((2, L, S, H, hd), float("nan"), dtype=torch.float32, device=DEV)
    outs = {}
    for pi, p in enumerate("kv"):
        out = torch.full_like(t["reuse_" + p], float("nan"))
        d = delta if p == "k" else None
        A, B = ab(case, p)
        log("per-head fit + apply", p)
        kv.kvfix_fit_mean(Plane.dense(t["fresh_" + p]), Plane.dense(t["reuse_" + p]),
                          Plane.dense(out), idx[pi], b, mu[pi], d, cfg.theta, kv.ROPE_HALF, A, B,
                          per_head=True)
        kv.kvfix_apply(Plane.dense(t["reuse_" + p]), Plane.dense(out), mask[pi], mu[pi],
                       scores[pi], cfg.w_lo, cfg.w_hi, d, cfg.theta, kv.ROPE_HALF, A, B,
                       per_head=True)
        outs[p] = out
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_mask = mask.cpu().numpy().view(np.uint32)
    for pi, p in enumerate("kv"):
        rope = (case["deltas"], cfg.theta) if p == "k" else (None, 0.0)
        o_s = K.score_l2(case["fresh_" + p], case["reuse_" + p], dtype, c, rope[0], rope[1],
                         per_head=True)
        err = np.abs(g_scores[pi].astype(np.float64) - o_s) / np.maximum(np.abs(o_s), 1e-30)
        assert err.max() <= 2.0 ** -23, (p, err.max())
        i1, m1 = K.select_topb(g_scores[pi].reshape(S * H, n), b)
        assert np.array_equal(g_idx[pi].reshape(S * H, b), i1)
        assert np.array_equal(g_mask[pi].reshape(S * H, words), m1)
        i2, _ = K.select_topb(o_s.reshape(S * H, n), b)
        assert np.array_equal(g_idx[pi].reshape(S * H, b), i2)
        o_mu = K.fit_mean(case["fresh_" + p], case["reuse_" + p], dtype, g_idx[pi], rope[0],
                          rope[1], "half", case["A_" + p], case["B_" + p], per_head=True)
        assert rel_err(mu[pi].cpu().numpy(), o_mu, "f32") <= 1e-5, p
        o_out, _ = K.correct(case["fresh_" + p], case["reuse_" + p], dtype, g_idx[pi], g_mask[pi],
                             o_s, cfg.w_lo, cfg.w_hi, case["A_" + p], case["B_" + p], rope[0],
                             rope[1], per_head=True)
        e = assert_values(to_np(outs[p]), o_out, dtype, f"per-head out {p}")
        log("per-head", dtype, p, "max rel err", e)


@pytest.mark.parametrize("rank", [0, 2, 4])
def test_cover_matches_oracle(rank):
    cfg = small(n_segs=5, rank=rank, weight="clip")
    case = correction_case(cfg)
    L, S, H, n, hd, b = cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, cfg.b
    cover = [150, 0, n, 10 ** 6, -3]               # inside, none, all, past n, negative
    rng = np.random.default_rng(rank)
    idx = np.stack([np.sort(rng.choice(n, b, replace=False)) for _ in range(S)]).astype(np.int32)
    mask = K.select_topb(np.zeros((S, n), np.float32), 0)[1]
    for s in range(S):
        for j in idx[s]:
            mask[s, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    sc = (rng.random((S, n)) * 3).astype(np.float32)
    t = {k: from_np(case[k], DEV) for k in ("reuse_k", "fresh_k")}
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV)
    A, B = ab(case, "k")
    out = torch.full_like(t["reuse_k"], float("nan"))
    mu = torch.full((L, S, H, hd), float("nan"), dtype=torch.float32, device=DEV)
    g_cover = torch.tensor(cover, dtype=torch.int32, device=DEV)
    log("cover", rank, cover)
    kv.kvfix_fit_mean(Plane.dense(t["fresh_k"]), Plane.dense(t["reuse_k"]), Plane.dense(out),
                      torch.from_numpy(idx).to(DEV), b, mu, delta, cfg.theta, kv.ROPE_HALF, A, B,
                      cover=g_cover)
    kv.kvfix_apply(Plane.dense(t["reuse_k"]), Plane.dense(out),
                   torch.from_numpy(mask.view(np.int32)).to(DEV), mu, torch.from_numpy(sc).to(DEV),
                   0.0, 2.0, delta, cfg.theta, kv.ROPE_HALF, A, B, cover=g_cover)
    torch.cuda.synchronize()
    o_out, o_mu = K.correct(case["fresh_k"], case["reuse_k"], "bf16", idx, mask, sc, 0.0, 2.0,
                            case["A_k"], case["B_k"], case["deltas"], cfg.theta, cover=cover)
    assert rel_err(mu.cpu().numpy(), o_mu, "f32") <= 1e-5
    e = assert_values(to_np(out), o_out, "bf16", "cover")
    log("cover max rel err", e)
    # past the covered prefix the rows are the rotary shift alone (apply rotates
    # bf16 rows in fp32 and the rotation-only call in fp64, each rounding once,
    # so the two agree within the bf16 tolerance rather than bit for bit)
    shifted = torch.empty_like(t["reuse_k"])
    kv.kvfix_rope_shift(Plane.dense(t["reuse_k"]), Plane.dense(shifted), delta, cfg.theta)
    torch.cuda.synchronize()
    g, r = to_np(out), to_np(shifted)
    for s in range(S):
        past = np.setdiff1d(np.arange(max(0, min(cover[s], n)), n), idx[s])
        assert_values(g[:, s][:, :, past], r[:, s][:, :, past], "bf16", f"past cover {s}")


def test_per_head_fresh_by_slot_matches_dense_fresh():
    cfg = small()
    case = correction_case(cfg)
    L, S, H, n, hd, b = cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, cfg.b
    rng = np.random.default_rng(5)
    idx = np.stack([np.stack([np.sort(rng.choice(n, b, replace=False)) for _ in range(H)])
                    for _ in range(S)]).astype(np.int32)
    fr = case["fresh_k"]
    compact = np.zeros((L, S, H, b, hd), dtype=fr.dtype)
    for s in range(S):
        for h in range(H):
            compact[:, s, h] = fr[:, s, h][:, idx[s, h]]
    t = {k: from_np(case[k], DEV) for k in ("reuse_k", "fresh_k")}
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV)
    g_idx = torch.from_numpy(idx).to(DEV)
    mus = []
    for fresh, by_slot in ((t["fresh_k"], False), (from_np(compact, DEV), True)):
        mu = torch.empty(L, S, H, hd, dtype=torch.float32, device=DEV)
        kv.kvfix_fit_mean(Plane.dense(fresh), Plane.dense(t["reuse_k"]), None, g_idx, b, mu, delta,
                          cfg.theta, fresh_by_slot=by_slot, per_head=True)
        mus.append(mu)
    torch.cuda.synchronize()
    assert torch.equal(mus[0], mus[1])


def test_no_scores_means_unit_weight_whatever_the_clip():
    cfg = small(n_segs=1)
    case = correction_case(cfg)
    L, S, H, n, hd = cfg.n_layers, 1, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim
    rng = np.random.default_rng(3)
    mu = (rng.standard_normal((L, S, H, hd)) * 0.5).astype(np.float32)
    t = from_np(case["reuse_v"], DEV)
    out = torch.empty_like(t)
    log("apply without scores, clip [0, 0.5]")
    kv.kvfix_apply(Plane.dense(t), Plane.dense(out), None, torch.from_numpy(mu).to(DEV), None,
                   0.0, 0.5)
    torch.cuda.synchronize()
    o = K.apply(case["reuse_v"], "bf16", None, mu)          # no scores: w = 1
    assert_values(to_np(out), o, "bf16", "w = 1 without scores")

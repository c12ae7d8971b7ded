"""GPU parity of the anchor-blended low-rank correction and the reliability
gate (KVCMAS eq. 8-11, App. A.3) against the CPU oracle.

Tolerances, from the arithmetic of the two sides:
  * token weights: |g - o| <= 2^-15.  A distance is a mean of absolute
    differences formed by the MFMA in fp32 (bf16 products are exact; 33
    roundings of at most 2^-24 (|x| + sum |a b|) each, about 1e-5 for unit
    data) and summed in fp32 (relative 1e-6); a softmax moves a weight by at
    most twice the largest distance error.
  * gate distances: relative 1e-4 (the same element errors, squared sums in
    fp32 per block, totals in fp64).  The decision is checked by running the
    oracle's decision rule on the GPU's distances (both in fp64).
  * corrected rows: the bf16 value bar, max |g - o| / (|o| + 1e-3) <= 8e-3,
    with the oracle run on the GPU's weights (a chain test).
"""
import math

import numpy as np
import pytest
import torch

from helpers import assert_values, from_np, log, to_np
from oracle import kvref as K
from synthetic import CONFIGS, draw_anchor_pool

import cross_context_kv_amd.kvfix as kv
from cross_context_kv_amd.kvfix import AnchorPool, Plane

pytestmark = pytest.mark.gpu
DEV = "cuda"
W_TOL = 2.0 ** -15
D_TOL = 1e-4
STYLES = {"half": kv.ROPE_HALF, "interleaved": kv.ROPE_INTERLEAVED}


def anchor_case(L=3, H=2, n=300, V=5, n_max=None, seed=61, src_off=1234, theta=5e5,
                style="half", device="cpu"):
    cfg = CONFIGS["c2"].replace(n_layers=L, n_kv_heads=H, n_tokens=n, seed=seed)
    raw = draw_anchor_pool(cfg, V, device, n_max=n_max)
    ck = raw["src_k"].double().cpu().numpy()
    cv = raw["src_v"].double().cpu().numpy()
    case = {k: to_np(raw[k]) for k in ("a_base", "bt_base", "a_delta", "bt_delta")}
    # keys are cached at positions src_off + j: the canonical content rotated forward
    case["src_k"] = K.store(K.rope_rotate(ck, src_off, theta, style), "bf16")
    case["src_v"] = K.store(cv, "bf16")
    case.update(L=L, H=H, n=n, V=V, src_off=src_off, theta=theta, style=style)
    return case


def gpu_match(case, lengths, k_gate, tau, src_k=None, src_v=None):
    L, n, V = case["L"], case["n"], case["V"]
    tk = from_np(case["src_k"], DEV) if src_k is None else None
    tv = from_np(case["src_v"], DEV) if src_v is None else None
    pk = Plane.dense(tk) if src_k is None else src_k
    pv = Plane.dense(tv) if src_v is None else src_v
    base = AnchorPool(from_np(case["a_base"], DEV), from_np(case["bt_base"], DEV), lengths)
    w = torch.full((L, 2, V, n), float("nan"), dtype=torch.float32, device=DEV)
    gate = torch.full((V + 1,), -1.0, dtype=torch.float64, device=DEV)
    acc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(kv.kvfix_anchor_match_workspace(L, case["H"], n, V), dtype=torch.uint8,
                     device=DEV)
    kv.kvfix_anchor_match(pk, pv, 0, base, case["src_off"], case["theta"], k_gate, tau, w, gate,
                          acc, ws, STYLES[case["style"]])
    torch.cuda.synchronize()
    return w, gate.cpu().numpy(), int(acc.item())


def gpu_apply(case, lengths, w, tgt_off):
    tk, tv = from_np(case["src_k"], DEV), from_np(case["src_v"], DEV)
    ok = torch.full_like(tk, float("nan"))
    ov = torch.full_like(tv, float("nan"))
    delta = AnchorPool(from_np(case["a_delta"], DEV), from_np(case["bt_delta"], DEV), lengths)
    kv.kvfix_anchor_apply(Plane.dense(tk), Plane.dense(tv), 0, delta, w, case["src_off"], tgt_off,
                          case["theta"], Plane.dense(ok), Plane.dense(ov), STYLES[case["style"]])
    torch.cuda.synchronize()
    return to_np(ok), to_np(ov)


def check_gate(case, lengths, k_gate, tau, g_gate, g_acc):
    o = K.anchor_gate(case["src_v"], case["a_base"], case["bt_base"], lengths, k_gate, tau, "bf16")
    V = case["V"]
    for v in range(V):
        if v in o["Ak"]:
            assert abs(g_gate[v] - o["d"][v]) <= D_TOL * max(o["d"][v], 1e-30) + 1e-12, \
                (v, g_gate[v], o["d"][v])
        else:
            assert math.isnan(g_gate[v]), (v, g_gate[v])
    dec = K.anchor_gate_decide(g_gate[o["Ak"]], tau)      # the rule on the GPU's distances
    if len(o["Ak"]) < 2:
        assert math.isnan(g_gate[V]) and g_acc == 0
        return o
    assert abs(g_gate[V] - dec["hbar"]) <= 1e-12, (g_gate[V], dec["hbar"])
    if abs(dec["hbar"] - tau) > 1e-12:
        assert g_acc == int(dec["accept"])
    return o


def weights_np(w):
    """GPU weights [L][2][V][n] -> the oracle's layout [L][2][n][V]."""
    return w.cpu().numpy().transpose(0, 1, 3, 2)


def check_weights(case, lengths, w):
    g = weights_np(w)
    o = K.anchor_weights(case["src_k"], case["src_v"], case["a_base"], case["bt_base"], lengths,
                         case["src_off"], case["theta"], case["style"], "bf16")
    err = np.abs(g.astype(np.float64) - o).max() if g.size else 0.0
    assert err <= W_TOL, err
    E, cover = K.anchor_eligible(lengths, case["n"])
    assert np.all(g[:, :, cover:] == 0)
    for v in range(case["V"]):
        if v not in E:
            assert np.all(g[..., v] == 0)
    if E and cover:
        assert np.abs(g[:, :, :cover].sum(axis=3) - 1).max() < 1e-5
    return err


def check_apply(case, lengths, w, tgt_off):
    gk, gv = gpu_apply(case, lengths, w, tgt_off)
    wn = weights_np(w).astype(np.float64)
    errs = []
    for plane, src, g in ((0, case["src_k"], gk), (1, case["src_v"], gv)):
        o = K.anchor_apply(src, plane, case["a_delta"], case["bt_delta"], wn, lengths,
                           case["src_off"], tgt_off, case["theta"], case["style"], "bf16")
        errs.append(assert_values(g, o, "bf16", f"anchor apply plane {plane}"))
    return errs


@pytest.mark.parametrize("H", [3, 4])
def test_odd_and_even_head_counts(H):
    """A match block takes two heads when the head count is even and one
    when it is odd: both against the oracle (weights, gate, apply)."""
    case = anchor_case(L=2, H=H, n=200, V=4, n_max=210, seed=67)
    lengths = [200, 210, 205, 200]
    log("anchor heads", H)
    w, gate, acc = gpu_match(case, lengths, 150, 0.5)
    check_weights(case, lengths, w)
    check_gate(case, lengths, 150, 0.5, gate, acc)
    check_apply(case, lengths, w, tgt_off=500)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_match_gate_and_apply_match_oracle(style):
    case = anchor_case(style=style, n_max=320)
    lengths = [300, 320, 310, 300, 320]
    log("anchor match", style)
    w, gate, acc = gpu_match(case, lengths, 200, 0.5)
    e = check_weights(case, lengths, w)
    check_gate(case, lengths, 200, 0.5, gate, acc)
    log("anchor apply", style, "weight err", e)
    errs = check_apply(case, lengths, w, tgt_off=777)
    log("anchor apply max rel err", errs)


def test_partial_cover_and_short_anchors():
    case = anchor_case(L=2, H=3, n=333, V=4, n_max=260, seed=62)
    lengths = [100, 250, 250, 40]            # E = {1, 2}, covered prefix 250
    for k_gate in (120, 50, 0):
        log("partial cover, k_gate", k_gate)
        w, gate, acc = gpu_match(case, lengths, k_gate, 0.9)
        check_weights(case, lengths, w)
        check_gate(case, lengths, k_gate, 0.9, gate, acc)
    check_apply(case, lengths, w, tgt_off=-500)


def test_gate_edge_cases():
    case = anchor_case(L=2, H=2, n=130, V=3, seed=63)
    n = case["n"]
    # one compared anchor: dense, NaN entropy
    w, gate, acc = gpu_match(case, [n, 10, 10], n, 1.0)
    check_gate(case, [n, 10, 10], n, 1.0, gate, acc)
    assert acc == 0 and math.isnan(gate[3]) and math.isnan(gate[1])
    # empty prefix: every anchor at distance 0, flat, accepted only at tau = 1
    w, gate, acc = gpu_match(case, [n] * 3, 0, 1.0)
    assert np.all(gate[:3] == 0) and abs(gate[3] - 1.0) < 1e-12 and acc == 1
    w, gate, acc = gpu_match(case, [n] * 3, 0, 0.999)
    assert acc == 0
    # k past the segment is the segment
    w, gate, acc = gpu_match(case, [n] * 3, 10 ** 9, 0.3)
    check_gate(case, [n] * 3, 10 ** 9, 0.3, gate, acc)


def test_no_eligible_anchor_only_realigns():
    case = anchor_case(L=2, H=2, n=100, V=2, seed=64)
    lengths = [0, 0]
    w, gate, acc = gpu_match(case, lengths, 50, 1.0)
    assert np.all(w.cpu().numpy() == 0) and acc == 0
    gk, gv = gpu_apply(case, lengths, None, tgt_off=4096)
    o = K.rope_shift(case["src_k"], "bf16", [4096 - case["src_off"]], case["theta"])
    assert_values(gk, o, "bf16", "realign only")
    assert np.array_equal(gv, case["src_v"])


def test_paged_source_and_in_place_apply():
    case = anchor_case(L=2, H=2, n=200, V=3, seed=65)
    L, H, n, hd = 2, 2, 200, 128
    lengths = [200, 200, 200]
    ps = 16
    pps = -(-n // ps)
    n_pages = pps + 5
    rng = np.random.default_rng(3)
    pt_np = rng.permutation(n_pages)[:pps].astype(np.int32)[None]
    pools = []
    for key in ("src_k", "src_v"):
        src = case[key][:, 0]                                   # [L, H, n, hd]
        pool = np.zeros((L, n_pages, ps, H, hd), dtype=np.uint16)
        for j in range(n):
            pool[:, pt_np[0, j // ps], j % ps] = src[:, :, j]
        pools.append(from_np(pool, DEV))
    pt = torch.from_numpy(pt_np).to(DEV)
    pk, pv = Plane.paged(pools[0], pt, ps, n), Plane.paged(pools[1], pt, ps, n)
    log("anchor match on a paged source")
    w_p, gate_p, acc_p = gpu_match(case, lengths, n, 0.5, src_k=pk, src_v=pv)
    w_d, gate_d, acc_d = gpu_match(case, lengths, n, 0.5)
    assert torch.equal(w_p, w_d) and np.array_equal(gate_p, gate_d) and acc_p == acc_d
    check_weights(case, lengths, w_d)
    # in place on the paged pool
    delta = AnchorPool(from_np(case["a_delta"], DEV), from_np(case["bt_delta"], DEV), lengths)
    kv.kvfix_anchor_apply(pk, pv, 0, delta, w_d, case["src_off"], 99, case["theta"], pk, pv)
    torch.cuda.synchronize()
    gk, gv = gpu_apply(case, lengths, w_d, 99)
    pk_np, pv_np = to_np(pools[0]), to_np(pools[1])
    for j in range(n):
        page = pt_np[0, j // ps]
        assert np.array_equal(pk_np[:, page, j % ps], gk[:, 0, :, j])
        assert np.array_equal(pv_np[:, page, j % ps], gv[:, 0, :, j])


@pytest.mark.parametrize("V", [1, 3, 16])
def test_list_lengths_and_ragged_tiles(V):
    """One, three and sixteen eligible anchors (the apply keeps three
    anchors' operands in a ring of LDS stages, so these reuse no stage, each
    once, and five times) over three token tiles of the apply, the last one
    ragged."""
    n = 600
    case = anchor_case(L=2, H=2, n=n, V=V, n_max=n, seed=70 + V)
    lengths = [n] * V
    log("anchor list length", V)
    w, gate, acc = gpu_match(case, lengths, n // 2, 0.5)
    check_weights(case, lengths, w)
    check_gate(case, lengths, n // 2, 0.5, gate, acc)
    check_apply(case, lengths, w, tgt_off=321)


def test_paged_one_token_pages_partial_cover():
    """A paged plane with one token per page (a tile spans 256 page ids) and
    a covered prefix that ends inside the first tile, so the second tile has
    no anchor work: in place on the pool against the dense apply."""
    case = anchor_case(L=2, H=2, n=300, V=3, n_max=300, seed=69)
    L, H, n, hd = 2, 2, 300, 128
    lengths = [150, 150, 90]                 # E = {0, 1}, covered prefix 150
    n_pages = n + 7
    rng = np.random.default_rng(9)
    pt_np = rng.permutation(n_pages)[:n].astype(np.int32)[None]
    pools = []
    for key in ("src_k", "src_v"):
        src = case[key][:, 0]                                   # [L, H, n, hd]
        pool = np.zeros((L, n_pages, 1, H, hd), dtype=np.uint16)
        pool[:, pt_np[0], 0] = src.transpose(0, 2, 1, 3)
        pools.append(from_np(pool, DEV))
    pt = torch.from_numpy(pt_np).to(DEV)
    pk, pv = Plane.paged(pools[0], pt, 1, n), Plane.paged(pools[1], pt, 1, n)
    log("anchor apply in place, one-token pages")
    w, gate, acc = gpu_match(case, lengths, 100, 0.5)
    check_weights(case, lengths, w)
    delta = AnchorPool(from_np(case["a_delta"], DEV), from_np(case["bt_delta"], DEV), lengths)
    kv.kvfix_anchor_apply(pk, pv, 0, delta, w, case["src_off"], 77, case["theta"], pk, pv)
    torch.cuda.synchronize()
    gk, gv = gpu_apply(case, lengths, w, 77)
    pk_np, pv_np = to_np(pools[0]), to_np(pools[1])
    assert np.array_equal(pk_np[:, pt_np[0], 0], gk[:, 0].transpose(0, 2, 1, 3))
    assert np.array_equal(pv_np[:, pt_np[0], 0], gv[:, 0].transpose(0, 2, 1, 3))
    check_apply(case, lengths, w, tgt_off=77)


def test_runs_are_bitwise_repeatable():
    case = anchor_case(L=2, H=2, n=257, V=4, seed=66)
    lengths = [257] * 4
    a = gpu_match(case, lengths, 257, 0.5)
    b = gpu_match(case, lengths, 257, 0.5)
    assert torch.equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(np.stack(gpu_apply(case, lengths, a[0], 5)),
                          np.stack(gpu_apply(case, lengths, a[0], 5)))


def test_llama3_8b_shape_ten_anchors_sampled():
    """The 8B-shaped segment (32 layers, 8 KV heads, 4096 tokens) with the
    pages' pool defaults, V = 10 and rank 32, in the benchmark's launch
    configuration.  Weights and corrected rows are checked on sampled layers
    and tokens against the oracle run on those rows alone (all anchors cover
    the segment, so a token's weights and rows depend only on that token);
    the gate distances against an fp64 evaluation of their definition."""
    cfg = CONFIGS["c2"]
    L, H, n, hd, V = cfg.n_layers, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim, 10
    src_off, tgt_off, theta = 3000, 5111, cfg.theta
    log("draw anchor pool, 8B shape")
    raw = draw_anchor_pool(cfg, V, DEV)
    # keys cached at src_off: canonical content rotated forward (in fp64 on the
    # device with the angles' definition; the library is not used for inputs)
    i = torch.arange(hd // 2, dtype=torch.float64, device=DEV)
    phi = src_off * theta ** (-2.0 * i / hd)
    c, s = torch.cos(phi).float(), torch.sin(phi).float()
    x = raw["src_k"]
    a_, b_ = x[..., : hd // 2], x[..., hd // 2:]
    src_k = torch.cat([a_ * c - b_ * s, b_ * c + a_ * s], dim=-1).to(torch.bfloat16)
    src_v = raw["src_v"].to(torch.bfloat16)
    del x, a_, b_
    lengths = [n] * V
    base = AnchorPool(raw["a_base"], raw["bt_base"], lengths)
    delta = AnchorPool(raw["a_delta"], raw["bt_delta"], lengths)
    w = torch.empty((L, 2, V, n), dtype=torch.float32, device=DEV)
    gate = torch.empty((V + 1,), dtype=torch.float64, device=DEV)
    acc = torch.empty((1,), dtype=torch.int32, device=DEV)
    ws = torch.empty(kv.kvfix_anchor_match_workspace(L, H, n, V), dtype=torch.uint8, device=DEV)
    out_k, out_v = torch.empty_like(src_k), torch.empty_like(src_v)
    log("anchor match + apply, 8B shape")
    kv.kvfix_anchor_match(Plane.dense(src_k), Plane.dense(src_v), 0, base, src_off, theta, n, 0.5,
                          w, gate, acc, ws)
    kv.kvfix_anchor_apply(Plane.dense(src_k), Plane.dense(src_v), 0, delta, w, src_off, tgt_off,
                          theta, Plane.dense(out_k), Plane.dense(out_v))
    torch.cuda.synchronize()
    # gate distances: fp64 evaluation of the definition, layer by layer
    d2 = torch.zeros(V, dtype=torch.float64, device=DEV)
    for l in range(L):
        xv = src_v[l, 0].double().transpose(0, 1).reshape(n, H * hd)
        for v in range(V):
            rec = raw["a_base"][v, l, 1].double() @ raw["bt_base"][v, l, 1].double().T
            d2[v] += ((xv - rec) ** 2).sum()
    g_gate = gate.cpu().numpy()
    d_ref = d2.sqrt().cpu().numpy()
    assert np.all(np.abs(g_gate[:V] - d_ref) <= D_TOL * d_ref), (g_gate[:V], d_ref)
    dec = K.anchor_gate_decide(g_gate[:V], 0.5)
    assert abs(g_gate[V] - dec["hbar"]) <= 1e-12 and int(acc.item()) == int(dec["accept"])
    log("gate", g_gate.tolist(), "accept", int(acc.item()))
    # sampled rows
    rng = np.random.default_rng(8)
    layers = [0, 17, L - 1]
    toks = np.sort(np.concatenate([rng.choice(n, 40, replace=False), [0, n - 1]]))
    sel = lambda t: to_np(t[layers][:, :, :, toks])                   # noqa: E731
    sk, sv = sel(src_k), sel(src_v)
    fac = {k: to_np(raw[k][:, layers][:, :, :, toks]) for k in ("a_base", "a_delta")}
    bt = {k: to_np(raw[k][:, layers]) for k in ("bt_base", "bt_delta")}
    m = len(toks)
    o_w = K.anchor_weights(sk, sv, fac["a_base"], bt["bt_base"], [m] * V, src_off, theta, "half",
                           "bf16")
    g_w = weights_np(w[layers][:, :, :, toks]).astype(np.float64)
    err = np.abs(g_w - o_w).max()
    log("8B-shape weights max abs err", err)
    assert err <= W_TOL
    for plane, src, out in ((0, sk, out_k), (1, sv, out_v)):
        o = K.anchor_apply(src, plane, fac["a_delta"], bt["bt_delta"], g_w, [m] * V, src_off,
                           tgt_off, theta, "half", "bf16")
        e = assert_values(sel(out), o, "bf16", f"8B-shape plane {plane}")
        log("8B-shape plane", plane, "max rel err", e)


def test_sixteen_anchors_and_single_token_segment():
    """The largest pool (16 anchors, lengths mixed around n) and a one-token
    segment (one ragged tile, every wave but one idle)."""
    case = anchor_case(L=2, H=3, n=129, V=16, n_max=140, seed=67)
    lengths = [129, 140, 135, 129, 60, 129, 140, 2, 129, 130, 131, 129, 129, 100, 140, 129]
    log("sixteen anchors")
    w, gate, acc = gpu_match(case, lengths, 100, 0.7)
    check_weights(case, lengths, w)
    check_gate(case, lengths, 100, 0.7, gate, acc)
    check_apply(case, lengths, w, tgt_off=31)
    one = anchor_case(L=1, H=1, n=1, V=2, n_max=4, seed=68)
    w, gate, acc = gpu_match(one, [1, 4], 1, 1.0)
    check_weights(one, [1, 4], w)
    check_gate(one, [1, 4], 1, 1.0, gate, acc)
    check_apply(one, [1, 4], w, tgt_off=7)

"""GPU parity of the draft attention-mass score (a3) and the block-sparse diff
encode / decode (a8, a9) against the CPU oracle."""
import numpy as np
import pytest
import torch

from helpers import assert_values, from_np, log, rel_err, to_np
from oracle import kvref as K
from synthetic import CONFIGS, draw_collective

import cross_context_kv_amd.kvfix as kv
from cross_context_kv_amd.kvfix import Plane

pytestmark = pytest.mark.gpu
DEV = "cuda"

# ----------------------------------------------------------------------------
# a3: draft attention mass
# ----------------------------------------------------------------------------


def draft_inputs(L, S, H, Hq, T, n, seed, theta, style="half"):
    rng = np.random.default_rng(seed)
    q = K.f64_to_bf16(rng.standard_normal((S, L, Hq, T, 128)))
    deltas = [int(d) for d in rng.integers(1, 32769, size=S)]
    x = rng.standard_normal((L, S, H, n, 128))
    k = K.store(K.align_plane_f64(x, [-d for d in deltas], theta, style), "bf16")
    return q, k, deltas


def gpu_draft(q, k, deltas, theta, first, style=kv.ROPE_HALF, paged=None):
    S, L, Hq, T, hd = q.shape
    n = k.shape[3]
    q_t = from_np(q, DEV)
    if paged is None:
        kp = Plane.dense(from_np(k, DEV))
    else:
        pool_t, pt_t, ps = paged
        kp = Plane.paged(pool_t, pt_t, ps, n)
    d = torch.tensor(deltas, dtype=torch.int64, device=DEV)
    ws = torch.empty(kv.kvfix_score_draft_workspace(S, L, first, Hq, T, n) // 4 + 64,
                     dtype=torch.float32, device=DEV)
    scores = torch.full((S, n), float("nan"), dtype=torch.float32, device=DEV)
    log("score_draft", q.shape, k.shape, first)
    kv.kvfix_score_draft(q_t, kp, first, d, theta, scores, ws, style)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def oracle_draft(q, k, deltas, theta, first, style="half"):
    S = q.shape[0]
    out = np.zeros((S, k.shape[3]), dtype=np.float32)
    for s in range(S):
        out[s] = K.score_draft(q[s], k[:, s:s + 1], [deltas[s]], theta, first, style)[0]
    return out


def check_selection(g_scores, o_scores, b):
    """Tier 1: selection on the GPU scores is the oracle's selection of them.
    Tier 2: end to end, it equals the oracle's selection of its own scores,
    bit for bit; any swap fails, with the oracle's scores on both sides of
    the b-th place printed."""
    gi = torch.empty(g_scores.shape[0], b, dtype=torch.int32, device=DEV)
    gm = torch.empty(g_scores.shape[0], (g_scores.shape[1] + 31) // 32, dtype=torch.int32,
                     device=DEV)
    kv.kvfix_select_topb(torch.from_numpy(g_scores).to(DEV), b, gi, gm)
    torch.cuda.synchronize()
    gi = gi.cpu().numpy()
    i1, m1 = K.select_topb(g_scores, b)
    assert np.array_equal(gi, i1)
    assert np.array_equal(gm.cpu().numpy().view(np.uint32), m1)
    i2, _ = K.select_topb(o_scores, b)
    for r in range(gi.shape[0]):
        srt = np.sort(o_scores[r].astype(np.float64))[::-1]
        gap = (srt[b - 1] - srt[b]) / srt[b - 1] if 0 < b < len(srt) else float("inf")
        log(f"selection row {r}: oracle relative gap at the b-th place {gap:.3g}")
        swapped = sorted(set(gi[r].tolist()) ^ set(i2[r].tolist()))
        assert not swapped, (r, swapped[:8], [float(o_scores[r, j]) for j in swapped[:8]],
                             float(srt[b - 1]), gap)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_draft_small_qwen_shape(style):
    L, S, H, Hq, T, n, theta = 4, 1, 2, 10, 2, 1100, 1e6
    q, k, deltas = draft_inputs(L, S, H, Hq, T, n, 51, theta, style)
    st = kv.ROPE_HALF if style == "half" else kv.ROPE_INTERLEAVED
    g = gpu_draft(q, k, deltas, theta, 1, st)
    o = oracle_draft(q, k, deltas, theta, 1, style)
    e = rel_err(g, o, "f32")
    log("draft rel err", e)
    assert e <= 1e-5
    assert abs(float(g.astype(np.float64).sum()) - (L - 1) * Hq * T) < 1e-3
    check_selection(g, o, K.probe_budget(0.1, n))


def test_draft_multi_segment_gqa_group_one_and_first_layer():
    L, S, H, Hq, T, n, theta = 3, 3, 4, 4, 2, 333, 5e5
    q, k, deltas = draft_inputs(L, S, H, Hq, T, n, 52, theta)
    for first in (0, 1, 2, 3):
        g = gpu_draft(q, k, deltas, theta, first)
        o = oracle_draft(q, k, deltas, theta, first)
        if first == L:
            assert not g.any()
        else:
            assert rel_err(g, o, "f32") <= 1e-5, first


def test_draft_paged_keys_equal_dense():
    L, S, H, Hq, T, n, theta, ps = 3, 2, 2, 6, 2, 96, 1e6, 16
    q, k, deltas = draft_inputs(L, S, H, Hq, T, n, 53, theta)
    rng = np.random.default_rng(54)
    n_pages = 17
    pt = rng.permutation(n_pages)[: S * n // ps].reshape(S, n // ps).astype(np.int32)
    pool = np.zeros(L * n_pages * ps * H * 128, dtype=np.uint16)
    K.paged_scatter(pool, k, pt, ps)
    pool_t = from_np(pool.reshape(L, n_pages, ps, H, 128), DEV)
    g_dense = gpu_draft(q, k, deltas, theta, 1)
    g_paged = gpu_draft(q, k, deltas, theta, 1,
                        paged=(pool_t, torch.from_numpy(pt).to(DEV), ps))
    assert np.array_equal(g_dense, g_paged)
    assert rel_err(g_paged, oracle_draft(q, k, deltas, theta, 1), "f32") <= 1e-5


def test_draft_deterministic():
    q, k, deltas = draft_inputs(3, 1, 2, 10, 2, 2048, 55, 1e6)
    a = gpu_draft(q, k, deltas, 1e6, 1)
    b = gpu_draft(q, k, deltas, 1e6, 1)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# a8 / a9: block-sparse diff
# ----------------------------------------------------------------------------


def collective_case(L=3, A=4, H=2, n=150, seed_cfg=None, style="half", dtype="bf16"):
    cfg = CONFIGS["c3"].replace(n_layers=L, n_segs=A, n_kv_heads=H, n_tokens=n)
    raw = draw_collective(cfg, "cpu")
    offs = [int(o) for o in raw["offsets"].tolist()]
    mk, mv = to_np(raw["master_k"]), to_np(raw["master_v"])
    yk, yv = to_np(raw["y_k"]), to_np(raw["y_v"])
    if dtype == "f32":
        mk, mv = K.bf16_to_f64(mk).astype(np.float32), K.bf16_to_f64(mv).astype(np.float32)
        yk, yv = K.bf16_to_f64(yk).astype(np.float32), K.bf16_to_f64(yv).astype(np.float32)
    sib_k = K.rope_shift(yk, dtype, offs, cfg.theta, style)
    return cfg, raw, offs, mk, mv, sib_k, yv


def gpu_encode(mk, mv, sk, sv, to_master, theta, eps, bt, capacity, style=kv.ROPE_HALF):
    L, A, H, n, hd = sk.shape
    t = {name: from_np(a, DEV) for name, a in (("mk", mk), ("mv", mv), ("sk", sk), ("sv", sv))}
    diff = kv.Diff(A, L, n, H, hd, bt, capacity, dtype=t["mk"].dtype)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    ws = torch.empty(kv.kvfix_diff_encode_workspace(A, L, n, bt) + 256, dtype=torch.uint8,
                     device=DEV)
    d = torch.tensor(to_master, dtype=torch.int64, device=DEV)
    log("diff_encode", sk.shape, bt, capacity)
    kv.kvfix_diff_encode(Plane.dense(t["mk"]), Plane.dense(t["mv"]), Plane.dense(t["sk"]),
                         Plane.dense(t["sv"]), d, theta, eps, diff, status, ws, style)
    torch.cuda.synchronize()
    return diff, int(status.item()), t


def gpu_decode(t, diff, from_master, theta, A, style=kv.ROPE_HALF):
    L, _, H, n, hd = t["mk"].shape
    ok = torch.full((L, A, H, n, hd), float("nan"), dtype=t["mk"].dtype, device=DEV)
    ov = torch.full_like(ok, float("nan"))
    ws = torch.empty(kv.kvfix_diff_decode_workspace(A, hd) + 256, dtype=torch.uint8, device=DEV)
    d = torch.tensor(from_master, dtype=torch.int64, device=DEV)
    log("diff_decode", (L, A, H, n, hd))
    kv.kvfix_diff_decode(Plane.dense(t["mk"]), Plane.dense(t["mv"]), diff, d, theta,
                         Plane.dense(ok), Plane.dense(ov), ws, style)
    torch.cuda.synchronize()
    return to_np(ok), to_np(ov)


def diff_np(diff):
    return {"mask": diff.mask.cpu().numpy().view(np.uint32),
            "offsets": diff.offsets.cpu().numpy(),
            "block_idx": diff.block_idx.cpu().numpy(),
            "vals_k": to_np(diff.vals_k), "vals_v": to_np(diff.vals_v)}


@pytest.mark.parametrize("style,dtype,hd_note", [("half", "bf16", ""), ("interleaved", "bf16", ""),
                                                 ("half", "f32", "")])
def test_diff_encode_decode_small_collective(style, dtype, hd_note):
    cfg, raw, offs, mk, mv, sk, sv = collective_case(style=style, dtype=dtype)
    A, L, bt, n = cfg.n_segs, cfg.n_layers, cfg.block_tokens, cfg.n_tokens
    st = kv.ROPE_HALF if style == "half" else kv.ROPE_INTERLEAVED
    o = K.diff_encode(mk, mv, sk, sv, [-x for x in offs], cfg.theta, cfg.eps, bt, style, dtype)
    diff, status, t = gpu_encode(mk, mv, sk, sv, [-x for x in offs], cfg.theta, cfg.eps, bt,
                                 o["total"] + 5, st)
    assert status == 0
    g = diff_np(diff)
    assert np.array_equal(g["mask"], o["mask"])
    assert np.array_equal(g["offsets"], o["offsets"])
    tot = o["total"]
    assert np.array_equal(g["block_idx"][:tot], o["block_idx"])
    # planted blocks recovered exactly, at every layer
    nb = -(-n // bt)
    for a in range(A):
        for l in range(L):
            assert [K.mask_bit(o["mask"][a, l], b) for b in range(nb)] == raw["planted"][a].tolist()
    # packed values: compare valid rows of each block
    for slot in range(tot):
        beta = o["block_idx"][slot]
        tb = min(bt, n - beta * bt)
        assert_values(g["vals_k"][slot][:, :tb], o["vals_k"][slot][:, :tb], dtype, "vals_k")
        assert np.array_equal(g["vals_v"][slot][:, :tb], o["vals_v"][slot][:, :tb])
    # decode against the oracle's decode of the same (GPU) diff
    ok, ov = gpu_decode(t, diff, offs, cfg.theta, A, st)
    gd = dict(g)
    ook, oov = K.diff_decode(mk, mv, gd, offs, cfg.theta, A, bt, style, dtype)
    assert_values(ok, ook, dtype, "decode K")
    assert np.array_equal(ov, oov)
    assert np.mean(ok == ook) > 0.999
    # the restored caches are the siblings: values exactly, keys within the
    # two roundings of a rotation there and back (fp32 storage: a few float
    # ulps of the largest element, an absolute bound)
    assert np.array_equal(ov, sv)
    if dtype == "f32":
        assert np.abs(ok.astype(np.float64) - sk).max() <= 8 * 2.0 ** -24 * np.abs(sk).max()


# listed agents per block of the decode's mixes below: every agent, none,
# two, only the first, and three across the boundary of the first 16-agent
# group (the last block is ragged: 11 of 16 tokens)
LISTED_MIX = {0: list(range(19)), 1: [], 2: [3, 11], 3: [0], 4: [15, 16, 18]}


@pytest.mark.parametrize("hd,dtype,style", [(128, "bf16", "half"), (64, "bf16", "interleaved"),
                                            (256, "bf16", "half"), (128, "f32", "half"),
                                            (64, "f32", "half"), (256, "f32", "interleaved")])
def test_diff_decode_listed_block_mixes(hd, dtype, style):
    rng = np.random.default_rng(83 + hd)
    L, A, H, n, bt, theta, eps = 2, 19, 3, 75, 16, 1e4, 0.0625
    offs = [int(o) for o in rng.integers(0, 16385, size=A)]
    master_k = K.store(rng.standard_normal((L, 1, H, n, hd)), dtype)
    master_v = K.store(rng.standard_normal((L, 1, H, n, hd)), dtype)
    yk = np.repeat(K.to_f64(master_k, dtype), A, axis=1)
    yv = np.repeat(K.to_f64(master_v, dtype), A, axis=1)
    for beta, agents in LISTED_MIX.items():
        tb = min(bt, n - beta * bt)
        for a in agents:
            for l in range(L):
                h, t, d = rng.integers(H), beta * bt + rng.integers(tb), rng.integers(hd)
                yk[l, a, h, t, d] += 1.0
                yv[l, a, h, (t + 1 - beta * bt) % tb + beta * bt, d] -= 1.0
    sk = K.rope_shift(K.store(yk, dtype), dtype, offs, theta, style)
    sv = K.store(yv, dtype)
    st = kv.ROPE_HALF if style == "half" else kv.ROPE_INTERLEAVED
    o = K.diff_encode(master_k, master_v, sk, sv, [-x for x in offs], theta, eps, bt, style,
                      dtype)
    for a in range(A):
        for l in range(L):
            listed = [b for b in range(5) if K.mask_bit(o["mask"][a, l], b)]
            assert listed == [b for b, ag in LISTED_MIX.items() if a in ag]
    diff, status, t = gpu_encode(master_k, master_v, sk, sv, [-x for x in offs], theta, eps, bt,
                                 o["total"] + 5, st)
    assert status == 0
    g = diff_np(diff)
    assert np.array_equal(g["mask"], o["mask"])
    assert np.array_equal(g["offsets"], o["offsets"])
    ok, ov = gpu_decode(t, diff, offs, theta, A, st)
    ook, oov = K.diff_decode(master_k, master_v, g, offs, theta, A, bt, style, dtype)
    assert_values(ok, ook, dtype, "decode K")
    assert np.array_equal(ov, oov)
    assert np.array_equal(ov, sv)
    # the same restore into a paged pool (its rows addressed through the
    # slot mapping, the master's loaded in place): equal bit for bit
    ps = 16
    pps = -(-n // ps)
    n_pages = A * pps + 3
    pt_np = np.random.default_rng(hd).permutation(n_pages)[: A * pps].reshape(A, pps)
    pt = torch.from_numpy(pt_np.astype(np.int32)).to(DEV)
    pool_k = torch.full((L, n_pages, ps, H, hd), float("nan"), dtype=t["mk"].dtype, device=DEV)
    pool_v = torch.full_like(pool_k, float("nan"))
    ws = torch.empty(kv.kvfix_diff_decode_workspace(A, hd) + 256, dtype=torch.uint8, device=DEV)
    d = torch.tensor(offs, dtype=torch.int64, device=DEV)
    log("diff_decode paged", (L, A, H, n, hd))
    kv.kvfix_diff_decode(Plane.dense(t["mk"]), Plane.dense(t["mv"]), diff, d, theta,
                         Plane.paged(pool_k, pt, ps, n), Plane.paged(pool_v, pt, ps, n), ws, st)
    torch.cuda.synchronize()
    tok = np.arange(n)
    for pool, dense in ((pool_k, ok), (pool_v, ov)):
        rows = to_np(pool)[:, pt_np[:, tok // ps], tok % ps]         # [L][A][n][H][hd]
        assert np.array_equal(rows.transpose(0, 1, 3, 2, 4), dense)


@pytest.mark.parametrize("bt,n", [(1, 9), (7, 50), (32, 97), (64, 130)])
def test_diff_block_sizes(bt, n):
    """Encode and restore with block sizes from one token to the largest,
    ragged tails, about a third of the (agent, layer, block) triples listed."""
    rng = np.random.default_rng(1000 + bt)
    L, A, H, hd, theta, eps = 2, 5, 2, 128, 1e4, 0.0625
    nb = -(-n // bt)
    offs = [int(o) for o in rng.integers(0, 16385, size=A)]
    master_k = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    master_v = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    yk = np.repeat(K.to_f64(master_k, "bf16"), A, axis=1)
    yv = np.repeat(K.to_f64(master_v, "bf16"), A, axis=1)
    planted = rng.random((A, L, nb)) < 0.35
    for a, l, beta in zip(*np.nonzero(planted)):
        t = beta * bt + rng.integers(min(bt, n - beta * bt))
        if rng.random() < 0.5:
            yk[l, a, rng.integers(H), t, rng.integers(hd)] += 1.0
        else:
            yv[l, a, rng.integers(H), t, rng.integers(hd)] -= 1.0
    sk = K.rope_shift(K.store(yk, "bf16"), "bf16", offs, theta)
    sv = K.store(yv, "bf16")
    o = K.diff_encode(master_k, master_v, sk, sv, [-x for x in offs], theta, eps, bt)
    for a in range(A):
        for l in range(L):
            assert [K.mask_bit(o["mask"][a, l], b) for b in range(nb)] == planted[a, l].tolist()
    diff, status, t = gpu_encode(master_k, master_v, sk, sv, [-x for x in offs], theta, eps, bt,
                                 o["total"] + 2)
    assert status == 0
    g = diff_np(diff)
    assert np.array_equal(g["mask"], o["mask"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["block_idx"][: o["total"]], o["block_idx"])
    ok, ov = gpu_decode(t, diff, offs, theta, A)
    ook, oov = K.diff_decode(master_k, master_v, g, offs, theta, A, bt)
    assert_values(ok, ook, "bf16", "decode K")
    assert np.array_equal(ov, oov) and np.array_equal(ov, sv)


def test_diff_lossless_roundtrip_zero_shift_zero_eps():
    rng = np.random.default_rng(61)
    L, A, H, n, hd, bt = 2, 3, 2, 37, 128, 16
    mk = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    mv = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    sk, sv = np.repeat(mk, A, axis=1), np.repeat(mv, A, axis=1)
    sk[1, 0, 1, 5, 3] ^= 1
    sv[0, 2, 0, 36, 0] ^= 4
    diff, status, t = gpu_encode(mk, mv, sk, sv, [0] * A, 1e4, 0.0, bt, 8)
    assert status == 0
    g = diff_np(diff)
    assert g["offsets"].tolist() == [0, 0, 1, 1, 1, 2, 2]
    assert g["block_idx"][:2].tolist() == [0, 2]
    ok, ov = gpu_decode(t, diff, [0] * A, 1e4, A)
    assert np.array_equal(ok, sk) and np.array_equal(ov, sv)


def test_diff_capacity_overflow_reports_and_stays_in_bounds():
    cfg, raw, offs, mk, mv, sk, sv = collective_case()
    o = K.diff_encode(mk, mv, sk, sv, [-x for x in offs], cfg.theta, cfg.eps, 16)
    cap = o["total"] - 3
    assert cap > 0
    diff, status, t = gpu_encode(mk, mv, sk, sv, [-x for x in offs], cfg.theta, cfg.eps, 16, cap)
    assert status == 3                                   # KVFIX_ERR_CAPACITY
    g = diff_np(diff)
    assert np.array_equal(g["mask"], o["mask"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["block_idx"][:cap], o["block_idx"][:cap])
    # decode restores the slots past the capacity from the master
    ok, ov = gpu_decode(t, diff, offs, cfg.theta, cfg.n_segs)
    gd = diff_np(diff)
    for a in range(cfg.n_segs):
        for l in range(cfg.n_layers):
            slot = int(gd["offsets"][a * cfg.n_layers + l])
            for beta in range(-(-cfg.n_tokens // 16)):
                if K.mask_bit(gd["mask"][a, l], beta):
                    if slot >= cap:
                        t0, t1 = beta * 16, min(cfg.n_tokens, beta * 16 + 16)
                        assert np.array_equal(ov[l, a][:, t0:t1], mv[l, 0][:, t0:t1])
                    slot += 1


def test_diff_empty_group_is_ok():
    mk = np.zeros((2, 1, 2, 0, 128), dtype=np.uint16)
    diff, status, _ = gpu_encode(mk, mk, np.zeros((2, 3, 2, 0, 128), dtype=np.uint16),
                                 np.zeros((2, 3, 2, 0, 128), dtype=np.uint16), [0, 0, 0], 1e4,
                                 0.0625, 16, 4)
    assert status == 0
    assert not diff.offsets.cpu().numpy().any()

"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Inputs are drawn on the GPU (seeded torch generators; stored
keys rotated with plain torch ops), copied to the host, and compared with the
oracle: whole planes where the oracle finishes in seconds (the 8B-shaped
cache), otherwise every index and mask plus a seeded sample of layers for
the values, and properties that hold at any size."""
import numpy as np
import pytest
import torch

from helpers import correction_case_gpu, log
from test_gpu_correct import check_chain, gpu_chain
from synthetic import CONFIGS

pytestmark = pytest.mark.gpu


def test_c2_llama3_8b_full_size_whole_planes():
    cfg = CONFIGS["c2"]
    log("c2 full: drawing inputs on the GPU")
    case = correction_case_gpu(cfg)
    log("c2 full: GPU chain")
    g = gpu_chain(cfg, case)
    log("c2 full: oracle comparison")
    rep = check_chain(cfg, case, g)
    log("c2 full:", rep)


# ----------------------------------------------------------------------------
# Llama-3-70B-shaped paged batch: 80 layers x 32 segments x 4096 tokens,
# corrected in place through the page tables (40 GiB of pool per call pair).
# ----------------------------------------------------------------------------


def _pool_gather(pool_l, pt, H, n, hd):
    """Logical plane [S][H][n][hd] of one layer of a paged pool [pages][ps][H][hd]."""
    S = pt.shape[0]
    return pool_l[pt.long()].reshape(S, n, H, hd).permute(0, 2, 1, 3)


def _pool_scatter(pool_l, pt, plane):
    S, H, n, hd = plane.shape
    pool_l[pt.long()] = plane.permute(0, 2, 1, 3).reshape(S, pt.shape[1], -1, H, hd)


def test_c5_llama3_70b_paged_in_place_full_size():
    from helpers import to_np, torch_rotate, assert_values, rel_err
    from oracle import kvref as K
    from synthetic import draw_correction, draw_page_table, draw_deltas
    import cross_context_kv_amd.kvfix as kv
    from cross_context_kv_amd.kvfix import Plane
    cfg = CONFIGS["c5"]
    L, S, H, n, hd, ps, NP, b, c = (cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens,
                                    cfg.head_dim, cfg.page_size, cfg.n_pages, cfg.b,
                                    cfg.check_layer)
    sample = [0, c, 11, 25, 40, 53, 66, L - 1]          # eight layers, every segment and head
    deltas = [int(d) for d in draw_deltas(cfg).tolist()]
    neg = [-d for d in deltas]
    dev = "cuda"
    pt = draw_page_table(cfg, dev)
    assert pt.shape == (S, n // ps)
    pools = {p: torch.empty(L, NP, ps, H, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    A = {p: torch.empty(L, S, H, n, cfg.rank, dtype=torch.float32, device=dev) for p in "kv"}
    B = {p: torch.empty(L, S, H, cfg.rank, hd, dtype=torch.float32, device=dev) for p in "kv"}
    before, fresh_check = {}, {}
    log("c5 full: drawing 80 layers into the paged pools")
    for l in range(L):
        raw = draw_correction(cfg, dev, layers=[l])
        for p in "kv":
            x = raw["x_" + p][0]
            stored = (torch_rotate(x, neg, cfg.theta) if p == "k" else x).to(torch.bfloat16)
            _pool_scatter(pools[p][l], pt, stored)
            A[p][l] = raw["a_" + p][0]
            B[p][l] = raw["b_" + p][0]
            if l == c:
                fresh_check[p] = raw["fresh_" + p]
            if l in sample:
                before[(p, l)] = to_np(stored)
        del raw
    d_t = torch.tensor(deltas, dtype=torch.int64, device=dev)
    planes = {p: Plane.paged(pools[p], pt, ps, n) for p in "kv"}
    scores = torch.empty(2, S, n, dtype=torch.float32, device=dev)
    log("c5 full: scores at the check layer, selection")
    kv.kvfix_score(Plane.dense(fresh_check["k"]), 0, planes["k"], c, scores[0], d_t, cfg.theta)
    kv.kvfix_score(Plane.dense(fresh_check["v"]), 0, planes["v"], c, scores[1])
    idx = torch.empty(2, S, b, dtype=torch.int32, device=dev)
    mask = torch.empty(2, S, (n + 31) // 32, dtype=torch.int32, device=dev)
    kv.kvfix_select_topb(scores.view(2 * S, n), b, idx.view(2 * S, b), mask.view(2 * S, -1))
    torch.cuda.synchronize()
    # fresh rows of the selected probes, for every layer (fresh indexed by slot)
    log("c5 full: fresh probe rows of every layer")
    fslot = {p: torch.empty(L, S, H, b, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    for l in range(L):
        raw = draw_correction(cfg, dev, layers=[l])
        for pi, p in enumerate("kv"):
            f = raw["fresh_" + p][0]                                   # [S][H][n][hd]
            gi = idx[pi].long()[:, None, :, None].expand(S, H, b, hd)
            fslot[p][l] = torch.gather(f, 2, gi)
        del raw
    mu = torch.empty(2, L, S, H, hd, dtype=torch.float32, device=dev)
    log("c5 full: fit_mean + apply in place, K and V")
    for pi, p in enumerate("kv"):
        d = d_t if p == "k" else None
        kv.kvfix_fit_mean(Plane.dense(fslot[p]), planes[p], planes[p], idx[pi], b, mu[pi], d,
                          cfg.theta, A=A[p], B=B[p], fresh_by_slot=True)
        kv.kvfix_apply(planes[p], planes[p], mask[pi], mu[pi], None, 0.0, 1.0, d, cfg.theta,
                       A=A[p], B=B[p])
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_mask = mask.cpu().numpy().view(np.uint32)
    # scores and selection over all 32 segments
    log("c5 full: oracle scores")
    for pi, p in enumerate("kv"):
        fc = to_np(fresh_check[p])
        rc = before[(p, c)][None]
        o_s = K.score_l2(fc, rc, "bf16", 0, deltas if p == "k" else None, cfg.theta)
        err = np.abs(g_scores[pi].astype(np.float64) - o_s) / np.maximum(np.abs(o_s), 1e-30)
        assert err.max() <= 2.0 ** -23, (p, err.max())
        i1, m1 = K.select_topb(g_scores[pi], b)
        assert np.array_equal(g_idx[pi], i1) and np.array_equal(g_mask[pi], m1)
        i2, _ = K.select_topb(o_s, b)
        assert np.array_equal(g_idx[pi], i2), p
    # values on the sampled layers, every segment and head
    for l in sample:
        for pi, p in enumerate("kv"):
            log("c5 full: oracle layer", l, p)
            rope = (deltas, cfg.theta, "half") if p == "k" else (None, 0.0, "half")
            fs = to_np(fslot[p][l])[None]
            Al, Bl = A[p][l].cpu().numpy()[None], B[p][l].cpu().numpy()[None]
            o_mu = K.fit_mean(fs, before[(p, l)][None], "bf16", g_idx[pi], rope[0], rope[1],
                              rope[2], Al, Bl, True)
            assert rel_err(mu[pi, l].cpu().numpy()[None], o_mu, "f32") <= 1e-5, (l, p)
            after = to_np(_pool_gather(pools[p][l], pt, H, n, hd))[None]
            o_out, _ = K.correct(fs, before[(p, l)][None], "bf16", g_idx[pi], g_mask[pi], None,
                                 0.0, 1.0, Al, Bl, rope[0], rope[1], rope[2], True)
            e = assert_values(after, o_out, "bf16", f"c5 layer {l} {p}")
            for s in range(S):
                assert np.array_equal(after[0, s][:, g_idx[pi, s]], fs[0, s])
            log("c5 full: layer", l, p, "max rel err", e)


# ----------------------------------------------------------------------------
# Qwen2.5-14B-shaped draft-selected repair: 48 layers, 40 query / 8 KV heads,
# 32768 tokens; one probe set from the draft attention mass for both planes.
# ----------------------------------------------------------------------------


def test_c4_qwen25_14b_draft_full_size():
    from helpers import to_np, torch_rotate, assert_values, rel_err
    from oracle import kvref as K
    from synthetic import draw_correction, draw_draft_queries, draw_deltas
    from test_gpu_draft_diff import check_selection
    import cross_context_kv_amd.kvfix as kv
    from cross_context_kv_amd.kvfix import Plane
    cfg = CONFIGS["c4"]
    L, S, H, Hq, T, n, hd, b = (cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_q_heads,
                                cfg.n_draft, cfg.n_tokens, cfg.head_dim, cfg.b)
    dev = "cuda"
    deltas = [int(d) for d in draw_deltas(cfg).tolist()]
    sample = [0, cfg.first_layer, 12, 23, 35, L - 1]          # six layers, every head
    reuse = {p: torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    fresh = {p: torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    log("c4 full: drawing 48 layers")
    for l in range(L):
        raw = draw_correction(cfg, dev, layers=[l])
        reuse["k"][l] = torch_rotate(raw["x_k"][0], [-d for d in deltas], cfg.theta).to(
            torch.bfloat16)
        reuse["v"][l] = raw["x_v"][0].to(torch.bfloat16)
        fresh["k"][l] = raw["fresh_k"][0]
        fresh["v"][l] = raw["fresh_v"][0]
        del raw
    q = draw_draft_queries(cfg, dev)[None].contiguous()                # [S][L][Hq][T][hd]
    d_t = torch.tensor(deltas, dtype=torch.int64, device=dev)
    ws = torch.empty(kv.kvfix_score_draft_workspace(S, L, cfg.first_layer, Hq, T, n) // 4 + 64,
                     dtype=torch.float32, device=dev)
    scores = torch.empty(S, n, dtype=torch.float32, device=dev)
    log("c4 full: draft score, selection, fit_mean + apply")
    kv.kvfix_score_draft(q, Plane.dense(reuse["k"]), cfg.first_layer, d_t, cfg.theta, scores, ws)
    idx = torch.empty(S, b, dtype=torch.int32, device=dev)
    mask = torch.empty(S, (n + 31) // 32, dtype=torch.int32, device=dev)
    kv.kvfix_select_topb(scores, b, idx, mask)
    out = {p: torch.empty_like(reuse[p]) for p in "kv"}
    mu = torch.empty(2, L, S, H, hd, dtype=torch.float32, device=dev)
    for pi, p in enumerate("kv"):
        d = d_t if p == "k" else None
        kv.kvfix_fit_mean(Plane.dense(fresh[p]), Plane.dense(reuse[p]), Plane.dense(out[p]), idx,
                          b, mu[pi], d, cfg.theta)
        kv.kvfix_apply(Plane.dense(reuse[p]), Plane.dense(out[p]), mask, mu[pi], None, 0.0, 1.0,
                       d, cfg.theta)
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_mask = mask.cpu().numpy().view(np.uint32)
    # every softmax sums to one: the masses add up to (L - first) Hq T
    total = float(g_scores.astype(np.float64).sum())
    assert abs(total - (L - cfg.first_layer) * Hq * T) <= 1e-5 * (L - cfg.first_layer) * Hq * T
    # the oracle's draft score over all 47 layers
    log("c4 full: oracle draft score")
    k_host = to_np(reuse["k"])
    o_scores = K.score_draft(to_np(q[0]), k_host, deltas, cfg.theta, cfg.first_layer)
    e = rel_err(g_scores, o_scores, "f32")
    log("c4 full: draft rel err", e)
    assert e <= 1e-5
    i1, m1 = K.select_topb(g_scores, b)
    assert np.array_equal(g_idx, i1) and np.array_equal(g_mask, m1)
    check_selection(g_scores, o_scores, b)
    del k_host
    for l in sample:
        for pi, p in enumerate("kv"):
            log("c4 full: oracle layer", l, p)
            rope = (deltas, cfg.theta, "half") if p == "k" else (None, 0.0, "half")
            fr, ru = to_np(fresh[p][l:l + 1]), to_np(reuse[p][l:l + 1])
            o_mu = K.fit_mean(fr, ru, "bf16", g_idx, rope[0], rope[1], rope[2], None, None)
            assert rel_err(mu[pi, l:l + 1].cpu().numpy(), o_mu, "f32") <= 1e-5, (l, p)
            o_out, _ = K.correct(fr, ru, "bf16", g_idx, g_mask, None, 0.0, 1.0, None, None,
                                 rope[0], rope[1], rope[2])
            e = assert_values(to_np(out[p][l:l + 1]), o_out, "bf16", f"c4 layer {l} {p}")
            log("c4 full: layer", l, p, "max rel err", e)


def test_c4_bcr_layouts_full_size():
    """The BCR layouts on the Qwen-14B-shaped draft scores (32768 tokens):
    64-token chunks at r = 0.1 (51 chunks), the coin at the same budget, and
    grown spans (b = 3277, tau = 0.25), each bit-exact against the oracle on
    the GPU's scores; then the chunk-layout and grow-layout corrections of all
    48 layers, checked on sampled layers."""
    from helpers import to_np, torch_rotate, assert_values, rel_err
    from oracle import kvref as K
    from synthetic import draw_correction, draw_draft_queries, draw_deltas
    from synthetic.workloads import draw_coin_keys
    import cross_context_kv_amd.kvfix as kv
    from cross_context_kv_amd.kvfix import Plane
    cfg = CONFIGS["c4"]
    L, S, H, Hq, T, n, hd, b = (cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_q_heads,
                                cfg.n_draft, cfg.n_tokens, cfg.head_dim, cfg.b)
    B, tau = 64, 0.25
    dev = "cuda"
    deltas = [int(d) for d in draw_deltas(cfg).tolist()]
    reuse = {p: torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    fresh = {p: torch.empty(L, S, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    log("c4 bcr: drawing 48 layers")
    for l in range(L):
        raw = draw_correction(cfg, dev, layers=[l])
        reuse["k"][l] = torch_rotate(raw["x_k"][0], [-d for d in deltas], cfg.theta).to(
            torch.bfloat16)
        reuse["v"][l] = raw["x_v"][0].to(torch.bfloat16)
        fresh["k"][l] = raw["fresh_k"][0]
        fresh["v"][l] = raw["fresh_v"][0]
        del raw
    q = draw_draft_queries(cfg, dev)[None].contiguous()
    d_t = torch.tensor(deltas, dtype=torch.int64, device=dev)
    ws = torch.empty(kv.kvfix_score_draft_workspace(S, L, cfg.first_layer, Hq, T, n) // 4 + 64,
                     dtype=torch.float32, device=dev)
    scores = torch.empty(S, n, dtype=torch.float32, device=dev)
    log("c4 bcr: draft score and the three layouts")
    kv.kvfix_score_draft(q, Plane.dense(reuse["k"]), cfg.first_layer, d_t, cfg.theta, scores, ws)
    nc = n // B
    c = kv.kvfix_chunk_budget(n, B, 1, 10, kv.BUDGET_SKIP)
    assert c == K.chunk_budget(n, B, 1, 10, "alg1") == 51
    words = (n + 31) // 32

    def chunk_rows(keys):
        cidx = torch.empty(S, c, dtype=torch.int32, device=dev)
        cmask = torch.empty(S, (nc + 31) // 32, dtype=torch.int32, device=dev)
        kv.kvfix_select_topb(keys, c, cidx, cmask)
        idx = torch.empty(S, c * B, dtype=torch.int32, device=dev)
        counts = torch.empty(S, dtype=torch.int32, device=dev)
        mask = torch.empty(S, words, dtype=torch.int32, device=dev)
        kv.kvfix_expand_chunks(cidx, n, B, idx, counts, mask)
        return idx, counts, mask

    means = torch.empty(S, nc, dtype=torch.float32, device=dev)
    kv.kvfix_chunk_means(scores, B, means)
    layouts = {"chunk": chunk_rows(means)}
    keys = draw_coin_keys(cfg.seed, S, nc, dev)
    layouts["coin"] = chunk_rows(keys)
    g_idx = torch.empty(S, b, dtype=torch.int32, device=dev)
    g_mask = torch.empty(S, words, dtype=torch.int32, device=dev)
    kv.kvfix_select_grow(scores, b, tau, g_idx, g_mask)
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    o_means = K.chunk_means(g_scores, B)
    assert np.array_equal(means.cpu().numpy().view(np.uint32), o_means.view(np.uint32))
    for name, ks in (("chunk", o_means), ("coin", keys.cpu().numpy())):
        o = K.expand_chunks(K.select_topb(ks, c)[0], n, B)
        got = [t.cpu().numpy() for t in layouts[name]]
        got[2] = got[2].view(np.uint32)
        for a, e in zip(got, o):
            assert np.array_equal(a, e), name
        log("c4 bcr:", name, "rows", int(got[1][0]))
    o_gi, o_gm = K.select_grow(g_scores, b, tau)
    assert np.array_equal(g_idx.cpu().numpy(), o_gi)
    assert np.array_equal(g_mask.cpu().numpy().view(np.uint32), o_gm)
    spans = int(np.sum(np.diff(o_gi[0]) > 1)) + 1
    log("c4 bcr: grow spans", spans)

    for name, idx, width, mask in (("chunk", layouts["chunk"][0], c * B, layouts["chunk"][2]),
                                   ("grow", g_idx, b, g_mask)):
        out = {p: torch.empty_like(reuse[p]) for p in "kv"}
        mu = torch.empty(2, L, S, H, hd, dtype=torch.float32, device=dev)
        log("c4 bcr:", name, "correction of 48 layers")
        for pi, p in enumerate("kv"):
            d = d_t if p == "k" else None
            kv.kvfix_fit_mean(Plane.dense(fresh[p]), Plane.dense(reuse[p]), Plane.dense(out[p]),
                              idx, width, mu[pi], d, cfg.theta)
            kv.kvfix_apply(Plane.dense(reuse[p]), Plane.dense(out[p]), mask, mu[pi], None, 0.0,
                           1.0, d, cfg.theta)
        torch.cuda.synchronize()
        h_idx = idx.cpu().numpy()
        h_mask = mask.cpu().numpy().view(np.uint32)
        for l, p in ((0, "k"), (L - 1, "v")) if name == "chunk" else ((23, "k"),):
            pi = "kv".index(p)
            rope = (deltas, cfg.theta, "half") if p == "k" else (None, 0.0, "half")
            fr, ru = to_np(fresh[p][l:l + 1]), to_np(reuse[p][l:l + 1])
            o_out, o_mu = K.correct(fr, ru, "bf16", h_idx, h_mask, None, 0.0, 1.0, None, None,
                                    rope[0], rope[1], rope[2])
            assert rel_err(mu[pi, l:l + 1].cpu().numpy(), o_mu, "f32") <= 1e-5, (name, l, p)
            e = assert_values(to_np(out[p][l:l + 1]), o_out, "bf16", f"{name} layer {l} {p}")
            log("c4 bcr:", name, "layer", l, p, "max rel err", e)
        del out


# ----------------------------------------------------------------------------
# Collective round: 16 agents x 32 layers x 8192 tokens, block-sparse diffs
# against one master, then the fused restore of all 16 caches.
# ----------------------------------------------------------------------------


def test_c3_collective_16_agents_full_size():
    from helpers import to_np, torch_rotate, assert_values
    from oracle import kvref as K
    from synthetic import draw_collective
    from test_gpu_draft_diff import diff_np
    import cross_context_kv_amd.kvfix as kv
    from cross_context_kv_amd.kvfix import Plane
    cfg = CONFIGS["c3"]
    L, A, H, n, hd, bt = (cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim,
                          cfg.block_tokens)
    nb = -(-n // bt)
    dev = "cuda"
    sample = [0, L - 1]
    master = {p: torch.empty(L, 1, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    sib = {p: torch.empty(L, A, H, n, hd, dtype=torch.bfloat16, device=dev) for p in "kv"}
    log("c3 full: drawing 32 layers x 16 agents")
    planted = offs = None
    for l in range(L):
        raw = draw_collective(cfg, dev, layers=[l])
        planted, offs = raw["planted"], [int(o) for o in raw["offsets"].tolist()]
        master["k"][l], master["v"][l] = raw["master_k"][0], raw["master_v"][0]
        sib["k"][l] = torch_rotate(raw["y_k"][0], offs, cfg.theta).to(torch.bfloat16)
        sib["v"][l] = raw["y_v"][0]
        del raw
    total_planted = int(planted.sum()) * L
    cap = total_planted + 64
    diff = kv.Diff(A, L, n, H, hd, bt, cap, dtype=torch.bfloat16)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(kv.kvfix_diff_encode_workspace(A, L, n, bt) + 256, dtype=torch.uint8,
                     device=dev)
    to_m = torch.tensor([-o for o in offs], dtype=torch.int64, device=dev)
    from_m = torch.tensor(offs, dtype=torch.int64, device=dev)
    log("c3 full: encode, decode")
    kv.kvfix_diff_encode(Plane.dense(master["k"]), Plane.dense(master["v"]), Plane.dense(sib["k"]),
                         Plane.dense(sib["v"]), to_m, cfg.theta, cfg.eps, diff, status, ws)
    out = {p: torch.empty_like(sib[p]) for p in "kv"}
    wsd = torch.empty(kv.kvfix_diff_decode_workspace(A, hd) + 256, dtype=torch.uint8, device=dev)
    kv.kvfix_diff_decode(Plane.dense(master["k"]), Plane.dense(master["v"]), diff, from_m,
                         cfg.theta, Plane.dense(out["k"]), Plane.dense(out["v"]), wsd)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    g = diff_np(diff)
    # every planted block is found and nothing else, at every layer (bit-exact)
    want = np.zeros((A, L, -(-nb // 32)), dtype=np.uint32)
    for a in range(A):
        for beta in np.nonzero(planted[a].numpy())[0]:
            want[a, :, beta // 32] |= np.uint32(1) << np.uint32(beta % 32)
    assert np.array_equal(g["mask"], want)
    per = np.array([sum(bin(int(w)).count("1") for w in want[a, l]) for a in range(A)
                    for l in range(L)])
    assert np.array_equal(g["offsets"], np.concatenate([[0], np.cumsum(per)]))
    assert g["offsets"][-1] == total_planted
    # values restore exactly; keys within the rotation's roundings
    assert torch.equal(out["v"], sib["v"])
    log("c3 full: restored keys equal to the siblings:",
        float((out["k"] == sib["k"]).float().mean()))
    # sampled layers against the oracle: encode, and decode of the GPU's diff
    for l in sample:
        log("c3 full: oracle layer", l)
        mk, mv = to_np(master["k"][l:l + 1]), to_np(master["v"][l:l + 1])
        sk, sv = to_np(sib["k"][l:l + 1]), to_np(sib["v"][l:l + 1])
        o = K.diff_encode(mk, mv, sk, sv, [-x for x in offs], cfg.theta, cfg.eps, bt)
        slots = np.concatenate([np.arange(g["offsets"][a * L + l], g["offsets"][a * L + l + 1])
                                for a in range(A)]).astype(np.int64)
        assert np.array_equal(g["mask"][:, l:l + 1], o["mask"])
        assert np.array_equal(g["block_idx"][slots], o["block_idx"])
        assert_values(g["vals_k"][slots], o["vals_k"], "bf16", f"c3 vals_k layer {l}")
        assert np.array_equal(g["vals_v"][slots], o["vals_v"])
        sub = {"mask": g["mask"][:, l:l + 1], "vals_k": g["vals_k"][slots],
               "vals_v": g["vals_v"][slots], "offsets": o["offsets"]}
        ok, ov = K.diff_decode(mk, mv, sub, offs, cfg.theta, A, bt)
        e = assert_values(to_np(out["k"][l:l + 1]), ok, "bf16", f"c3 decode K layer {l}")
        assert np.array_equal(to_np(out["v"][l:l + 1]), ov)
        log("c3 full: layer", l, "decode K max rel err", e)

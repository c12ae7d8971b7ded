"""GPU test of kvfix_fit_mean_noalloc, the fit without a workspace argument
(its slice partials live in the library's per-device buffer): through the C
ABI, against kvfix_fit_mean with a caller workspace on the same inputs, on
two calls in a row, the second with a smaller input (so stale partials of the
first call sit in the buffer), and the capacity error past the buffer."""
import numpy as np
import pytest
import torch

from helpers import correction_case, from_np, log
from oracle import kvref as K
from synthetic import CONFIGS

import cross_context_kv_amd.kvfix as kv
from cross_context_kv_amd.kvfix import Plane

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_both(cfg, case, p, b, rng, fresh_by_slot=False):
    L, S, H, n, hd = cfg.n_layers, cfg.n_segs, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim
    idx = np.sort(np.stack([rng.choice(n, b, replace=False) for _ in range(S)]), axis=1)
    idx_t = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    fresh, reuse = from_np(case["fresh_" + p], DEV), from_np(case["reuse_" + p], DEV)
    if fresh_by_slot:
        fresh = torch.stack([fresh[:, s][:, :, idx_t[s].long()] for s in range(S)], dim=1)
    A = None if case["A_" + p] is None else torch.from_numpy(case["A_" + p]).to(DEV)
    B = None if case["B_" + p] is None else torch.from_numpy(case["B_" + p]).to(DEV)
    delta = torch.tensor(case["deltas"], dtype=torch.int64, device=DEV) if p == "k" else None
    res = []
    for noalloc in (False, True):
        out = torch.full_like(reuse, float("nan"))
        mu = torch.full((L, S, H, hd), float("nan"), dtype=torch.float32, device=DEV)
        args = (Plane.dense(fresh), Plane.dense(reuse), Plane.dense(out), idx_t, b, mu, delta,
                cfg.theta, kv.ROPE_HALF, A, B, fresh_by_slot)
        log("fit_mean", "noalloc" if noalloc else "workspace", (L, S, H, n, hd), b, p)
        if noalloc:
            kv.kvfix_fit_mean_noalloc(*args)
        else:
            kv.kvfix_fit_mean(*args)
        torch.cuda.synchronize()
        res.append((mu.cpu().numpy(), out.cpu()))
    return res, idx


def test_noalloc_fit_equals_workspace_fit_on_two_calls_in_a_row():
    rng = np.random.default_rng(90)
    big = CONFIGS["c2"].replace(n_layers=4, n_kv_heads=4, n_tokens=2000, b=600, n_segs=2,
                                per_segment_delta=True)
    small = CONFIGS["c2"].replace(n_layers=2, n_kv_heads=2, n_tokens=300, b=45, n_segs=1)
    for cfg, p, slot in ((big, "k", False), (small, "v", False), (small, "k", True)):
        case = correction_case(cfg)
        (ws_res, na_res), idx = run_both(cfg, case, p, cfg.b, rng, slot)
        assert np.array_equal(ws_res[0].view(np.uint32), na_res[0].view(np.uint32))
        assert torch.equal(ws_res[1].view(torch.int16), na_res[1].view(torch.int16))
        # and to the parity bar against the oracle
        rope = (case["deltas"], cfg.theta) if p == "k" else (None, 0.0)
        fresh = case["fresh_" + p]
        if slot:
            fresh = np.stack([fresh[:, s][:, :, idx[s]] for s in range(cfg.n_segs)], axis=1)
        o_mu = K.fit_mean(fresh, case["reuse_" + p], cfg.dtype, idx, rope[0], rope[1], "half",
                          case["A_" + p], case["B_" + p], slot)
        e = float(np.max(np.abs(na_res[0].astype(np.float64) - o_mu) / (np.abs(o_mu) + 1e-3)))
        log("noalloc mu rel err", e)
        assert e <= 1e-5


def test_noalloc_fit_rejects_sizes_past_its_buffer():
    # 64 layers x 128 segments x 8 heads with b = 256: 65,536 units of one
    # 1,096-byte partial each, 68.5 MiB
    L, S, H, n, hd, b = 64, 128, 8, 256, 128, 256
    need = kv.kvfix_fit_mean_workspace(L, S, H, hd, b)
    assert need > kv.NOALLOC_SCRATCH_BYTES
    plane = torch.zeros(hd, dtype=torch.bfloat16, device=DEV).as_strided((L, S, H, n, hd),
                                                                        (0, 0, 0, 0, 1))
    idx = torch.zeros(S, b, dtype=torch.int32, device=DEV)
    mu = torch.empty(L, S, H, hd, dtype=torch.float32, device=DEV)
    with pytest.raises(kv.KvfixError) as e:
        kv.kvfix_fit_mean_noalloc(Plane.dense(plane), Plane.dense(plane), None, idx, b, mu)
    assert e.value.status == 3

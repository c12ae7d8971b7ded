"""Pins of the CPU oracle against things other than itself.

Each test fixes one oracle function to a value printed on the pages, a closed
form, an invariant, a library special case or a brute-force enumeration, so
that a dropped term, a wrong sign or index, or a transposed operand anywhere in
the oracle fails at least one of them.  All of these run on the CPU.
"""
import cmath
import itertools
import json
import math
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

from oracle import kvref as K

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# bf16 codec: a library special case (torch's float32 -> bfloat16 is RNE)
# ----------------------------------------------------------------------------


def test_bf16_encode_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    specials = np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, 3.3961e38,
                         1e-40, -1e-40, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
                         np.float32(np.inf), -np.inf], dtype=np.float32)
    x32 = np.concatenate([x32, specials, rng.standard_normal(100_000).astype(np.float32)])
    ours = K.f64_to_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_is_exact_and_roundtrips():
    allbits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    vals = K.bf16_to_f64(allbits)
    finite = np.isfinite(vals)
    back = K.f64_to_bf16(vals[finite])
    assert np.array_equal(back, allbits[finite])
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(vals[finite], ref[finite])


def test_bf16_rounds_once_from_float64():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between two bf16 values:
    # a single rounding goes up; rounding through float32 first would tie
    # back down to 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert K.bf16_to_f64(K.f64_to_bf16(np.array([x])))[0] == 1.0 + 2.0 ** -7


# ----------------------------------------------------------------------------
# a1: rotary re-alignment
# ----------------------------------------------------------------------------


def test_rope_hand_example():
    g = golden("rope_hand_example.json")
    x = np.array(g["input"], dtype=np.float64)
    out = K.rope_rotate(x, g["delta"], g["theta"], "half")
    np.testing.assert_allclose(out, g["expected_half_values"], rtol=0, atol=5e-14)
    np.testing.assert_allclose(K.rope_angles(g["delta"], g["theta"], g["head_dim"]),
                               g["angles_rad"], rtol=1e-15)


def _complex_rotate(x, delta, theta, style):
    """Textbook form: pair (a, b) is the complex number a + ib times e^(i phi)."""
    hd = x.shape[-1]
    out = np.empty_like(x)
    for i in range(hd // 2):
        ia, ib = (i, i + hd // 2) if style == "half" else (2 * i, 2 * i + 1)
        phi = delta * theta ** (-2.0 * i / hd)
        z = (x[..., ia] + 1j * x[..., ib]) * cmath.exp(1j * phi)
        out[..., ia], out[..., ib] = z.real, z.imag
    return out


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("hd", [4, 64, 128])
def test_rope_equals_complex_multiplication(style, hd):
    rng = np.random.default_rng(hd)
    x = rng.standard_normal((5, hd))
    for delta, theta in [(37, 1e4), (8191, 5e5), (-32768, 1e6)]:
        # angles reach |delta| radians: fp64 keeps them to about |delta| * 1e-16
        np.testing.assert_allclose(K.rope_rotate(x, delta, theta, style),
                                   _complex_rotate(x, delta, theta, style), rtol=0,
                                   atol=1e-14 * max(1, abs(delta)))


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_rope_composition_inverse_and_norm(style):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 128))
    p, d, theta = 1234, 4321, 5e5
    two_step = K.rope_rotate(K.rope_rotate(x, p, theta, style), d, theta, style)
    np.testing.assert_allclose(two_step, K.rope_rotate(x, p + d, theta, style), atol=1e-11)
    back = K.rope_rotate(K.rope_rotate(x, d, theta, style), -d, theta, style)
    np.testing.assert_allclose(back, x, atol=1e-13)
    ia, ib = K._pairs(128, style)
    y = K.rope_rotate(x, d, theta, style)
    np.testing.assert_allclose(y[:, ia] ** 2 + y[:, ib] ** 2, x[:, ia] ** 2 + x[:, ib] ** 2,
                               rtol=1e-13)


def test_rope_relative_position_property():
    # <R(p) q, R(p') k> depends only on p' - p.
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = None
    for p in [0, 17, 5000]:
        v = K.rope_rotate(q, p, 1e4) @ K.rope_rotate(k, p + 300, 1e4)
        base = v if base is None else base
        assert abs(v - base) < 1e-9


def test_rope_interleaved_is_half_after_permutation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 64))
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])   # interleaved -> half
    y_int = K.rope_rotate(x, 99, 1e4, "interleaved")
    y_half = K.rope_rotate(x[:, perm], 99, 1e4, "half")
    np.testing.assert_allclose(y_int[:, perm], y_half, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_shift_zero_delta_is_bitwise_identity(dtype):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 2, 9, 64))
    plane = K.store(x, dtype)
    assert np.array_equal(K.rope_shift(plane, dtype, [0, 0, 0], 1e4), plane)


def test_rope_shift_rounds_once_per_segment():
    rng = np.random.default_rng(5)
    x = K.store(rng.standard_normal((1, 2, 1, 4, 8)), "bf16")
    out = K.rope_shift(x, "bf16", [3, -7], 1e4)
    for s, d in enumerate([3, -7]):
        exp = K.f64_to_bf16(_complex_rotate(K.bf16_to_f64(x[:, s]), d, 1e4, "half"))
        assert np.array_equal(out[:, s], exp)


# ----------------------------------------------------------------------------
# a2: L2 score
# ----------------------------------------------------------------------------


def test_score_l2_hand_example():
    # Two rows, one head, hd = 2, V plane (no rotation):
    # row 0 differs by (3, 4) -> 5; row 1 by (0, 0) -> 0.
    fresh = np.array([[[[[3.0, 4.0], [1.0, 1.0]]]]], dtype=np.float32)
    reuse = np.array([[[[[0.0, 0.0], [1.0, 1.0]]]]], dtype=np.float32)
    d = K.score_l2(fresh, reuse, "f32", 0)
    assert d.tolist() == [[5.0, 0.0]]


def test_score_l2_spans_heads_and_uses_aligned_keys():
    rng = np.random.default_rng(6)
    L, S, H, n, hd, theta = 2, 2, 3, 11, 8, 1e4
    reuse = K.store(rng.standard_normal((L, S, H, n, hd)), "f32")
    fresh = K.store(rng.standard_normal((L, S, H, n, hd)), "f32")
    deltas = [5, 900]
    d = K.score_l2(fresh, reuse, "f32", 1, deltas, theta)
    for s in range(S):
        for j in range(n):
            al = _complex_rotate(reuse[1, s, :, j].astype(np.float64), deltas[s], theta, "half")
            ref = np.linalg.norm((fresh[1, s, :, j].astype(np.float64) - al).ravel())
            assert abs(d[s, j] - ref) <= 1e-6 * ref
    # fresh equal to the aligned reuse -> all zero
    fresh_eq = np.stack([K.rope_rotate(reuse[:, s].astype(np.float64), deltas[s], theta)
                         for s in range(S)], axis=1)
    d0 = K.score_l2(fresh_eq.astype(np.float64), reuse.astype(np.float64), "f32", 1, deltas, theta)
    assert np.abs(d0).max() < 1e-5


# ----------------------------------------------------------------------------
# a4: top-b selection (brute force over all subsets)
# ----------------------------------------------------------------------------


def _brute_topb(scores, b):
    """The unique b-subset S with (s_i > s_j) or (s_i == s_j and i < j) for i in S, j not in S."""
    n = len(scores)
    found = []
    for sub in itertools.combinations(range(n), b):
        inside = set(sub)
        ok = all((scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
                 for i in inside for j in range(n) if j not in inside)
        if ok:
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


def test_select_topb_brute_force_with_ties():
    rng = np.random.default_rng(8)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        s = rng.integers(-2, 3, size=n).astype(np.float32)   # many ties
        for b in range(n + 1):
            idx, mask = K.select_topb(s[None, :], b)
            assert idx[0].tolist() == _brute_topb(s.tolist(), b)
            for j in range(n):
                assert K.mask_bit(mask[0], j) == (j in idx[0])


def test_select_topb_negative_zero_ties_with_zero():
    idx, _ = K.select_topb(np.array([[-0.0, 0.0, -1.0]], dtype=np.float32), 1)
    assert idx.tolist() == [[0]]


def test_probe_budget_formula():
    # b = ceil(r n): configuration 1 states b = 26 for r = 0.1, n = 256.
    assert K.probe_budget(0.1, 256) == 26
    assert K.probe_budget(0.15, 4096) == 615
    assert K.probe_budget(0.1, 32768) == 3277
    assert K.probe_budget(0.1, 4096) == 410
    assert K.probe_budget(0.3, 10) == 3        # exact product, no float ceil spill
    assert K.probe_budget(1.0, 77) == 77
    assert K.probe_budget(0.0, 77) == 0


# ----------------------------------------------------------------------------
# a5 / a6: probe mean and apply
# ----------------------------------------------------------------------------


def _scalar_plane(values, hd=2):
    """[1][1][1][n][hd] float32 plane with `values` in coordinate 0."""
    p = np.zeros((1, 1, 1, len(values), hd), dtype=np.float32)
    p[0, 0, 0, :, 0] = values
    return p


def test_worked_example_printed_on_the_page():
    g = golden("aks_worked_example.json")
    # rows 0, 1 are the probes (reused 0, fresh = their residual); rows 2..4 are A, B, C
    reuse = _scalar_plane([0.0, 0.0] + [r["reused"] for r in g["rows"]])
    fresh = _scalar_plane(g["probe_residuals"] + [r["fresh"] for r in g["rows"]])
    idx = np.array([[0, 1]], dtype=np.int32)
    mask = np.array([[0b11]], dtype=np.uint32)
    # weights enter as min(d, 1): feed the printed weights as the check-layer scores
    scores = np.array([[9.0, 9.0] + [r["weight"] for r in g["rows"]]], dtype=np.float32)
    out, mu = K.correct(fresh, reuse, "f32", idx, mask, scores, w_lo=0.0, w_hi=1.0)
    assert mu[0, 0, 0, 0] == np.float32(g["mu_hat"])
    assert mu[0, 0, 0, 1] == 0.0
    for k, r in enumerate(g["rows"]):
        assert out[0, 0, 0, 2 + k, 0] == np.float32(r["corrected"])
        res = abs(r["fresh"] - float(out[0, 0, 0, 2 + k, 0]))
        assert abs(res - g["residual_after"][r["token"]]) < 1e-5
    # probes keep their fresh values exactly
    assert out[0, 0, 0, 0, 0] == fresh[0, 0, 0, 0, 0]
    assert out[0, 0, 0, 1, 0] == fresh[0, 0, 0, 1, 0]


def _random_case(rng, L=2, S=2, H=2, n=40, hd=8):
    x = rng.standard_normal((L, S, H, n, hd))
    return x


def test_mean_fit_brute_force_loops_with_rank_state():
    rng = np.random.default_rng(9)
    L, S, H, n, hd, r, b, theta = 2, 2, 2, 12, 4, 2, 5, 1e4
    reuse = K.store(rng.standard_normal((L, S, H, n, hd)), "f32")
    fresh = K.store(rng.standard_normal((L, S, H, n, hd)), "f32")
    A = rng.standard_normal((L, S, H, n, r)).astype(np.float32)
    B = rng.standard_normal((L, S, H, r, hd)).astype(np.float32)
    idx = np.array([sorted(rng.choice(n, b, replace=False)) for _ in range(S)], dtype=np.int32)
    deltas = [3, -11]
    mu = K.fit_mean(fresh, reuse, "f32", idx, deltas, theta, "half", A, B)
    for l in range(L):
        for s in range(S):
            for h in range(H):
                for d in range(hd):
                    acc = 0.0
                    for j in idx[s]:
                        al = _complex_rotate(reuse[l, s, h, j].astype(np.float64), deltas[s],
                                             theta, "half")[d]
                        ab = sum(float(A[l, s, h, j, k]) * float(B[l, s, h, k, d]) for k in range(r))
                        acc += float(fresh[l, s, h, j, d]) - al - ab
                    assert abs(mu[l, s, h, d] - acc / b) <= 1e-6 * max(1.0, abs(acc / b))


def test_full_budget_reproduces_fresh_bitwise():
    rng = np.random.default_rng(10)
    for dtype in ["f32", "bf16"]:
        reuse = K.store(rng.standard_normal((2, 1, 2, 16, 8)), dtype)
        fresh = K.store(rng.standard_normal((2, 1, 2, 16, 8)), dtype)
        scores = rng.random((1, 16)).astype(np.float32)
        idx, mask = K.select_topb(scores, 16)
        out, _ = K.correct(fresh, reuse, dtype, idx, mask, scores, 0, 2, deltas=[7], theta=1e4)
        assert np.array_equal(out, fresh)


def test_zero_residual_gives_aligned_reuse():
    rng = np.random.default_rng(11)
    reuse = K.store(rng.standard_normal((2, 1, 2, 20, 8)), "f32")
    deltas, theta = [13], 1e4
    fresh = K.store(K.align_plane_f64(reuse.astype(np.float64), deltas, theta), "f32")
    scores = K.score_l2(fresh, reuse, "f32", 1, deltas, theta)
    assert scores.max() < 1e-5
    idx, mask = K.select_topb(scores, 4)
    out, mu = K.correct(fresh, reuse, "f32", idx, mask, None, deltas=deltas, theta=theta)
    assert np.abs(mu).max() < 1e-6
    np.testing.assert_allclose(out, K.rope_shift(reuse, "f32", deltas, theta), atol=1e-6)
    # with delta = 0 the whole path is a bitwise identity
    out0, mu0 = K.correct(reuse.copy(), reuse, "f32", idx, mask, None, deltas=[0], theta=theta)
    assert np.array_equal(out0, reuse) and not mu0.any()


def test_pure_offset_and_rank_state_are_removed_exactly():
    rng = np.random.default_rng(12)
    L, S, H, n, hd, r = 2, 1, 2, 64, 8, 3
    x = rng.standard_normal((L, S, H, n, hd))
    mu_true = rng.standard_normal((L, S, H, 1, hd))
    A = rng.standard_normal((L, S, H, n, r)).astype(np.float32)
    B = rng.standard_normal((L, S, H, r, hd)).astype(np.float32)
    ab = np.einsum("lshnr,lshrd->lshnd", A.astype(np.float64), B.astype(np.float64))
    deltas, theta = [321], 1e4
    reuse = np.stack([K.rope_rotate(x[:, s], -deltas[s], theta) for s in range(S)], axis=1)
    fresh = x + mu_true + ab                       # float64 "storage" for an exact identity
    idx = np.array([[3, 9, 20, 41]], dtype=np.int32)
    mask = np.zeros((1, 2), dtype=np.uint32)
    for j in idx[0]:
        mask[0, j // 32] |= np.uint32(1 << (j % 32))
    mu = K.fit_mean(fresh.astype(np.float32), reuse.astype(np.float32), "f32", idx, deltas,
                    theta, "half", A, B)
    np.testing.assert_allclose(mu, mu_true[:, :, :, 0].astype(np.float32), atol=1e-5)
    out, _ = K.correct(fresh.astype(np.float32), reuse.astype(np.float32), "f32", idx, mask,
                       None, A=A, B=B, deltas=deltas, theta=theta)
    np.testing.assert_allclose(out, fresh, atol=2e-5)
    # without the state the same mean leaves exactly A B behind on non-probe rows
    out2, _ = K.correct(fresh.astype(np.float32), reuse.astype(np.float32), "f32", idx, mask,
                        None, deltas=deltas, theta=theta)
    keep = np.setdiff1d(np.arange(n), idx[0])
    resid = fresh[:, :, :, keep] - out2[:, :, :, keep]
    centred = ab[:, :, :, keep] - ab[:, :, :, idx[0]].mean(axis=3, keepdims=True)
    np.testing.assert_allclose(resid, centred, atol=5e-5)


def test_error_identity_for_unweighted_mean():
    # AgentKVShift: with w = 1, e = mu_hat - mu and the corrected residual of
    # a non-probe row is xi_j - e.
    rng = np.random.default_rng(13)
    n, hd = 50, 6
    reuse = rng.standard_normal((1, 1, 1, n, hd))
    mu = rng.standard_normal(hd)
    xi = 0.1 * rng.standard_normal((n, hd))
    fresh = reuse.copy()
    fresh[0, 0, 0] += mu + xi
    idx = np.array([[1, 7, 30]], dtype=np.int32)
    mask = np.zeros((1, 2), dtype=np.uint32)
    for j in idx[0]:
        mask[0, j // 32] |= np.uint32(1 << (j % 32))
    out, mu_hat = K.correct(fresh.astype(np.float32), reuse.astype(np.float32), "f32", idx, mask)
    e = mu_hat[0, 0, 0].astype(np.float64) - mu
    keep = np.setdiff1d(np.arange(n), idx[0])
    r_corr = fresh[0, 0, 0, keep] - out[0, 0, 0, keep]
    np.testing.assert_allclose(r_corr, xi[keep] - e, atol=2e-6)


def test_weights_clip_and_scope():
    # w multiplies only the mean; the rank term is added unweighted; no
    # scores means w = 1.
    w = K.weights(np.array([-1.0, 0.5, 3.0], dtype=np.float32), 0.0, 2.0, 3)
    assert w.tolist() == [0.0, 0.5, 2.0]
    assert K.weights(None, 0.0, 2.0, 4).tolist() == [1.0] * 4
    reuse = np.zeros((1, 1, 1, 3, 2), dtype=np.float32)
    mu = np.full((1, 1, 1, 2), 1.0, dtype=np.float32)
    A = np.ones((1, 1, 1, 3, 1), dtype=np.float32)
    B = np.full((1, 1, 1, 1, 2), 10.0, dtype=np.float32)
    out = K.apply(reuse, "f32", None, mu, np.array([[0.0, 0.5, 5.0]], dtype=np.float32),
                  0.0, 2.0, A, B)
    assert out[0, 0, 0, :, 0].tolist() == [10.0, 10.5, 12.0]


def test_empty_budget_is_pure_realignment():
    rng = np.random.default_rng(14)
    reuse = K.store(rng.standard_normal((1, 1, 2, 10, 8)), "bf16")
    fresh = K.store(rng.standard_normal((1, 1, 2, 10, 8)), "bf16")
    idx = np.zeros((1, 0), dtype=np.int32)
    mask = np.zeros((1, 1), dtype=np.uint32)
    out, mu = K.correct(fresh, reuse, "bf16", idx, mask, deltas=[5], theta=1e4)
    assert not mu.any()
    assert np.array_equal(out, K.rope_shift(reuse, "bf16", [5], 1e4))


def test_fresh_by_slot_matches_dense_fresh():
    rng = np.random.default_rng(15)
    reuse = K.store(rng.standard_normal((2, 2, 2, 30, 8)), "bf16")
    fresh = K.store(rng.standard_normal((2, 2, 2, 30, 8)), "bf16")
    idx = np.array([[0, 4, 29], [2, 3, 17]], dtype=np.int32)
    compact = np.stack([fresh[:, s][:, :, idx[s]] for s in range(2)], axis=1)
    a = K.fit_mean(fresh, reuse, "bf16", idx, [1, 2], 1e4)
    b = K.fit_mean(compact, reuse, "bf16", idx, [1, 2], 1e4, fresh_by_slot=True)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------
# a3: draft attention mass
# ----------------------------------------------------------------------------


def test_softmax_counterexample_printed_on_the_page():
    g = golden("aks_softmax_l1.json")
    d = np.abs(K.softmax(np.array(g["z_prime"])) - K.softmax(np.array(g["z"]))).sum()
    assert round(float(d), g["printed_decimals"]) == g["l1_printed"]
    # closed form: 2 (sigma(0.2) - 1/2)
    assert abs(d - 2 * (1 / (1 + math.exp(-0.2)) - 0.5)) < 1e-15


def _draft_case(rng, L=3, H=2, Hq=4, T=2, n=13, hd=8):
    q = K.f64_to_bf16(rng.standard_normal((L, Hq, T, hd)))
    k = K.f64_to_bf16(rng.standard_normal((L, 1, H, n, hd)))
    return q, k


def test_draft_mass_sums_to_rows_times_layers():
    rng = np.random.default_rng(16)
    q, k = _draft_case(rng)
    a = K.score_draft(q, k, [17], 1e4, first_layer=1)
    assert abs(float(a.astype(np.float64).sum()) - (3 - 1) * 4 * 2) < 1e-5
    assert (a > 0).all()


def test_draft_brute_force_scalar_loops():
    rng = np.random.default_rng(17)
    L, H, Hq, T, n, hd, theta, delta = 3, 2, 4, 2, 7, 4, 1e4, 9
    q, k = _draft_case(rng, L, H, Hq, T, n, hd)
    a = K.score_draft(q, k, [delta], theta, first_layer=1)
    qf, kf = K.bf16_to_f64(q), K.bf16_to_f64(k)
    ref = [0.0] * n
    for l in range(1, L):
        for h in range(Hq):
            g = h // (Hq // H)
            keys = [_complex_rotate(kf[l, 0, g, j], delta, theta, "half") for j in range(n)]
            for t in range(T):
                z = [sum(qf[l, h, t, d] * keys[j][d] for d in range(hd)) / math.sqrt(hd)
                     for j in range(n)]
                m = max(z)
                e = [math.exp(v - m) for v in z]
                tot = sum(e)
                for j in range(n):
                    ref[j] += e[j] / tot
    np.testing.assert_allclose(a[0], np.array(ref, dtype=np.float32), rtol=2e-7)


def test_draft_common_key_shift_invariance():
    # AgentKVShift, "Limitations": adding one vector to every visible key
    # leaves the softmax unchanged.  A common shift c of the stored keys of a
    # segment is a common shift R(delta) c of its aligned keys.  Small integer
    # keys and shifts keep k + c exact in bf16.
    rng = np.random.default_rng(18)
    L, H, Hq, T, n, hd = 3, 2, 4, 2, 11, 8
    q = K.f64_to_bf16(rng.standard_normal((L, Hq, T, hd)))
    k = rng.integers(-4, 5, size=(L, 1, H, n, hd)).astype(np.float64)
    c = rng.integers(-2, 3, size=(L, 1, H, 1, hd)).astype(np.float64)
    a0 = K.score_draft(q, K.f64_to_bf16(k), [5], 1e4)
    a1 = K.score_draft(q, K.f64_to_bf16(k + c), [5], 1e4)
    np.testing.assert_allclose(a1, a0, rtol=2e-6)
    assert not np.allclose(K.score_draft(q, K.f64_to_bf16(k + rng.integers(-2, 3, size=k.shape)),
                                         [5], 1e4), a0, rtol=1e-3)


def test_draft_gqa_group_one_is_plain_multihead():
    rng = np.random.default_rng(19)
    q, k = _draft_case(rng, H=4, Hq=4, n=9)
    a = K.score_draft(q, k, [3], 1e4)
    # With 8 query heads over 4 key heads, query heads 2h and 2h+1 read key
    # head h.  Make both copies of the old query head h: the mass doubles.
    q2 = np.repeat(q, 2, axis=1)
    a2 = K.score_draft(q2, k, [3], 1e4)
    np.testing.assert_allclose(a2, 2 * a, rtol=1e-6)


def test_query_rotation_identity():
    # q . R(d) k = R(-d) q . k  (the kernel scores without rotating keys)
    rng = np.random.default_rng(20)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    lhs = q @ K.rope_rotate(k, 777, 1e6)
    rhs = K.rope_rotate(q, -777, 1e6) @ k
    assert abs(lhs - rhs) < 1e-11


# ----------------------------------------------------------------------------
# a7: paged addressing
# ----------------------------------------------------------------------------


def test_paged_offsets_hand_computed():
    # 2 segments x 4 tokens, page size 2, 2 heads, hd 3, 4 pages, 1 layer.
    pt = np.array([[2, 0], [3, 1]], dtype=np.int32)
    # s_token = H*hd = 6, s_page = 2*6 = 12, s_layer = 4*12 = 48
    cases = {  # (l, s, h, j) -> offset worked by hand
        (0, 0, 0, 0): 2 * 12,
        (0, 0, 1, 1): 2 * 12 + 6 + 3,
        (0, 0, 0, 2): 0,
        (0, 1, 1, 3): 1 * 12 + 6 + 3,
        (1, 1, 0, 0): 48 + 3 * 12,
    }
    for (l, s, h, j), off in cases.items():
        assert K.paged_offset(pt, 2, 48, 12, 6, 3, l, s, h, j) == off


def test_paged_tagging_roundtrip():
    rng = np.random.default_rng(21)
    L, S, H, n, hd, ps = 2, 3, 2, 8, 4, 2
    n_pages = 14
    pt = rng.permutation(n_pages)[: S * n // ps].reshape(S, n // ps).astype(np.int32)
    tag = np.zeros((L, S, H, n, hd), dtype=np.float32)
    for l, s, h, j in itertools.product(range(L), range(S), range(H), range(n)):
        tag[l, s, h, j] = [l, s, h, j]
    pool = np.full(L * n_pages * ps * H * hd, -1.0, dtype=np.float32)
    K.paged_scatter(pool, tag, pt, ps)
    assert np.array_equal(K.paged_gather(pool, pt, ps, L, H, n, hd), tag)
    # every untouched page stays untouched
    used = np.zeros(n_pages, dtype=bool)
    used[pt.ravel()] = True
    pv = pool.reshape(L, n_pages, -1)
    assert (pv[:, ~used] == -1).all() and (pv[:, used] != -1).any()


# ----------------------------------------------------------------------------
# a8 / a9: block-sparse diff
# ----------------------------------------------------------------------------


def test_diff_roundtrip_lossless_with_zero_shift_and_zero_eps():
    rng = np.random.default_rng(22)
    L, A, H, n, hd, bt = 2, 3, 2, 37, 8, 16      # ragged last block
    master_k = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    master_v = K.store(rng.standard_normal((L, 1, H, n, hd)), "bf16")
    sib_k = np.repeat(master_k, A, axis=1)
    sib_v = np.repeat(master_v, A, axis=1)
    sib_k[1, 0, 1, 5, 3] ^= 1                      # one bit flipped -> block 0 listed
    sib_v[0, 2, 0, 36, 0] ^= 4                     # the ragged tail block
    d = K.diff_encode(master_k, master_v, sib_k, sib_v, [0] * A, 1e4, 0.0, bt)
    assert d["total"] == 2
    assert d["offsets"].tolist() == [0, 0, 1, 1, 1, 2, 2]
    assert d["block_idx"].tolist() == [0, 2]
    ok, ov = K.diff_decode(master_k, master_v, d, [0] * A, 1e4, A, bt)
    assert np.array_equal(ok, sib_k) and np.array_equal(ov, sib_v)


def test_diff_recovers_planted_blocks_and_empty_diff_is_rotated_master():
    from synthetic import CONFIGS, draw_collective
    cfg = CONFIGS["c3"].replace(n_layers=2, n_kv_heads=2, n_tokens=160, n_segs=3)
    raw = draw_collective(cfg, "cpu")
    theta, bt = cfg.theta, cfg.block_tokens
    offs = raw["offsets"].tolist()
    yk = raw["y_k"].view(torch.int16).numpy().view(np.uint16)
    yv = raw["y_v"].view(torch.int16).numpy().view(np.uint16)
    mk = raw["master_k"].view(torch.int16).numpy().view(np.uint16)
    mv = raw["master_v"].view(torch.int16).numpy().view(np.uint16)
    sib_k = K.rope_shift(yk, "bf16", offs, theta)
    d = K.diff_encode(mk, mv, sib_k, yv, [-o for o in offs], theta, cfg.eps, bt)
    nb = 10
    for a in range(3):
        for l in range(2):
            flagged = [K.mask_bit(d["mask"][a, l], beta) for beta in range(nb)]
            assert flagged == raw["planted"][a].tolist()
    ok, ov = K.diff_decode(mk, mv, d, offs, theta, 3, bt)
    assert np.array_equal(ov, yv)
    err = np.abs(K.bf16_to_f64(ok) - K.bf16_to_f64(sib_k))
    assert err.max() < 0.1                           # two roundings of a rotation
    empty = {"mask": np.zeros_like(d["mask"]), "offsets": np.zeros(7, dtype=np.int64),
             "vals_k": d["vals_k"][:0], "vals_v": d["vals_v"][:0], "block_idx": d["block_idx"][:0]}
    ek, ev = K.diff_decode(mk, mv, empty, offs, theta, 3, bt)
    for a in range(3):
        assert np.array_equal(ek[:, a:a + 1], K.rope_shift(mk, "bf16", [offs[a]], theta))
        assert np.array_equal(ev[:, a], mv[:, 0])


def test_storage_formulas_printed_on_the_page():
    g = golden("td_storage.json")
    for c in g["cases"]:
        full = 1.0
        diff = full / c["R"]
        assert abs(K.mirror_ratio(full, diff) - c["R"]) < 1e-12
        if "mirror_percent" in c:
            assert round(100 * diff) == c["mirror_percent"]
        cost = K.group_cost(c["N"], c["R"])
        assert round(cost, 1) == c["cost_printed"]
        assert round(c["N"] / round(cost, 1), 1) == c["reduction_printed"]


def test_diff_roundtrip_lossless_fp32_storage():
    rng = np.random.default_rng(23)
    L, A, H, n, hd, bt = 2, 2, 2, 21, 8, 16
    mk = rng.standard_normal((L, 1, H, n, hd)).astype(np.float32)
    mv = rng.standard_normal((L, 1, H, n, hd)).astype(np.float32)
    sk, sv = np.repeat(mk, A, axis=1), np.repeat(mv, A, axis=1)
    sk[0, 1, 0, 17, 2] += np.float32(1e-3)         # tail block of agent 1, layer 0
    d = K.diff_encode(mk, mv, sk, sv, [0] * A, 1e4, 0.0, bt, dtype="f32")
    assert d["total"] == 1 and d["offsets"].tolist() == [0, 0, 0, 1, 1]
    assert d["vals_k"].dtype == np.float32
    ok, ov = K.diff_decode(mk, mv, d, [0] * A, 1e4, A, bt, dtype="f32")
    assert np.array_equal(ok, sk) and np.array_equal(ov, sv)


# ----------------------------------------------------------------------------
# BCR layouts: chunk budget, chunk means, chunk rows, grown spans, coin
# ----------------------------------------------------------------------------


def test_chunk_budget_reproduces_the_printed_budget_column():
    g = golden("bcr_table8_budget.json")
    M, (num, den) = g["segment_rows"], g["rho"]
    for unit, pct in zip(g["units"], g["budget_percent_printed"]):
        c = K.chunk_budget(M, unit, num, den, "table8")
        assert round(100.0 * c * unit / M, g["printed_decimals"]) == pct, (unit, c)


def test_chunk_budget_algorithm1_skip_rule_and_rounding():
    # skip when M < 2B ...
    assert K.chunk_budget(127, 64, 1, 5, "alg1") == 0
    # ... or when rho M < B (0.2 * 319 = 63.8 < 64); rho M = B is repaired
    assert K.chunk_budget(319, 64, 1, 5, "alg1") == 0
    assert K.chunk_budget(320, 64, 1, 5, "alg1") == 1
    # round(rho M / B): 0.2 * 2048 / 64 = 6.4 -> 6, the 64-row line of the table
    assert K.chunk_budget(2048, 64, 1, 5, "alg1") == 6 == K.chunk_budget(2048, 64, 1, 5, "table8")
    # 0.2 * 2240 / 64 = 7.0 exactly; 0.5 * 192 / 64 = 1.5 rounds up
    assert K.chunk_budget(2240, 64, 1, 5, "alg1") == 7
    assert K.chunk_budget(192, 64, 1, 2, "alg1") == 2
    # rho = 1 takes every chunk (1000 / 64 = 15.625 -> 16 = ceil(1000 / 64))
    assert K.chunk_budget(1000, 64, 1, 1, "alg1") == 16
    # rho = 0: Algorithm 1 serves unrepaired; the table's rule keeps one chunk
    assert K.chunk_budget(2048, 64, 0, 1, "alg1") == 0
    assert K.chunk_budget(2048, 64, 0, 1, "table8") == 1
    assert K.chunk_budget(0, 64, 1, 5, "table8") == 0


def test_chunk_means_closed_forms():
    n, B = 100, 64
    ramp = np.arange(n, dtype=np.float32)[None, :]
    m = K.chunk_means(ramp, B)
    # the mean of the integers lo..hi-1 is (lo + hi - 1) / 2; the short last
    # chunk (rows 64..99) is divided by its own 36 rows, not by 64
    assert m.tolist() == [[31.5, 81.5]]
    const = np.full((2, 130), 0.375, dtype=np.float32)
    assert np.all(K.chunk_means(const, 16) == np.float32(0.375))
    # random: within one float32 ulp of the exactly rounded mean
    rng = np.random.default_rng(21)
    x = rng.random((3, 200)).astype(np.float32) * 10.0 ** rng.integers(-3, 3, (3, 200))
    got = K.chunk_means(x.astype(np.float32), 48)
    for r in range(3):
        for i in range(got.shape[1]):
            vals = [float(v) for v in x[r, i * 48:(i + 1) * 48]]
            exact = np.float32(math.fsum(vals) / len(vals))
            assert abs(float(got[r, i]) - float(exact)) <= float(np.spacing(exact))


def test_expand_chunks_hand_example():
    idx, counts, mask = K.expand_chunks(np.array([[1, 3]], dtype=np.int32), 100, 32)
    # chunk 1 = rows 32..63, chunk 3 = rows 96..99 (a short last chunk), then padding
    assert idx[0].tolist() == list(range(32, 64)) + [96, 97, 98, 99] + [-1] * 28
    assert counts.tolist() == [36]
    assert mask[0].tolist() == [0, 0xFFFFFFFF, 0, 0xF]


def test_chunk_layout_keeps_the_best_means():
    rng = np.random.default_rng(22)
    a = rng.random((4, 1000)).astype(np.float32)
    a[:, 300:364] += 5.0                       # one chunk of clearly higher scores
    m = K.chunk_means(a, 64)
    c = K.chunk_budget(1000, 64, 1, 5, "alg1")
    cidx, _ = K.select_topb(m, c)
    for r in range(4):
        assert 300 // 64 in cidx[r] or 364 // 64 in cidx[r]
        chosen = set(cidx[r].tolist())
        worst_in = min(m[r, i] for i in chosen)
        best_out = max(m[r, i] for i in range(m.shape[1]) if i not in chosen)
        assert worst_in >= best_out


def test_select_grow_hand_example():
    # seed 3 (9), threshold 2.25: left 3 >= 2.25, right 2 < 2.25 -> row 2;
    # left 8 -> row 1; left 1 and right 2 both fail; seed 1 is taken already;
    # seed 5 (7) uses the last row of the budget of 4
    idx, mask = K.select_grow(np.array([[1, 8, 3, 9, 2, 7, 0.5, 6]], np.float32), 4, 0.25)
    assert idx.tolist() == [[1, 2, 3, 5]]
    assert mask.tolist() == [[0b101110]]


def test_select_grow_tie_goes_left_and_budget_stops_mid_span():
    a = np.array([[5, 4, 10, 4, 1]], np.float32)
    assert K.select_grow(a, 1, 0.25)[0].tolist() == [[2]]
    assert K.select_grow(a, 2, 0.25)[0].tolist() == [[1, 2]]        # 4 | 4: the left one
    assert K.select_grow(a, 3, 0.25)[0].tolist() == [[0, 1, 2]]     # 5 beats 4
    assert K.select_grow(a, 4, 0.25)[0].tolist() == [[0, 1, 2, 3]]


def test_select_grow_spans_stop_at_chosen_rows():
    # seed 0 (9) cannot grow (0.1 < 4.5); seed 3 (8) takes row 2 (5 >= 4) and
    # stops at 0.1 on both sides; row 2 is then skipped as a seed; seed 1
    # (0.1, threshold 0.05) is boxed in by chosen rows 0 and 2
    a = np.array([[9, 0.1, 5, 8, 0.1]], np.float32)
    assert K.select_grow(a, 4, 0.5)[0].tolist() == [[0, 1, 2, 3]]
    assert K.select_grow(a, 3, 0.5)[0].tolist() == [[0, 2, 3]]


@pytest.mark.parametrize("b", [0, 1, 7, 40, 100])
def test_select_grow_with_tau_above_one_is_topb(b):
    # an unchosen neighbour never beats the seed, so no span grows
    rng = np.random.default_rng(23 + b)
    a = np.round(rng.random((3, 100)) * 20).astype(np.float32) + 1.0   # ties
    gi, gm = K.select_grow(a, b, 1.5)
    ti, tm = K.select_topb(a, b)
    assert np.array_equal(gi, ti) and np.array_equal(gm, tm)


def _window_by_prefix_minimum_merge(a, b):
    """tau = 0: one window around the best row.  Its left and right parts are
    the first b-1 rows of the merge of the two outward runs, where each run is
    replaced by its running minimum (a non-increasing sequence) and equal
    values go to the left run."""
    s = int(np.lexsort((np.arange(len(a)), -a.astype(np.float64)))[0])
    X = list(np.minimum.accumulate(a[:s][::-1].astype(np.float64))) if s > 0 else []
    Y = list(np.minimum.accumulate(a[s + 1:].astype(np.float64))) if s + 1 < len(a) else []
    i = j = 0
    for _ in range(b - 1):
        if j >= len(Y) or (i < len(X) and X[i] >= Y[j]):
            i += 1
        else:
            j += 1
    return list(range(s - i, s + j + 1))


def test_select_grow_zero_tau_is_one_window_by_prefix_minimum_merge():
    rng = np.random.default_rng(24)
    for trial in range(20):
        n = int(rng.integers(2, 60))
        a = (rng.random(n) * 10).astype(np.float32)
        if trial % 3 == 0:
            a = np.round(a).astype(np.float32)       # ties
        b = int(rng.integers(1, n + 1))
        got = K.select_grow(a[None, :], b, 0.0)[0][0].tolist()
        assert got == _window_by_prefix_minimum_merge(a, b)


def test_select_grow_invariants():
    rng = np.random.default_rng(25)
    a = rng.random((5, 300)).astype(np.float32) ** 4
    for b in [0, 1, 30, 299, 300]:
        idx, mask = K.select_grow(a, b, 0.25)
        assert idx.shape == (5, b)
        for r in range(5):
            assert np.all(np.diff(idx[r]) > 0)
            assert K.mask_to_bool(mask[r], 300).sum() == b
            if b:
                assert int(np.argmax(a[r])) in idx[r]


def test_fit_mean_padding_entries_are_not_probes():
    rng = np.random.default_rng(26)
    reuse = K.store(rng.standard_normal((2, 2, 2, 40, 8)), "bf16")
    fresh = K.store(rng.standard_normal((2, 2, 2, 40, 8)), "bf16")
    real = np.array([[3, 9, 20], [0, 5, 39]], dtype=np.int32)
    padded = np.array([[3, 9, 20, -1, -1], [0, 5, 39, -1, 40]], dtype=np.int32)
    a = K.fit_mean(fresh, reuse, "bf16", real, [4, 7], 1e4)
    b = K.fit_mean(fresh, reuse, "bf16", padded, [4, 7], 1e4)
    assert np.array_equal(a, b)
    # a list of padding only is an empty probe set: mu = 0
    z = K.fit_mean(fresh, reuse, "bf16", np.full((2, 4), -1, np.int32), [4, 7], 1e4)
    assert not z.any()
    # by slot: padding slots hold no fresh row
    compact = np.zeros((2, 2, 2, 5, 8), dtype=fresh.dtype)
    for s in range(2):
        for k in range(5):
            if 0 <= padded[s, k] < 40:
                compact[:, s, :, k] = fresh[:, s, :, padded[s, k]]
    c = K.fit_mean(compact, reuse, "bf16", padded, [4, 7], 1e4, fresh_by_slot=True)
    assert np.array_equal(a, c)


def test_coin_control_draws_exactly_c_uniform_chunks():
    from synthetic.workloads import draw_coin_keys
    nc, c, trials = 10, 3, 3000
    hits = np.zeros(nc)
    keys = draw_coin_keys(77, trials, nc).numpy()
    idx, mask = K.select_topb(keys, c)
    for r in range(trials):
        assert len(set(idx[r].tolist())) == c
        hits[idx[r]] += 1
    p = c / nc
    sd = math.sqrt(trials * p * (1 - p))
    assert np.all(np.abs(hits - trials * p) < 5 * sd)


# ----------------------------------------------------------------------------
# Probe granularity per head (AKS: the construction for one attention head)
# and the covered prefix (KVCMAS App. A.3 "Variable Segment Lengths")
# ----------------------------------------------------------------------------


def _case(seed, L=2, S=2, H=3, n=40, hd=8, r=2, dtype="bf16"):
    rng = np.random.default_rng(seed)
    reuse = K.store(rng.standard_normal((L, S, H, n, hd)), dtype)
    fresh = K.store(rng.standard_normal((L, S, H, n, hd)), dtype)
    A = rng.standard_normal((L, S, H, n, r)).astype(np.float32)
    B = rng.standard_normal((L, S, H, r, hd)).astype(np.float32)
    return rng, reuse, fresh, A, B


def test_per_head_scores_add_up_in_squares_to_the_shared_score():
    rng, reuse, fresh, _, _ = _case(40)
    d = K.score_l2(fresh, reuse, "bf16", 1, [3, 9], 1e4)
    dh = K.score_l2(fresh, reuse, "bf16", 1, [3, 9], 1e4, per_head=True)
    assert dh.shape == (2, 3, 40)
    sq = (dh.astype(np.float64) ** 2).sum(axis=1)
    assert np.allclose(np.sqrt(sq), d, rtol=2e-7, atol=0)
    # one head: the per-head score is the shared score
    d1 = K.score_l2(fresh[:, :, :1], reuse[:, :, :1], "bf16", 1, [3, 9], 1e4)
    assert np.array_equal(K.score_l2(fresh[:, :, :1], reuse[:, :, :1], "bf16", 1, [3, 9], 1e4,
                                     per_head=True)[:, 0], d1)


def test_per_head_fit_with_one_probe_set_for_all_heads_is_the_shared_fit():
    rng, reuse, fresh, A, B = _case(41)
    idx = np.array([[1, 7, 30, 39], [0, 2, 3, 20]], np.int32)
    idx_h = np.repeat(idx[:, None, :], 3, axis=1)
    a = K.fit_mean(fresh, reuse, "bf16", idx, [4, -2], 1e4, "half", A, B)
    b = K.fit_mean(fresh, reuse, "bf16", idx_h, [4, -2], 1e4, "half", A, B, per_head=True)
    assert np.array_equal(a, b)


def test_per_head_fit_and_apply_use_each_heads_own_probes():
    rng, reuse, fresh, A, B = _case(42)
    S, H, n = 2, 3, 40
    idx_h = np.stack([np.stack([np.sort(rng.choice(n, 5, replace=False)) for _ in range(H)])
                      for _ in range(S)]).astype(np.int32)
    mask_h = np.zeros((S, H, (n + 31) // 32), np.uint32)
    for s in range(S):
        for h in range(H):
            for j in idx_h[s, h]:
                mask_h[s, h, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    out, mu = K.correct(fresh, reuse, "bf16", idx_h, mask_h, None, 0.0, 1.0, A, B, [5, 6], 1e4,
                        per_head=True)
    # each head equals the shared correction of that head alone with its probes
    for h in range(H):
        o1, m1 = K.correct(fresh[:, :, h:h + 1], reuse[:, :, h:h + 1], "bf16", idx_h[:, h],
                           mask_h[:, h], None, 0.0, 1.0, A[:, :, h:h + 1], B[:, :, h:h + 1],
                           [5, 6], 1e4)
        assert np.array_equal(out[:, :, h:h + 1], o1) and np.array_equal(mu[:, :, h:h + 1], m1)


def test_cover_full_is_no_cover_and_zero_is_pure_realignment():
    rng, reuse, fresh, A, B = _case(43)
    idx = np.array([[1, 7, 30, 39], [0, 2, 3, 20]], np.int32)
    mask = np.zeros((2, 2), np.uint32)
    for s in range(2):
        for j in idx[s]:
            mask[s, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    sc = rng.random((2, 40)).astype(np.float32) * 3
    base = K.correct(fresh, reuse, "bf16", idx, mask, sc, 0.0, 2.0, A, B, [7, 8], 1e4)
    full = K.correct(fresh, reuse, "bf16", idx, mask, sc, 0.0, 2.0, A, B, [7, 8], 1e4,
                     cover=[40, 40])
    assert np.array_equal(base[0], full[0]) and np.array_equal(base[1], full[1])
    zero, mu0 = K.correct(fresh, reuse, "bf16", idx, mask, sc, 0.0, 2.0, A, B, [7, 8], 1e4,
                          cover=[0, 0])
    shifted = K.rope_shift(reuse, "bf16", [7, 8], 1e4)
    for s in range(2):
        rows = np.setdiff1d(np.arange(40), idx[s])
        assert np.array_equal(zero[:, s][:, :, rows], shifted[:, s][:, :, rows])
    # no rank state anywhere: the mean is the mean without A B
    assert np.array_equal(mu0, K.fit_mean(fresh, reuse, "bf16", idx, [7, 8], 1e4))


def test_cover_splits_the_segment_at_the_covered_prefix():
    rng, reuse, fresh, A, B = _case(44)
    idx = np.array([[1, 7, 30, 39], [0, 2, 3, 20]], np.int32)
    mask = np.zeros((2, 2), np.uint32)
    for s in range(2):
        for j in idx[s]:
            mask[s, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    cover = [25, 10]
    out, mu = K.correct(fresh, reuse, "bf16", idx, mask, None, 0.0, 1.0, A, B, [7, 8], 1e4,
                        cover=cover)
    shifted = K.rope_shift(reuse, "bf16", [7, 8], 1e4)
    # A rows past the prefix set to zero give the same mean (the state is absent there)
    A0 = A.copy()
    for s in range(2):
        A0[:, s, :, cover[s]:] = 0.0
    assert np.array_equal(mu, K.fit_mean(fresh, reuse, "bf16", idx, [7, 8], 1e4, "half", A0, B))
    full, _ = K.correct(fresh, reuse, "bf16", idx, mask, None, 0.0, 1.0, A0, B, [7, 8], 1e4)
    for s in range(2):
        rows = np.setdiff1d(np.arange(40), idx[s])
        inside, past = rows[rows < cover[s]], rows[rows >= cover[s]]
        assert np.array_equal(out[:, s][:, :, past], shifted[:, s][:, :, past])
        assert np.array_equal(out[:, s][:, :, inside], full[:, s][:, :, inside])


# ----------------------------------------------------------------------------
# Master selection (TD §4.2 "reuse plan output")
# ----------------------------------------------------------------------------


def test_select_master_hand_example_and_ties():
    m, tot = K.select_master(np.array([[1, 2, 3], [0.5, 0.5, 0.5], [1, 1, 1]], np.float32))
    assert m == 1 and tot.tolist() == [6.0, 1.5, 3.0]
    # equal totals go to the lower request index
    m, _ = K.select_master(np.array([[2, 2], [1, 3], [4, 0], [5, 5]], np.float32))
    assert m == 0
    m, _ = K.select_master(np.array([[9, 9], [1, 3], [4, 0]], np.float32))
    assert m == 1


def test_select_master_prefers_the_request_without_deviation():
    # a request whose cache equals the shared blocks has zero divergence at
    # every token: it is the master whatever the others look like
    rng = np.random.default_rng(50)
    sc = rng.random((6, 500)).astype(np.float32) + 0.01
    sc[4] = 0.0
    assert K.select_master(sc)[0] == 4


def test_select_master_total_is_the_exact_sum_of_the_l2_scores():
    # the deviation of a request against the shared blocks: per-token L2
    # divergence of its keys from the shared keys re-aligned to its frame
    rng = np.random.default_rng(51)
    A, H, n, hd = 4, 2, 300, 8
    shared = K.store(rng.standard_normal((1, 1, H, n, hd)), "f32")
    agents = np.repeat(shared, A, axis=1).copy()
    planted = [5, 1, 3, 0]
    for a, nb in enumerate(planted):
        rows = rng.choice(n, nb * 4, replace=False)
        agents[0, a][:, rows] += np.float32(0.5)
    sc = K.score_l2(agents, np.repeat(shared, A, axis=1), "f32", 0)
    m, tot = K.select_master(sc)
    assert m == 3 and tot[3] == 0.0
    assert np.argsort(tot, kind="stable").tolist() == np.argsort(planted, kind="stable").tolist()
    # the total is the sum itself: the exact rational sum of the float32
    # scores, rounded once to float64 (Python's Fraction -> float rounds
    # correctly), whatever order a machine adds them in
    for a in range(A):
        exact = float(sum((Fraction(float(x)) for x in sc[a]), Fraction(0)))
        assert tot[a] == exact, a


def test_select_master_total_does_not_depend_on_the_order_of_the_tokens():
    # scores spanning 40 binades: a left-to-right float64 sum loses the small
    # terms, the total does not; reversing or shuffling the tokens of a
    # request leaves its total bit for bit unchanged
    rng = np.random.default_rng(52)
    sc = (np.exp(rng.standard_normal((3, 1000)) * 9.0)).astype(np.float32)
    sc[0, 0] = np.float32(1e30)
    _, tot = K.select_master(sc)
    _, rev = K.select_master(sc[:, ::-1].copy())
    _, shuf = K.select_master(sc[:, rng.permutation(1000)].copy())
    assert np.array_equal(tot.view(np.uint64), rev.view(np.uint64))
    assert np.array_equal(tot.view(np.uint64), shuf.view(np.uint64))
    exact = float(sum((Fraction(float(x)) for x in sc[0]), Fraction(0)))
    assert tot[0] == exact


# ----------------------------------------------------------------------------
# Anchor-blended correction and the reliability gate (KVCMAS eq. 8-11,
# App. A.3).  Pools are built from small exactly representable factors so that
# reconstructions, distances and corrected rows have closed forms.
# ----------------------------------------------------------------------------


def _rows_to_plane(rows, H, hd):
    """[n][H*hd] float64 -> [H][n][hd]."""
    n = rows.shape[0]
    return rows.reshape(n, H, hd).transpose(1, 0, 2)


def _const_pool(V, L, n_max, H, hd, r, fill):
    """Pool whose anchor v reconstructs, at (l, p), every row as the vector
    fill(v, l, p) [H*hd]: A rows = e_0, B row 0 = that vector.  All values
    must be bf16-exact."""
    D = H * hd
    a = np.zeros((V, L, 2, n_max, r))
    bt = np.zeros((V, L, 2, D, r))
    a[..., 0] = 1.0
    for v in range(V):
        for l in range(L):
            for p in range(2):
                bt[v, l, p, :, 0] = fill(v, l, p)
    return K.f64_to_bf16(a), K.f64_to_bf16(bt)


def test_anchor_eligible_full_cover_else_longest_prefix():
    assert K.anchor_eligible([5, 10, 10, 3], 8) == ([1, 2], 8)
    assert K.anchor_eligible([5, 10, 10, 3], 10) == ([1, 2], 10)
    assert K.anchor_eligible([5, 10, 12, 3], 8) == ([1, 2], 8)
    assert K.anchor_eligible([5, 10, 10, 3], 12) == ([1, 2], 10)   # longest covered prefix
    assert K.anchor_eligible([5, 7, 3], 12) == ([1], 7)
    assert K.anchor_eligible([0, 0], 4) == ([], 0)
    assert K.anchor_eligible([], 4) == ([], 0)


def test_anchor_gate_decide_closed_forms():
    # g = (3/4, 1/4): binary entropy of 1/4 = 2 - (3/4) log2 3
    r = K.anchor_gate_decide([0.0, math.log(3.0)], 0.9)
    assert np.allclose(r["g"], [0.75, 0.25], rtol=0, atol=1e-15)
    assert abs(r["hbar"] - (2 - 0.75 * math.log2(3))) < 1e-14 and r["accept"]
    assert not K.anchor_gate_decide([0.0, math.log(3.0)], 0.8)["accept"]
    # g = (1/2, 1/4, 1/4): 1.5 bits out of log2 3
    r = K.anchor_gate_decide([0.0, math.log(2.0), math.log(2.0)], 0.95)
    assert abs(r["hbar"] - 1.5 / math.log2(3)) < 1e-14 and r["accept"]
    # equal distances: the flat distribution, Hbar = 1; tau = 1 never refuses
    for V in (2, 3, 7, 10):
        r = K.anchor_gate_decide([2.5] * V, 1.0)
        assert r["hbar"] == 1.0 and r["accept"]
        assert not K.anchor_gate_decide([2.5] * V, 0.999)["accept"]
    # a distinctive match: entropy near 0
    r = K.anchor_gate_decide([0.0, 50.0, 60.0], 0.01)
    assert r["hbar"] < 1e-15 and r["accept"]
    # fewer than two compared anchors: dense
    assert not K.anchor_gate_decide([0.0], 1.0)["accept"]
    assert not K.anchor_gate_decide([], 1.0)["accept"]


def test_anchor_gate_distance_is_the_frobenius_norm_over_layers_and_prefix():
    L, H, n, hd, r = 3, 2, 7, 4, 2
    D = H * hd
    rng = np.random.default_rng(11)
    base = np.round(rng.standard_normal(D) * 4) / 4                 # bf16-exact
    off = [0.0, 0.5, -0.25, 1.0]
    # value factors reconstruct base + off[v]; key factors hold unrelated data
    a, bt = _const_pool(4, L, 9, H, hd, r,
                        lambda v, l, p: base + off[v] if p == 1 else base * 3 - 7 + v)
    src_v = K.f64_to_bf16(np.stack([_rows_to_plane(np.tile(base, (n, 1)), H, hd)[None]] * L))
    lengths = [9, 9, 5, 9]
    k = 5
    g = K.anchor_gate(src_v, a, bt, lengths, k, 1.0, "bf16")
    assert g["Ak"] == [0, 1, 2, 3]
    for v in range(4):
        assert abs(g["d"][v] - abs(off[v]) * math.sqrt(L * k * D)) < 1e-12
    # the rows past the prefix do not matter
    src2 = src_v.copy()
    src2[:, :, :, k:] = K.f64_to_bf16(np.full(src2[:, :, :, k:].shape, 9.0))
    assert np.array_equal(K.anchor_gate(src2, a, bt, lengths, k, 1.0, "bf16")["d"], g["d"])
    # a longer prefix drops the short anchor; k past the segment is the segment
    g6 = K.anchor_gate(src_v, a, bt, lengths, 6, 1.0, "bf16")
    assert g6["Ak"] == [0, 1, 3] and np.isnan(g6["d"][2])
    g99 = K.anchor_gate(src_v, a, bt, [9, 9, 7, 9], 99, 1.0, "bf16")
    assert g99["Ak"] == [0, 1, 2, 3]
    assert abs(g99["d"][3] - math.sqrt(L * n * D)) < 1e-12
    # decision: distances above give a distinctive match to anchor 0
    assert g["accept"] == (g["hbar"] <= 1.0)
    one = K.anchor_gate(src_v, a, bt, [9, 2, 2, 2], 5, 1.0, "bf16")
    assert one["Ak"] == [0] and not one["accept"]


def test_anchor_gate_flat_when_anchors_are_equally_far():
    L, H, n, hd, r = 2, 1, 4, 4, 2
    a, bt = _const_pool(3, L, n, H, hd, r, lambda v, l, p: np.full(hd, 0.5 if v < 2 else -0.5))
    src_v = K.f64_to_bf16(np.zeros((L, 1, H, n, hd)))
    g = K.anchor_gate(src_v, a, bt, [n] * 3, n, 1.0, "bf16")
    assert g["hbar"] == 1.0 and g["accept"]
    assert not K.anchor_gate(src_v, a, bt, [n] * 3, n, 0.99, "bf16")["accept"]


def test_anchor_weights_closed_form_mean_absolute_distance():
    L, H, n, hd, r = 2, 2, 6, 4, 2
    D = H * hd
    rng = np.random.default_rng(12)
    base = np.round(rng.standard_normal(D) * 4) / 4
    # anchor 0 exact; anchor 1 off by 0.5 in head 0 only (mean 0.25 over all
    # heads); anchor 2 off by 1 everywhere; anchor 3 too short to be eligible
    def fill(v, l, p):
        x = base.copy()
        if v == 1:
            x[:hd] += 0.5
        if v >= 2:
            x += 1.0
        return x
    a, bt = _const_pool(4, L, n, H, hd, r, fill)
    plane = K.f64_to_bf16(np.stack([_rows_to_plane(np.tile(base, (n, 1)), H, hd)[None]] * L))
    w = K.anchor_weights(plane, plane, a, bt, [n, n, n, n - 1], 0, 1e4, "half", "bf16")
    e = np.exp(-np.array([0.0, 0.25, 1.0]))
    want = e / e.sum()
    for l in range(L):
        for p in range(2):
            assert np.allclose(w[l, p, :, :3], want, rtol=0, atol=1e-15)
            assert np.all(w[l, p, :, 3] == 0)
    assert np.allclose(w.sum(axis=3), 1.0, rtol=0, atol=1e-15)


def test_anchor_weights_compare_keys_in_canonical_positions():
    L, H, n, hd, r = 1, 2, 5, 8, 2
    D = H * hd
    rng = np.random.default_rng(13)
    base = np.round(rng.standard_normal(D) * 4) / 4
    a, bt = _const_pool(2, L, n, H, hd, r,
                        lambda v, l, p: base if v == 0 else base + 0.75)
    src_off, theta = 37, 100.0
    canon = _rows_to_plane(np.tile(base, (n, 1)), H, hd)
    keys = K.rope_rotate(canon, src_off, theta, "half")[None, None].astype(np.float32)
    vals = canon[None, None].astype(np.float32)
    w = K.anchor_weights(keys, vals, a, bt, [n, n], src_off, theta, "half", "f32")
    e = np.exp(-np.array([0.0, 0.75]))
    assert np.allclose(w[0, 0], e / e.sum(), rtol=0, atol=1e-6)      # keys: f32 rounding only
    assert np.allclose(w[0, 1], e / e.sum(), rtol=0, atol=1e-15)
    # matched at the cached positions instead, the keys would not fit anchor 0
    w_wrong = K.anchor_weights(keys, vals, a, bt, [n, n], 0, theta, "half", "f32")
    assert w_wrong[0, 0, :, 0].max() < 0.6


def test_anchor_weights_are_token_wise_and_stop_at_the_covered_prefix():
    L, H, n, hd, r = 1, 1, 6, 4, 2
    rng = np.random.default_rng(14)
    rows = np.round(rng.standard_normal((n, hd)) * 4) / 4
    # anchor 0 reconstructs the first three rows exactly, anchor 1 the last three
    a = np.zeros((2, L, 2, 8, r))
    bt = np.zeros((2, L, 2, hd, r))
    for v, sl in ((0, slice(0, 3)), (1, slice(3, 6))):
        a[v, 0, :, sl, 0] = 1.0
        bt[v, 0, :, :, 0] = rows[sl][0]
    rows[1:3] = rows[0]
    rows[4:6] = rows[3]
    a, bt = K.f64_to_bf16(a), K.f64_to_bf16(bt)
    plane = K.f64_to_bf16(rows[None, None, None])
    w = K.anchor_weights(plane, plane, a, bt, [8, 8], 0, 1e4, "half", "bf16")
    assert np.all(w[0, :, :3, 0] > 0.5) and np.all(w[0, :, 3:, 1] > 0.5)
    # no anchor covers the segment: weights only on the longest covered prefix
    w4 = K.anchor_weights(plane, plane, a, bt, [4, 2], 0, 1e4, "half", "bf16")
    assert np.all(w4[0, :, :4, 0] == 1.0) and np.all(w4[0, :, 4:] == 0) and np.all(w4[..., 1] == 0)


def _integer_delta_pool(V, L, n_max, H, hd, r, rng):
    a = rng.integers(-2, 3, (V, L, 2, n_max, r)).astype(np.float64)
    bt = rng.integers(-2, 3, (V, L, 2, H * hd, r)).astype(np.float64)
    return a, bt, K.f64_to_bf16(a), K.f64_to_bf16(bt)


def test_anchor_apply_values_add_the_weighted_low_rank_deltas_exactly():
    L, H, n, hd, r, V = 2, 2, 5, 4, 3, 3
    rng = np.random.default_rng(15)
    af, btf, a, bt = _integer_delta_pool(V, L, n, H, hd, r, rng)
    x = rng.integers(-8, 9, (L, 1, H, n, hd)).astype(np.float32)
    w = np.zeros((L, 2, n, V))
    w[:, :, :, 0] = 0.25
    w[:, :, :, 2] = 0.75
    w[:, :, :, 1] = 0.5          # anchor 1 is too short to be eligible: ignored
    out = K.anchor_apply(x, 1, a, bt, w, [n, n - 1, n], 3, 9, 1e4, "half", "f32")
    for l in range(L):
        dhat = 0.25 * af[0, l, 1] @ btf[0, l, 1].T + 0.75 * af[2, l, 1] @ btf[2, l, 1].T
        want = x[l, 0].astype(np.float64) + _rows_to_plane(dhat, H, hd)
        assert np.array_equal(out[l, 0], want.astype(np.float32))
    # one anchor at full weight
    w1 = np.zeros((L, 2, n, V))
    w1[:, :, :, 1] = 1.0
    out1 = K.anchor_apply(x, 1, a, bt, w1, [n - 2, n, n - 1], 0, 0, 1e4, "half", "f32")
    for l in range(L):
        want = x[l, 0].astype(np.float64) + _rows_to_plane(af[1, l, 1] @ btf[1, l, 1].T, H, hd)
        assert np.array_equal(out1[l, 0], want.astype(np.float32))


def test_anchor_apply_keys_add_the_delta_in_canonical_positions():
    L, H, n, hd, r, V = 1, 2, 6, 8, 2, 2
    rng = np.random.default_rng(16)
    af, btf, a, bt = _integer_delta_pool(V, L, n, H, hd, r, rng)
    x = rng.standard_normal((L, 1, H, n, hd)).astype(np.float32)
    w = np.zeros((L, 2, n, V))
    w[..., 0] = 0.375
    w[..., 1] = 0.625
    src_off, tgt_off, theta = 19, 301, 50.0
    out = K.anchor_apply(x, 0, a, bt, w, [n, n], src_off, tgt_off, theta, "half", "f32")
    dhat = 0.375 * af[0, 0, 0] @ btf[0, 0, 0].T + 0.625 * af[1, 0, 0] @ btf[1, 0, 0].T
    canon = K.rope_rotate(x[0, 0].astype(np.float64), -src_off, theta, "half") + \
        _rows_to_plane(dhat, H, hd)
    back = K.rope_rotate(out[0, 0].astype(np.float64), -tgt_off, theta, "half")
    assert np.abs(back - canon).max() < 1e-5 * np.abs(canon).max()
    # with no delta the keys are the rotary shift alone
    z = np.zeros_like(w)
    o0 = K.anchor_apply(x, 0, a, bt, z, [n, n], src_off, tgt_off, theta, "half", "f32")
    assert np.array_equal(o0, K.rope_shift(x, "f32", [tgt_off - src_off], theta))
    o0v = K.anchor_apply(x, 1, a, bt, z, [n, n], src_off, tgt_off, theta, "half", "f32")
    assert np.array_equal(o0v, x)


def test_anchor_apply_rows_past_the_covered_prefix_are_only_realigned():
    L, H, n, hd, r, V = 1, 1, 8, 4, 2, 2
    rng = np.random.default_rng(17)
    af, btf, a, bt = _integer_delta_pool(V, L, n, H, hd, r, rng)
    x = rng.integers(-8, 9, (L, 1, H, n, hd)).astype(np.float32)
    w = np.full((L, 2, n, V), 0.5)                   # nonzero past the prefix too
    src_off, tgt_off, theta = 4, 10, 1e4
    out = K.anchor_apply(x, 0, a, bt, w, [5, 3], src_off, tgt_off, theta, "half", "f32")
    shifted = K.rope_shift(x, "f32", [tgt_off - src_off], theta)
    assert np.array_equal(out[:, :, :, 5:], shifted[:, :, :, 5:])
    assert not np.array_equal(out[:, :, :, :5], shifted[:, :, :, :5])
    # only anchor 0 covers the prefix: its delta at full weight 0.5 on rows < 5
    outv = K.anchor_apply(x, 1, a, bt, w, [5, 3], 0, 0, theta, "half", "f32")
    want = x[0, 0].astype(np.float64)
    want[:, :5] += 0.5 * _rows_to_plane(af[0, 0, 1, :5] @ btf[0, 0, 1].T, H, hd)
    assert np.array_equal(outv[0, 0], want.astype(np.float32))

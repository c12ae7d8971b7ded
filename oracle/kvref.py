"""CPU oracle for cross-context KV correction — TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The product path never does: it runs on the GPU
through the compiled library and fails loudly if that library is missing.

What it is: a plain, slow, single-threaded numpy implementation of every step
of the correction path, written from the definitions on the source pages:

  KVCMAS  = "KVCMAS: Efficient KV cache Correction for Shared Context in
            Multi-Agent Systems" (arXiv 2609.34060)
  AKS     = "AgentKVShift: Correcting Reused KV" (review page)
  TD      = "TokenDance: Scaling Multi-Agent LLM Serving via Collective KV
            Cache Sharing" (summary page, in Chinese)
  BCR     = "Budgeted Cache Repair for Cross-Context KV-Cache Reuse"
            (arXiv 2610.02233)

Conventions
  * A "plane" is one K or V cache, a numpy array [layer][segment][kv_head]
    [token][head_dim] holding either float32 values ("f32") or bfloat16 bit
    patterns as uint16 ("bf16").
  * Every computation is in float64; each output element is rounded ONCE to
    its storage type (round-to-nearest-even).  Scores and means are returned
    as float32 (rounded once from float64).
  * Rotary pairing: "half" pairs dims (i, i + hd/2); "interleaved" pairs
    (2i, 2i + 1).  Frequency of pair i is theta^(-2i/hd).  A shift by delta
    positions rotates pair i by delta * theta^(-2i/hd) radians.

Every function below is pinned by a CPU test against something other than
itself (worked examples printed on the pages, closed forms, invariants,
library special cases or brute force); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# storage codecs
# ----------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):            # NaN patterns stay NaN
        return u32.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one round-to-nearest-even step.

    bfloat16 keeps 8 significant bits and float32's exponent range.  A finite
    x = f * 2^e with 0.5 <= |f| < 1 has spacing 2^(e-8) between neighbours;
    below the smallest normal (2^-126) the spacing is fixed at 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    _, e = np.frexp(np.where(finite, x, 1.0))
    step_exp = np.maximum(e - 8, -133)
    step = np.ldexp(1.0, step_exp)
    r = np.rint(np.where(finite, x, 0.0) / step) * step          # np.rint: ties to even
    with np.errstate(over="ignore"):               # overflow is mapped to inf below
        r32 = r.astype(np.float32)                 # exact unless it overflows
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    too_big = finite & (np.abs(r) >= 2.0 ** 128)
    sign = np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))
    bits = np.where(too_big, sign | np.uint16(0x7F80), bits)
    bits = np.where(np.isinf(x), sign | np.uint16(0x7F80), bits)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    out[...] = bits
    return out


def to_f64(plane: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(plane)
    if dtype == "f32":
        return plane.astype(np.float64)
    raise ValueError(dtype)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage type."""
    if dtype == "bf16":
        return f64_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# a1: rotary re-alignment
# (KVCMAS §2.2 and App. A.3 "Correction Weighting and Positional Alignment":
#  cached keys are re-aligned to their target positions before reuse, values
#  are never rotated; TD §4.2: one batched rotary call for the whole group,
#  TD Algorithm 1: RoPERecover(P_old -> P_new))
# ----------------------------------------------------------------------------


def rope_angles(delta: float, theta: float, head_dim: int) -> np.ndarray:
    """Rotation angle of each of the hd/2 pairs for a shift of `delta` positions."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return float(delta) * inv_freq


def _pairs(head_dim: int, style: str):
    half = head_dim // 2
    if style == "half":
        return np.arange(half), np.arange(half) + half
    if style == "interleaved":
        return np.arange(half) * 2, np.arange(half) * 2 + 1
    raise ValueError(style)


def rope_rotate(x: np.ndarray, delta: float, theta: float, style: str = "half") -> np.ndarray:
    """Rotate float64 vectors x[..., hd] forward by `delta` positions.

    Each pair (a, b) of dims turns by angle phi:  a' = a cos phi - b sin phi,
    b' = b cos phi + a sin phi.
    """
    hd = x.shape[-1]
    ia, ib = _pairs(hd, style)
    phi = rope_angles(delta, theta, hd)
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., ia], x[..., ib]
    out = np.empty_like(x, dtype=np.float64)
    out[..., ia] = a * c - b * s
    out[..., ib] = b * c + a * s
    return out


def align_plane_f64(plane_f64: np.ndarray, deltas: Sequence[int], theta: float,
                    style: str = "half") -> np.ndarray:
    """Re-align a float64 plane [L][S][H][n][hd]: segment s shifts by deltas[s]."""
    out = np.empty_like(plane_f64)
    for s in range(plane_f64.shape[1]):
        out[:, s] = rope_rotate(plane_f64[:, s], deltas[s], theta, style)
    return out


def rope_shift(plane: np.ndarray, dtype: str, deltas: Sequence[int], theta: float,
               style: str = "half") -> np.ndarray:
    """a1 as a stand-alone batched call: every segment of the plane rotated by its shift."""
    return store(align_plane_f64(to_f64(plane, dtype), deltas, theta, style), dtype)


# ----------------------------------------------------------------------------
# a2: L2 divergence score at a check layer
# (AKS "Core idea and method", step 1 and the equation for d: the norm of
#  fresh minus reused state at the check layer, keys and values separately;
#  TD §4.2: one batched difference pass against the aligned keys)
# ----------------------------------------------------------------------------


def score_l2(fresh: np.ndarray, reuse: np.ndarray, dtype: str, check_layer: int,
             deltas: Optional[Sequence[int]] = None, theta: float = 0.0,
             style: str = "half", per_head: bool = False) -> np.ndarray:
    """d[s][j] = || fresh_j - align(reuse_j) || over all heads and dims of row j.

    per_head: d[s][h][j] over the head_dim elements of head h alone (AKS
    builds its correction for one attention head).  deltas=None scores a
    value plane (no rotation).  Returns float32 [S][n], or [S][H][n].
    """
    f = to_f64(fresh[check_layer], dtype)          # [S][H][n][hd]
    r = to_f64(reuse[check_layer], dtype)
    if deltas is not None:
        r = np.stack([rope_rotate(r[s], deltas[s], theta, style) for s in range(r.shape[0])])
    diff = f - r
    sq = (diff * diff).sum(axis=3 if per_head else (1, 3))
    return np.sqrt(sq).astype(np.float32)


# ----------------------------------------------------------------------------
# a4: top-b probe selection
# (AKS step 2 and the equation b = ceil(r n): the b rows with the largest
#  score; ties go to the lower token index; BCR-single: per-row top budget)
# ----------------------------------------------------------------------------


def probe_budget(ratio, n: int) -> int:
    """b = ceil(r * n), with r taken as the decimal it is written as."""
    return int(math.ceil(Fraction(repr(float(ratio))) * n))


def select_topb(scores: np.ndarray, b: int):
    """Exactly b indices per row with the largest score, ties to the lower index.

    scores: float32 [rows][n] (no NaN).  Returns (idx int32 [rows][b] in
    ascending order, mask uint32 [rows][ceil(n/32)] with bit j%32 of word j//32
    set for every selected j).
    """
    scores = np.asarray(scores, dtype=np.float32)
    if np.isnan(scores).any():
        raise ValueError("NaN score")
    rows, n = scores.shape
    if not 0 <= b <= n:
        raise ValueError("b out of range")
    idx = np.zeros((rows, b), dtype=np.int32)
    mask = np.zeros((rows, (n + 31) // 32), dtype=np.uint32)
    for r in range(rows):
        s = scores[r].astype(np.float64)
        order = np.lexsort((np.arange(n), -s))      # primary: score desc, then index asc
        chosen = np.sort(order[:b])
        idx[r] = chosen
        for j in chosen:
            mask[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return idx, mask


def mask_bit(mask_row: np.ndarray, j: int) -> bool:
    return bool((int(mask_row[j // 32]) >> (j % 32)) & 1)


def mask_to_bool(mask_row: np.ndarray, n: int) -> np.ndarray:
    """Bit j%32 of word j//32, for every j < n."""
    j = np.arange(n)
    return ((mask_row[j // 32].astype(np.uint64) >> (j % 32).astype(np.uint64)) & 1).astype(bool)


# ----------------------------------------------------------------------------
# BCR layouts: the chunk budget, chunk scores, whole chunks as rows, grown
# spans, and the coin control
# (BCR §3 "The layouts": BCR-chunk repairs the best-scoring fixed chunks,
#  BCR-grow seeds on the best row and widens the span while a neighbour scores
#  at least tau of the seed, BCR-single spends the budget row by row; §3 "The
#  repair": a group of rows scores the mean of its rows; §4.3: tau = 0.25;
#  App. A.2 "The policy" step 2 (the mean keeps a short last chunk from being
#  penalised) and "The random control" (chunks drawn by coin at the same
#  budget); App. A.2 Table 8 (the budget kept by unit of choice:
#  max(1, round(0.2 n_chunks)) chunks); App. B Algorithm 1 (skip rule
#  M < 2B or rho M < B, else round(rho M / B) chunks of B = 64 rows))
# ----------------------------------------------------------------------------


def _round_half_up(x: Fraction) -> int:
    """Nearest integer to x >= 0; a half rounds up (away from zero)."""
    return int(math.floor(x + Fraction(1, 2)))


def chunk_budget(M: int, B: int, rho_num: int, rho_den: int, rule: str) -> int:
    """Chunks of B rows to repair among M cached rows at budget rho = rho_num / rho_den.

    rule "alg1"  : 0 (serve unrepaired) when M < 2B or rho M < B, otherwise
                   round(rho M / B)                      [BCR App. B Algorithm 1]
    rule "table8": max(1, round(rho n_chunks)), n_chunks = ceil(M / B)
                                                        [BCR App. A.2 Table 8]
    Never more than n_chunks.  rho is exact (a fraction), so halves are exact.
    """
    if M < 0 or B < 1 or rho_den < 1 or not 0 <= rho_num <= rho_den:
        raise ValueError("bad budget arguments")
    rho = Fraction(rho_num, rho_den)
    n_chunks = -(-M // B)
    if rule == "alg1":
        if M < 2 * B or rho * M < B:
            return 0
        c = _round_half_up(rho * M / B)
    elif rule == "table8":
        c = max(1, _round_half_up(rho * n_chunks))
    else:
        raise ValueError(rule)
    return min(c, n_chunks)


def chunk_means(scores: np.ndarray, B: int) -> np.ndarray:
    """Chunk score a-bar_i = mean of a_j over the rows j of chunk i.

    Chunk i holds rows [iB, min((i+1)B, n)); the last one may be short and is
    divided by its own length.  The sum runs in float64 over the rows in
    ascending order and the mean is rounded once to float32.
    scores: float32 [rows][n].  Returns float32 [rows][ceil(n/B)].
    """
    scores = np.asarray(scores, dtype=np.float32)
    rows, n = scores.shape
    nc = -(-n // B)
    out = np.zeros((rows, nc), dtype=np.float32)
    for r in range(rows):
        for i in range(nc):
            lo, hi = i * B, min((i + 1) * B, n)
            acc = 0.0
            for j in range(lo, hi):
                acc += float(scores[r, j])
            out[r, i] = np.float32(acc / (hi - lo))
    return out


def expand_chunks(chunk_idx: np.ndarray, n: int, B: int):
    """The rows of the chosen chunks.

    chunk_idx: int32 [rows][c], ascending (as select_topb returns it); an id
    outside [0, ceil(n/B)) names no chunk and lists no rows.  Returns (idx int32 [rows][c*B]: the rows in ascending order, then -1 for
    the rows a short last chunk does not have; counts int32 [rows]; mask
    uint32 [rows][ceil(n/32)]).
    """
    rows, c = chunk_idx.shape
    nc = -(-n // B)
    idx = np.full((rows, c * B), -1, dtype=np.int32)
    counts = np.zeros(rows, dtype=np.int32)
    mask = np.zeros((rows, (n + 31) // 32), dtype=np.uint32)
    for r in range(rows):
        k = 0
        for ci in chunk_idx[r]:
            if not 0 <= int(ci) < nc:          # not a chunk of the row: no rows
                continue
            for j in range(int(ci) * B, min((int(ci) + 1) * B, n)):
                idx[r, k] = j
                mask[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
                k += 1
        counts[r] = k
    return idx, counts, mask


def select_grow(scores: np.ndarray, b: int, tau: float):
    """Exactly b rows per score row, spent in grown spans.

    While fewer than b rows are chosen: the seed is the best-scoring row not
    yet chosen (ties to the lower index); it is chosen, and its span then
    widens one row at a time, taking the higher-scoring of the two rows just
    outside it (the left one on a tie), as long as that row is not chosen yet
    and scores at least tau times the seed (compared in float64), and rows
    remain in the budget.
    scores: float32 [rows][n] (no NaN).  Returns (idx int32 [rows][b]
    ascending, mask uint32 [rows][ceil(n/32)]).
    """
    scores = np.asarray(scores, dtype=np.float32)
    if np.isnan(scores).any():
        raise ValueError("NaN score")
    rows, n = scores.shape
    if not 0 <= b <= n:
        raise ValueError("b out of range")
    idx = np.zeros((rows, b), dtype=np.int32)
    mask = np.zeros((rows, (n + 31) // 32), dtype=np.uint32)
    for r in range(rows):
        a = scores[r].astype(np.float64)
        chosen = np.zeros(n, dtype=bool)
        left = b
        for seed in np.lexsort((np.arange(n), -a)):     # score desc, then index asc
            if left == 0:
                break
            if chosen[seed]:
                continue
            chosen[seed] = True
            left -= 1
            thr = float(tau) * a[seed]
            lo = hi = int(seed)
            while left > 0:
                cl = lo - 1 if lo > 0 and not chosen[lo - 1] and a[lo - 1] >= thr else -1
                cr = hi + 1 if hi + 1 < n and not chosen[hi + 1] and a[hi + 1] >= thr else -1
                if cl < 0 and cr < 0:
                    break
                if cl >= 0 and (cr < 0 or a[cl] >= a[cr]):
                    lo = cl
                    chosen[cl] = True
                else:
                    hi = cr
                    chosen[cr] = True
                left -= 1
        sel = np.nonzero(chosen)[0]
        idx[r] = sel
        for j in sel:
            mask[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return idx, mask


# ----------------------------------------------------------------------------
# a5: probe mean residual (+ fresh scatter)
# (AKS step 3 and the equation for mu-hat: the mean of fresh minus reused over
#  the probe set, re-estimated at every layer; KVCMAS eq. 7-8: a rank-r state
#  A B, which the mean is taken after removing)
# ----------------------------------------------------------------------------


def lowrank_rows(A: Optional[np.ndarray], B: Optional[np.ndarray], l: int, s: int, h: int,
                 rows) -> Optional[np.ndarray]:
    """A[l][s][h][rows] @ B[l][s][h] in float64, or None without a state."""
    if A is None:
        return None
    return A[l, s, h][rows].astype(np.float64) @ B[l, s, h].astype(np.float64)


def _probe_list(idx: np.ndarray, s: int, h: int, per_head: bool) -> np.ndarray:
    return idx[s][h] if per_head else idx[s]


def _covered(rows: np.ndarray, cover, s: int) -> np.ndarray:
    """1.0 for rows inside segment s's covered prefix, 0.0 past it."""
    if cover is None:
        return np.ones(len(rows))
    return (rows < int(cover[s])).astype(np.float64)


def fit_mean(fresh: np.ndarray, reuse: np.ndarray, dtype: str, idx: np.ndarray,
             deltas: Optional[Sequence[int]] = None, theta: float = 0.0, style: str = "half",
             A: Optional[np.ndarray] = None, B: Optional[np.ndarray] = None,
             fresh_by_slot: bool = False, per_head: bool = False,
             cover: Optional[Sequence[int]] = None) -> np.ndarray:
    """mu[l][s][h] = (1/|S|) sum_{j in S} (fresh_j - align(reuse_j) - A_j B).

    idx: int32 [S][w], or [S][H][w] with per_head (a probe set per head).  An
    entry outside [0, n) is padding, not a member of the probe set S (a
    layout whose row count depends on the data, such as whole chunks with a
    short last chunk, pads its fixed-width list with -1); mu is the mean over
    the members, 0 when there are none.  cover: rows at or past cover[s] have
    no rank state (A_j = 0 there; KVCMAS App. A.3 "Variable Segment Lengths":
    no extrapolation past the covered prefix).  fresh_by_slot: fresh holds
    the probe rows by slot, row k being token idx[s]([h])[k] (padding slots
    unused).  Returns float32 [L][S][H][hd].
    """
    L, S, H, n, hd = reuse.shape
    mu = np.zeros((L, S, H, hd), dtype=np.float64)
    for s in range(S):
        for h in range(H):
            lst = _probe_list(idx, s, h, per_head)
            slots = np.array([k for k in range(len(lst)) if 0 <= int(lst[k]) < n], dtype=np.int64)
            if len(slots) == 0:
                continue
            rows = lst[slots].astype(np.int64)
            fr_rows = slots if fresh_by_slot else rows
            cov = _covered(rows, cover, s)
            for l in range(L):
                f = to_f64(fresh[l, s, h][fr_rows], dtype)
                r = to_f64(reuse[l, s, h][rows], dtype)
                if deltas is not None:
                    r = rope_rotate(r, deltas[s], theta, style)
                res = f - r
                ab = lowrank_rows(A, B, l, s, h, rows)
                if ab is not None:
                    res = res - cov[:, None] * ab
                mu[l, s, h] = res.sum(axis=0) / len(rows)
    return mu.astype(np.float32)


def scatter_fresh(out: np.ndarray, fresh: np.ndarray, idx: np.ndarray,
                  fresh_by_slot: bool = False, per_head: bool = False) -> None:
    """Copy the fresh rows into the probe positions of `out` (in place, exact);
    padding entries of idx (outside [0, n)) are skipped."""
    L, S, H, n, hd = out.shape
    for s in range(S):
        for h in range(H):
            lst = _probe_list(idx, s, h, per_head)
            slots = np.array([k for k in range(len(lst)) if 0 <= int(lst[k]) < n], dtype=np.int64)
            if len(slots) == 0:
                continue
            rows = lst[slots].astype(np.int64)
            src = slots if fresh_by_slot else rows
            out[:, s, h][:, rows] = fresh[:, s, h][:, src]


# ----------------------------------------------------------------------------
# a6: correction apply
# (AKS equation for K_corr: probes keep their fresh rows, every other row gets
#  reuse + w_j * mu-hat with w_j = min(d_j, 1) from the check layer;
#  KVCMAS eq. 3 (selective recompute) and eq. 4 / eq. 8 (add the estimated
#  deviation A B to the aligned source cache))
# ----------------------------------------------------------------------------


def weights(scores_row: Optional[np.ndarray], w_lo: float, w_hi: float, n: int) -> np.ndarray:
    """w_j = clip(d_j, lo, hi); no scores means w = 1 (mean-only correction)."""
    if scores_row is None:
        return np.ones(n, dtype=np.float64)
    return np.minimum(np.maximum(scores_row.astype(np.float64), float(w_lo)), float(w_hi))


def apply(reuse: np.ndarray, dtype: str, mask: Optional[np.ndarray], mu: np.ndarray,
          scores: Optional[np.ndarray] = None, w_lo: float = 0.0, w_hi: float = 1.0,
          A: Optional[np.ndarray] = None, B: Optional[np.ndarray] = None,
          deltas: Optional[Sequence[int]] = None, theta: float = 0.0, style: str = "half",
          out: Optional[np.ndarray] = None, per_head: bool = False,
          cover: Optional[Sequence[int]] = None) -> np.ndarray:
    """out_j = round(align(reuse_j) + w_j mu + A_j B) for every non-probe row j.

    Probe rows (mask bit set) are left as they are in `out` (a copy of `reuse`
    when out is None); the fresh scatter fills them.  mu: float32 [L][S][H][hd];
    scores: float32 [S][n] or None (w = 1); mask [S][words].  per_head: mask
    [S][H][words] and scores [S][H][n].  cover: rows at or past cover[s] are
    only re-aligned, out_j = round(align(reuse_j)) (KVCMAS App. A.3 "Variable
    Segment Lengths").
    """
    L, S, H, n, hd = reuse.shape
    res = reuse.copy() if out is None else out
    for s in range(S):
        for h in range(H):
            m = None if mask is None else (mask[s][h] if per_head else mask[s])
            keep = np.ones(n, dtype=bool) if m is None else ~mask_to_bool(m, n)
            rows = np.nonzero(keep)[0]
            sc = None if scores is None else (scores[s][h] if per_head else scores[s])
            cov = _covered(rows, cover, s)
            w = weights(sc, w_lo, w_hi, n)[rows] * cov
            for l in range(L):
                x = to_f64(reuse[l, s, h][rows], dtype)
                if deltas is not None:
                    x = rope_rotate(x, deltas[s], theta, style)
                y = x + w[:, None] * mu[l, s, h].astype(np.float64)[None, :]
                ab = lowrank_rows(A, B, l, s, h, rows)
                if ab is not None:
                    y = y + cov[:, None] * ab
                res[l, s, h][rows] = store(y, dtype)
    return res


def correct(fresh, reuse, dtype, idx, mask, scores=None, w_lo=0.0, w_hi=1.0, A=None, B=None,
            deltas=None, theta=0.0, style="half", fresh_by_slot=False, per_head=False,
            cover=None):
    """The whole correction of one plane: fit the mean, scatter, apply.

    Returns (out plane, mu).
    """
    mu = fit_mean(fresh, reuse, dtype, idx, deltas, theta, style, A, B, fresh_by_slot,
                  per_head, cover)
    out = reuse.copy()
    scatter_fresh(out, fresh, idx, fresh_by_slot, per_head)
    apply(reuse, dtype, mask, mu, scores, w_lo, w_hi, A, B, deltas, theta, style, out=out,
          per_head=per_head, cover=cover)
    return out, mu


# ----------------------------------------------------------------------------
# Anchor-blended low-rank correction and the reliability gate
# (KVCMAS eq. 7: low-rank factors A B of each anchor's base cache and delta
#  correction; eq. 8: the correction is the weighted sum of the anchors'
#  deltas; App. A.3 "Reliability Gate" eq. 9-11, "Correction Weighting and
#  Positional Alignment" (token-wise weights from the mean absolute source
#  distance, softmax with T = 1, keys compared in canonical positions) and
#  "Variable Segment Lengths"; eq. 4, 6 and 12: the correction is added to
#  the aligned source cache)
#
# Layouts: an anchor pool of V anchors holds, per anchor v, layer l and plane
# p (0 = K, 1 = V), A factors a[v][l][p][n_max][r] and the transposed B
# factors bt[v][l][p][H*hd][r], both bf16 bit patterns; a row's feature
# index is h*hd + d (all heads of a token).  Factors are in canonical
# (segment-relative) positions; the source plane holds one segment.
# ----------------------------------------------------------------------------


def anchor_eligible(lengths: Sequence[int], n: int):
    """Anchors that correct an n-token segment, and the covered prefix: those
    covering the whole segment; if none does, those covering the longest
    prefix, which is then the covered prefix."""
    full = [v for v, ln in enumerate(lengths) if ln >= n]
    if full:
        return full, n
    m = max(list(lengths) + [0])
    if m <= 0:
        return [], 0
    return [v for v, ln in enumerate(lengths) if ln == m], m


def anchor_recon(a: np.ndarray, bt: np.ndarray, v: int, l: int, p: int, rows) -> np.ndarray:
    """Anchor v's reconstruction A B (eq. 7) of `rows` at layer l, plane p:
    float64 [len(rows)][H*hd]."""
    A = bf16_to_f64(a[v, l, p][np.asarray(rows, dtype=np.int64)])     # [m][r]
    Bt = bf16_to_f64(bt[v, l, p])                                       # [D][r]
    return A @ Bt.T


def _token_rows(x: np.ndarray) -> np.ndarray:
    """[H][n][hd] -> [n][H*hd] (all heads of a token in one row)."""
    H, n, hd = x.shape
    return x.transpose(1, 0, 2).reshape(n, H * hd)


def anchor_gate_decide(d: Sequence[float], tau: float) -> dict:
    """Gate weights, normalized entropy and decision from the distances of
    the compared anchors (KVCMAS eq. 10-11 and the rule after them):
    g = softmax(-d / T) with T = 1; Hbar = -sum g log2 g / log2 |A_k|,
    clamped to [0, 1], its mathematical range, so that tau >= 1 never
    refuses; accept iff |A_k| >= 2 and Hbar <= tau."""
    d = np.asarray(d, dtype=np.float64)
    if d.size < 2:
        return {"g": np.ones(d.size), "hbar": float("nan"), "accept": False}
    z = -d
    e = np.exp(z - z.max())
    g = e / e.sum()
    terms = np.where(g > 0, g * np.log2(np.where(g > 0, g, 1.0)), 0.0)
    hbar = float(min(1.0, max(0.0, -terms.sum() / math.log2(d.size))))
    return {"g": g, "hbar": hbar, "accept": hbar <= tau}


def anchor_gate(src_v: np.ndarray, a_base: np.ndarray, bt_base: np.ndarray,
                lengths: Sequence[int], k: int, tau: float, dtype: str) -> dict:
    """The reliability gate (KVCMAS App. A.3, eq. 9-11).

    The comparison prefix is the first k tokens of the segment (k is clamped
    to the segment length).  Compared anchors A_k: those storing at least k
    tokens.  d_v = the Frobenius norm, over all layers, of the source value
    states of the prefix (all heads and dims) minus anchor v's reconstructed
    base value states (eq. 9).  src_v: value plane [L][1][H][n][hd].
    Returns the compared anchors, d [V] (NaN outside A_k), g, Hbar, accept.
    """
    L, _, H, n, hd = src_v.shape
    k = max(0, min(int(k), n))
    Ak = [v for v, ln in enumerate(lengths) if ln >= k]
    d = np.full(len(lengths), np.nan)
    for v in Ak:
        acc = 0.0
        for l in range(L):
            x = _token_rows(to_f64(src_v[l, 0], dtype))[:k]
            diff = x - anchor_recon(a_base, bt_base, v, l, 1, np.arange(k))
            acc += float((diff * diff).sum())
        d[v] = math.sqrt(acc)
    dec = anchor_gate_decide(d[Ak], tau)
    return {"Ak": Ak, "d": d, "g": dec["g"], "hbar": dec["hbar"], "accept": dec["accept"]}


def anchor_weights(src_k: np.ndarray, src_v: np.ndarray, a_base: np.ndarray,
                   bt_base: np.ndarray, lengths: Sequence[int], src_off: int,
                   theta: float, style: str, dtype: str) -> np.ndarray:
    """Token-wise interpolation weights (KVCMAS App. A.3).

    For each layer, plane and covered token j: dist_v = the mean, over all
    heads and dims, of |source row - anchor v's reconstructed base row| for
    the eligible anchors (source keys, cached at positions src_off + j, are
    first turned to canonical, segment-relative positions: rotated by
    -src_off), and w_v = softmax(-dist / T), T = 1.  Returns float64
    w [L][2][n][V], zero for anchors outside the eligible set and for rows
    past the covered prefix.
    """
    L, _, H, n, hd = src_k.shape
    V = len(lengths)
    E, cover = anchor_eligible(lengths, n)
    w = np.zeros((L, 2, n, V))
    if not E:
        return w
    for l in range(L):
        for p, plane in enumerate((src_k, src_v)):
            x = to_f64(plane[l, 0], dtype)
            if p == 0:
                x = rope_rotate(x, -src_off, theta, style)
            rows = _token_rows(x)[:cover]
            dist = np.stack([np.abs(rows - anchor_recon(a_base, bt_base, v, l, p, np.arange(cover)))
                             .mean(axis=1) for v in E], axis=1)
            z = -dist
            e = np.exp(z - z.max(axis=1, keepdims=True))
            wl = w[l, p]
            for i, v in enumerate(E):
                wl[:cover, v] = e[:, i] / e.sum(axis=1)
    return w


def anchor_apply(src: np.ndarray, plane: int, a_delta: np.ndarray, bt_delta: np.ndarray,
                 w: np.ndarray, lengths: Sequence[int], src_off: int, tgt_off: int,
                 theta: float, style: str, dtype: str) -> np.ndarray:
    """The corrected target cache (KVCMAS eq. 8 with the token-wise weights,
    added to the aligned source cache, eq. 4 / 6 / 12).

    delta_hat_j = sum over eligible v of w[l][plane][j][v] A_v[j] B_v, in
    canonical positions.  Keys: out_j = R(tgt_off) (R(-src_off) x_j +
    delta_hat_j) = R(tgt_off - src_off) x_j + R(tgt_off) delta_hat_j; values:
    out_j = x_j + delta_hat_j; rows past the covered prefix keep the
    re-aligned source row.  Rounded once.  src: [L][1][H][n][hd].
    """
    L, _, H, n, hd = src.shape
    E, cover = anchor_eligible(lengths, n)
    out = np.empty_like(src)
    for l in range(L):
        x = to_f64(src[l, 0], dtype)
        dhat = np.zeros((n, H * hd))
        for v in E:
            dhat[:cover] += w[l, plane, :cover, v][:, None] * anchor_recon(
                a_delta, bt_delta, v, l, plane, np.arange(cover))
        dh = dhat.reshape(n, H, hd).transpose(1, 0, 2)
        if plane == 0:
            y = rope_rotate(x, tgt_off - src_off, theta, style) + rope_rotate(dh, tgt_off, theta,
                                                                              style)
        else:
            y = x + dh
        out[l, 0] = store(y, dtype)
    return out


# ----------------------------------------------------------------------------
# a3: draft attention-mass score
# (BCR §3 "The repair": a_j = sum over layers l > 1 of the attention the two
#  kept draft query rows pay row j, softmax(Q K~^T / sqrt(d_head)), with
#  grouped-query keys expanded to the query heads (App. B, Algorithm 2 and
#  "The policy", step 2); K~ are the predicted (re-aligned) keys.)
# ----------------------------------------------------------------------------


def softmax(z: np.ndarray) -> np.ndarray:
    """Two-pass softmax over the last axis: subtract the max, exponentiate, normalise."""
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def score_draft(q: np.ndarray, k_plane: np.ndarray, deltas: Sequence[int], theta: float,
                first_layer: int = 1, style: str = "half") -> np.ndarray:
    """a[s][j] = sum_{l >= first_layer} sum_t sum_h softmax_j(q_{l,h,t} . K~_{l,g(h),j} / sqrt(hd)).

    q: bf16 bits [L][Hq][T][hd]; k_plane: bf16 bits [L][S][H][n][hd].  Query
    head h reads key head g(h) = h // (Hq / H).  Returns float32 [S][n].
    """
    L, S, H, n, hd = k_plane.shape
    Hq = q.shape[1]
    group = Hq // H
    a = np.zeros((S, n), dtype=np.float64)
    for s in range(S):
        for l in range(first_layer, L):
            kt = rope_rotate(bf16_to_f64(k_plane[l, s]), deltas[s], theta, style)   # [H][n][hd]
            for h in range(Hq):
                qh = bf16_to_f64(q[l, h])                                           # [T][hd]
                logits = (qh @ kt[h // group].T) / math.sqrt(hd)                   # [T][n]
                a[s] += softmax(logits).sum(axis=0)
    return a.astype(np.float32)


# ----------------------------------------------------------------------------
# a7: paged addressing
# (TD Algorithm 1: the restored rows are written through the slot mapping S
#  into paged KV memory)
# Layout [layer][page][page_size][kv_head][head_dim]; token j of segment s
# lives on page page_table[s][j // page_size], slot j % page_size.
# ----------------------------------------------------------------------------


def paged_offset(page_table: np.ndarray, page_size: int, s_layer: int, s_page: int,
                 s_token: int, s_head: int, l: int, s: int, h: int, j: int) -> int:
    """Element offset of row (layer l, segment s, head h, token j) in the pool."""
    page = int(page_table[s, j // page_size])
    return l * s_layer + page * s_page + (j % page_size) * s_token + h * s_head


def paged_gather(pool: np.ndarray, page_table: np.ndarray, page_size: int, n_layers: int,
                 n_heads: int, n_tokens: int, head_dim: int) -> np.ndarray:
    """Logical plane [L][S][H][n][hd] read row by row from a paged pool.

    pool: flat array laid out [layer][page][page_size][kv_head][head_dim].
    """
    S = page_table.shape[0]
    n_pages = pool.size // (n_layers * page_size * n_heads * head_dim)
    s_token, s_head = n_heads * head_dim, head_dim
    s_page = page_size * s_token
    s_layer = n_pages * s_page
    out = np.empty((n_layers, S, n_heads, n_tokens, head_dim), dtype=pool.dtype)
    for l in range(n_layers):
        for s in range(S):
            for h in range(n_heads):
                for j in range(n_tokens):
                    o = paged_offset(page_table, page_size, s_layer, s_page, s_token, s_head,
                                     l, s, h, j)
                    out[l, s, h, j] = pool[o:o + head_dim]
    return out


def paged_scatter(pool: np.ndarray, plane: np.ndarray, page_table: np.ndarray,
                  page_size: int) -> None:
    """Write a logical plane row by row into a paged pool (in place)."""
    L, S, H, n, hd = plane.shape
    n_pages = pool.size // (L * page_size * H * hd)
    s_token, s_head = H * hd, hd
    s_page = page_size * s_token
    s_layer = n_pages * s_page
    for l in range(L):
        for s in range(S):
            for h in range(H):
                for j in range(n):
                    o = paged_offset(page_table, page_size, s_layer, s_page, s_token, s_head,
                                     l, s, h, j)
                    pool[o:o + hd] = plane[l, s, h, j]


# ----------------------------------------------------------------------------
# a8 / a9: master-mirror block-sparse diff
# (TD §4.3 "master-mirror layout" and "block-sparse diff representation": one
#  dense master, each sibling stored as the blocks that differ from it, with
#  one shared index list when K and V touch the same blocks (§5); TD §4.4 and
#  Algorithm 1: restore = load master block, overwrite the diff blocks,
#  RoPERecover, write — no dense mirror is built first)
# ----------------------------------------------------------------------------


def diff_encode(master_k: np.ndarray, master_v: np.ndarray, sib_k: np.ndarray,
                sib_v: np.ndarray, to_master: Sequence[int], theta: float, eps: float,
                block_tokens: int, style: str = "half", dtype: str = "bf16") -> dict:
    """Block-sparse diff of every sibling against the master (storage `dtype`).

    master_*: [L][1][H][n][hd]; sib_*: [L][A][H][n][hd].  Sibling a's keys are
    first re-aligned into the master's frame by to_master[a] positions.  Block
    (a, l, beta) = tokens [beta*bt, min(n, beta*bt+bt)) of every head; it is
    listed when any element of K or V differs from the master by more than
    eps.  Listed blocks are packed in (agent, layer, block)-ascending order.

    Returns dict: mask uint32 [A][L][ceil(nb/32)], offsets int64 [A*L+1]
    (exclusive prefix count per (agent, layer)), block_idx int32 [total],
    vals_k / vals_v [total][H][bt][hd] in the storage dtype (rows past a
    ragged tail = 0), total int.
    """
    L, A, H, n, hd = sib_k.shape
    bt = block_tokens
    nb = (n + bt - 1) // bt
    mask = np.zeros((A, L, (nb + 31) // 32), dtype=np.uint32)
    listed = []                                          # (a, l, beta) in ascending order
    packed_k, packed_v = [], []
    mk_all = to_f64(master_k[:, 0], dtype)               # [L][H][n][hd]
    mv_all = to_f64(master_v[:, 0], dtype)
    for a in range(A):
        for l in range(L):
            xk = rope_rotate(to_f64(sib_k[l, a], dtype), to_master[a], theta, style)
            xv = to_f64(sib_v[l, a], dtype)
            for beta in range(nb):
                t0, t1 = beta * bt, min(n, beta * bt + bt)
                dk = np.abs(xk[:, t0:t1] - mk_all[l][:, t0:t1]).max()
                dv = np.abs(xv[:, t0:t1] - mv_all[l][:, t0:t1]).max()
                if dk > eps or dv > eps:
                    mask[a, l, beta // 32] |= np.uint32(1) << np.uint32(beta % 32)
                    listed.append((a, l, beta))
                    pk = np.zeros((H, bt, hd), dtype=sib_k.dtype)
                    pv = np.zeros((H, bt, hd), dtype=sib_v.dtype)
                    pk[:, : t1 - t0] = store(xk[:, t0:t1], dtype)
                    pv[:, : t1 - t0] = sib_v[l, a][:, t0:t1]
                    packed_k.append(pk)
                    packed_v.append(pv)
    counts = np.zeros(A * L, dtype=np.int64)
    for a, l, _ in listed:
        counts[a * L + l] += 1
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    total = len(listed)
    empty = np.zeros((0, H, bt, hd), dtype=sib_k.dtype)
    return {
        "mask": mask,
        "offsets": offsets,
        "block_idx": np.array([beta for _, _, beta in listed], dtype=np.int32),
        "vals_k": np.stack(packed_k) if total else empty,
        "vals_v": np.stack(packed_v) if total else empty.copy(),
        "total": total,
    }


def diff_decode(master_k: np.ndarray, master_v: np.ndarray, diff: dict,
                from_master: Sequence[int], theta: float, n_agents: int, block_tokens: int,
                style: str = "half", dtype: str = "bf16"):
    """Restore every sibling: master, overwritten by its listed blocks, keys rotated.

    Returns (out_k, out_v) [L][A][H][n][hd] in the storage dtype.
    """
    L, _, H, n, hd = master_k.shape
    A, bt = n_agents, block_tokens
    nb = (n + bt - 1) // bt
    out_k = np.empty((L, A, H, n, hd), dtype=master_k.dtype)
    out_v = np.empty((L, A, H, n, hd), dtype=master_v.dtype)
    offsets, mask = diff["offsets"], diff["mask"]
    for a in range(A):
        for l in range(L):
            k = master_k[l, 0].copy()
            v = master_v[l, 0].copy()
            slot = int(offsets[a * L + l])
            for beta in range(nb):
                if mask_bit(mask[a, l], beta):
                    t0, t1 = beta * bt, min(n, beta * bt + bt)
                    k[:, t0:t1] = diff["vals_k"][slot][:, : t1 - t0]
                    v[:, t0:t1] = diff["vals_v"][slot][:, : t1 - t0]
                    slot += 1
            out_k[l, a] = store(rope_rotate(to_f64(k, dtype), from_master[a], theta, style), dtype)
            out_v[l, a] = v
    return out_k, out_v


def select_master(scores: np.ndarray):
    """The group's master: the request with the lowest total deviation.

    TD §4.2 "reuse plan output": the reuse path accumulates a deviation score
    per request, and the master is the request whose restored cache is
    closest to the group's shared structure, usually the one with the lowest
    total deviation from the shared blocks.  Reading: the total of request a
    is the sum of its per-token deviation scores (the check-layer divergence
    of a2).  The pages fix no order of addition, so the oracle takes the sum
    itself: the exact sum of the float32 scores, rounded once to float64
    (math.fsum).  The master has the lowest total, ties to the lower request
    index.  scores: float32 [A][n] (no NaN).  Returns (master, totals float64 [A]).
    """
    scores = np.asarray(scores, dtype=np.float32)
    if np.isnan(scores).any():
        raise ValueError("NaN score")
    A, n = scores.shape
    if A == 0:
        raise ValueError("empty group")
    totals = np.array([math.fsum(float(x) for x in scores[a]) for a in range(A)],
                      dtype=np.float64)
    master = min(range(A), key=lambda a: (totals[a], a))
    return master, totals


def mirror_ratio(full_bytes: int, diff_bytes: int) -> float:
    """Compression R of one mirror: its dense size over its diff size
    (TD §6.4: R = 11.2 means a mirror costs about 9 % of a full cache)."""
    return full_bytes / diff_bytes


def group_cost(n_agents: int, ratio: float) -> float:
    """KV memory of a round in full caches under the master-mirror layout:
    one master plus N - 1 mirrors at 1/R each (TD §6.4, implied capacity)."""
    return 1.0 + (n_agents - 1) / ratio

"""Thin Python binding of the kvfix C ABI (include/kvfix.h).

Argument marshalling only: every function here builds the C structs from
torch tensors that already live in device memory, calls the function of the
same name in libkvfix.so on torch's current stream, and raises KvfixError on
a non-OK status.  No step of the correction is computed in Python.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvfix.so")

F32, BF16 = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
STATUS = {0: "KVFIX_OK", 1: "KVFIX_ERR_ARG", 2: "KVFIX_ERR_ALIGN", 3: "KVFIX_ERR_CAPACITY",
          4: "KVFIX_ERR_HIP", 5: "KVFIX_ERR_UNSUPPORTED"}

EXPORTS = ("kvfix_rope_shift", "kvfix_score", "kvfix_score_draft_workspace", "kvfix_score_draft",
           "kvfix_select_topb", "kvfix_chunk_budget", "kvfix_chunk_means", "kvfix_expand_chunks",
           "kvfix_select_grow", "kvfix_score_ex", "kvfix_fit_mean_ex", "kvfix_apply_ex",
           "kvfix_select_master", "kvfix_anchor_match_workspace", "kvfix_anchor_match",
           "kvfix_anchor_apply",
           "kvfix_fit_mean_workspace", "kvfix_fit_mean", "kvfix_fit_mean_noalloc", "kvfix_apply",
           "kvfix_diff_encode_workspace",
           "kvfix_diff_encode", "kvfix_diff_decode_workspace", "kvfix_diff_decode",
           "kvfix_status_string", "kvfix_version")


class KvfixError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class c_plane(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_segs", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("s_layer", ctypes.c_int64), ("s_seg", ctypes.c_int64),
                ("s_head", ctypes.c_int64), ("s_token", ctypes.c_int64),
                ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_seg", ctypes.c_int32), ("s_page", ctypes.c_int64),
                ("n_pool_pages", ctypes.c_int64)]


class c_rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("style", ctypes.c_int32),
                ("delta", ctypes.c_void_p)]


class c_lowrank(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("rank", ctypes.c_int32),
                ("sA_layer", ctypes.c_int64), ("sA_seg", ctypes.c_int64),
                ("sA_head", ctypes.c_int64), ("sB_layer", ctypes.c_int64),
                ("sB_seg", ctypes.c_int64), ("sB_head", ctypes.c_int64)]


class c_diff(ctypes.Structure):
    _fields_ = [("mask", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("block_idx", ctypes.c_void_p), ("vals_k", ctypes.c_void_p),
                ("vals_v", ctypes.c_void_p), ("capacity_blocks", ctypes.c_int64),
                ("block_tokens", ctypes.c_int32)]


class c_anchor_pool(ctypes.Structure):
    _fields_ = [("n_anchors", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("n_max", ctypes.c_int64), ("lengths", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("bt", ctypes.c_void_p)]


class c_granularity(ctypes.Structure):
    _fields_ = [("per_head", ctypes.c_int32), ("cover", ctypes.c_void_p)]


def _granularity(per_head: bool, cover: Optional[torch.Tensor]):
    """ctypes options for the _ex calls, or None for the plain calls."""
    if not per_head and cover is None:
        return None
    return c_granularity(int(per_head), None if cover is None else cover.data_ptr())


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"kvfix library not built: {_LIB_PATH} is missing "
                              "(run python -m cross_context_kv_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "kvfix_rope_shift": [P, P, P, P],
            "kvfix_score": [P, I32, P, I32, P, P, P],
            "kvfix_score_draft_workspace": [I32, I32, I32, I32, I32, I32],
            "kvfix_score_draft": [P, I32, I32, P, I32, P, P, P, ctypes.c_size_t, P],
            "kvfix_select_topb": [P, I32, I32, I32, P, P, P],
            "kvfix_chunk_budget": [I64, I32, I64, I64, I32],
            "kvfix_chunk_means": [P, I32, I32, I32, P, P],
            "kvfix_expand_chunks": [P, I32, I32, I32, I32, P, P, P, P],
            "kvfix_select_grow": [P, I32, I32, I32, ctypes.c_double, P, P, P],
            "kvfix_score_ex": [P, I32, P, I32, P, P, P, P],
            "kvfix_fit_mean_ex": [P, I32, P, P, P, I32, P, P, P, P, P, ctypes.c_size_t, P],
            "kvfix_apply_ex": [P, P, P, P, F, F, P, P, P, P, P],
            "kvfix_select_master": [P, I32, I32, P, P, P],
            "kvfix_anchor_match_workspace": [I32, I32, I32, I32],
            "kvfix_anchor_match": [P, P, I32, P, I64, ctypes.c_double, I32, I64, ctypes.c_double,
                                   P, P, P, P, ctypes.c_size_t, P],
            "kvfix_anchor_apply": [P, P, I32, P, P, I64, I64, ctypes.c_double, I32, P, P, P],
            "kvfix_fit_mean_workspace": [I32, I32, I32, I32, I32],
            "kvfix_fit_mean": [P, I32, P, P, P, I32, P, P, P, P, ctypes.c_size_t, P],
            "kvfix_fit_mean_noalloc": [P, I32, P, P, P, I32, P, P, P, P],
            "kvfix_apply": [P, P, P, P, F, F, P, P, P, P],
            "kvfix_diff_encode_workspace": [I32, I32, I32, I32],
            "kvfix_diff_encode": [P, P, P, P, P, F, P, P, P, ctypes.c_size_t, P],
            "kvfix_diff_decode_workspace": [I32, I32],
            "kvfix_diff_decode": [P, P, P, P, P, P, P, ctypes.c_size_t, P],
            "kvfix_status_string": [I32],
            "kvfix_version": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        L.kvfix_chunk_budget.restype = ctypes.c_int64
        L.kvfix_score_draft_workspace.restype = ctypes.c_size_t
        L.kvfix_fit_mean_workspace.restype = ctypes.c_size_t
        L.kvfix_diff_encode_workspace.restype = ctypes.c_size_t
        L.kvfix_diff_decode_workspace.restype = ctypes.c_size_t
        L.kvfix_anchor_match_workspace.restype = ctypes.c_size_t
        L.kvfix_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvfixError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported plane dtype {t.dtype}")


class Plane:
    """A K or V plane over device memory.

    dense(t):  t shaped [L, S, H, n, hd] with any element strides (hd contiguous).
    paged(pool, page_table, page_size, n_tokens): pool shaped
      [L, n_pages, page_size, H, hd]; page_table int32 [S, pages_per_seg].
    """

    def __init__(self, struct: c_plane, keep: Sequence[torch.Tensor]):
        self.c = struct
        self._keep = list(keep)          # keep the tensors alive with the struct

    @staticmethod
    def dense(t: torch.Tensor) -> "Plane":
        if t.dim() != 5:
            raise ValueError("dense plane must be [L, S, H, n, hd]")
        L, S, H, n, hd = t.shape
        sl, ss, sh, sn, sd = t.stride()
        if sd != 1 and hd > 1 and t.numel() > 0:
            raise ValueError("head_dim must be contiguous")
        c = c_plane(t.data_ptr(), _dtype(t), L, S, H, n, hd, sl, ss, sh, sn,
                    None, 0, 0, 0, 0)
        return Plane(c, [t])

    @staticmethod
    def paged(pool: torch.Tensor, page_table: torch.Tensor, page_size: int,
              n_tokens: int) -> "Plane":
        if pool.dim() != 5 or not pool.is_contiguous():
            raise ValueError("pool must be a contiguous [L, n_pages, page_size, H, hd] tensor")
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 [S, pages_per_seg] tensor")
        L, n_pages, ps, H, hd = pool.shape
        if ps != page_size:
            raise ValueError("pool page dimension differs from page_size")
        S, pps = page_table.shape
        sl, sp, st, sh, _ = pool.stride()
        c = c_plane(pool.data_ptr(), _dtype(pool), L, S, H, n_tokens, hd, sl, 0, sh, st,
                    page_table.data_ptr(), page_size, pps, sp, n_pages)
        return Plane(c, [pool, page_table])

    def ref(self):
        return ctypes.byref(self.c)


def make_rope(delta: torch.Tensor, theta: float, style: int = ROPE_HALF):
    """Rotary shift description over a device int64 [n_segs] tensor of shifts."""
    if delta.dtype != torch.int64 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous int64 tensor")
    r = c_rope(float(theta), int(style), delta.data_ptr())
    return r, delta


def make_lowrank(A: Optional[torch.Tensor], B: Optional[torch.Tensor]):
    """Rank-r state over fp32 A [L, S, H, n, r] and B [L, S, H, r, hd] (dense strides)."""
    if A is None:
        return None
    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise TypeError("rank state must be float32")
    if A.stride(-1) != 1 or A.stride(-2) != A.shape[-1] or B.stride(-1) != 1 or \
            B.stride(-2) != B.shape[-1]:
        raise ValueError("A rows and B rows must be contiguous")
    r = A.shape[-1]
    c = c_lowrank(A.data_ptr(), B.data_ptr(), r, A.stride(0), A.stride(1), A.stride(2),
                  B.stride(0), B.stride(1), B.stride(2))
    return c, (A, B)


def kvfix_rope_shift(src: Plane, dst: Plane, delta: torch.Tensor, theta: float,
                     style: int = ROPE_HALF) -> None:
    r, _ = make_rope(delta, theta, style)
    _check("kvfix_rope_shift", lib().kvfix_rope_shift(src.ref(), dst.ref(), ctypes.byref(r),
                                                      _stream()))


def kvfix_score(fresh: Plane, fresh_layer: int, reuse: Plane, reuse_layer: int,
                scores: torch.Tensor, delta: Optional[torch.Tensor] = None, theta: float = 0.0,
                style: int = ROPE_HALF, per_head: bool = False) -> None:
    """per_head: scores [n_segs][n_heads][n] (kvfix_score_ex)."""
    rr = None
    if delta is not None:
        r, _ = make_rope(delta, theta, style)
        rr = ctypes.byref(r)
    g = _granularity(per_head, None)
    if g is None:
        _check("kvfix_score", lib().kvfix_score(fresh.ref(), fresh_layer, reuse.ref(),
                                                reuse_layer, rr, _ptr(scores), _stream()))
    else:
        _check("kvfix_score_ex", lib().kvfix_score_ex(fresh.ref(), fresh_layer, reuse.ref(),
                                                      reuse_layer, rr, ctypes.byref(g),
                                                      _ptr(scores), _stream()))


def kvfix_select_topb(scores: torch.Tensor, b: int, idx: torch.Tensor,
                      mask: torch.Tensor) -> None:
    n_rows, n = scores.shape
    _check("kvfix_select_topb", lib().kvfix_select_topb(_ptr(scores), n_rows, n, b, _ptr(idx),
                                                        _ptr(mask), _stream()))


BUDGET_SKIP, BUDGET_AT_LEAST_ONE = 0, 1


def kvfix_chunk_budget(n_tokens: int, chunk: int, rho_num: int, rho_den: int,
                       rule: int = BUDGET_SKIP) -> int:
    c = int(lib().kvfix_chunk_budget(n_tokens, chunk, rho_num, rho_den, rule))
    if c < 0:
        raise KvfixError("kvfix_chunk_budget", 1)
    return c


def kvfix_chunk_means(scores: torch.Tensor, chunk: int, means: torch.Tensor) -> None:
    n_rows, n = scores.shape
    _check("kvfix_chunk_means", lib().kvfix_chunk_means(_ptr(scores), n_rows, n, chunk,
                                                        _ptr(means), _stream()))


def kvfix_expand_chunks(chunk_idx: torch.Tensor, n: int, chunk: int, idx: torch.Tensor,
                        counts: torch.Tensor, mask: torch.Tensor) -> None:
    n_rows, c = chunk_idx.shape
    _check("kvfix_expand_chunks", lib().kvfix_expand_chunks(
        _ptr(chunk_idx), n_rows, c, n, chunk, _ptr(idx), _ptr(counts), _ptr(mask), _stream()))


def kvfix_select_grow(scores: torch.Tensor, b: int, tau: float, idx: torch.Tensor,
                      mask: torch.Tensor) -> None:
    n_rows, n = scores.shape
    _check("kvfix_select_grow", lib().kvfix_select_grow(_ptr(scores), n_rows, n, b, float(tau),
                                                        _ptr(idx), _ptr(mask), _stream()))


def kvfix_select_master(scores: torch.Tensor, totals: torch.Tensor, master: torch.Tensor) -> None:
    """scores fp32 [n_agents][n]; totals fp64 [n_agents]; master int32 [1] (all device)."""
    A, n = scores.shape
    _check("kvfix_select_master", lib().kvfix_select_master(_ptr(scores), A, n, _ptr(totals),
                                                            _ptr(master), _stream()))


def kvfix_fit_mean_workspace(n_layers: int, n_segs: int, n_heads: int, head_dim: int,
                             b: int) -> int:
    return int(lib().kvfix_fit_mean_workspace(n_layers, n_segs, n_heads, head_dim, b))


def kvfix_fit_mean(fresh: Plane, reuse: Plane, out: Optional[Plane], idx: torch.Tensor, b: int,
                   mu: torch.Tensor, delta: Optional[torch.Tensor] = None, theta: float = 0.0,
                   style: int = ROPE_HALF, A=None, B=None, fresh_by_slot: bool = False,
                   ws: Optional[torch.Tensor] = None, per_head: bool = False,
                   cover: Optional[torch.Tensor] = None) -> None:
    """ws: device workspace (any dtype) of at least kvfix_fit_mean_workspace bytes; a
    fresh one is allocated through torch when omitted.  per_head / cover: the
    kvfix_fit_mean_ex options (idx [n_segs][n_heads][b]; cover int32 [n_segs])."""
    rr = None
    if delta is not None:
        r, _ = make_rope(delta, theta, style)
        rr = ctypes.byref(r)
    lr = make_lowrank(A, B)
    lrp = ctypes.byref(lr[0]) if lr else None
    c = reuse.c
    need = kvfix_fit_mean_workspace(c.n_layers, c.n_segs, c.n_heads, c.head_dim, b)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=mu.device)
    g = _granularity(per_head, cover)
    if g is None:
        _check("kvfix_fit_mean", lib().kvfix_fit_mean(
            fresh.ref(), int(fresh_by_slot), reuse.ref(), out.ref() if out else None, _ptr(idx),
            b, rr, lrp, _ptr(mu), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    else:
        _check("kvfix_fit_mean_ex", lib().kvfix_fit_mean_ex(
            fresh.ref(), int(fresh_by_slot), reuse.ref(), out.ref() if out else None, _ptr(idx),
            b, rr, lrp, ctypes.byref(g), _ptr(mu), _ptr(ws), ws.numel() * ws.element_size(),
            _stream()))


NOALLOC_SCRATCH_BYTES = 64 << 20


def kvfix_fit_mean_noalloc(fresh: Plane, reuse: Plane, out: Optional[Plane], idx: torch.Tensor,
                           b: int, mu: torch.Tensor, delta: Optional[torch.Tensor] = None,
                           theta: float = 0.0, style: int = ROPE_HALF, A=None, B=None,
                           fresh_by_slot: bool = False) -> None:
    """kvfix_fit_mean with the library's own per-device buffer instead of a
    workspace (no allocation by the library or here)."""
    rr = None
    if delta is not None:
        r, _ = make_rope(delta, theta, style)
        rr = ctypes.byref(r)
    lr = make_lowrank(A, B)
    lrp = ctypes.byref(lr[0]) if lr else None
    _check("kvfix_fit_mean_noalloc", lib().kvfix_fit_mean_noalloc(
        fresh.ref(), int(fresh_by_slot), reuse.ref(), out.ref() if out else None, _ptr(idx), b,
        rr, lrp, _ptr(mu), _stream()))


def kvfix_apply(reuse: Plane, out: Plane, mask: Optional[torch.Tensor], mu: torch.Tensor,
                scores: Optional[torch.Tensor] = None, w_lo: float = 0.0, w_hi: float = 1.0,
                delta: Optional[torch.Tensor] = None, theta: float = 0.0, style: int = ROPE_HALF,
                A=None, B=None, per_head: bool = False,
                cover: Optional[torch.Tensor] = None) -> None:
    """per_head / cover: the kvfix_apply_ex options (mask [n_segs][n_heads][words],
    scores [n_segs][n_heads][n]; cover int32 [n_segs])."""
    rr = None
    if delta is not None:
        r, _ = make_rope(delta, theta, style)
        rr = ctypes.byref(r)
    lr = make_lowrank(A, B)
    lrp = ctypes.byref(lr[0]) if lr else None
    g = _granularity(per_head, cover)
    if g is None:
        _check("kvfix_apply", lib().kvfix_apply(reuse.ref(), out.ref(), _ptr(mask), _ptr(scores),
                                                float(w_lo), float(w_hi), _ptr(mu), lrp, rr,
                                                _stream()))
    else:
        _check("kvfix_apply_ex", lib().kvfix_apply_ex(reuse.ref(), out.ref(), _ptr(mask),
                                                      _ptr(scores), float(w_lo), float(w_hi),
                                                      _ptr(mu), lrp, rr, ctypes.byref(g),
                                                      _stream()))


def kvfix_score_draft_workspace(n_segs: int, n_layers: int, first_layer: int, n_q_heads: int,
                                n_draft: int, n_tokens: int) -> int:
    return int(lib().kvfix_score_draft_workspace(n_segs, n_layers, first_layer, n_q_heads,
                                                 n_draft, n_tokens))


def kvfix_score_draft(q: torch.Tensor, k: Plane, first_layer: int, delta: torch.Tensor,
                      theta: float, scores: torch.Tensor, ws: torch.Tensor,
                      style: int = ROPE_HALF) -> None:
    """q: bf16 [S, L, Hq, T, hd] contiguous."""
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 5:
        raise ValueError("q must be a contiguous bf16 [S, L, Hq, T, hd] tensor")
    r, _ = make_rope(delta, theta, style)
    _check("kvfix_score_draft", lib().kvfix_score_draft(
        _ptr(q), q.shape[2], q.shape[3], k.ref(), first_layer, ctypes.byref(r), _ptr(scores),
        _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def kvfix_diff_encode_workspace(n_agents: int, n_layers: int, n_tokens: int,
                                block_tokens: int) -> int:
    return int(lib().kvfix_diff_encode_workspace(n_agents, n_layers, n_tokens, block_tokens))


class Diff:
    """Device buffers of a block-sparse diff (see kvfix_diff in include/kvfix.h)."""

    def __init__(self, n_agents: int, n_layers: int, n_tokens: int, n_heads: int, head_dim: int,
                 block_tokens: int, capacity_blocks: int, dtype=torch.bfloat16, device="cuda"):
        nb = -(-n_tokens // block_tokens)
        self.n_agents, self.n_layers, self.n_blocks = n_agents, n_layers, nb
        self.block_tokens, self.capacity = block_tokens, capacity_blocks
        self.mask = torch.zeros(n_agents, n_layers, -(-nb // 32), dtype=torch.int32,
                                device=device)
        self.offsets = torch.zeros(n_agents * n_layers + 1, dtype=torch.int64, device=device)
        self.block_idx = torch.zeros(max(capacity_blocks, 1), dtype=torch.int32, device=device)
        shape = (max(capacity_blocks, 1), n_heads, block_tokens, head_dim)
        self.vals_k = torch.zeros(shape, dtype=dtype, device=device)
        self.vals_v = torch.zeros(shape, dtype=dtype, device=device)

    def c(self) -> c_diff:
        return c_diff(self.mask.data_ptr(), self.offsets.data_ptr(), self.block_idx.data_ptr(),
                      self.vals_k.data_ptr(), self.vals_v.data_ptr(), self.capacity,
                      self.block_tokens)


def kvfix_diff_encode(master_k: Plane, master_v: Plane, sib_k: Plane, sib_v: Plane,
                      to_master: torch.Tensor, theta: float, eps: float, diff: Diff,
                      dev_status: torch.Tensor, ws: torch.Tensor, style: int = ROPE_HALF) -> None:
    r, _ = make_rope(to_master, theta, style)
    d = diff.c()
    _check("kvfix_diff_encode", lib().kvfix_diff_encode(
        master_k.ref(), master_v.ref(), sib_k.ref(), sib_v.ref(), ctypes.byref(r), float(eps),
        ctypes.byref(d), _ptr(dev_status), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def kvfix_diff_decode_workspace(n_agents: int, head_dim: int) -> int:
    return int(lib().kvfix_diff_decode_workspace(n_agents, head_dim))


def kvfix_diff_decode(master_k: Plane, master_v: Plane, diff: Diff, from_master: torch.Tensor,
                      theta: float, out_k: Plane, out_v: Plane, ws: torch.Tensor,
                      style: int = ROPE_HALF) -> None:
    r, _ = make_rope(from_master, theta, style)
    d = diff.c()
    _check("kvfix_diff_decode", lib().kvfix_diff_decode(
        master_k.ref(), master_v.ref(), ctypes.byref(d), ctypes.byref(r), out_k.ref(),
        out_v.ref(), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


ANCHOR_MAX, ANCHOR_RANK = 16, 32


class AnchorPool:
    """Factors of an anchor pool: a [V, L, 2, n_max, r] and bt [V, L, 2, H*hd, r],
    device tensors of bfloat16 (or their uint16/int16 bit patterns), plus the
    host list of stored lengths."""

    def __init__(self, a: torch.Tensor, bt: torch.Tensor, lengths: Sequence[int]):
        if a.dim() != 5 or bt.dim() != 5 or not a.is_contiguous() or not bt.is_contiguous():
            raise ValueError("a and bt must be contiguous 5-d tensors")
        if a.element_size() != 2 or bt.element_size() != 2:
            raise ValueError("a and bt must hold bf16 values")
        V = a.shape[0]
        if bt.shape[0] != V or len(lengths) != V:
            raise ValueError("a, bt and lengths disagree on the anchor count")
        self.a, self.bt = a, bt
        self.lengths = [int(x) for x in lengths]
        self._len = (ctypes.c_int32 * max(V, 1))(*self.lengths)
        self.c = c_anchor_pool(V, a.shape[4], a.shape[3], ctypes.addressof(self._len),
                               a.data_ptr(), bt.data_ptr())

    def ref(self):
        return ctypes.byref(self.c)


def kvfix_anchor_match_workspace(n_layers: int, n_heads: int, n_tokens: int,
                                 n_anchors: int) -> int:
    return int(lib().kvfix_anchor_match_workspace(n_layers, n_heads, n_tokens, n_anchors))


def kvfix_anchor_match(src_k: Plane, src_v: Plane, seg: int, base: AnchorPool, src_off: int,
                       theta: float, k_gate: int, tau: float, weights: torch.Tensor,
                       gate: torch.Tensor, accept: torch.Tensor, ws: torch.Tensor,
                       style: int = ROPE_HALF) -> None:
    _check("kvfix_anchor_match", lib().kvfix_anchor_match(
        src_k.ref(), src_v.ref(), seg, base.ref(), int(src_off), float(theta), style, int(k_gate),
        float(tau), _ptr(weights), _ptr(gate), _ptr(accept), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def kvfix_anchor_apply(src_k: Plane, src_v: Plane, seg: int, delta: AnchorPool,
                       weights: Optional[torch.Tensor], src_off: int, tgt_off: int, theta: float,
                       out_k: Plane, out_v: Plane, style: int = ROPE_HALF) -> None:
    _check("kvfix_anchor_apply", lib().kvfix_anchor_apply(
        src_k.ref(), src_v.ref(), seg, delta.ref(), _ptr(weights), int(src_off), int(tgt_off),
        float(theta), style, out_k.ref(), out_v.ref(), _stream()))

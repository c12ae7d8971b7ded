"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments with a status before touching a GPU."""
import ctypes
import os
import re

import pytest

import cross_context_kv_amd.kvfix as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfix.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kv._LIB_PATH),
                                reason="libkvfix.so not built (run the build first)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvfix_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_calls():
    names = declared_functions()
    assert set(names) == set(kv.EXPORTS), names


def test_library_exports_every_declared_symbol():
    L = kv.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.kvfix_version() == 100


def test_status_strings():
    L = kv.lib()
    for code, name in kv.STATUS.items():
        assert L.kvfix_status_string(code).decode().startswith(name)


def plane(**kw):
    base = dict(data=256, dtype=kv.BF16, n_layers=2, n_segs=1, n_heads=2, n_tokens=64,
                head_dim=128, s_layer=2 * 64 * 128, s_seg=2 * 64 * 128, s_head=64 * 128,
                s_token=128, page_table=None, page_size=0, pages_per_seg=0, s_page=0,
                n_pool_pages=0)
    base.update(kw)
    return kv.c_plane(**base)


def rope(**kw):
    base = dict(theta=1e4, style=kv.ROPE_HALF, delta=4096)
    base.update(kw)
    return kv.c_rope(**base)


R = ctypes.byref


@pytest.mark.parametrize("bad,status", [
    (dict(data=None), 1),
    (dict(dtype=7), 5),
    (dict(head_dim=96), 5),
    (dict(head_dim=100), 5),
    (dict(n_tokens=-1), 1),
    (dict(s_token=-128), 1),
    (dict(data=258), 2),
    (dict(s_token=129), 2),
    (dict(page_table=4096, page_size=16, pages_per_seg=3, s_page=4096, n_pool_pages=8), 1),
    (dict(page_table=4096, page_size=0, pages_per_seg=4, s_page=4096, n_pool_pages=8), 1),
    (dict(page_table=4096, page_size=16, pages_per_seg=4, s_page=4097, n_pool_pages=8), 2),
])
def test_plane_validation(bad, status):
    L = kv.lib()
    p, good = plane(**bad), plane()
    mu = ctypes.c_void_p(512)
    assert L.kvfix_apply(R(p), R(good), None, None, 0.0, 1.0, mu, None, None, None) == status
    assert L.kvfix_rope_shift(R(p), R(good), R(rope()), None) == status


def test_call_level_validation():
    L = kv.lib()
    p, mu = plane(), ctypes.c_void_p(512)
    # shapes must agree
    assert L.kvfix_apply(R(p), R(plane(n_heads=3)), None, None, 0.0, 1.0, mu, None, None, None) == 1
    assert L.kvfix_apply(R(p), R(p), None, None, 0.0, 1.0, None, None, None, None) == 1
    # the mean must be 16-byte aligned (it is read as vectors)
    assert L.kvfix_apply(R(p), R(p), None, None, 0.0, 1.0, ctypes.c_void_p(516), None, None,
                         None) == 2
    # weights need lo <= hi
    assert L.kvfix_apply(R(p), R(p), None, ctypes.c_void_p(512), 2.0, 1.0, mu, None, None, None) == 1
    # rotary arguments
    assert L.kvfix_rope_shift(R(p), R(p), None, None) == 1
    assert L.kvfix_rope_shift(R(p), R(p), R(rope(delta=None)), None) == 1
    assert L.kvfix_rope_shift(R(p), R(p), R(rope(style=3)), None) == 1
    assert L.kvfix_rope_shift(R(p), R(p), R(rope(theta=0.0)), None) == 1
    assert L.kvfix_rope_shift(R(p), R(plane(n_layers=3)), R(rope()), None) == 1
    # rank state
    lr = kv.c_lowrank(A=512, B=512, rank=9)
    assert L.kvfix_apply(R(p), R(p), None, None, 0.0, 1.0, mu, R(lr), None, None) == 5
    lr = kv.c_lowrank(A=None, B=512, rank=2)
    assert L.kvfix_apply(R(p), R(p), None, None, 0.0, 1.0, mu, R(lr), None, None) == 1
    # score layers in range
    sc = ctypes.c_void_p(512)
    assert L.kvfix_score(R(p), 2, R(p), 0, None, sc, None) == 1
    assert L.kvfix_score(R(p), 0, R(p), -1, None, sc, None) == 1
    assert L.kvfix_score(R(p), 0, R(p), 0, None, None, None) == 1
    # select: 0 <= b <= n
    assert L.kvfix_select_topb(sc, 1, 10, 11, ctypes.c_void_p(512), ctypes.c_void_p(512), None) == 1
    assert L.kvfix_select_topb(sc, 1, 10, -1, ctypes.c_void_p(512), ctypes.c_void_p(512), None) == 1
    assert L.kvfix_select_topb(None, 1, 10, 3, ctypes.c_void_p(512), ctypes.c_void_p(512), None) == 1
    # fit_mean: b (the list width) >= 0, idx needed when b > 0, fresh rows by
    # slot need >= b rows
    assert L.kvfix_fit_mean(R(p), 0, R(p), None, None, 3, None, None, mu, None, 0, None) == 1
    assert L.kvfix_fit_mean(R(p), 0, R(p), None, ctypes.c_void_p(512), -1, None, None, mu, None, 0, None) == 1
    assert L.kvfix_fit_mean(R(plane(n_tokens=2)), 1, R(p), None, ctypes.c_void_p(512), 3, None,
                            None, mu, None, 0, None) == 1
    assert L.kvfix_fit_mean(R(plane(n_tokens=3)), 0, R(p), None, ctypes.c_void_p(512), 3, None,
                            None, mu, None, 0, None) == 1
    # the workspace must hold every slice's partial sums
    need = L.kvfix_fit_mean_workspace(2, 1, 2, 128, 3)
    assert need == 2 * 1 * 2 * 1 * (128 + 8 + 1) * 8      # sums, rank-state sums, member count
    # a list wider than n (padded whole chunks) is accepted
    assert L.kvfix_fit_mean_workspace(2, 1, 2, 128, 100) == need
    assert L.kvfix_fit_mean(R(p), 0, R(p), None, ctypes.c_void_p(512), 3, None, None, mu,
                            ctypes.c_void_p(4096), need - 8, None) == 1
    assert L.kvfix_fit_mean(R(p), 0, R(p), None, ctypes.c_void_p(512), 3, None, None, mu,
                            None, need, None) == 1


def test_empty_shapes_are_noops_without_launch():
    L = kv.lib()
    mu = ctypes.c_void_p(512)
    for kw in (dict(n_tokens=0), dict(n_layers=0), dict(n_segs=0), dict(n_heads=0)):
        p = plane(**kw)
        assert L.kvfix_apply(R(p), R(p), None, None, 0.0, 1.0, mu, None, None, None) == 0
        assert L.kvfix_rope_shift(R(p), R(p), R(rope()), None) == 0
    assert L.kvfix_select_topb(None, 0, 10, 3, None, None, None) == 0
    assert L.kvfix_select_topb(None, 4, 0, 0, None, None, None) == 0


def anchor_pool(V=3, rank=32, n_max=64, lengths=None, a=4096, bt=8192):
    lens = (ctypes.c_int32 * max(V, 1))(*(lengths if lengths is not None else [n_max] * V))
    pool = kv.c_anchor_pool(V, rank, n_max, ctypes.addressof(lens), a, bt)
    pool._lens = lens                   # keep the host array alive
    return pool


def test_anchor_call_validation():
    L = kv.lib()
    p = plane()
    w, gate, acc = ctypes.c_void_p(512), ctypes.c_void_p(1024), ctypes.c_void_p(2048)
    up = lambda x: (x + 255) // 256 * 256                       # noqa: E731
    # distance sums per head group [L][2][V][G][n] (G = H / 2 for even H, else
    # H) and the gate's fp64 partials, [L][128-token blocks][G][V] then
    # [L][256-token blocks][V]
    need = L.kvfix_anchor_match_workspace(2, 2, 64, 3)
    assert need == up(2 * 2 * 3 * 1 * 64 * 4) + up(2 * 1 * 1 * 3 * 8) + up(2 * 1 * 3 * 8) + 256
    assert L.kvfix_anchor_match_workspace(2, 2, 300, 3) == \
        up(2 * 2 * 3 * 1 * 300 * 4) + up(2 * 3 * 1 * 3 * 8) + up(2 * 2 * 3 * 8) + 256
    assert L.kvfix_anchor_match_workspace(2, 3, 64, 3) == \
        up(2 * 2 * 3 * 3 * 64 * 4) + up(2 * 1 * 3 * 3 * 8) + up(2 * 1 * 3 * 8) + 256
    ws = ctypes.c_void_p(4096)

    def match(pk=p, pv=p, seg=0, pool=None, src_off=100, theta=1e4, style=kv.ROPE_HALF, k=64,
              tau=0.5, wts=w, g=gate, a=acc, wsp=ws, wsb=need):
        pool = anchor_pool() if pool is None else pool
        return L.kvfix_anchor_match(R(pk), R(pv), seg, R(pool), src_off, theta, style, k, tau,
                                    wts, g, a, wsp, wsb, None)

    def apply(pk=p, pv=p, seg=0, pool=None, wts=w, src_off=100, tgt_off=900, theta=1e4,
              style=kv.ROPE_HALF, ok=p, ov=p):
        pool = anchor_pool() if pool is None else pool
        return L.kvfix_anchor_apply(R(pk), R(pv), seg, R(pool), wts, src_off, tgt_off, theta,
                                    style, R(ok), R(ov), None)

    for call in (match, apply):
        assert call(pool=anchor_pool(rank=16)) == 5                 # rank must be 32
        assert call(pool=anchor_pool(V=17)) == 1                    # at most 16 anchors
        assert call(pool=anchor_pool(lengths=[64, 65, 3])) == 1     # a length past n_max
        assert call(pool=anchor_pool(lengths=[64, -1, 3])) == 1
        assert call(pool=anchor_pool(a=None)) == 1
        assert call(pool=anchor_pool(bt=8200)) == 2                 # factors 16-byte aligned
        assert call(pk=plane(dtype=kv.F32, s_layer=4 * 64 * 128, s_seg=4 * 64 * 128,
                             s_head=64 * 128, s_token=128)) == 1    # K and V must agree
        f32 = plane(dtype=kv.F32)
        assert call(pk=f32, pv=f32) == 5                            # bf16 planes only
        hd64 = plane(head_dim=64, s_token=64)
        assert call(pk=hd64, pv=hd64) == 5                          # head_dim 128 only
        assert call(seg=1) == 1 and call(seg=-1) == 1
        assert call(pv=plane(n_tokens=32)) == 1
        assert call(style=3) == 1 and call(theta=0.0) == 1
        assert call(src_off=(1 << 23) + 1) == 1                     # rotary angle range
    assert match(g=None) == 1 and match(a=None) == 1 and match(wsp=None) == 1
    assert match(wsb=need - 8) == 1
    assert match(wsp=ctypes.c_void_p(4096 + 128)) == 2              # 256-byte aligned
    assert match(tau=float("nan")) == 1
    assert match(wts=None) == 1                                     # weights needed with anchors
    assert apply(tgt_off=-(1 << 23) - 50) == 1                      # tgt - src out of range too
    assert apply(wts=None) == 1                                     # eligible anchors need weights
    assert apply(ok=plane(n_heads=3)) == 1
    # more blocks than one launch takes (heads x 256-token tiles x layer-plane
    # slots past 2^31 - 1): refused before any launch
    n_big, h_big = (1 << 31) - 1, 64
    big = plane(n_layers=2, n_heads=h_big, n_tokens=n_big, s_token=128, s_head=n_big * 128,
                s_seg=h_big * n_big * 128, s_layer=h_big * n_big * 128)
    assert apply(pk=big, pv=big, ok=big, ov=big, pool=anchor_pool(n_max=n_big)) == 1
    # no eligible anchor and no rows: nothing to launch
    assert apply(wts=None, pool=anchor_pool(lengths=[0, 0, 0]), pk=plane(n_layers=0),
                 pv=plane(n_layers=0), ok=plane(n_layers=0), ov=plane(n_layers=0)) == 0

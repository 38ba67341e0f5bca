"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host before any launch (no GPU needed: every
check runs before the first HIP call)."""
import ctypes
import os
import re

import pytest

from eagle_draft_trees_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "eagle_mi355x.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(d=256, H=4, Hkv=4, hd=64, F=688, V=4096, dtype=L.EAGLE_F32, B=1, D=3, k=2, m=6,
                max_prefix=70)
    base.update(kw)
    dims = L.EagleDims(base["d"], base["H"], base["Hkv"], base["hd"], base["F"], base["V"],
                       base["dtype"], 1e-6, 1e4)
    tc = L.EagleTreeCfg(base["B"], base["D"], base["k"], base["m"], base["max_prefix"])
    return dims, tc


def test_workspace_bytes_and_shape_checks():
    dims, tc = _cfg()
    n = L.eagle_workspace_bytes(dims, tc)
    assert n > 0 and n % 256 == 0
    bad = [dict(d=250), dict(hd=96, d=384), dict(H=4, Hkv=3), dict(k=0), dict(k=17),
           dict(m=1), dict(m=65), dict(D=1), dict(D=17), dict(k=2, D=2, m=8),  # m-1 > pool 6
           dict(max_prefix=6), dict(F=100), dict(F=0), dict(V=1, k=2), dict(dtype=7)]
    for kw in bad:
        d2, t2 = _cfg(**kw)
        assert L.eagle_workspace_bytes(d2, t2) == 0, kw
    # larger trees need more workspace
    d3, t3 = _cfg(B=4, k=4, m=16)
    assert L.eagle_workspace_bytes(d3, t3) > n


def _expect(status, fn):
    with pytest.raises(L.EagleError) as e:
        fn()
    assert e.value.status == status, str(e.value)


def test_entry_points_reject_bad_arguments_before_launch():
    dims, tc = _cfg()
    n = L.eagle_workspace_bytes(dims, tc)
    fake = 1 << 40  # never dereferenced: validation fails first
    ws = ctypes.c_void_p(fake)
    w = L.EagleWeights(*([fake] * 12), L.EAGLE_PACKED_WEIGHTS)
    st = L.EagleSeqState(fake, fake, fake, fake, fake)
    lib = L.lib()

    def level(level=2, flags=0, wsb=n, ws_ptr=fake, weights=w, state=st, dims_=dims, tc_=tc):
        return L._check(lib.eagle_draft_level(ctypes.byref(dims_), ctypes.byref(weights),
                                              ctypes.byref(tc_), ctypes.byref(state), level, flags,
                                              ws_ptr, wsb, None), "level")

    _expect(L.EAGLE_ERR_WORKSPACE, lambda: level(wsb=n - 256))
    _expect(L.EAGLE_ERR_ARG, lambda: level(ws_ptr=fake + 16))          # misaligned
    _expect(L.EAGLE_ERR_ARG, lambda: level(ws_ptr=None))
    _expect(L.EAGLE_ERR_ARG, lambda: level(level=0))
    _expect(L.EAGLE_ERR_ARG, lambda: level(level=4))
    _expect(L.EAGLE_ERR_ARG, lambda: level(flags=5))
    _expect(L.EAGLE_ERR_ARG, lambda: level(weights=L.EagleWeights(*([fake] * 11 + [0]), L.EAGLE_PACKED_WEIGHTS)))
    _expect(L.EAGLE_ERR_ARG, lambda: level(weights=L.EagleWeights(*([fake] * 12))))  # row-major
    assert "not packed" in L.eagle_last_error()
    _expect(L.EAGLE_ERR_ARG, lambda: level(state=L.EagleSeqState(fake, 0, fake, fake, fake)))
    d_bad, _ = _cfg(d=320)
    _expect(L.EAGLE_ERR_SHAPE, lambda: level(dims_=d_bad))
    assert "d 320" in L.eagle_last_error()
    _expect(L.EAGLE_ERR_ARG, lambda: L._check(
        lib.eagle_verify_greedy(ctypes.byref(tc), 4096, None, fake, fake, fake, fake, fake, None),
        "verify"))
    _expect(L.EAGLE_ERR_SHAPE, lambda: L._check(
        lib.eagle_verify_greedy(ctypes.byref(tc), 0, fake, fake, fake, fake, fake, fake, None),
        "verify"))
    need = lib.eagle_verify_relaxed_scratch_bytes(ctypes.byref(tc))
    assert need == tc.batch * tc.m * 16 * 8

    def relaxed(vocab=4096, T=1.0, thr=0.1, uni=fake, scr=fake, scr_bytes=need):
        return L._check(lib.eagle_verify_relaxed(ctypes.byref(tc), vocab, fake, fake, fake, T, thr,
                                                 uni, fake, fake, fake, scr, scr_bytes, None),
                        "relaxed")

    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(T=0.0))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(T=-1.0))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(T=float("inf")))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(T=float("nan")))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(thr=float("nan")))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(uni=None))
    _expect(L.EAGLE_ERR_SHAPE, lambda: relaxed(vocab=0))
    _expect(L.EAGLE_ERR_WORKSPACE, lambda: relaxed(scr_bytes=need - 8))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(scr=None))
    _expect(L.EAGLE_ERR_ARG, lambda: relaxed(scr=fake + 4))  # misaligned
    _expect(L.EAGLE_ERR_ARG, lambda: L._check(
        lib.eagle_draft_extend(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(tc),
                               ctypes.byref(st), None, fake, fake, fake, fake, fake, n, None),
        "extend"))
    _expect(L.EAGLE_ERR_ARG, lambda: L._check(
        lib.eagle_rerank_build_tree(ctypes.byref(dims), ctypes.byref(tc), ctypes.byref(st), fake,
                                    n, None, fake, None, None, None, None, None), "rerank"))
    assert L.eagle_status_str(L.EAGLE_ERR_WORKSPACE) == "workspace too small"


def test_ws_view_regions_are_inside_the_workspace():
    dims, tc = _cfg(B=2, k=3, D=4, m=9, V=1003, d=192, H=3, Hkv=1, F=400, max_prefix=49)
    n = L.eagle_workspace_bytes(dims, tc)
    base = 1 << 40
    spans = []
    for what in range(10):
        p, sz = ctypes.c_void_p(), ctypes.c_size_t()
        assert L.lib().eagle_ws_view(ctypes.byref(dims), ctypes.byref(tc), base, what,
                                     ctypes.byref(p), ctypes.byref(sz)) == 0
        off = p.value - base
        assert off % 256 == 0 and off + sz.value <= n
        spans.append((off, off + sz.value))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))  # regions do not overlap
    assert L.POOL_DTYPE.itemsize == 24 and L.FRONTIER_DTYPE.itemsize == 80


def _packed_bytes_formula(d, H, Hkv, hd, F, V, es):
    ks = 32 if es == 2 else 16
    cd = lambda a, b: -(-a // b)
    # the FC's feature half [d][d] is packed; its token half is the fp32 table [V][d]
    mats = [(d, d), (H * hd, d), (Hkv * hd, d), (Hkv * hd, d), (d, H * hd), (F, d), (F, d), (d, F), (V, d)]
    return (sum(cd(cd(n, 16) * 16 * cd(k, ks) * ks * es, 256) * 256 for n, k in mats)
            + cd(V * d * 4, 256) * 256)


def test_packed_weights_bytes_and_pack_validation():
    for dt, es in ((L.EAGLE_BF16, 2), (L.EAGLE_F32, 4)):
        dims, _ = _cfg(d=192, H=3, Hkv=1, F=400, V=1003)
        dims.dtype = dt
        assert L.eagle_packed_weights_bytes(dims) == _packed_bytes_formula(192, 3, 1, 64, 400, 1003, es)
    dims, _ = _cfg()
    need = L.eagle_packed_weights_bytes(dims)
    assert need > 0
    fake = 1 << 40
    src = L.EagleWeights(*([fake] * 12))
    out = L.EagleWeights()
    lib = L.lib()

    def pack(src_=src, dst=fake, n=need):
        return L._check(lib.eagle_pack_weights(ctypes.byref(dims), ctypes.byref(src_), dst, n,
                                                ctypes.byref(out), None), "pack")

    _expect(L.EAGLE_ERR_ARG, lambda: pack(dst=None))
    _expect(L.EAGLE_ERR_ARG, lambda: pack(dst=fake + 16))               # misaligned
    _expect(L.EAGLE_ERR_WORKSPACE, lambda: pack(n=need - 1))
    _expect(L.EAGLE_ERR_ARG, lambda: pack(src_=L.EagleWeights(*([fake] * 12),
                                                             packed=L.EAGLE_PACKED_WEIGHTS)))
    _expect(L.EAGLE_ERR_ARG, lambda: pack(src_=L.EagleWeights(*([fake] * 2 + [0] + [fake] * 9))))
    assert "wq" in L.eagle_last_error()
    _expect(L.EAGLE_ERR_ARG, lambda: pack(src_=L.EagleWeights(*([fake] * 2 + [fake + 8] + [fake] * 9))))
    assert "aligned" in L.eagle_last_error()

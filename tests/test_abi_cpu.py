"""The C ABI on the host: the library loads without a GPU, exports every
function include/*.h declares, and rejects bad arguments with the documented
status codes before touching the GPU (no call here passes validation)."""
import ctypes
import glob
import os
import re

import pytest

from routed_expert_prefill_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000000  # a 16-byte-aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return _lib.load()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"\b(moe_[a-z0-9_]+)\s*\(", src):
            names.add(m.group(1))
    return names


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.moe_abi_version() == 2


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.moe_status_string(code).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(7)


def test_route_build_workspace_query(lib):
    assert lib.moe_route_build_workspace(0, 6, 16) == 0
    assert lib.moe_route_build_workspace(4, 6, 300) == 0
    small = lib.moe_route_build_workspace(32, 6, 16)
    big = lib.moe_route_build_workspace(8192, 6, 256)
    assert 0 < small < big and big % 256 == 0


def _rb(lib, ids=A, mask=0, T=8, k=2, E=4, c=A, o=A, s=A, r=A, ws=A, wsb=1 << 20):
    return lib.moe_route_build(ids, mask or None, T, k, E, c, o, s, r, ws, wsb, None)


def test_route_build_errors(lib):
    assert _rb(lib, ids=0) == _lib.MOE_EINVAL
    assert _rb(lib, r=0) == _lib.MOE_EINVAL
    assert _rb(lib, T=0) == _lib.MOE_EINVAL
    assert _rb(lib, k=0) == _lib.MOE_EINVAL
    assert _rb(lib, T=1 << 28, k=16, E=256) == _lib.MOE_EINVAL  # T*k >= 2^31
    assert _rb(lib, E=0) == _lib.MOE_EUNSUPPORTED
    assert _rb(lib, E=257) == _lib.MOE_EUNSUPPORTED
    assert _rb(lib, k=17, E=64) == _lib.MOE_EUNSUPPORTED
    assert _rb(lib, k=5, E=4) == _lib.MOE_EUNSUPPORTED  # k > E, as moe_grouped_ffn and moe_route_topk
    assert _rb(lib, k=4, E=4, ids=0) == _lib.MOE_EINVAL  # k == E passes the shape check
    assert _rb(lib, ids=A + 4) == _lib.MOE_EALIGN
    assert _rb(lib, mask=A + 1) == _lib.MOE_EALIGN
    assert _rb(lib, ws=0) == _lib.MOE_EWORKSPACE
    assert _rb(lib, wsb=16) == _lib.MOE_EWORKSPACE


def _rbn(lib, ids=A, mask=0, T=8, k=2, E=4, c=A, o=A, s=A, r=A):
    return lib.moe_route_build_noalloc(ids, mask or None, T, k, E, c, o, s, r, None)


def test_route_build_noalloc_errors(lib):
    assert _rbn(lib, ids=0) == _lib.MOE_EINVAL
    assert _rbn(lib, c=0) == _lib.MOE_EINVAL
    assert _rbn(lib, T=0) == _lib.MOE_EINVAL
    assert _rbn(lib, E=257) == _lib.MOE_EUNSUPPORTED
    assert _rbn(lib, k=5, E=4) == _lib.MOE_EUNSUPPORTED
    assert _rbn(lib, T=1 << 28, k=16, E=256) == _lib.MOE_EINVAL  # T*k >= 2^31
    # beyond the fixed scratch: rejected before any HIP call
    big = _lib.MOE_ROUTE_NOALLOC_MAX_ROUTES
    assert _rbn(lib, T=big // 4 + 1, k=4, E=256) == _lib.MOE_ETOOLARGE
    assert _rbn(lib, T=big // 4, k=4, E=256, ids=A + 4) == _lib.MOE_EALIGN  # the largest size passes
    assert _rbn(lib, mask=A + 2) == _lib.MOE_EALIGN


def _desc(T=32, k=6, E=16, d=512, f=256, w=0, a=0):
    return _lib.MoeFfnDesc(T, k, E, d, f, w, a)


def test_ffn_workspace_query(lib):
    q = lambda **kw: lib.moe_grouped_ffn_workspace(ctypes.byref(_desc(**kw)))  # noqa: E731
    assert q() > 0
    assert q(d=500) == 0 and q(f=100) == 0 and q(E=257) == 0 and q(k=17, E=32) == 0
    assert q(k=7, E=6) == 0 and q(T=0) == 0
    assert q(w=1, a=0) == 0 and q(w=0, a=1) == 0 and q(w=2, a=2) == 0
    # h dominates: T*k rows of f bf16
    assert q(T=8192, k=6, E=256, d=4096, f=2048) >= 8192 * 6 * 2048 * 2
    assert q(w=1, a=1) > q()
    assert lib.moe_grouped_ffn_workspace(None) == 0


def _ffn(lib, desc=None, x=A, offs=A, sr=A, wg=A, wu=A, wd=A, sg=0, su=0, sd=0, y=A, ws=A,
         wsb=1 << 40):
    desc = desc or _desc()
    return lib.moe_grouped_ffn(ctypes.byref(desc), x, offs, sr, wg, wu, wd, sg or None, su or None,
                               sd or None, y, ws, wsb, None)


def test_grouped_ffn_errors(lib):
    assert lib.moe_grouped_ffn(None, A, A, A, A, A, A, None, None, None, A, A, 1 << 30, None) == _lib.MOE_EINVAL
    assert _ffn(lib, x=0) == _lib.MOE_EINVAL
    assert _ffn(lib, y=0) == _lib.MOE_EINVAL
    assert _ffn(lib, desc=_desc(T=0)) == _lib.MOE_EINVAL
    assert _ffn(lib, desc=_desc(d=384 + 64)) == _lib.MOE_EUNSUPPORTED
    assert _ffn(lib, desc=_desc(E=300)) == _lib.MOE_EUNSUPPORTED
    assert _ffn(lib, desc=_desc(w=1, a=0)) == _lib.MOE_EUNSUPPORTED
    assert _ffn(lib, desc=_desc(w=1, a=1)) == _lib.MOE_EINVAL  # fp8 without scales
    assert _ffn(lib, wg=A + 2) == _lib.MOE_EALIGN
    assert _ffn(lib, desc=_desc(w=1, a=1), sg=A, su=A + 4, sd=A) == _lib.MOE_EALIGN
    assert _ffn(lib, ws=0) == _lib.MOE_EWORKSPACE
    assert _ffn(lib, wsb=1024) == _lib.MOE_EWORKSPACE


def test_ffn_stage_errors(lib):
    d = ctypes.byref(_desc())
    # plan needs offsets; gate/up needs x, sorted_routes and both weights; down needs offsets, w_down, y
    assert lib.moe_ffn_plan(d, None, None, A, 1 << 40, None) == _lib.MOE_EINVAL
    assert lib.moe_ffn_gate_up(d, A, A, A, None, None, None, A, 1 << 40, None) == _lib.MOE_EINVAL
    assert lib.moe_ffn_down(d, A, A, None, None, A, 1 << 40, None) == _lib.MOE_EINVAL
    assert lib.moe_ffn_down(d, A, A, None, A + 4, A, 1 << 40, None) == _lib.MOE_EALIGN
    assert lib.moe_ffn_gate_up(d, A, A, A, A, None, None, A, 64, None) == _lib.MOE_EWORKSPACE
    d8 = ctypes.byref(_desc(w=1, a=1))
    assert lib.moe_ffn_plan(d8, None, A, A, 1 << 40, None) == _lib.MOE_EINVAL  # fp8 plan quantises x
    assert lib.moe_ffn_down(d8, A, A, None, A, A, 1 << 40, None) == _lib.MOE_EINVAL  # no s_down


def test_combine_errors(lib):
    c = lambda y=A, rr=A, w=A, m=0, lim=0, T=4, k=2, d=64, out=A: lib.moe_combine(  # noqa: E731
        y, rr, w, m or None, lim or None, T, k, d, out, None)
    assert c(y=0) == _lib.MOE_EINVAL
    assert c(out=0) == _lib.MOE_EINVAL
    assert c(T=0) == _lib.MOE_EINVAL
    assert c(d=6) == _lib.MOE_EINVAL
    assert c(k=17) == _lib.MOE_EUNSUPPORTED
    assert c(w=A + 4) == _lib.MOE_EALIGN
    assert c(m=A + 3) == _lib.MOE_EALIGN
    assert c(lim=A + 2) == _lib.MOE_EALIGN  # the row limit is one int32: 4-byte aligned
    assert c(lim=A + 4, y=0) == _lib.MOE_EINVAL  # 4-byte aligned passes the alignment check


def test_combine_shared_errors(lib):
    c = lambda y=A, rr=A, w=A, m=0, lim=0, sh=0, T=4, k=2, d=64, out=A, ob=0: lib.moe_combine_shared(  # noqa: E731
        y, rr, w, m or None, lim or None, sh or None, T, k, d, out or None, ob or None, None)
    assert c(y=0) == _lib.MOE_EINVAL
    assert c(out=0, ob=0) == _lib.MOE_EINVAL  # no output at all
    assert c(T=0) == _lib.MOE_EINVAL
    assert c(d=6) == _lib.MOE_EINVAL
    assert c(k=17) == _lib.MOE_EUNSUPPORTED
    assert c(sh=A + 4) == _lib.MOE_EALIGN
    assert c(out=0, ob=A + 2) == _lib.MOE_EALIGN
    assert c(lim=A + 1) == _lib.MOE_EALIGN


def test_quant_errors(lib):
    qf = lambda x=A, rows=4, cols=256, q=A, s=A: lib.moe_quant_rows_fp8(x, rows, cols, q, s, None)  # noqa: E731
    assert qf(x=0) == _lib.MOE_EINVAL
    assert qf(rows=0) == _lib.MOE_EINVAL
    assert qf(cols=100) == _lib.MOE_EUNSUPPORTED
    assert qf(cols=32768) == _lib.MOE_EUNSUPPORTED
    assert qf(q=A + 8) == _lib.MOE_EALIGN


def test_route_topk_errors(lib):
    r = lambda lg=A, b=0, T=4, E=16, k=6, ids=A, w=A: lib.moe_route_topk(  # noqa: E731
        lg, b or None, T, E, k, ids, w, None)
    assert r(lg=0) == _lib.MOE_EINVAL
    assert r(ids=0) == _lib.MOE_EINVAL
    assert r(w=0) == _lib.MOE_EINVAL
    assert r(T=0) == _lib.MOE_EINVAL
    assert r(E=0) == _lib.MOE_EINVAL
    assert r(k=0) == _lib.MOE_EINVAL
    assert r(T=1 << 24, E=256) == _lib.MOE_EINVAL  # T*E overflows int
    assert r(E=257) == _lib.MOE_EUNSUPPORTED
    assert r(k=17, E=64) == _lib.MOE_EUNSUPPORTED
    assert r(k=9, E=8) == _lib.MOE_EUNSUPPORTED
    assert r(lg=A + 4) == _lib.MOE_EALIGN
    assert r(b=A + 4) == _lib.MOE_EALIGN
    assert r(w=A + 8) == _lib.MOE_EALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(_lib.LibraryNotBuilt):
        _lib.load()

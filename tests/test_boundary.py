"""The C ABI on the CPU: the library loads, exports exactly what the header
declares, and rejects every invalid argument with its documented status
before any HIP call (no call here reaches the GPU)."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from sparse_long_context_page_amd import _lib, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagesparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libpagesparse.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(ps_[a-z_0-9]+)\s*\(", text)


def test_header_declares_the_bound_entry_points():
    assert tuple(declared_functions()) == _lib.ENTRY_POINTS


def test_library_exports_exactly_the_header():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {e for e in exported if e.startswith("ps_")} == set(declared_functions())


def test_abi_version_and_strerror():
    assert ops.ps_abi_version() >> 16 == 2
    for code in range(0, -8, -1):
        assert ops.ps_strerror(code).startswith("PS_")
    assert "unknown" in ops.ps_strerror(17)


def geom(**kw):
    base = dict(batch=2, num_q_heads=12, num_kv_heads=2, head_dim=128, page_size=16,
                max_pages=64, num_phys_pages=128, kv_dtype=_lib.PS_BF16,
                meta_format=_lib.PS_META_KV, meta_layout=_lib.PS_META_PHYSICAL)
    base.update(kw)
    return _lib.PsGeom(**base)


X = ctypes.c_void_p(4096)  # a non-NULL pointer that is never dereferenced


def score(g):
    return _lib.load().ps_score_pages(g, X, X, X, X, X, None)


@pytest.mark.parametrize("kw,code", [
    (dict(meta_format=2), _lib.PS_ERR_SHAPE),
    (dict(meta_format=-1), _lib.PS_ERR_SHAPE),
    (dict(meta_layout=2), _lib.PS_ERR_SHAPE),
    (dict(meta_layout=-1), _lib.PS_ERR_SHAPE),
    # logical metadata B * Hkv * max_pages * 2 * D * 4 bytes beyond int64 (the
    # physical layout of the same geometry is in range)
    (dict(batch=(1 << 31) - 1, num_q_heads=8, num_kv_heads=8, max_pages=(1 << 26) - 1,
          kv_dtype=_lib.PS_F32, meta_layout=_lib.PS_META_LOGICAL), _lib.PS_ERR_OVERFLOW),
    (dict(batch=-1), _lib.PS_ERR_SHAPE),
    (dict(num_q_heads=0), _lib.PS_ERR_SHAPE),
    (dict(num_q_heads=13), _lib.PS_ERR_SHAPE),
    (dict(num_q_heads=32, num_kv_heads=2), _lib.PS_ERR_UNSUPPORTED),
    (dict(head_dim=96), _lib.PS_ERR_UNSUPPORTED),
    (dict(head_dim=0), _lib.PS_ERR_SHAPE),
    (dict(page_size=32), _lib.PS_ERR_UNSUPPORTED),
    (dict(page_size=0), _lib.PS_ERR_SHAPE),
    (dict(kv_dtype=7), _lib.PS_ERR_UNSUPPORTED),
    (dict(max_pages=0), _lib.PS_ERR_SHAPE),
    (dict(num_phys_pages=0), _lib.PS_ERR_SHAPE),
    (dict(num_phys_pages=1 << 60), _lib.PS_ERR_OVERFLOW),
    (dict(num_phys_pages=1 << 31), _lib.PS_ERR_OVERFLOW),
    (dict(max_pages=1 << 28), _lib.PS_ERR_OVERFLOW),
    (dict(batch=(1 << 31) - 1, num_q_heads=16, num_kv_heads=16, max_pages=(1 << 27) - 1),
     _lib.PS_ERR_OVERFLOW),
    (dict(num_q_heads=16, num_kv_heads=16, max_pages=1 << 27), _lib.PS_ERR_OVERFLOW),
])
def test_geometry_validation(kw, code):
    assert score(geom(**kw)) == code


@pytest.mark.parametrize("layout", [_lib.PS_META_PHYSICAL, _lib.PS_META_LOGICAL])
@pytest.mark.parametrize("kv", [_lib.PS_BF16, _lib.PS_F32])
def test_fp8_metadata_geometry_accepted(kv, layout):
    """8-bit metadata with bf16 or fp32 pools, in either layout, passes the
    geometry checks (a call with batch 0 validates and enqueues nothing)."""
    g = geom(meta_format=_lib.PS_META_FP8_E4M3, batch=0, kv_dtype=kv, meta_layout=layout)
    lib = _lib.load()
    assert lib.ps_score_pages(g, X, X, X, X, X, None) == _lib.PS_OK
    assert lib.ps_build_page_meta(g, X, X, X, None, 4, X, None) == _lib.PS_OK
    assert lib.ps_refresh_score_pages(g, X, X, X, X, X, X, None) == _lib.PS_OK


def test_null_geometry():
    assert _lib.load().ps_score_pages(None, X, X, X, X, X, None) == _lib.PS_ERR_NULL


def test_null_pointers():
    lib = _lib.load()
    g = geom()
    assert lib.ps_build_page_meta(g, None, X, X, None, 4, X, None) == _lib.PS_ERR_NULL
    assert lib.ps_build_page_meta(g, X, X, X, None, 4, None, None) == _lib.PS_ERR_NULL
    assert lib.ps_score_pages(g, X, None, X, X, X, None) == _lib.PS_ERR_NULL
    assert lib.ps_select_topk(g, X, X, 8, 0, 0, None, X, None) == _lib.PS_ERR_NULL
    assert lib.ps_sparse_decode(g, X, X, X, X, X, X, None, 8, 0.1, 2, X, X, None) == \
        _lib.PS_ERR_NULL
    assert lib.ps_full_decode(g, X, X, None, X, X, 0.1, 2, X, X, None) == _lib.PS_ERR_NULL
    assert lib.ps_combine(g, X, X, 2, None, None, None, None) == _lib.PS_ERR_NULL


def test_topdelta_validation():
    lib = _lib.load()
    g = geom()
    f = lib.ps_select_topdelta
    assert f(g, None, X, X, X, X, 8, 0, 1, 0.1, 1.0, X, X, None) == _lib.PS_ERR_NULL
    assert f(g, X, None, X, X, X, 8, 0, 1, 0.1, 1.0, X, X, None) == _lib.PS_ERR_NULL
    assert f(g, X, X, X, X, X, 8, 0, 1, 0.1, -1.0, X, X, None) == _lib.PS_ERR_BUDGET
    assert f(g, X, X, X, X, X, 8, 0, 1, 0.1, float("nan"), X, X, None) == _lib.PS_ERR_BUDGET
    assert f(g, X, X, X, X, X, 8, 0, 1, 0.0, 1.0, X, X, None) == _lib.PS_ERR_BUDGET
    assert f(g, X, X, X, X, X, 8, 0, 1, float("inf"), 1.0, X, X, None) == _lib.PS_ERR_BUDGET
    assert f(g, X, X, X, X, X, 8, 5, 4, 0.1, 1.0, X, X, None) == _lib.PS_ERR_BUDGET
    assert f(geom(max_pages=65537), X, X, X, X, X, 8, 0, 1, 0.1, 1.0, X, X, None) == \
        _lib.PS_ERR_UNSUPPORTED
    assert f(geom(batch=0), X, X, X, X, X, 8, 0, 1, 0.1, float("inf"), X, X, None) == _lib.PS_OK


def test_budget_and_split_validation():
    lib = _lib.load()
    g = geom()
    assert lib.ps_build_page_meta(g, X, X, X, None, 0, X, None) == _lib.PS_ERR_SHAPE
    assert lib.ps_select_topk(g, X, X, 0, 0, 0, X, X, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_select_topk(g, X, X, 8, -1, 0, X, X, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_select_topk(g, X, X, 8, 0, -1, X, X, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_select_topk(g, X, X, 8, 5, 4, X, X, None) == _lib.PS_ERR_BUDGET
    # the selection holds a request's scores in registers: at most 65536 pages
    assert lib.ps_select_topk(geom(max_pages=65537), X, X, 8, 0, 0, X, X, None) == \
        _lib.PS_ERR_UNSUPPORTED
    assert lib.ps_sparse_decode(g, X, X, X, X, X, X, X, 8, 0.1, 0, X, X, None) == \
        _lib.PS_ERR_BUDGET
    assert lib.ps_sparse_decode(g, X, X, X, X, X, X, X, 8, 0.1, 9, X, X, None) == \
        _lib.PS_ERR_BUDGET
    assert lib.ps_sparse_decode(g, X, X, X, X, X, X, X, 0, 0.1, 1, X, X, None) == \
        _lib.PS_ERR_BUDGET
    assert lib.ps_full_decode(g, X, X, X, X, X, 0.1, 65, X, X, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_full_decode(g, X, X, X, X, X, 0.1, 0, X, X, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_combine(g, X, X, 0, None, X, None, None) == _lib.PS_ERR_BUDGET
    assert lib.ps_combine(g, X, X, 5000, None, X, None, None) == _lib.PS_ERR_BUDGET


def test_refresh_score_validation():
    lib = _lib.load()
    g = geom()
    assert lib.ps_refresh_score_pages(g, X, None, X, X, X, X, None) == _lib.PS_ERR_NULL
    assert lib.ps_refresh_score_pages(g, X, X, None, X, X, X, None) == _lib.PS_ERR_NULL
    # fp32 pools are accepted (validated, nothing enqueued for an empty batch)
    assert lib.ps_refresh_score_pages(geom(kv_dtype=_lib.PS_F32, batch=0), X, X, X, X, X, X,
                                      None) == _lib.PS_OK
    assert lib.ps_refresh_score_pages(geom(batch=0), X, X, X, X, X, X, None) == _lib.PS_OK


def test_fused_select_decode_validation():
    lib = _lib.load()
    g = geom()

    def call(g=g, sel=X, cnt=X, budget=8, ns=1, nl=2, splits=2, scores=X, acc=X, ml=X,
             sink=None, out=None, lse=None, arr=None):
        return lib.ps_select_sparse_decode(g, X, X, X, X, X, scores, budget, ns, nl, 0.1, splits,
                                           sel, cnt, acc, ml, sink, out, lse, arr, None)
    assert call(scores=None) == _lib.PS_ERR_NULL
    assert call(sel=None) == _lib.PS_ERR_NULL           # one of the pair
    assert call(cnt=None) == _lib.PS_ERR_NULL
    assert call(budget=0) == _lib.PS_ERR_BUDGET
    assert call(ns=5, nl=4) == _lib.PS_ERR_BUDGET
    assert call(splits=9) == _lib.PS_ERR_BUDGET
    assert call(splits=0) == _lib.PS_ERR_BUDGET
    assert call(g=geom(kv_dtype=_lib.PS_F32, batch=0)) == _lib.PS_OK
    assert call(g=geom(kv_dtype=_lib.PS_F32, max_pages=8193)) == _lib.PS_ERR_UNSUPPORTED
    assert call(g=geom(max_pages=8193)) == _lib.PS_ERR_UNSUPPORTED
    assert call(budget=1026, ns=0, nl=0, splits=2) == _lib.PS_ERR_UNSUPPORTED  # 513 per split
    assert call(acc=None) == _lib.PS_ERR_NULL           # partials needed without out
    assert call(out=X) == _lib.PS_ERR_BUDGET            # several splits merge with arrivals
    assert call(sink=X) == _lib.PS_ERR_BUDGET           # sink, lse, arrivals only with out
    assert call(lse=X) == _lib.PS_ERR_BUDGET
    assert call(arr=X) == _lib.PS_ERR_BUDGET
    assert call(out=X, arr=X, acc=None) == _lib.PS_ERR_NULL  # several splits write partials
    assert call(out=X, arr=X, ml=None) == _lib.PS_ERR_NULL
    assert call(g=geom(batch=0), sel=None, cnt=None) == _lib.PS_OK
    assert call(g=geom(batch=0), splits=1, acc=None, ml=None, sink=X, out=X, lse=X) == \
        _lib.PS_OK
    assert call(g=geom(batch=0), splits=4, sink=X, out=X, lse=X, arr=X) == _lib.PS_OK
    assert call(g=geom(batch=0, kv_dtype=_lib.PS_F32), splits=4, out=X, arr=X) == _lib.PS_OK


def test_noalloc_select_decode_validation():
    """The entry point without allocation: the checks of the fused decode with
    out set, out required, and PS_ERR_WORKSPACE (before any HIP call) when the
    partials and counters would not fit in the library's 8 MiB array."""
    lib = _lib.load()

    def call(g=None, sel=X, cnt=X, budget=8, ns=1, nl=2, splits=2, scores=X, sink=None, out=X,
             lse=None):
        g = geom() if g is None else g
        return lib.ps_select_sparse_decode_noalloc(g, X, X, X, X, X, scores, budget, ns, nl, 0.1,
                                                   splits, sel, cnt, sink, out, lse, None)
    assert call(out=None) == _lib.PS_ERR_NULL
    assert call(scores=None) == _lib.PS_ERR_NULL
    assert call(sel=None) == _lib.PS_ERR_NULL
    assert call(budget=0) == _lib.PS_ERR_BUDGET
    assert call(splits=9) == _lib.PS_ERR_BUDGET
    assert call(g=geom(max_pages=8193)) == _lib.PS_ERR_UNSUPPORTED
    assert call(g=geom(batch=0)) == _lib.PS_OK
    assert call(g=geom(batch=0), sel=None, cnt=None, sink=X, lse=X) == _lib.PS_OK
    # B*Hq*S*(D+2)*4 bytes of partials: 64 x 64 heads x 8 splits x 130 x 4 = 17 MB
    big = geom(batch=64, num_q_heads=64, num_kv_heads=8, max_pages=64)
    assert call(g=big, budget=64, splits=8) == _lib.PS_ERR_WORKSPACE
    # one split needs no partials, only the counters
    assert call(g=geom(batch=0, num_q_heads=64, num_kv_heads=8), budget=64, splits=1) == \
        _lib.PS_OK
    assert call(g=geom(batch=0, num_q_heads=64, num_kv_heads=8), budget=64, splits=4) == \
        _lib.PS_OK


def test_fused_topdelta_decode_validation():
    lib = _lib.load()
    g = geom()

    def call(g=g, sel=X, cnt=X, budget=8, ns=1, nl=2, scale=0.1, delta=1.0, splits=2, acc=X,
             ml=X, sink=None, out=None, lse=None, arr=None):
        return lib.ps_select_topdelta_sparse_decode(g, X, X, X, X, X, X, budget, ns, nl, scale,
                                                    delta, splits, sel, cnt, acc, ml, sink, out,
                                                    lse, arr, None)
    assert call(sel=None) == _lib.PS_ERR_NULL
    assert call(acc=None) == _lib.PS_ERR_NULL
    assert call(ns=5, nl=4) == _lib.PS_ERR_BUDGET
    assert call(splits=9) == _lib.PS_ERR_BUDGET
    assert call(out=X) == _lib.PS_ERR_BUDGET
    assert call(arr=X) == _lib.PS_ERR_BUDGET
    assert call(out=X, arr=X, acc=None) == _lib.PS_ERR_NULL
    assert call(out=X, arr=X, delta=-1.0) == _lib.PS_ERR_BUDGET
    assert call(delta=-1.0) == _lib.PS_ERR_BUDGET
    assert call(delta=float("nan")) == _lib.PS_ERR_BUDGET
    assert call(scale=0.0) == _lib.PS_ERR_BUDGET
    assert call(scale=float("inf")) == _lib.PS_ERR_BUDGET
    assert call(g=geom(max_pages=8193)) == _lib.PS_ERR_UNSUPPORTED
    assert call(budget=1026, ns=0, nl=0, splits=2) == _lib.PS_ERR_UNSUPPORTED
    assert call(g=geom(batch=0), delta=float("inf")) == _lib.PS_OK
    assert call(g=geom(batch=0, kv_dtype=_lib.PS_F32), splits=1, acc=None, ml=None, sink=X,
                out=X, lse=X) == _lib.PS_OK
    assert call(g=geom(batch=0), splits=3, out=X, lse=X, arr=X) == _lib.PS_OK


def test_partials_overflow():
    lib = _lib.load()
    g = geom(batch=1 << 20, num_q_heads=8, num_kv_heads=8, max_pages=4096)
    assert lib.ps_combine(g, X, X, 4096, None, X, None, None) == _lib.PS_ERR_OVERFLOW


def test_empty_batch_is_a_no_op():
    # validated, nothing enqueued, no HIP call: the pointers are never touched
    lib = _lib.load()
    g = geom(batch=0)
    assert lib.ps_build_page_meta(g, X, X, X, None, 4, X, None) == _lib.PS_OK
    assert lib.ps_score_pages(g, X, X, X, X, X, None) == _lib.PS_OK
    assert lib.ps_select_topk(g, X, X, 8, 1, 2, X, X, None) == _lib.PS_OK
    assert lib.ps_sparse_decode(g, X, X, X, X, X, X, X, 8, 0.1, 2, X, X, None) == _lib.PS_OK
    assert lib.ps_full_decode(g, X, X, X, X, X, 0.1, 2, X, X, None) == _lib.PS_OK
    assert lib.ps_combine(g, X, X, 2, None, X, None, None) == _lib.PS_OK


def test_binding_rejects_host_tensors():
    g = ops.Geometry(1, 4, 1, 64, 4, 4, torch.float32)
    q = torch.zeros(1, 4, 64)
    meta = torch.zeros(4, 1, 2, 64)
    pt = torch.zeros(1, 4, dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    sc = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError, match="device tensor"):
        ops.ps_score_pages(g, q, meta, pt, sl, sc)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libpagesparse.so")
    with pytest.raises(_lib.NativeLibraryMissing):
        _lib.load()

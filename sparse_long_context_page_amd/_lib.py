"""ctypes loader of libpagesparse.so (the C ABI in include/pagesparse.h).

There is no fallback: if the library has not been built, loading raises.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagesparse.so")

PS_OK = 0
PS_ERR_NULL = -1
PS_ERR_SHAPE = -2
PS_ERR_UNSUPPORTED = -3
PS_ERR_OVERFLOW = -4
PS_ERR_BUDGET = -5
PS_ERR_HIP = -6
PS_ERR_WORKSPACE = -7

PS_F32 = 0
PS_BF16 = 1

#: Every entry point the header declares, in declaration order.
ENTRY_POINTS = (
    "ps_build_page_meta",
    "ps_score_pages",
    "ps_refresh_score_pages",
    "ps_select_topk",
    "ps_select_topdelta",
    "ps_sparse_decode",
    "ps_select_sparse_decode",
    "ps_select_sparse_decode_noalloc",
    "ps_select_topdelta_sparse_decode",
    "ps_full_decode",
    "ps_combine",
    "ps_strerror",
    "ps_abi_version",
)


PS_META_KV = 0
PS_META_FP8_E4M3 = 1
PS_META_PHYSICAL = 0
PS_META_LOGICAL = 1

ABI_MAJOR = 2  # the ps_abi_version() major that PsGeom matches


class PsGeom(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("meta_format", ctypes.c_int32),
        ("meta_layout", ctypes.c_int32),
    ]


class NativeLibraryMissing(RuntimeError):
    pass


class PsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status
        self.fn = fn


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_G = ctypes.POINTER(PsGeom)

_SIGS = {
    "ps_build_page_meta": [_G, _P, _P, _P, _P, _I, _P, _P],
    "ps_score_pages": [_G, _P, _P, _P, _P, _P, _P],
    "ps_refresh_score_pages": [_G, _P, _P, _P, _P, _P, _P, _P],
    "ps_select_topk": [_G, _P, _P, _I, _I, _I, _P, _P, _P],
    "ps_select_topdelta": [_G, _P, _P, _P, _P, _P, _I, _I, _I, _F, _F, _P, _P, _P],
    "ps_sparse_decode": [_G, _P, _P, _P, _P, _P, _P, _P, _I, _F, _I, _P, _P, _P],
    "ps_select_sparse_decode": [_G, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _I, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P],
    "ps_select_sparse_decode_noalloc": [_G, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _I, _P,
                                        _P, _P, _P, _P, _P],
    "ps_select_topdelta_sparse_decode": [_G, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _F, _I,
                                         _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "ps_full_decode": [_G, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P],
    "ps_combine": [_G, _P, _P, _I, _P, _P, _P, _P],
    "ps_strerror": [ctypes.c_int],
    "ps_abi_version": [],
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library once (raises NativeLibraryMissing if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NativeLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m sparse_long_context_page_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "ps_strerror" else ctypes.c_int
    major = lib.ps_abi_version() >> 16
    if major != ABI_MAJOR:  # PsGeom above mirrors this major version's ps_geom
        raise NativeLibraryMissing(
            f"{LIB_PATH} has ABI {major}.x, this binding needs {ABI_MAJOR}.x; rebuild it")
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().ps_strerror(status).decode()


def check(fn: str, status: int) -> None:
    if status != PS_OK:
        raise PsError(fn, status, strerror(status))

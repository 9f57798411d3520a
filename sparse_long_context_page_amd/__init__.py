"""Page-selected sparse decode attention on AMD Instinct MI355X (gfx950).

The compute path is the HIP library libpagesparse.so (C ABI in
include/pagesparse.h); `ops` binds each entry point under the same name and
`decode.DecodeStep` runs one decode step. Importing this package does not load
the library; the first call does, and raises if it has not been built.
"""

from .ops import (  # noqa: F401
    Geometry,
    ps_abi_version,
    ps_build_page_meta,
    ps_combine,
    ps_full_decode,
    ps_refresh_score_pages,
    ps_score_pages,
    ps_select_sparse_decode,
    ps_select_topdelta,
    ps_select_topdelta_sparse_decode,
    ps_select_topk,
    ps_sparse_decode,
    ps_strerror,
)
from .decode import DecodeStep, build_meta  # noqa: F401

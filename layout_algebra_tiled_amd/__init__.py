"""Layout-algebra tiled GEMM for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``liblt.so`` (declared in include/lt.h):
a host Shape:Stride layout algebra, device layout maps, and hand-written
gfx950 GEMM kernels. This package is its thin Python binding. Importing it
loads nothing; the library is loaded on first use and must have been built
(``python -m layout_algebra_tiled_amd.build``). GEMM and device maps live in
``layout_algebra_tiled_amd.gemm`` (they need torch for device memory).
"""

from ._lib import LtError, lib  # noqa: F401
from .layout import Layout  # noqa: F401


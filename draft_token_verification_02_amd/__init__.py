"""Target-side verification step of speculative decoding on MI355X (gfx950).

The compute lives in ``libspecverify.so`` (hand-written HIP kernels behind a C
ABI, include/specverify.h); this package is its ctypes binding.
"""

from ._lib import (Dims, SVError, accept_and_draw, accept_greedy, debug_views, dims_of, library,
                   lmhead, new_workspace, verify, verify_greedy, workspace_bytes)

__all__ = ["Dims", "SVError", "accept_and_draw", "accept_greedy", "debug_views", "dims_of",
           "library", "lmhead", "new_workspace", "verify", "verify_greedy", "workspace_bytes"]

"""Target-side verification step of speculative decoding on MI355X (gfx950).

The compute lives in ``libspecverify.so`` (hand-written HIP kernels behind a C
ABI, include/specverify.h); this package is its ctypes binding.
"""

from ._lib import (Dims, HeadDims, SVError, TiledW, accept_and_draw, accept_and_draw_sparse_q,
                   accept_greedy, debug_views, dims_of, library, lmhead, new_workspace,
                   sparse_head, sparse_head_workspace_bytes, tile_w, tiled_w_bytes, tree_shape,
                   tree_workspace_bytes, verify, verify_greedy, verify_sparse_q, verify_static,
                   verify_tree, workspace_bytes)

__all__ = ["Dims", "HeadDims", "SVError", "TiledW", "accept_and_draw", "accept_and_draw_sparse_q",
           "accept_greedy", "debug_views", "dims_of", "library", "lmhead", "new_workspace",
           "sparse_head", "sparse_head_workspace_bytes", "tile_w", "tiled_w_bytes", "tree_shape",
           "tree_workspace_bytes", "verify", "verify_greedy", "verify_sparse_q", "verify_static",
           "verify_tree", "workspace_bytes"]

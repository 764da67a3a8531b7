"""ctypes binding of libspecverify (include/specverify.h).

Argument marshalling only: every step of the verification runs in the HIP
library.  Tensors are torch tensors on one ROCm device; PyTorch provides the
device memory and the stream.  If the library is not built this module raises
instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SV_OK, SV_ERR_NULL, SV_ERR_DIMS, SV_ERR_WORKSPACE, SV_ERR_ALIGN, SV_ERR_DEVICE = range(6)
SV_DEV_BAD_DRAFT, SV_DEV_FALLBACK, SV_DEV_NONFINITE, SV_DEV_BAD_QID = 1, 2, 4, 8
SV_LMHEAD_LOGITS, SV_LMHEAD_ARGMAX = 1, 2
SV_W_ROWS, SV_W_TILED = 0, 1
ABI_VERSION = 5
STATIC_SCRATCH_BYTES = 49 << 20
EXPORTS = ("sv_abi_version", "sv_status_string", "sv_workspace_bytes", "spec_verify", "sv_lmhead",
           "sv_accept_and_draw", "spec_verify_greedy", "sv_accept_greedy", "sv_debug_views",
           "spec_verify_sparse_q", "sv_accept_and_draw_sparse_q", "sv_sparse_head_workspace_bytes",
           "sv_sparse_head", "sv_tree_shape", "sv_tree_workspace_bytes", "spec_verify_tree",
           "spec_verify_static", "sv_lmhead_ex", "sv_tiled_w_bytes", "sv_tile_w")


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("gamma", ctypes.c_int32), ("d", ctypes.c_int32),
                ("V", ctypes.c_int32), ("w_layout", ctypes.c_int32)]


class HeadDims(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("d", ctypes.c_int32), ("V", ctypes.c_int32),
                ("C", ctypes.c_int32), ("M", ctypes.c_int32), ("k", ctypes.c_int32)]


class SVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_load().sv_status_string(status).decode()}")


_LIB = None


def _load():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.sv_abi_version.restype = ctypes.c_int32
        lib.sv_abi_version.argtypes = []
        lib.sv_status_string.restype = ctypes.c_char_p
        lib.sv_status_string.argtypes = [st]
        lib.sv_workspace_bytes.restype = sz
        lib.sv_workspace_bytes.argtypes = [Dims]
        lib.sv_tiled_w_bytes.restype = sz
        lib.sv_tiled_w_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        lib.sv_tile_w.restype = st
        lib.sv_tile_w.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, sz, vp]
        lib.spec_verify.restype = st
        lib.spec_verify.argtypes = [vp, vp, vp, vp, vp, Dims, vp, vp, vp, sz, vp]
        lib.spec_verify_static.restype = st
        lib.spec_verify_static.argtypes = [vp, vp, vp, vp, vp, Dims, vp, vp, vp]
        lib.sv_lmhead_ex.restype = st
        lib.sv_lmhead_ex.argtypes = [vp, vp, Dims, ctypes.c_int32, vp, sz, vp]
        lib.sv_lmhead.restype = st
        lib.sv_lmhead.argtypes = [vp, vp, Dims, vp, sz, vp]
        lib.sv_accept_and_draw.restype = st
        lib.sv_accept_and_draw.argtypes = [vp, vp, vp, Dims, vp, vp, vp, sz, vp]
        lib.spec_verify_greedy.restype = st
        lib.spec_verify_greedy.argtypes = [vp, vp, vp, Dims, vp, vp, vp, vp, sz, vp]
        lib.sv_accept_greedy.restype = st
        lib.sv_accept_greedy.argtypes = [vp, Dims, vp, vp, vp, vp, sz, vp]
        lib.spec_verify_sparse_q.restype = st
        lib.spec_verify_sparse_q.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int32, vp, Dims, vp, vp,
                                             vp, sz, vp]
        lib.sv_accept_and_draw_sparse_q.restype = st
        lib.sv_accept_and_draw_sparse_q.argtypes = [vp, vp, vp, ctypes.c_int32, vp, Dims, vp, vp,
                                                    vp, sz, vp]
        lib.sv_sparse_head_workspace_bytes.restype = sz
        lib.sv_sparse_head_workspace_bytes.argtypes = [HeadDims]
        lib.sv_sparse_head.restype = st
        lib.sv_sparse_head.argtypes = [vp, vp, vp, vp, HeadDims, vp, vp, vp, vp, sz, vp]
        lib.sv_tree_shape.restype = st
        lib.sv_tree_shape.argtypes = [vp, ctypes.c_int32, vp, vp, vp]
        lib.sv_tree_workspace_bytes.restype = sz
        lib.sv_tree_workspace_bytes.argtypes = [Dims]
        lib.spec_verify_tree.restype = st
        lib.spec_verify_tree.argtypes = [vp, vp, vp, vp, vp, vp, Dims, vp, vp, vp, vp, sz, vp]
        lib.sv_debug_views.restype = st
        lib.sv_debug_views.argtypes = [vp, Dims, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                       ctypes.POINTER(vp), ctypes.POINTER(vp)]
        if lib.sv_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH}: unexpected ABI version {lib.sv_abi_version()}")
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


class TiledW:
    """W [V, d] in the SV_W_TILED layout (1 KB tiles of 16 rows x 32 columns),
    as sv_tile_w writes it.  Every entry point except sparse_head takes it in
    place of the row-major W; its results are bitwise those of the row-major
    form.  ``data`` is the tiled buffer (int16, sv_tiled_w_bytes / 2 entries)."""

    def __init__(self, data, V: int, d: int):
        self.data, self.V, self.d = data, int(V), int(d)

    @property
    def shape(self):
        return (self.V, self.d)

    @property
    def device(self):
        return self.data.device

    @property
    def dtype(self):
        return self.data.dtype

    def dim(self) -> int:
        return 2

    def is_contiguous(self) -> bool:
        return self.data.is_contiguous()

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def tiled_w_bytes(V: int, d: int) -> int:
    return int(_load().sv_tiled_w_bytes(V, d))


def tile_w(W, *, out=None, stream=None) -> TiledW:
    """sv_tile_w: the SV_W_TILED copy of the row-major W [V, d] (bf16 or int16
    bits), written into ``out`` (int16, at least sv_tiled_w_bytes / 2 entries)
    or a new tensor.  Done once per matrix; enqueued on the stream."""
    import torch
    if W.dim() != 2 or not W.is_contiguous() or W.dtype not in (torch.bfloat16, torch.int16,
                                                                  torch.uint16):
        raise ValueError("W must be a contiguous 2-D bf16/int16 tensor")
    V, d = W.shape
    n = tiled_w_bytes(V, d)
    if n == 0:
        raise SVError(SV_ERR_DIMS, "sv_tiled_w_bytes")
    if out is None:
        out = torch.empty(n // 2, dtype=torch.int16, device=W.device)
    st = _load().sv_tile_w(_ptr(W), V, d, _ptr(out), out.numel() * out.element_size(),
                           _stream_handle(W.device, stream))
    if st != SV_OK:
        raise SVError(st, "sv_tile_w")
    return TiledW(out, V, d)


def dims_of(hidden, W, draft=None) -> Dims:
    B, g1, d = hidden.shape
    return Dims(B, g1 - 1, d, W.shape[0], SV_W_TILED if isinstance(W, TiledW) else SV_W_ROWS)


def workspace_bytes(dims: Dims) -> int:
    return int(_load().sv_workspace_bytes(dims))


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(device, stream) -> ctypes.c_void_p:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check_inputs(hidden, W, draft=None, q=None, uniforms=None):
    import torch
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a ROCm device")
    for name, t, dt in (("hidden", hidden, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("W", W, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("draft", draft, (torch.int32,)), ("q", q, (torch.float32,)),
                        ("uniforms", uniforms, (torch.float32,))):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, W on {dev}")
        if t.dtype not in dt:
            raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dt}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, g1, d = hidden.shape
    if W.dim() != 2 or W.shape[1] != d:
        raise ValueError(f"W must be [V, {d}], got {tuple(W.shape)}")
    V = W.shape[0]
    if draft is not None and tuple(draft.shape) != (B, g1 - 1):
        raise ValueError(f"draft must be [{B}, {g1 - 1}]")
    if q is not None and tuple(q.shape) != (B, g1 - 1, V):
        raise ValueError(f"q must be [{B}, {g1 - 1}, {V}]")
    if uniforms is not None and tuple(uniforms.shape) != (B, g1):
        raise ValueError(f"uniforms must be [{B}, {g1}]")


def new_workspace(dims: Dims, device):
    import torch
    n = workspace_bytes(dims)
    if n == 0:
        raise SVError(SV_ERR_DIMS, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def verify(hidden, W, draft, q, uniforms, *, out_tokens=None, n_accepted=None, workspace=None,
           stream=None):
    """The whole verification step; returns (out_tokens [B, gamma+1], n_accepted [B]).

    hidden bf16 [B, gamma+1, d]; W bf16 [V, d]; draft int32 [B, gamma];
    q float32 [B, gamma, V]; uniforms float32 [B, gamma+1] in (0, 1].
    """
    import torch
    _check_inputs(hidden, W, draft, q, uniforms)
    dims = dims_of(hidden, W)
    dev = W.device
    if out_tokens is None:
        out_tokens = torch.empty((dims.B, dims.gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((dims.B,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(dims, dev)
    st = _load().spec_verify(_ptr(hidden), _ptr(W), _ptr(draft), _ptr(q), _ptr(uniforms), dims,
                             _ptr(out_tokens), _ptr(n_accepted), _ptr(workspace),
                             workspace.numel(), _stream_handle(dev, stream))
    if st != SV_OK:
        raise SVError(st, "spec_verify")
    return out_tokens, n_accepted


def verify_static(hidden, W, draft, q, uniforms, *, out_tokens=None, n_accepted=None,
                  stream=None):
    """spec_verify_static: the whole step with the library's static device
    workspace (no workspace argument; the C call allocates nothing).  Pass
    preallocated outputs to allocate nothing here either.  Calls on one device
    share that workspace: serialise them."""
    import torch
    _check_inputs(hidden, W, draft, q, uniforms)
    dims = dims_of(hidden, W)
    dev = W.device
    if out_tokens is None:
        out_tokens = torch.empty((dims.B, dims.gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((dims.B,), dtype=torch.int32, device=dev)
    st = _load().spec_verify_static(_ptr(hidden), _ptr(W), _ptr(draft), _ptr(q), _ptr(uniforms),
                                    dims, _ptr(out_tokens), _ptr(n_accepted),
                                    _stream_handle(dev, stream))
    if st == SV_ERR_WORKSPACE:
        raise SVError(st, f"spec_verify_static: these dims need {workspace_bytes(dims)} bytes of "
                          f"workspace, more than the static {STATIC_SCRATCH_BYTES}")
    if st != SV_OK:
        raise SVError(st, "spec_verify_static")
    return out_tokens, n_accepted


def verify_greedy(hidden, W, draft, *, out_tokens=None, n_accepted=None, target_tokens=None,
                  workspace=None, stream=None):
    """Greedy (match) verification; returns (out_tokens, n_accepted, target_tokens).

    hidden bf16 [B, gamma+1, d]; W bf16 [V, d]; draft int32 [B, gamma].
    target_tokens int32 [B, gamma+1] receives every row's greedy token.
    """
    import torch
    _check_inputs(hidden, W, draft)
    dims = dims_of(hidden, W)
    dev = W.device
    if out_tokens is None:
        out_tokens = torch.empty((dims.B, dims.gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((dims.B,), dtype=torch.int32, device=dev)
    if target_tokens is None:
        target_tokens = torch.empty((dims.B, dims.gamma + 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(dims, dev)
    st = _load().spec_verify_greedy(_ptr(hidden), _ptr(W), _ptr(draft), dims, _ptr(out_tokens),
                                    _ptr(n_accepted), _ptr(target_tokens), _ptr(workspace),
                                    workspace.numel(), _stream_handle(dev, stream))
    if st != SV_OK:
        raise SVError(st, "spec_verify_greedy")
    return out_tokens, n_accepted, target_tokens


def accept_greedy(dims: Dims, draft, out_tokens, n_accepted, workspace, *, target_tokens=None,
                  stream=None):
    """Greedy stage 2 from the partials stage 1 left in ``workspace``."""
    tp = _ptr(target_tokens) if target_tokens is not None else ctypes.c_void_p(None)
    st = _load().sv_accept_greedy(_ptr(draft), dims, _ptr(out_tokens), _ptr(n_accepted), tp,
                                  _ptr(workspace), workspace.numel(),
                                  _stream_handle(draft.device, stream))
    if st != SV_OK:
        raise SVError(st, "sv_accept_greedy")


def lmhead(hidden, W, workspace, *, stream=None, logits=True, argmax=True):
    """Stage 1: softmax partials into ``workspace``, with the logits and the
    argmax partials unless asked not to (sv_lmhead, or sv_lmhead_ex with the
    matching flags: logits=True, argmax=False launches what spec_verify does)."""
    _check_inputs(hidden, W)
    dims = dims_of(hidden, W)
    if logits and argmax:
        st = _load().sv_lmhead(_ptr(hidden), _ptr(W), dims, _ptr(workspace), workspace.numel(),
                               _stream_handle(W.device, stream))
    else:
        flags = (SV_LMHEAD_LOGITS if logits else 0) | (SV_LMHEAD_ARGMAX if argmax else 0)
        st = _load().sv_lmhead_ex(_ptr(hidden), _ptr(W), dims, flags, _ptr(workspace),
                                  workspace.numel(), _stream_handle(W.device, stream))
    if st != SV_OK:
        raise SVError(st, "sv_lmhead")


def accept_and_draw(dims: Dims, draft, q, uniforms, out_tokens, n_accepted, workspace, *,
                    stream=None):
    """Stage 2: accept tests, first rejection and the draw, from stage 1's workspace."""
    st = _load().sv_accept_and_draw(_ptr(draft), _ptr(q), _ptr(uniforms), dims, _ptr(out_tokens),
                                    _ptr(n_accepted), _ptr(workspace), workspace.numel(),
                                    _stream_handle(q.device, stream))
    if st != SV_OK:
        raise SVError(st, "sv_accept_and_draw")


def _check_sparse_q(dims: Dims, q_ids, q_vals):
    import torch
    if q_ids.dtype != torch.int32 or q_vals.dtype != torch.float32:
        raise TypeError("q_ids must be int32 and q_vals float32")
    if q_ids.dim() != 3 or tuple(q_ids.shape[:2]) != (dims.B, dims.gamma):
        raise ValueError(f"q_ids must be [{dims.B}, {dims.gamma}, K], got {tuple(q_ids.shape)}")
    if q_vals.shape != q_ids.shape:
        raise ValueError("q_vals must have the shape of q_ids")
    if not (q_ids.is_contiguous() and q_vals.is_contiguous()):
        raise ValueError("q_ids and q_vals must be contiguous")
    return int(q_ids.shape[2])


def verify_sparse_q(hidden, W, draft, q_ids, q_vals, uniforms, *, out_tokens=None,
                    n_accepted=None, workspace=None, stream=None):
    """Verification with sparse q; returns (out_tokens [B, gamma+1], n_accepted [B]).

    q_ids int32 [B, gamma, K] (ids < 0 are padding), q_vals float32 [B, gamma, K]:
    the same result as ``verify`` on the dense q holding those values at those ids.
    """
    import torch
    _check_inputs(hidden, W, draft, None, uniforms)
    dims = dims_of(hidden, W)
    K = _check_sparse_q(dims, q_ids, q_vals)
    dev = W.device
    if out_tokens is None:
        out_tokens = torch.empty((dims.B, dims.gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((dims.B,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = new_workspace(dims, dev)
    st = _load().spec_verify_sparse_q(_ptr(hidden), _ptr(W), _ptr(draft), _ptr(q_ids),
                                      _ptr(q_vals), K, _ptr(uniforms), dims, _ptr(out_tokens),
                                      _ptr(n_accepted), _ptr(workspace), workspace.numel(),
                                      _stream_handle(dev, stream))
    if st != SV_OK:
        raise SVError(st, "spec_verify_sparse_q")
    return out_tokens, n_accepted


def accept_and_draw_sparse_q(dims: Dims, draft, q_ids, q_vals, uniforms, out_tokens, n_accepted,
                             workspace, *, stream=None):
    """Stage 2 with sparse q, from stage 1's workspace."""
    K = _check_sparse_q(dims, q_ids, q_vals)
    st = _load().sv_accept_and_draw_sparse_q(_ptr(draft), _ptr(q_ids), _ptr(q_vals), K,
                                             _ptr(uniforms), dims, _ptr(out_tokens),
                                             _ptr(n_accepted), _ptr(workspace), workspace.numel(),
                                             _stream_handle(q_vals.device, stream))
    if st != SV_OK:
        raise SVError(st, "sv_accept_and_draw_sparse_q")


def sparse_head_workspace_bytes(dims: HeadDims) -> int:
    return int(_load().sv_sparse_head_workspace_bytes(dims))


def sparse_head(h, W, centroids, members, k: int, *, q_ids=None, q_vals=None, clusters=None,
                workspace=None, stream=None):
    """The drafter's clustered sparse head; returns (q_ids [N, k*M], q_vals [N, k*M], clusters [N, k]).

    h bf16 [N, d]; W bf16 [V, d] row-major (not a TiledW); centroids bf16 [C, d];
    members int32 [C, M].
    """
    import torch
    if isinstance(W, TiledW):
        raise TypeError("sparse_head reads W row-major: pass the [V, d] tensor, not a TiledW")
    dev = W.device
    for name, t, dt in (("h", h, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("W", W, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("centroids", centroids, (torch.bfloat16, torch.int16, torch.uint16)),
                        ("members", members, (torch.int32,))):
        if t.device != dev or t.dtype not in dt or not t.is_contiguous() or t.dim() != 2:
            raise ValueError(f"{name}: expected a contiguous 2-d {dt} tensor on {dev}")
    N, d = h.shape
    C, M = members.shape
    if W.shape[1] != d or tuple(centroids.shape) != (C, d):
        raise ValueError("W must be [V, d] and centroids [C, d] with the hidden size of h")
    dims = HeadDims(N, d, W.shape[0], C, M, k)
    nbytes = sparse_head_workspace_bytes(dims)
    if nbytes == 0:
        raise SVError(SV_ERR_DIMS, "sv_sparse_head_workspace_bytes")
    if q_ids is None:
        q_ids = torch.empty((N, k * M), dtype=torch.int32, device=dev)
    if q_vals is None:
        q_vals = torch.empty((N, k * M), dtype=torch.float32, device=dev)
    if clusters is None:
        clusters = torch.empty((N, k), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = _load().sv_sparse_head(_ptr(h), _ptr(W), _ptr(centroids), _ptr(members), dims,
                                _ptr(q_ids), _ptr(q_vals), _ptr(clusters), _ptr(workspace),
                                workspace.numel(), _stream_handle(dev, stream))
    if st != SV_OK:
        raise SVError(st, "sv_sparse_head")
    return q_ids, q_vals, clusters


def _host_parent(parent):
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    if arr.ndim != 1:
        raise ValueError("parent must be a 1-d list of node parents")
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def tree_shape(parent):
    """(depth D, q rows P, launch rounds) of a topology; raises SVError if invalid."""
    arr, ptr = _host_parent(parent)
    out = [ctypes.c_int32() for _ in range(3)]
    st = _load().sv_tree_shape(ptr, int(arr.size), *[ctypes.byref(o) for o in out])
    if st != SV_OK:
        raise SVError(st, "sv_tree_shape")
    return tuple(int(o.value) for o in out)


def tree_workspace_bytes(dims: Dims) -> int:
    return int(_load().sv_tree_workspace_bytes(dims))


def verify_tree(hidden, W, parent, tokens, q, uniforms, *, out_tokens=None, n_accepted=None,
                path_nodes=None, workspace=None, stream=None):
    """Tree verification; returns (out_tokens [B, D+1], n_accepted [B], path_nodes [B, D]).

    hidden bf16 [B, T+1, d]; W bf16 [V, d] or its TiledW; parent host ints [T]; tokens int32
    [B, T]; q float32 [B, P, V] (rows with children); uniforms float32 [B, T+1].
    """
    import torch
    arr, pptr = _host_parent(parent)
    D, P, _ = tree_shape(arr)
    _check_inputs(hidden, W, None, None, uniforms)
    B, T1, d = hidden.shape
    V = W.shape[0]
    if T1 - 1 != arr.size:
        raise ValueError(f"hidden has {T1} rows per sequence, the tree {arr.size} nodes + root")
    if tokens.dtype != torch.int32 or tuple(tokens.shape) != (B, T1 - 1) or not tokens.is_contiguous():
        raise ValueError(f"tokens must be contiguous int32 [{B}, {T1 - 1}]")
    if q.dtype != torch.float32 or tuple(q.shape) != (B, P, V) or not q.is_contiguous():
        raise ValueError(f"q must be contiguous float32 [{B}, {P}, {V}]")
    dims = dims_of(hidden, W)
    dev = W.device
    if out_tokens is None:
        out_tokens = torch.empty((B, D + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if path_nodes is None:
        path_nodes = torch.empty((B, D), dtype=torch.int32, device=dev)
    if workspace is None:
        n = tree_workspace_bytes(dims)
        if n == 0:
            raise SVError(SV_ERR_DIMS, "sv_tree_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    st = _load().spec_verify_tree(_ptr(hidden), _ptr(W), pptr, _ptr(tokens), _ptr(q),
                                  _ptr(uniforms), dims, _ptr(out_tokens), _ptr(n_accepted),
                                  _ptr(path_nodes), _ptr(workspace), workspace.numel(),
                                  _stream_handle(dev, stream))
    if st != SV_OK:
        raise SVError(st, "spec_verify_tree")
    return out_tokens, n_accepted, path_nodes


def debug_views(workspace, dims: Dims) -> dict:
    """Views of the last call's logits [R, V], row_max [R], row_sumexp [R], status [B]."""
    import torch
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    st = _load().sv_debug_views(_ptr(workspace), dims, *[ctypes.byref(p) for p in ptrs])
    if st != SV_OK:
        raise SVError(st, "sv_debug_views")
    R = dims.B * (dims.gamma + 1)
    base = workspace.data_ptr()

    def view(p, n, dtype, shape):
        off = p.value - base
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype).view(*shape)

    return {"logits": view(ptrs[0], R * dims.V, torch.float32, (R, dims.V)),
            "row_max": view(ptrs[1], R, torch.float32, (R,)),
            "row_sumexp": view(ptrs[2], R, torch.float32, (R,)),
            "status": view(ptrs[3], dims.B, torch.int32, (dims.B,))}

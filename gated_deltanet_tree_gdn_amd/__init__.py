"""Python binding of ``libgdn_tree.so``: rollback-free tree verification of
Gated DeltaNet layers on MI355X (gfx950).

Argument marshalling only.  Every step of verify and commit runs in the HIP
kernels of the C library (``include/gdn_tree.h``); PyTorch is used for device
memory and for the current stream.  There is no CPU fallback: if the library
is missing or fails to load, every call raises.

The names mirror the C ABI: :func:`gdn_tree_verify`, :func:`gdn_commit_path`,
:func:`gdn_tree_ancestors`, :func:`gdn_ctx_status`, plus :class:`GdnContext`
for ``gdn_ctx_create`` / ``gdn_ctx_destroy``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn_tree.so")

GDN_BF16, GDN_F32 = 0, 1
STATUS = ["GDN_OK", "GDN_ERR_NULL", "GDN_ERR_SHAPE", "GDN_ERR_DTYPE", "GDN_ERR_ALIGN",
          "GDN_ERR_WORKSPACE", "GDN_ERR_TREE", "GDN_ERR_ACCEPT", "GDN_ERR_STATE", "GDN_ERR_HIP"]
EXPORTS = ["gdn_tree_workspace_bytes", "gdn_ctx_create", "gdn_ctx_destroy", "gdn_tree_verify",
           "gdn_tree_verify_branches", "gdn_commit_path", "gdn_commit_verify", "gdn_tree_ancestors", "gdn_accept_path", "gdn_tree_build", "gdn_tree_verify_static", "gdn_ctx_status",
           "gdn_status_string", "gdn_last_error"]


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        self.code = code
        self.status = STATUS[code] if 0 <= code < len(STATUS) else f"status {code}"
        super().__init__(f"{self.status}: {msg}")


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("H_k", ctypes.c_int32),
                ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_deltanet_tree_gdn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    dp = ctypes.POINTER(Dims)
    lib.gdn_tree_workspace_bytes.argtypes = [dp]
    lib.gdn_tree_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_ctx_create.argtypes = [dp, vp, ctypes.c_size_t, ctypes.POINTER(vp)]
    lib.gdn_ctx_create.restype = i32
    lib.gdn_ctx_destroy.argtypes = [vp]
    lib.gdn_ctx_destroy.restype = i32
    lib.gdn_tree_verify.argtypes = [vp] * 10
    lib.gdn_tree_verify.restype = i32
    lib.gdn_tree_verify_branches.argtypes = [vp] * 10
    lib.gdn_tree_verify_branches.restype = i32
    lib.gdn_commit_path.argtypes = [vp] * 4
    lib.gdn_commit_path.restype = i32
    lib.gdn_tree_ancestors.argtypes = [dp, vp, vp, vp, vp, vp]
    lib.gdn_tree_ancestors.restype = i32
    lib.gdn_accept_path.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_accept_path.restype = i32
    lib.gdn_tree_build.argtypes = [dp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_tree_build.restype = i32
    lib.gdn_commit_verify.argtypes = [vp] * 11
    lib.gdn_commit_verify.restype = i32
    lib.gdn_tree_verify_static.argtypes = [dp] + [vp] * 9
    lib.gdn_tree_verify_static.restype = i32
    lib.gdn_ctx_status.argtypes = [vp, vp]
    lib.gdn_ctx_status.restype = i32
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code: int):
    if code != 0:
        raise GdnError(code, load_library().gdn_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _require(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class GdnContext:
    """``gdn_ctx``: ties a verify to its delayed commit.  Owns its device
    workspace (allocated once, through torch, at construction)."""

    def __init__(self, B, N, H_k, H_v, d_k, d_v, qkv_dtype=GDN_BF16, device="cuda"):
        torch = _torch()
        lib = load_library()
        self.dims = Dims(B, N, H_k, H_v, d_k, d_v, qkv_dtype)
        nbytes = lib.gdn_tree_workspace_bytes(ctypes.byref(self.dims))
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        handle = ctypes.c_void_p()
        _check(lib.gdn_ctx_create(ctypes.byref(self.dims), self.workspace.data_ptr(), nbytes,
                                  ctypes.byref(handle)))
        self.handle = handle
        self._keep = ()

    def close(self):
        if self.handle:
            load_library().gdn_ctx_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @classmethod
    def for_tensors(cls, q, v, parent):
        B, N, H_k, d_k = q.shape
        H_v, d_v = v.shape[2], v.shape[3]
        return cls(B, N, H_k, H_v, d_k, d_v, _dtype_code(q), device=q.device)


def gdn_tree_verify(ctx: GdnContext, q, k, v, g, beta, parent, S0, o=None, stream=None):
    """o[B][N][H_v][d_v] (fp32): every tree node's output, in one pass, with
    S0 untouched.  Shapes and dtypes as in gdn_tree.h; returns ``o``."""
    torch = _torch()
    d = ctx.dims
    B, N, Hk, Hv, dk, dv = d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v
    qkv = torch.bfloat16 if d.qkv_dtype == GDN_BF16 else torch.float32
    _require(q, "q", qkv, (B, N, Hk, dk))
    _require(k, "k", qkv, (B, N, Hk, dk))
    _require(v, "v", qkv, (B, N, Hv, dv))
    _require(g, "g", torch.float32, (B, N, Hv))
    _require(beta, "beta", torch.float32, (B, N, Hv))
    _require(parent, "parent", torch.int32, (B, N))
    _require(S0, "S0", torch.float32, (B, Hv, dv, dk))
    if o is None:
        o = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _require(o, "o", torch.float32, (B, N, Hv, dv))
    lib = load_library()
    _check(lib.gdn_tree_verify(ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(parent),
                               _ptr(S0), _ptr(o), _stream(stream)))
    ctx._keep = (k, v, g, beta, parent, S0)  # borrowed by the pending commit
    return o


def gdn_tree_verify_branches(ctx: GdnContext, q, k, v, g, beta, parent, S0, o=None, stream=None):
    """The per-branch recurrent baseline: same contract and result as
    :func:`gdn_tree_verify` (for comparison)."""
    torch = _torch()
    d = ctx.dims
    B, N, Hk, Hv, dk, dv = d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v
    qkv = torch.bfloat16 if d.qkv_dtype == GDN_BF16 else torch.float32
    _require(q, "q", qkv, (B, N, Hk, dk))
    _require(k, "k", qkv, (B, N, Hk, dk))
    _require(v, "v", qkv, (B, N, Hv, dv))
    _require(g, "g", torch.float32, (B, N, Hv))
    _require(beta, "beta", torch.float32, (B, N, Hv))
    _require(parent, "parent", torch.int32, (B, N))
    _require(S0, "S0", torch.float32, (B, Hv, dv, dk))
    if o is None:
        o = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _require(o, "o", torch.float32, (B, N, Hv, dv))
    _check(load_library().gdn_tree_verify_branches(ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                                   _ptr(parent), _ptr(S0), _ptr(o), _stream(stream)))
    ctx._keep = (k, v, g, beta, parent, S0)
    return o


def gdn_commit_path(ctx: GdnContext, accepted, S_new=None, stream=None):
    """S_new[B][H_v][d_v][d_k] (fp32): the state at accepted[b] (S0 where
    accepted[b] == -1), for the tree of the last verify on ``ctx``.
    ``S_new`` may be the S0 tensor itself (in-place commit)."""
    torch = _torch()
    d = ctx.dims
    _require(accepted, "accepted", torch.int32, (d.B,))
    if S_new is None:
        S_new = torch.empty((d.B, d.H_v, d.d_v, d.d_k), dtype=torch.float32, device=accepted.device)
    _require(S_new, "S_new", torch.float32, (d.B, d.H_v, d.d_v, d.d_k))
    _check(load_library().gdn_commit_path(ctx.handle, _ptr(accepted), _ptr(S_new), _stream(stream)))
    return S_new


def gdn_commit_verify(ctx: GdnContext, accepted, q, k, v, g, beta, parent, S_next=None, o=None, stream=None):
    """(o, S_next): the delayed commit of the tree recorded on ``ctx`` at
    ``accepted`` fused into the verify of the new tree (q .. parent) on the
    committed state.  ``S_next`` may be the recorded S0 tensor (in place).
    Afterwards ``ctx`` records the new tree with S0 = S_next."""
    torch = _torch()
    d = ctx.dims
    B, N, Hk, Hv, dk, dv = d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v
    qkv = torch.bfloat16 if d.qkv_dtype == GDN_BF16 else torch.float32
    _require(accepted, "accepted", torch.int32, (B,))
    _require(q, "q", qkv, (B, N, Hk, dk))
    _require(k, "k", qkv, (B, N, Hk, dk))
    _require(v, "v", qkv, (B, N, Hv, dv))
    _require(g, "g", torch.float32, (B, N, Hv))
    _require(beta, "beta", torch.float32, (B, N, Hv))
    _require(parent, "parent", torch.int32, (B, N))
    if S_next is None:
        S_next = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=q.device)
    _require(S_next, "S_next", torch.float32, (B, Hv, dv, dk))
    if o is None:
        o = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _require(o, "o", torch.float32, (B, N, Hv, dv))
    _check(load_library().gdn_commit_verify(ctx.handle, _ptr(accepted), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                            _ptr(beta), _ptr(parent), _ptr(S_next), _ptr(o), _stream(stream)))
    ctx._keep = (k, v, g, beta, parent, S_next)
    return o, S_next


def gdn_tree_ancestors(parent, stream=None):
    """(anc [B][N][ceil(N/32)] uint32 as int32, depth [B][N] int32,
    tree_status [B] int32) computed on the device."""
    torch = _torch()
    _require(parent, "parent", torch.int32)
    B, N = parent.shape
    W = max((N + 31) // 32, 1)
    anc = torch.zeros((B, N, W), dtype=torch.int32, device=parent.device)
    depth = torch.zeros((B, N), dtype=torch.int32, device=parent.device)
    status = torch.zeros((max(B, 1),), dtype=torch.int32, device=parent.device)
    dims = Dims(B, N, 1, 1, 64, 64, GDN_BF16)
    _check(load_library().gdn_tree_ancestors(ctypes.byref(dims), _ptr(parent), _ptr(anc), _ptr(depth),
                                             _ptr(status), _stream(stream)))
    return anc, depth, status[:B]


def gdn_accept_path(parent, draft_token, target_token, stream=None):
    """(accepted [B], accept_len [B], tree_status [B]) int32 device tensors:
    the greedy accepted node of every sequence, computed on the device."""
    torch = _torch()
    _require(parent, "parent", torch.int32)
    B, N = parent.shape
    _require(draft_token, "draft_token", torch.int32, (B, N))
    _require(target_token, "target_token", torch.int32, (B, N + 1))
    dev = parent.device
    accepted, accept_len, status = (torch.empty((max(B, 1),), dtype=torch.int32, device=dev) for _ in range(3))
    dims = Dims(B, N, 1, 1, 64, 64, GDN_BF16)
    _check(load_library().gdn_accept_path(ctypes.byref(dims), _ptr(parent), _ptr(draft_token),
                                          _ptr(target_token), _ptr(accepted), _ptr(accept_len), _ptr(status),
                                          _stream(stream)))
    return accepted[:B], accept_len[:B], status[:B]


def gdn_tree_build(root_logp, node_logp, w, max_depth, stream=None):
    """(parent, cand_rank, score, steps, build_status) device tensors: the
    top-w best-first tree of every sequence, built on the device.
    root_logp [B][C] and node_logp [B][N][C] float32, rows non-increasing."""
    torch = _torch()
    _require(root_logp, "root_logp", torch.float32)
    B, C = root_logp.shape
    _require(node_logp, "node_logp", torch.float32)
    N = node_logp.shape[1]
    _require(node_logp, "node_logp", torch.float32, (B, N, C))
    dev = root_logp.device
    parent = torch.empty((B, N), dtype=torch.int32, device=dev)
    rank = torch.empty((B, N), dtype=torch.int32, device=dev)
    score = torch.empty((B, N), dtype=torch.float32, device=dev)
    steps = torch.empty((max(B, 1),), dtype=torch.int32, device=dev)
    status = torch.empty((max(B, 1),), dtype=torch.int32, device=dev)
    dims = Dims(B, N, 1, 1, 64, 64, GDN_BF16)
    _check(load_library().gdn_tree_build(ctypes.byref(dims), int(C), int(w), int(max_depth), _ptr(root_logp),
                                         _ptr(node_logp), _ptr(parent), _ptr(rank), _ptr(score), _ptr(steps),
                                         _ptr(status), _stream(stream)))
    return parent, rank, score, steps[:B], status[:B]


def gdn_tree_verify_static(q, k, v, g, beta, parent, S0, o=None, stream=None):
    """:func:`gdn_tree_verify` for callers that cannot allocate device memory:
    no context, no workspace (the library's fixed device array takes the
    per-sequence verdicts).  ``o`` must be passed in to allocate nothing."""
    torch = _torch()
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    code = _dtype_code(q)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (parent, "parent"), (S0, "S0")):
        _require(t, name)
    if o is None:
        o = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _require(o, "o", torch.float32, (B, N, Hv, dv))
    dims = Dims(B, N, Hk, Hv, dk, dv, code)
    _check(load_library().gdn_tree_verify_static(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                                 _ptr(beta), _ptr(parent), _ptr(S0), _ptr(o), _stream(stream)))
    return o


def gdn_ctx_status(ctx: GdnContext, stream=None):
    """Synchronises and raises GdnError if the last verify saw an invalid
    tree (GDN_ERR_TREE) or the last commit an invalid accepted node."""
    _check(load_library().gdn_ctx_status(ctx.handle, _stream(stream)))


def verify(q, k, v, g, beta, parent, S0, o=None, stream=None, ctx: Optional[GdnContext] = None):
    """Convenience: :func:`gdn_tree_verify` with a context made for the
    tensors' shapes; returns ``(o, ctx)`` so the caller can commit later."""
    ctx = ctx or GdnContext.for_tensors(q, v, parent)
    return gdn_tree_verify(ctx, q, k, v, g, beta, parent, S0, o=o, stream=stream), ctx

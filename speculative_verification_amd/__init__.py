"""Deterministic small-batch speculative verification for AMD MI355X.

Thin torch-facing wrappers over libspecv.so (see include/specv.h): they check
tensor dtypes, devices and shapes, pass raw device pointers and the current
HIP stream, and raise SpecvError on a non-zero status. All computation runs
in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import CM_WEIGHT, LIB, SpecvError, check, cm_params
from .model import DeviceModel

__all__ = ["SpecvError", "DeviceModel", "CTRL_FIELDS", "new_ctrl", "quantize_act", "linear", "linear_argmax",
           "linear_argmax_noalloc", "linear_argmax_accept", "tree_accept", "tree_argmax_accept",
           "argmax_accept_workspace_bytes", "kv_compact", "linear_workspace", "cm_params", "cm_draft", "CM_WEIGHT",
           "quantize_act_blocks", "linear_blocks", "Packed", "pack_weights"]

CTRL_FIELDS = ("committed_len", "n_nodes", "ctx_len", "done", "accept_len", "root_token", "step",
               "ring_head")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def new_ctrl(committed_len: int, n_nodes: int, ctx_len: int, root_token: int = 0,
             device="cuda") -> torch.Tensor:
    """int32[8] control block with the layout of specv_ctrl."""
    v = [committed_len, n_nodes, ctx_len, 0, 0, root_token, 0, 0]
    return torch.tensor(v, dtype=torch.int32, device=device)


def quantize_act(x: torch.Tensor, xq: torch.Tensor | None = None, xs: torch.Tensor | None = None):
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.int8, device=x.device) if xq is None else xq
    xs = torch.empty((T,), dtype=torch.float32, device=x.device) if xs is None else xs
    check("w4a8_quantize_act", LIB.w4a8_quantize_act(_dev(x, "x", torch.float32), T, K,
                                                     _dev(xq, "xq", torch.int8),
                                                     _dev(xs, "xs", torch.float32), _stream()))
    return xq, xs


class Packed:
    """A W4A8 matrix of N rows and K inputs in the library's packed tile
    layout (w4a8_pack_weights): flat uint8 nibbles and int16 fp16-bit scales."""

    def __init__(self, wp: torch.Tensor, sp: torch.Tensor, N: int, K: int):
        self.wp, self.sp, self.N, self.K = wp, sp, int(N), int(K)

    def rows(self, n: int) -> "Packed":
        """The first n rows (n a multiple of 16): a prefix of both buffers."""
        if n % 16 or not 0 < n <= self.N:
            raise ValueError("a row prefix must be a positive multiple of 16 within the matrix")
        return Packed(self.wp[: n * self.K // 2], self.sp[: n * self.K // 32], n, self.K)


def packed_sizes(N: int, K: int) -> tuple[int, int]:
    """(weight bytes, scale elements) of an N x K matrix in the packed layout."""
    wb, sb = int(LIB.w4a8_packed_weight_bytes(N, K)), int(LIB.w4a8_packed_scale_bytes(N, K))
    if wb == 0 or sb == 0:
        raise ValueError(f"no packed layout for N={N}, K={K}")
    return wb, sb // 2


def pack_weights(wq: torch.Tensor, ws: torch.Tensor, wp: torch.Tensor | None = None,
                 sp: torch.Tensor | None = None) -> Packed:
    """Packs interchange nibbles wq uint8 [N][K/2] and fp16 scale bits ws
    [N][K/32] (device tensors) into the packed tile layout; wp / sp may be
    given (flat, at least the packed sizes) to pack in place."""
    N, half = wq.shape
    K = 2 * half
    if ws.shape != (N, K // 32):
        raise ValueError("ws must be [N][K/32]")
    if ws.dtype not in (torch.int16, torch.uint16, torch.float16):
        raise TypeError("ws must hold fp16 bit patterns")
    wb, se = packed_sizes(N, K)
    wp = torch.empty(wb, dtype=torch.uint8, device=wq.device) if wp is None else wp
    sp = torch.empty(se, dtype=torch.int16, device=wq.device) if sp is None else sp
    if wp.numel() < wb or sp.numel() < se:
        raise ValueError("packed buffers too small")
    check("w4a8_pack_weights", LIB.w4a8_pack_weights(_dev(wq, "wq", torch.uint8), _dev(ws, "ws", ws.dtype), N, K,
                                                     _dev(wp, "wp", torch.uint8), _dev(sp, "sp", sp.dtype),
                                                     _stream()))
    return Packed(wp, sp, N, K)


_WORKSPACES: dict = {}


def linear_workspace(T: int, N: int, K: int, device) -> torch.Tensor | None:
    """A zero-filled workspace for w4a8_linear_T on `device`, shared by calls
    on one stream (the library leaves it zeroed after every call)."""
    need = int(LIB.w4a8_linear_workspace(T, N, K))
    if need == 0:
        return None
    dev = torch.device(device)
    ws = _WORKSPACES.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=dev)
        _WORKSPACES[dev] = ws
    return ws


def _check_packed(w: Packed, xq: torch.Tensor, xs_shape: tuple) -> tuple[int, int, int]:
    if not isinstance(w, Packed):
        raise TypeError("weights must be a Packed matrix (pack_weights)")
    T, K = xq.shape
    if w.K != K or xs_shape[0] != T:
        raise ValueError("shape mismatch between the packed weights, xq and xs")
    return T, w.N, K


def linear(w: Packed, xq: torch.Tensor, xs: torch.Tensor, y: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [T][N] fp32 from a packed matrix, codes xq int8 [T][K] and token
    scales xs [T]."""
    T, N, K = _check_packed(w, xq, tuple(xs.shape))
    if xs.shape != (T,):
        raise ValueError("xs must be [T]")
    wq, ws = w.wp, w.sp
    y = torch.empty((T, N), dtype=torch.float32, device=xq.device) if y is None else y
    if workspace is None:
        workspace = linear_workspace(T, N, K, xq.device)
    wsp = _dev(workspace, "workspace", torch.uint8) if workspace is not None else None
    wsb = workspace.numel() if workspace is not None else 0
    check("w4a8_linear_T", LIB.w4a8_linear_T(_dev(wq, "wq", torch.uint8), _dev(ws, "ws", ws.dtype),
                                             _dev(xq, "xq", torch.int8), _dev(xs, "xs", torch.float32),
                                             _dev(y, "y", torch.float32), T, N, K, wsp, wsb, _stream()))
    return y


def quantize_act_blocks(x: torch.Tensor, xq: torch.Tensor | None = None, xs: torch.Tensor | None = None):
    """Per-block codes int8 [T][K] and scales fp32 [T][K/32]."""
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.int8, device=x.device) if xq is None else xq
    xs = torch.empty((T, K // 32), dtype=torch.float32, device=x.device) if xs is None else xs
    check("w4a8_quantize_act_blocks", LIB.w4a8_quantize_act_blocks(_dev(x, "x", torch.float32), T, K,
                                                                   _dev(xq, "xq", torch.int8),
                                                                   _dev(xs, "xs", torch.float32), _stream()))
    return xq, xs


def linear_blocks(w: Packed, xq: torch.Tensor, xs: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """As linear, with per-block activation scales xs [T][K/32]."""
    T, N, K = _check_packed(w, xq, tuple(xs.shape))
    if xs.shape != (T, K // 32):
        raise ValueError("xs must be [T][K/32]")
    wq, ws = w.wp, w.sp
    y = torch.empty((T, N), dtype=torch.float32, device=xq.device) if y is None else y
    check("w4a8_linear_blocks_T", LIB.w4a8_linear_blocks_T(_dev(wq, "wq", torch.uint8), _dev(ws, "ws", ws.dtype),
                                                           _dev(xq, "xq", torch.int8),
                                                           _dev(xs, "xs", torch.float32),
                                                           _dev(y, "y", torch.float32), T, N, K, _stream()))
    return y


def linear_argmax(w: Packed, xq: torch.Tensor, xs: torch.Tensor, y: torch.Tensor | None = None,
                  argmax: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """argmax int32 [T] of the W4A8 linear's outputs (w4a8_linear_argmax_T);
    the outputs are written to y only when y is given."""
    T, N, K = _check_packed(w, xq, tuple(xs.shape))
    if xs.shape != (T,):
        raise ValueError("xs must be [T]")
    wq, ws = w.wp, w.sp
    need = int(LIB.w4a8_linear_argmax_workspace(T, N, K))
    if need == 0:
        raise ValueError("shape not supported by the fused argmax linear")
    dev = xq.device
    argmax = torch.empty(T, dtype=torch.int32, device=dev) if argmax is None else argmax
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    yp = _dev(y, "y", torch.float32) if y is not None else None
    check("w4a8_linear_argmax_T", LIB.w4a8_linear_argmax_T(
        _dev(wq, "wq", torch.uint8), _dev(ws, "ws", ws.dtype), _dev(xq, "xq", torch.int8),
        _dev(xs, "xs", torch.float32), yp, _dev(argmax, "argmax", torch.int32), T, N, K,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream()))
    return argmax


def linear_argmax_noalloc(w: Packed, xq: torch.Tensor, xs: torch.Tensor, argmax: torch.Tensor,
                          y: torch.Tensor | None = None) -> torch.Tensor:
    """linear_argmax through w4a8_linear_argmax_T_noalloc: the caller passes
    the output buffer and the library uses its static device scratch, so
    nothing is allocated (calls that overlap on one device race)."""
    T, N, K = _check_packed(w, xq, tuple(xs.shape))
    if xs.shape != (T,):
        raise ValueError("xs must be [T]")
    yp = _dev(y, "y", torch.float32) if y is not None else None
    check("w4a8_linear_argmax_T_noalloc", LIB.w4a8_linear_argmax_T_noalloc(
        _dev(w.wp, "wq", torch.uint8), _dev(w.sp, "ws", w.sp.dtype), _dev(xq, "xq", torch.int8),
        _dev(xs, "xs", torch.float32), yp, _dev(argmax, "argmax", torch.int32), T, N, K, _stream()))
    return argmax


def tree_accept(argmax: torch.Tensor, parent: torch.Tensor, token: torch.Tensor, ctrl: torch.Tensor,
                path: torch.Tensor | None = None, stats: torch.Tensor | None = None,
                ring: torch.Tensor | None = None) -> torch.Tensor:
    """Acceptance from each node's greedy prediction (tree_accept); returns path."""
    n_max = argmax.numel()
    path = torch.zeros(n_max, dtype=torch.int32, device=argmax.device) if path is None else path
    st = _dev(stats, "stats", torch.int32) if stats is not None else None
    rp = _dev(ring, "ring", torch.int32) if ring is not None else None
    check("tree_accept", LIB.tree_accept(
        _dev(argmax, "argmax", torch.int32), n_max, _dev(parent, "parent", torch.int32),
        _dev(token, "token", torch.int32), _dev(path, "path", torch.int32), _dev(ctrl, "ctrl", torch.int32),
        st, rp, ring.numel() if ring is not None else 0, _stream()))
    return path


def linear_argmax_accept(w: Packed, xq: torch.Tensor, xs: torch.Tensor, parent: torch.Tensor, token: torch.Tensor,
                         ctrl: torch.Tensor, argmax: torch.Tensor | None = None, path: torch.Tensor | None = None,
                         stats: torch.Tensor | None = None, ring: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None):
    """The lm_head's argmax epilogue, then acceptance from its pairs
    (w4a8_linear_argmax_accept_T); returns (argmax, path), allocated when not
    given."""
    T, N, K = _check_packed(w, xq, tuple(xs.shape))
    if xs.shape != (T,):
        raise ValueError("xs must be [T]")
    need = int(LIB.w4a8_linear_argmax_workspace(T, N, K))
    if need == 0:
        raise ValueError("shape not supported by the fused argmax linear")
    dev = xq.device
    argmax = torch.empty(T, dtype=torch.int32, device=dev) if argmax is None else argmax
    path = torch.zeros(T, dtype=torch.int32, device=dev) if path is None else path
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _dev(stats, "stats", torch.int32) if stats is not None else None
    rp = _dev(ring, "ring", torch.int32) if ring is not None else None
    wq, ws = w.wp, w.sp
    check("w4a8_linear_argmax_accept_T", LIB.w4a8_linear_argmax_accept_T(
        _dev(wq, "wq", torch.uint8), _dev(ws, "ws", ws.dtype), _dev(xq, "xq", torch.int8),
        _dev(xs, "xs", torch.float32), T, N, K, _dev(parent, "parent", torch.int32),
        _dev(token, "token", torch.int32), _dev(argmax, "argmax", torch.int32), _dev(path, "path", torch.int32),
        _dev(ctrl, "ctrl", torch.int32), st, rp, ring.numel() if ring is not None else 0,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream()))
    return argmax, path


def argmax_accept_workspace_bytes(V: int, n_max: int) -> int:
    return int(LIB.tree_argmax_accept_workspace(V, n_max))


def tree_argmax_accept(logits: torch.Tensor, parent: torch.Tensor, token: torch.Tensor,
                       ctrl: torch.Tensor, argmax: torch.Tensor | None = None,
                       path: torch.Tensor | None = None, stats: torch.Tensor | None = None,
                       ring: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    n_max, V = logits.shape
    dev = logits.device
    argmax = torch.empty(n_max, dtype=torch.int32, device=dev) if argmax is None else argmax
    path = torch.zeros(n_max, dtype=torch.int32, device=dev) if path is None else path
    if workspace is None:
        workspace = torch.empty(argmax_accept_workspace_bytes(V, n_max), dtype=torch.uint8, device=dev)
    st = _dev(stats, "stats", torch.int32) if stats is not None else None
    rp = _dev(ring, "ring", torch.int32) if ring is not None else None
    check("tree_argmax_accept", LIB.tree_argmax_accept(
        _dev(logits, "logits", torch.float32), V, n_max, _dev(parent, "parent", torch.int32),
        _dev(token, "token", torch.int32), _dev(argmax, "argmax", torch.int32),
        _dev(path, "path", torch.int32), _dev(ctrl, "ctrl", torch.int32), st, rp,
        ring.numel() if ring is not None else 0, _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream()))
    return argmax, path


def kv_compact(k_cache: torch.Tensor, v_cache: torch.Tensor, path: torch.Tensor,
               ctrl: torch.Tensor) -> None:
    """Caches: fp16 (or int16 bits) [layers][kv_heads][capacity][head_dim]."""
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must share a 4-D shape")
    if k_cache.element_size() != 2 or v_cache.element_size() != 2:
        raise TypeError("caches must hold fp16 values (2-byte elements)")
    layers, heads, cap, hd = k_cache.shape
    check("kv_compact", LIB.kv_compact(_dev(k_cache, "k_cache", k_cache.dtype),
                                       _dev(v_cache, "v_cache", v_cache.dtype), layers, heads, cap, hd,
                                       _dev(path, "path", torch.int32), _dev(ctrl, "ctrl", torch.int32),
                                       _stream()))


def cm_draft(stream: torch.Tensor, width: int, params=None, workspace: torch.Tensor | None = None):
    """Context-mixing drafter on a token stream (committed tokens, then the
    root): returns (parent, token) int32 [width] device tensors, of which the
    first n are the tree, and an int32 [2] device tensor (n, best match)."""
    p = params if params is not None else cm_params()
    n = stream.numel()
    need = int(LIB.cm_draft_workspace(n, ctypes.byref(p)))
    if need == 0:
        raise ValueError("cm_draft_workspace rejected its arguments")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=stream.device)
    parent = torch.empty(width, dtype=torch.int32, device=stream.device)
    token = torch.empty(width, dtype=torch.int32, device=stream.device)
    out = torch.empty(2, dtype=torch.int32, device=stream.device)
    check("cm_draft", LIB.cm_draft(_dev(stream, "stream", torch.int32), n, ctypes.byref(p), width, parent.data_ptr(),
                                   token.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream()))
    return parent, token, out

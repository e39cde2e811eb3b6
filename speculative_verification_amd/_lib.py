"""ctypes binding of libspecv.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels. There is no
Python or CPU fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecv.so")

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/specv.h
SIGNATURES = {
    "specv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a8_quantize_act": (ctypes.c_int, [P, I32, I32, P, P, P]),
    "w4a8_quantize_act_blocks": (ctypes.c_int, [P, I32, I32, P, P, P]),
    "w4a8_linear_blocks_T": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, P]),
    "w4a8_packed_weight_bytes": (SZ, [I32, I32]),
    "w4a8_packed_scale_bytes": (SZ, [I32, I32]),
    "w4a8_pack_weights": (ctypes.c_int, [P, P, I32, I32, P, P, P]),
    "w4a8_linear_workspace": (SZ, [I32, I32, I32]),
    "w4a8_linear_T": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, P, SZ, P]),
    "specv_time_next_linear": (ctypes.c_int, [P, P]),
    "specv_stream_read": (ctypes.c_int, [P, SZ, P, I32, P]),
    "w4a8_linear_argmax_workspace": (SZ, [I32, I32, I32]),
    "w4a8_linear_argmax_T": (ctypes.c_int, [P, P, P, P, P, P, I32, I32, I32, P, SZ, P]),
    "w4a8_linear_argmax_T_noalloc": (ctypes.c_int, [P, P, P, P, P, P, I32, I32, I32, P]),
    "tree_accept": (ctypes.c_int, [P, I32, P, P, P, P, P, P, I32, P]),
    "w4a8_linear_argmax_accept_T": (ctypes.c_int, [P, P, P, P, I32, I32, I32, P, P, P, P, P, P, P, I32, P, SZ, P]),
    "tree_argmax_accept_workspace": (SZ, [I64, I32]),
    "tree_argmax_accept": (ctypes.c_int, [P, I64, I32, P, P, P, P, P, P, P, I32, P, SZ, P]),
    "kv_compact": (ctypes.c_int, [P, P, I32, I32, I32, I32, P, P, P]),
    "specv_rope_table": (ctypes.c_int, [P, P, I32, I32, ctypes.c_double]),
    "spec_step_workspace": (SZ, [P, I32]),
    "spec_tree_step": (ctypes.c_int, [P, P, P, P, I32, P, P, P, P, P, I32, P, SZ, P]),
    "spec_window_workspace": (SZ, [P, I32]),
    "spec_window_run": (ctypes.c_int, [P, P, P, P, I32, P, I32, I32, P, SZ, P, P]),
    "cm_draft_workspace": (SZ, [I32, P]),
    "cm_draft": (ctypes.c_int, [P, I32, P, I32, P, P, P, P, SZ, P]),
    "spec_window_cm_workspace": (SZ, [P, I32, I32, P]),
    "spec_window_run_cm": (ctypes.c_int, [P, P, P, P, I32, P, I32, I32, P, SZ, P, P]),
}


class SpecvModel(ctypes.Structure):
    """Mirror of specv_model."""
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim",
                                              "inter", "vocab", "max_pos")] + \
               [("eps", ctypes.c_float), ("kv_capacity", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu", "w_down", "s_down",
                                              "norm_attn", "norm_mlp", "norm_final", "w_lm", "s_lm", "rope_cos",
                                              "rope_sin", "k_cache", "v_cache")]


class SpecvDrafter(ctypes.Structure):
    """Mirror of specv_drafter."""
    _fields_ = [("reference", ctypes.c_void_p), ("reference_len", ctypes.c_int32), ("draw_rows", ctypes.c_int32),
                ("draws", ctypes.c_void_p), ("accept_threshold", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


class SpecvCmParams(ctypes.Structure):
    """Mirror of specv_cm_params."""
    _fields_ = [("max_order", ctypes.c_int32), ("candidates", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("weight", ctypes.c_uint32 * 9)]


# Default candidate weight by match length l = 0..8: 2^(l - 1), so a match
# one token longer counts as much as two shorter ones.
CM_WEIGHT = (0, 1, 2, 4, 8, 16, 32, 64, 128)


def cm_params(max_order: int = 8, candidates: int = 16, depth: int = 8, weight=CM_WEIGHT) -> SpecvCmParams:
    p = SpecvCmParams(max_order, candidates, depth)
    for i, w in enumerate(weight):
        p.weight[i] = int(w)
    return p


class SpecvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    if not os.path.exists(SO):
        raise ImportError(f"{SO} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(SO)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


LIB = load()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise SpecvError(fn, status, LIB.specv_status_string(status).decode())

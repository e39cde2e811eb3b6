"""ctypes loader for liboracle.so, the plain CPU reference.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
CPU-baseline leg of bench.py. The product package never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")
SOURCES = ["oracle.c"]
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile the oracle with gcc (no -march, no contraction)."""
    out = out or SO
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), "-o", out,
           *[os.path.join(HERE, s) for s in SOURCES], "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            build()
        _lib = ctypes.CDLL(SO)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64


def _declare(L: ctypes.CDLL) -> None:
    L.orc_f16_to_f32.argtypes, L.orc_f16_to_f32.restype = [ctypes.c_uint16], ctypes.c_float
    L.orc_f32_to_f16.argtypes, L.orc_f32_to_f16.restype = [ctypes.c_float], ctypes.c_uint16
    L.orc_r16.argtypes, L.orc_r16.restype = [P, I64], ctypes.c_float
    L.orc_quantize_act.argtypes = [P, I, I, P, P]
    L.orc_group_dots.argtypes = [P, P, I, I, I, P]
    L.orc_w4a8_linear.argtypes = [P, P, P, P, P, I, I, I]
    L.orc_w4a8_linear_rows.argtypes = [P, P, P, P, P, I, I, I, P, I]
    L.orc_argmax.argtypes = [P, I, I64, P]
    L.orc_tree_accept.argtypes = [P, P, P, I, P, P]
    L.orc_kv_compact.argtypes = [P, I, I, I, I, I, P, I]
    for f in ("orc_quantize_act", "orc_group_dots", "orc_w4a8_linear", "orc_w4a8_linear_rows",
              "orc_argmax", "orc_tree_accept", "orc_kv_compact"):
        getattr(L, f).restype = I


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc < 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def f16_to_f32(bits: int) -> float:
    return lib().orc_f16_to_f32(bits)


def f32_to_f16(x: float) -> int:
    return lib().orc_f32_to_f16(x)


def r16(v: np.ndarray) -> np.float32:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(lib().orc_r16(_p(v), v.size))


def quantize_act(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, K = x.shape
    xq = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    _check(lib().orc_quantize_act(_p(x), T, K, _p(xq), _p(xs)), "quantize_act")
    return xq, xs


def group_dots(wq: np.ndarray, xq: np.ndarray) -> np.ndarray:
    N, Kh = wq.shape
    T, K = xq.shape
    assert Kh * 2 == K
    d = np.empty((T, N, K // 32), np.int32)
    _check(lib().orc_group_dots(_p(wq), _p(xq), T, N, K, _p(d)), "group_dots")
    return d


def w4a8_linear(wq: np.ndarray, ws: np.ndarray, xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    wq, ws = np.ascontiguousarray(wq), np.ascontiguousarray(ws)
    xq, xs = np.ascontiguousarray(xq), np.ascontiguousarray(xs, dtype=np.float32)
    N = wq.shape[0]
    T, K = xq.shape
    y = np.empty((T, N), np.float32)
    _check(lib().orc_w4a8_linear(_p(wq), _p(ws), _p(xq), _p(xs), _p(y), T, N, K), "w4a8_linear")
    return y


def w4a8_linear_rows(wq, ws, xq, xs, rows) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    N = wq.shape[0]
    T, K = xq.shape
    y = np.empty((T, rows.size), np.float32)
    _check(lib().orc_w4a8_linear_rows(_p(wq), _p(ws), _p(xq), _p(np.ascontiguousarray(xs, np.float32)),
                                      _p(y), T, N, K, _p(rows), rows.size), "w4a8_linear_rows")
    return y


def argmax(logits: np.ndarray) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    N, V = logits.shape
    out = np.empty(N, np.int32)
    _check(lib().orc_argmax(_p(logits), N, V, _p(out)), "argmax")
    return out


def tree_accept(parent, token, amax):
    parent = np.ascontiguousarray(parent, np.int32)
    token = np.ascontiguousarray(token, np.int32)
    amax = np.ascontiguousarray(amax, np.int32)
    N = parent.size
    path = np.zeros(max(N, 1), np.int32)
    bonus = np.zeros(1, np.int32)
    m = lib().orc_tree_accept(_p(parent), _p(token), _p(amax), N, _p(path), _p(bonus))
    _check(m, "tree_accept")
    return m, path[: m + 1].copy(), int(bonus[0])


def kv_compact(cache: np.ndarray, L: int, path: np.ndarray, m: int) -> None:
    """In place on cache uint16 [layers][heads][cap][hd]."""
    assert cache.dtype == np.uint16 and cache.flags["C_CONTIGUOUS"]
    layers, heads, cap, hd = cache.shape
    path = np.ascontiguousarray(path, np.int32)
    _check(lib().orc_kv_compact(_p(cache), layers, heads, cap, hd, L, _p(path), m), "kv_compact")

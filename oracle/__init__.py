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
SOURCES = ["oracle.c", "forward.c", "drafter.c"]
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
    """The oracle library: liboracle.so, or the build named by SPECV_ORACLE_SO
    (e.g. one compiled with sanitizers)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SPECV_ORACLE_SO") or SO
        if path == SO and not os.path.exists(SO):
            build()
        _lib = ctypes.CDLL(path)
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
    L.orc_quantize_act_blocks.argtypes = [P, I, I, P, P]
    L.orc_w4a8_linear_blocks.argtypes = [P, P, P, P, P, I, I, I]
    L.orc_argmax.argtypes = [P, I, I64, P]
    L.orc_tree_accept.argtypes = [P, P, P, I, P, P]
    L.orc_kv_compact.argtypes = [P, I, I, I, I, I, P, I]
    L.orc_det_exp.argtypes, L.orc_det_exp.restype = [ctypes.c_float], ctypes.c_float
    L.orc_silu.argtypes, L.orc_silu.restype = [ctypes.c_float], ctypes.c_float
    L.orc_rmsnorm.argtypes, L.orc_rmsnorm.restype = [P, P, I, ctypes.c_float, P], None
    L.orc_rope_table.argtypes = [P, P, I, I, ctypes.c_double]
    L.orc_attention.argtypes = [P, P, P, I, P, I, P]
    L.orc_forward.argtypes = [P, P, P, I, I, I, P, P, P]
    L.orc_tree_step.argtypes = [P, P, P, I, P, I, P, P, P, P, P, P]
    L.orc_draft_tree.argtypes = [I, I, ctypes.c_int32, P, I, P, ctypes.c_uint32, I, P, P, P]
    L.orc_cm_draft.argtypes = [P, I, I, I, I, P, I, P, P, P]
    for f in ("orc_quantize_act_blocks", "orc_w4a8_linear_blocks", "orc_quantize_act", "orc_group_dots", "orc_w4a8_linear", "orc_w4a8_linear_rows",
              "orc_argmax", "orc_tree_accept", "orc_kv_compact", "orc_rope_table", "orc_attention",
              "orc_forward", "orc_tree_step", "orc_draft_tree", "orc_cm_draft"):
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


def w4a8_linear_threads(wq: np.ndarray, ws: np.ndarray, xq: np.ndarray, xs: np.ndarray,
                        threads: int) -> np.ndarray:
    """w4a8_linear over blocks of output rows on `threads` host threads (the
    C call releases the interpreter lock). Every row is computed by the same
    code on the same inputs, so the result equals w4a8_linear bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    wq, ws = np.ascontiguousarray(wq), np.ascontiguousarray(ws)
    N = wq.shape[0]
    T = xq.shape[0]
    bounds = np.linspace(0, N, max(1, min(threads, N)) + 1).astype(int)
    y = np.empty((T, N), np.float32)

    def block(i):
        r0, r1 = bounds[i], bounds[i + 1]
        y[:, r0:r1] = w4a8_linear(wq[r0:r1], ws[r0:r1], xq, xs)

    with ThreadPoolExecutor(max_workers=len(bounds) - 1) as ex:
        list(ex.map(block, range(len(bounds) - 1)))
    return y


def quantize_act_blocks(x: np.ndarray):
    """Per-block (32 inputs) int8 codes and scales [T][K/32]."""
    x = np.ascontiguousarray(x, np.float32)
    T, K = x.shape
    xq = np.zeros((T, K), np.int8)
    xs = np.zeros((T, K // 32), np.float32)
    _check(lib().orc_quantize_act_blocks(_p(x), T, K, _p(xq), _p(xs)), "quantize_act_blocks")
    return xq, xs


def w4a8_linear_blocks(wq: np.ndarray, ws: np.ndarray, xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """W4A8 linear with per-block activation scales xs [T][K/32]."""
    wq, ws = np.ascontiguousarray(wq, np.uint8), np.ascontiguousarray(ws, np.uint16)
    xq, xs = np.ascontiguousarray(xq, np.int8), np.ascontiguousarray(xs, np.float32)
    N, T, K = wq.shape[0], xq.shape[0], xq.shape[1]
    y = np.zeros((T, N), np.float32)
    _check(lib().orc_w4a8_linear_blocks(_p(wq), _p(ws), _p(xq), _p(xs), _p(y), T, N, K), "w4a8_linear_blocks")
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


# ---------------------------------------------------------------- forward

def det_exp(x: float) -> np.float32:
    return np.float32(lib().orc_det_exp(x))


def silu(g: float) -> np.float32:
    return np.float32(lib().orc_silu(g))


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(w), x.size, eps, _p(y))
    return y


def rope_table(max_pos: int, head_dim: int, theta: float = 1e6):
    c = np.empty((max_pos, head_dim // 2), np.float32)
    s = np.empty((max_pos, head_dim // 2), np.float32)
    _check(lib().orc_rope_table(_p(c), _p(s), max_pos, head_dim, theta), "rope_table")
    return c, s


def attention(q: np.ndarray, kplane: np.ndarray, vplane: np.ndarray, rows) -> np.ndarray:
    """One query head over rows of one KV head plane [cap][hd] (fp16 bits)."""
    q = np.ascontiguousarray(q, np.float32)
    rows = np.ascontiguousarray(rows, np.int32)
    hd = q.size
    out = np.empty(hd, np.float32)
    _check(lib().orc_attention(_p(q), _p(np.ascontiguousarray(kplane)), _p(np.ascontiguousarray(vplane)),
                               hd, _p(rows), rows.size, _p(out)), "attention")
    return out


class _OrcModel(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim",
                                            "inter", "vocab", "max_pos")] + [("eps", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in ("wq", "sq", "wk", "sk", "wv", "sv", "wo", "so", "wg", "sg",
                                              "wu", "su", "wd", "sd", "norm_attn", "norm_mlp", "norm_final",
                                              "wlm", "slm", "rope_cos", "rope_sin")]


class Model:
    """Holds a model's host arrays (canonical layouts: nibbles [rows][K/2],
    scales [rows][K/32]) and the C struct that points into them."""

    def __init__(self, arrays: dict, cfg: dict):
        self.cfg, self.arrays = cfg, arrays
        self._keep = []
        c = _OrcModel()
        for k in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab", "max_pos"):
            setattr(c, k, int(cfg[k]))
        c.eps = float(cfg["eps"])
        for k in ("wq", "sq", "wk", "sk", "wv", "sv", "wo", "so", "wg", "sg", "wu", "su", "wd", "sd",
                  "norm_attn", "norm_mlp"):
            arr = (ctypes.c_void_p * cfg["n_layers"])(*[_p(a) for a in arrays[k]])
            self._keep.append(arr)
            setattr(c, k, ctypes.cast(arr, ctypes.c_void_p))
        for k in ("norm_final", "wlm", "slm", "rope_cos", "rope_sin"):
            setattr(c, k, _p(arrays[k]))
        self.c = c

    def ptr(self):
        return ctypes.addressof(self.c)


def forward(model: Model, kc: np.ndarray, vc: np.ndarray, L: int, parent, token) -> np.ndarray:
    """Forward over a tree; writes K/V rows L+i in place; returns logits [N][V]."""
    parent = np.ascontiguousarray(parent, np.int32)
    token = np.ascontiguousarray(token, np.int32)
    N = parent.size
    logits = np.empty((N, model.cfg["vocab"]), np.float32)
    cap = kc.shape[2]
    _check(lib().orc_forward(model.ptr(), _p(kc), _p(vc), cap, L, N, _p(parent), _p(token), _p(logits)),
           "forward")
    return logits


def tree_step(model: Model, kc: np.ndarray, vc: np.ndarray, L: int, parent, token, want_logits=False):
    """Forward + argmax + acceptance + compaction. Returns dict with m, path,
    bonus, amax, new L (and logits)."""
    parent = np.ascontiguousarray(parent, np.int32)
    token = np.ascontiguousarray(token, np.int32)
    N = parent.size
    logits = np.empty((N, model.cfg["vocab"]), np.float32) if want_logits else None
    amax = np.empty(N, np.int32)
    path = np.zeros(N, np.int32)
    bonus = np.zeros(1, np.int32)
    Lb = ctypes.c_int(L)
    m = lib().orc_tree_step(model.ptr(), _p(kc), _p(vc), kc.shape[2], ctypes.byref(Lb), N, _p(parent),
                            _p(token), _p(logits) if logits is not None else None, _p(amax), _p(path),
                            _p(bonus))
    _check(m, "tree_step")
    return {"m": m, "path": path[: m + 1].copy(), "bonus": int(bonus[0]), "amax": amax, "L": Lb.value,
            "logits": logits}


def draft_tree(width, L, root_token, greedy, draws, threshold, vocab):
    greedy = np.ascontiguousarray(greedy, np.int32)
    draws = np.ascontiguousarray(draws, np.uint32)
    parent = np.zeros(width, np.int32)
    token = np.zeros(width, np.int32)
    bm = ctypes.c_int(0)
    _check(lib().orc_draft_tree(width, L, root_token, _p(greedy), greedy.size, _p(draws), threshold, vocab,
                                _p(parent), _p(token), ctypes.byref(bm)), "draft_tree")
    return parent, token, bm.value


def cm_draft(stream, width: int, max_order: int = 8, cands: int = 16, depth: int = 8, weight=None):
    """Context-mixing drafter: (parent, token, n_nodes, best_match) of the
    next tree from the token stream (committed tokens + pending root)."""
    s = np.ascontiguousarray(stream, np.int32)
    w = np.ascontiguousarray(CM_WEIGHT if weight is None else weight, np.uint32)
    assert w.size == 9
    parent = np.zeros(width, np.int32)
    token = np.zeros(width, np.int32)
    bm = ctypes.c_int32(0)
    n = lib().orc_cm_draft(_p(s), s.size, max_order, cands, depth, _p(w), width, _p(parent), _p(token),
                           ctypes.byref(bm))
    _check(n, "cm_draft")
    return parent[:n].copy(), token[:n].copy(), n, bm.value


# Default candidate weight by match length l = 0..8: 2^(l-1), so one match
# one token longer counts as much as two shorter ones.
CM_WEIGHT = [0, 1, 2, 4, 8, 16, 32, 64, 128]


def window(model: Model, kc, vc, ctrl: dict, width: int, W: int, greedy, draws_table, threshold):
    """W speculation steps of the device-resident window, driven by the
    control state (committed_len, root_token, step, done, ctx_len, ring):
    each step drafts a tree, verifies it, accepts and compacts. Steps after
    `done` do nothing. Returns the per-step statistics and emitted tokens."""
    stats, emitted = [], []
    for _ in range(W):
        if ctrl["done"]:
            stats.append((-1, 0, width))
            ctrl["accept_len"] = 0
            continue
        L = ctrl["committed_len"]
        parent, token, bm = draft_tree(width, L, ctrl["root_token"], greedy,
                                       draws_table[ctrl["step"] % len(draws_table)], threshold,
                                       model.cfg["vocab"])
        r = tree_step(model, kc, vc, L, parent, token)
        m = r["m"]
        out = [int(token[p]) for p in r["path"][1:]] + [r["bonus"]]
        emitted.extend(out)
        ctrl.update(committed_len=r["L"], accept_len=m, root_token=r["bonus"], step=ctrl["step"] + 1,
                    ring_head=ctrl["ring_head"] + m + 1)
        if r["L"] + width > ctrl["ctx_len"]:
            ctrl["done"] = 1
        stats.append((m, bm, width))
    return stats, emitted


def window_cm(model: Model, kc, vc, ctrl: dict, width: int, W: int, history, max_order: int = 8,
              cands: int = 16, depth: int = 8, weight=None):
    """W speculation steps drafted by the context-mixing drafter. `history`
    (a list, extended in place) holds the token stream: history[i] is the
    token at position i, history[committed_len] the pending root. Returns the
    per-step statistics (m, best match, nodes) and the emitted tokens."""
    stats, emitted = [], []
    for _ in range(W):
        if ctrl["done"]:
            stats.append((-1, 0, ctrl["n_nodes"]))
            ctrl["accept_len"] = 0
            continue
        L = ctrl["committed_len"]
        assert len(history) == L + 1 and history[L] == ctrl["root_token"]
        parent, token, n, bm = cm_draft(history, width, max_order, cands, depth, weight)
        r = tree_step(model, kc, vc, L, parent, token)
        m = r["m"]
        out = [int(token[p]) for p in r["path"][1:]] + [r["bonus"]]
        emitted.extend(out)
        history.extend(out)
        ctrl.update(committed_len=r["L"], n_nodes=n, accept_len=m, root_token=r["bonus"], step=ctrl["step"] + 1,
                    ring_head=ctrl["ring_head"] + m + 1)
        if r["L"] + n > ctrl["ctx_len"]:   # the step's own node count, as the acceptance rule states
            ctrl["done"] = 1
        stats.append((m, bm, n))
    return stats, emitted

"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and shapes them into arrays. It holds
none of the arithmetic of the verification method: no quantisation, no dot
products, no reductions. Both sides receive the same arrays from here.

The generator is SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used in counter mode: the i-th
output of a stream is the SplitMix64 finaliser applied to key + (i+1)*gamma,
so any slice of a stream can be produced independently of the rest.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> np.uint64:
    """Key of the stream for one (config seed, tensor id) pair."""
    with np.errstate(over="ignore"):
        a = _mix(np.array([(seed * 0x100000001B3 + 0x51) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))
        b = _mix(a ^ np.uint64(tensor_id & 0xFFFFFFFFFFFFFFFF))
    return b[0]


_CHUNK = 1 << 20


def u64(key: np.uint64, n: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+n-1 of stream `key` as uint64."""
    out = np.empty(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for c0 in range(0, n, _CHUNK):
            c1 = min(n, c0 + _CHUNK)
            ctr = np.arange(start + c0 + 1, start + c1 + 1, dtype=np.uint64)
            out[c0:c1] = _mix(np.uint64(key) + ctr * GAMMA)
    return out


def uniform(key: np.uint64, n: int, start: int = 0) -> np.ndarray:
    """Doubles uniform in [0, 1) from the top 53 bits."""
    return (u64(key, n, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_f32(key: np.uint64, n: int) -> np.ndarray:
    """float32 N(0,1) by the Box-Muller transform evaluated in double."""
    m = (n + 1) // 2
    u = uniform(key, 2 * m)
    u1 = 1.0 - u[0::2]            # (0, 1]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return z[:n].astype(np.float32)


def uniform_f32(key: np.uint64, n: int, lo: float, hi: float) -> np.ndarray:
    return (lo + (hi - lo) * uniform(key, n)).astype(np.float32)


def packed_nibbles(key: np.uint64, rows: int, k: int) -> np.ndarray:
    """uint8 [rows][k/2]: every nibble uniform in 0..15 (two per byte)."""
    assert k % 2 == 0
    nbytes = rows * (k // 2)
    words = u64(key, (nbytes + 7) // 8)
    return words.view(np.uint8)[:nbytes].reshape(rows, k // 2).copy()


def fp16_bits_uniform(key: np.uint64, n: int, lo: float, hi: float) -> np.ndarray:
    """uint16 bit patterns of fp16 values U(lo, hi), rounded to nearest even."""
    v = lo + (hi - lo) * uniform(key, n)
    return v.astype(np.float16).view(np.uint16)


def fp16_bits_normal(key: np.uint64, n: int) -> np.ndarray:
    return normal_f32(key, n).astype(np.float16).view(np.uint16)


def tokens(key: np.uint64, n: int, vocab: int) -> np.ndarray:
    """int32 token ids uniform in [0, vocab) (multiply-shift on the top 32 bits)."""
    hi = u64(key, n) >> np.uint64(32)
    return ((hi * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)


def random_tree_parents(key: np.uint64, n: int) -> np.ndarray:
    """Topologically ordered parent array: parent[0] = -1, parent[i] ~ U{0..i-1}."""
    u = uniform(key, n)
    p = np.floor(u * np.arange(n)).astype(np.int32)
    p[0] = -1
    return p


def u32(key: np.uint64, n: int) -> np.ndarray:
    return (u64(key, n) >> np.uint64(32)).astype(np.uint32)


# Tensor ids used across tests and the benchmark, so every consumer of a
# config draws the same bytes.
TID_WQ, TID_WS, TID_X, TID_LOGITS, TID_PARENT, TID_TOKEN, TID_KV = 1, 2, 3, 4, 5, 6, 7
TID_NORM, TID_DRAFT = 8, 9


def linear_case(seed: int, T: int, N: int, K: int, layer: int = 0):
    """One W4A8 linear workload: int4 g32 weights with fp16 scales drawn
    U(0.005, 0.02), fp32 N(0,1) activations. Returns (wq, ws_bits, x)."""
    base = layer * 16
    wq = packed_nibbles(stream_key(seed, base + TID_WQ), N, K)
    ws = fp16_bits_uniform(stream_key(seed, base + TID_WS), N * (K // 32), 0.005, 0.02)
    x = normal_f32(stream_key(seed, base + TID_X), T * K).reshape(T, K)
    return wq, ws.reshape(N, K // 32), x


# ---------------------------------------------------------------- models

QWEN05 = dict(n_layers=24, hidden=896, n_heads=14, n_kv_heads=2, head_dim=64, inter=4864, vocab=151936,
              eps=1e-6, max_pos=4096 + 64)
TINY = dict(n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, inter=96, vocab=300,
            eps=1e-6, max_pos=640)


def model_case(seed: int, cfg: dict, distinct_layers: int | None = None) -> dict:
    """Random W4A8 model arrays of a Qwen2.5-shaped decoder: int4 g32 weights
    (codes uniform, fp16 scales U(0.005, 0.02), scales row-major
    [rows][K/32]), RMSNorm weights U(0.9, 1.1). distinct_layers < n_layers
    reuses layer l % distinct_layers (the copies are separate arrays)."""
    H, nh, nkv, hd, I, V = (cfg[k] for k in ("hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab"))
    nd = distinct_layers or cfg["n_layers"]
    shapes = {"q": (nh * hd, H), "k": (nkv * hd, H), "v": (nkv * hd, H), "o": (H, nh * hd),
              "g": (I, H), "u": (I, H), "d": (H, I)}
    out = {f"{p}{n}": [] for n in shapes for p in ("w", "s")}
    out["norm_attn"], out["norm_mlp"] = [], []
    gen = []
    for l in range(nd):
        layer = {}
        for i, (n, (rows, K)) in enumerate(shapes.items()):
            layer["w" + n] = packed_nibbles(stream_key(seed, 1000 + 40 * l + 2 * i), rows, K)
            layer["s" + n] = fp16_bits_uniform(stream_key(seed, 1001 + 40 * l + 2 * i), rows * (K // 32),
                                               0.005, 0.02).reshape(rows, K // 32)
        layer["norm_attn"] = uniform_f32(stream_key(seed, 1030 + 40 * l), H, 0.9, 1.1)
        layer["norm_mlp"] = uniform_f32(stream_key(seed, 1031 + 40 * l), H, 0.9, 1.1)
        gen.append(layer)
    for l in range(cfg["n_layers"]):
        src = gen[l % nd]
        for k, v in src.items():
            out[k].append(v if l < nd else v.copy())
    out["norm_final"] = uniform_f32(stream_key(seed, 90), H, 0.9, 1.1)
    out["wlm"] = packed_nibbles(stream_key(seed, 91), V, H)
    out["slm"] = fp16_bits_uniform(stream_key(seed, 92), V * (H // 32), 0.005, 0.02).reshape(V, H // 32)
    return out


def kv_prefix(seed: int, cfg: dict, L: int, cap: int):
    """fp16 K and V caches [layers][kv_heads][cap][hd] whose first L rows are
    N(0,1) values; rows >= L are zero."""
    shape = (cfg["n_layers"], cfg["n_kv_heads"], cap, cfg["head_dim"])
    kc = np.zeros(shape, np.uint16)
    vc = np.zeros(shape, np.uint16)
    n = cfg["n_layers"] * cfg["n_kv_heads"] * L * cfg["head_dim"]
    kc[:, :, :L] = fp16_bits_normal(stream_key(seed, 95), n).reshape(shape[0], shape[1], L, shape[3])
    vc[:, :, :L] = fp16_bits_normal(stream_key(seed, 96), n).reshape(shape[0], shape[1], L, shape[3])
    return kc, vc


def draft_draws(seed: int, steps: int, width: int = 16) -> np.ndarray:
    """Per-step, per-node uint32 draws of the synthetic drafter [steps][16]."""
    return u32(stream_key(seed, 97), steps * width).reshape(steps, width)

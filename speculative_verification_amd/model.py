"""Device model for the tree-masked verification step.

Packs a decoder given in the interchange layout (per layer: nibbles
[rows][K/2] and scales [rows][K/32] for q, k, v, o, gate, up, down; norms;
lm_head) into the library's device layout (q/k/v rows concatenated, gate and
up rows alternating in blocks of 8, each matrix in the packed tile layout of
w4a8_pack_weights, layers one after another), and exposes the step. Layout conversion only:
all arithmetic runs in libspecv.so.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import LIB, SpecvDrafter, SpecvModel, check, cm_params

CFG_KEYS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "vocab", "max_pos")


def _gate_up_blocks(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Gate and up rows [I][...] alternating in blocks of 8 (gate rows 8b..8b+7,
    then up rows 8b..8b+7): the row order of the library's gate_up matrix,
    whose epilogue pairs gate row i with up row i."""
    I = g.shape[0]
    if I % 8 or u.shape != g.shape:
        raise ValueError("gate and up need the same shape with a multiple of 8 rows")
    return np.ascontiguousarray(np.stack([g.reshape(I // 8, 8, -1), u.reshape(I // 8, 8, -1)], axis=1)
                                .reshape(2 * I, -1))


def _pack_layers(nl: int, wfn, sfn, dev) -> tuple[torch.Tensor, torch.Tensor]:
    """Layers' interchange matrices (wfn(l): nibbles [rows][K/2], sfn(l):
    scales [rows][K/32]) packed one after another into flat device buffers."""
    from . import pack_weights, packed_sizes
    w0 = wfn(0)
    rows, K = w0.shape[0], 2 * w0.shape[1]
    wb, se = packed_sizes(rows, K)
    wp = torch.empty(nl * wb, dtype=torch.uint8, device=dev)
    sp = torch.empty(nl * se, dtype=torch.int16, device=dev)
    for l in range(nl):
        wq = torch.from_numpy(np.ascontiguousarray(wfn(l))).to(dev)
        ws = torch.from_numpy(np.ascontiguousarray(sfn(l)).view(np.int16)).to(dev)
        pack_weights(wq, ws, wp[l * wb:(l + 1) * wb], sp[l * se:(l + 1) * se])
    torch.cuda.synchronize(dev)
    return wp, sp


class DeviceModel:
    def __init__(self, arrays: dict, cfg: dict, kv_capacity: int, k_cache=None, v_cache=None,
                 rope_theta: float = 1e6, device="cuda"):
        self.cfg = dict(cfg)
        dev = torch.device(device)
        nl = cfg["n_layers"]

        def stack(fn):
            return torch.from_numpy(np.ascontiguousarray(np.stack([fn(l) for l in range(nl)]))).to(dev)

        a = arrays
        self.w_qkv, self.s_qkv = _pack_layers(nl, lambda l: np.concatenate([a["wq"][l], a["wk"][l], a["wv"][l]]),
                                              lambda l: np.concatenate([a["sq"][l], a["sk"][l], a["sv"][l]]), dev)
        self.w_o, self.s_o = _pack_layers(nl, lambda l: a["wo"][l], lambda l: a["so"][l], dev)
        self.w_gu, self.s_gu = _pack_layers(nl, lambda l: _gate_up_blocks(a["wg"][l], a["wu"][l]),
                                            lambda l: _gate_up_blocks(a["sg"][l], a["su"][l]), dev)
        self.w_down, self.s_down = _pack_layers(nl, lambda l: a["wd"][l], lambda l: a["sd"][l], dev)
        self.norm_attn = stack(lambda l: arrays["norm_attn"][l])
        self.norm_mlp = stack(lambda l: arrays["norm_mlp"][l])
        self.norm_final = torch.from_numpy(arrays["norm_final"]).to(dev)
        self.w_lm, self.s_lm = _pack_layers(1, lambda l: a["wlm"], lambda l: a["slm"], dev)
        half = cfg["head_dim"] // 2
        c = np.empty((cfg["max_pos"], half), np.float32)
        s = np.empty((cfg["max_pos"], half), np.float32)
        check("specv_rope_table", LIB.specv_rope_table(c.ctypes.data, s.ctypes.data, cfg["max_pos"],
                                                       cfg["head_dim"], rope_theta))
        self.rope_cos = torch.from_numpy(c).to(dev)
        self.rope_sin = torch.from_numpy(s).to(dev)
        shape = (nl, cfg["n_kv_heads"], kv_capacity, cfg["head_dim"])
        self.k_cache = (torch.from_numpy(k_cache.view(np.int16)).to(dev) if k_cache is not None
                        else torch.zeros(shape, dtype=torch.int16, device=dev))
        self.v_cache = (torch.from_numpy(v_cache.view(np.int16)).to(dev) if v_cache is not None
                        else torch.zeros(shape, dtype=torch.int16, device=dev))
        assert tuple(self.k_cache.shape) == shape and tuple(self.v_cache.shape) == shape
        m = SpecvModel()
        for k in CFG_KEYS:
            setattr(m, k, int(cfg[k]))
        m.eps = float(cfg["eps"])
        m.kv_capacity = kv_capacity
        for k in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gu", "s_gu", "w_down", "s_down", "norm_attn", "norm_mlp",
                  "norm_final", "w_lm", "s_lm", "rope_cos", "rope_sin", "k_cache", "v_cache"):
            setattr(m, k, getattr(self, k).data_ptr())
        self.c = m
        self._ws = {}

    def ptr(self):
        return ctypes.addressof(self.c)

    def workspace(self, n_max: int) -> torch.Tensor:
        need = int(LIB.spec_step_workspace(self.ptr(), n_max))
        if need == 0:
            raise ValueError("model or n_max rejected by spec_step_workspace")
        ws = self._ws.get(n_max)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(need, dtype=torch.uint8, device=self.k_cache.device)
            self._ws[n_max] = ws
        return ws

    def tree_step(self, ctrl: torch.Tensor, parent: torch.Tensor, token: torch.Tensor, n_max: int,
                  logits: torch.Tensor | None = None, stats: torch.Tensor | None = None,
                  ring: torch.Tensor | None = None, want_logits: bool = True):
        """One verification step (spec_tree_step). Returns (logits, argmax,
        path); logits is None when want_logits is false (not written)."""
        dev = self.k_cache.device
        V = self.cfg["vocab"]
        if want_logits and logits is None:
            logits = torch.empty((n_max, V), dtype=torch.float32, device=dev)
        argmax = torch.empty(n_max, dtype=torch.int32, device=dev)
        path = torch.zeros(n_max, dtype=torch.int32, device=dev)
        ws = self.workspace(n_max)
        check("spec_tree_step", LIB.spec_tree_step(
            self.ptr(), ctrl.data_ptr(), parent.data_ptr(), token.data_ptr(), n_max,
            logits.data_ptr() if want_logits else None,
            argmax.data_ptr(), path.data_ptr(), stats.data_ptr() if stats is not None else None,
            ring.data_ptr() if ring is not None else None, ring.numel() if ring is not None else 0,
            ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream))
        return logits, argmax, path

    def window_cm(self, ctrl: torch.Tensor, stats: torch.Tensor, width: int, W: int, ring: torch.Tensor,
                  params=None, readback: torch.Tensor | None = None):
        """W speculation steps drafted by the context-mixing drafter
        (spec_window_run_cm). `ring` int32 holds the token stream: ring[i] is
        the token at position i (committed tokens, then the root), with
        ctrl's ring_head = committed_len + 1."""
        p = params if params is not None else cm_params()
        assert ring.dtype == torch.int32 and stats.dtype == torch.int32 and stats.numel() >= 3 * W
        if readback is not None:
            assert readback.device.type == "cpu" and readback.numel() * readback.element_size() >= 32 + 12 * W
        need = int(LIB.spec_window_cm_workspace(self.ptr(), width, ring.numel(), ctypes.byref(p)))
        if need == 0:
            raise ValueError("spec_window_cm_workspace rejected its arguments")
        key = ("cm", width, ring.numel())
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(need, dtype=torch.uint8, device=self.k_cache.device)
            self._ws[key] = ws
        check("spec_window_run_cm", LIB.spec_window_run_cm(
            self.ptr(), ctrl.data_ptr(), stats.data_ptr(), ring.data_ptr(), ring.numel(), ctypes.byref(p), width, W,
            ws.data_ptr(), ws.numel(), readback.data_ptr() if readback is not None else None,
            torch.cuda.current_stream().cuda_stream))

    def window(self, ctrl: torch.Tensor, stats: torch.Tensor, width: int, W: int,
               reference: torch.Tensor | None = None, draws: torch.Tensor | None = None, threshold: int = 0,
               ring: torch.Tensor | None = None, readback: torch.Tensor | None = None):
        """W device-resident speculation steps (spec_window_run). `reference`
        int32 and `draws` uint32-as-int32 [rows][16] feed the synthetic
        drafter (not needed for width 1); `stats` is int32 [>= W][3];
        `readback`, if given, is a pinned uint8 host tensor of >= 32 + 12*W
        bytes that receives ctrl and stats[0..W) on the current stream."""
        d = None
        if reference is not None:
            assert reference.dtype == torch.int32 and draws.dtype == torch.int32 and draws.shape[-1] == 16
            d = SpecvDrafter(reference.data_ptr(), reference.numel(), draws.shape[0], draws.data_ptr(),
                             int(threshold) & 0xFFFFFFFF, 0)
        assert stats.dtype == torch.int32 and stats.numel() >= 3 * W
        if readback is not None:
            assert readback.device.type == "cpu" and readback.numel() * readback.element_size() >= 32 + 12 * W
        ws = self.workspace(width)
        check("spec_window_run", LIB.spec_window_run(
            self.ptr(), ctrl.data_ptr(), stats.data_ptr(), ring.data_ptr() if ring is not None else None,
            ring.numel() if ring is not None else 0, ctypes.byref(d) if d is not None else None, width, W,
            ws.data_ptr(), ws.numel(), readback.data_ptr() if readback is not None else None,
            torch.cuda.current_stream().cuda_stream))

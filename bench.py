#!/usr/bin/env python3
"""Benchmark of one deterministic small-batch verification step on one GPU.

A step verifies a T-node tree (default T = 8) through a W4A8 linear stack of
a Llama-3-8B-shaped model and then accepts on the GPU:
  the per-token int8 quantisation of every input row of the step (each
  linear has its own fp32 N(0,1) input; one launch per input width K, as a
  model fuses this quantisation into the kernel producing the activations);
  per layer (32): qkv (6144x4096, q/k/v rows concatenated), o (4096x4096),
  gate_up (28672x4096, gate/up rows concatenated), down (4096x14336);
  then lm_head (128256x4096) with the fused argmax epilogue (the logits are
  not written) and tree acceptance from its (value, row) pairs, then KV
  compaction of the accepted rows (32 layers x 8 KV heads x head_dim 128).
Weights are int4 in groups of 32 with fp16 scales U(0.005, 0.02). The
weights of 4 distinct generated layer sets are copied into 32 separate layer
buffers plus one lm_head, 4.22 GB in total, so every step streams each byte
from HBM once (far above the 256 MB last-level cache). The step is captured
once as a HIP graph and replayed.

The line also times the same step on the Qwen2.5-0.5B linear set
(`small_set`: 24 layers of qkv 1152x896, o 896x896, gate_up 9728x896,
down 896x4864, then lm_head 151936x896; four copies of its 278 MB of weights
in rotation, so that each step reads its copy cold) at T = 1, 2, 4, 8.

The line also times the 32-token prefill bucket on the same 8B weights
(`prefill`: the quantisation and the 129 linears at T = 32, the lm_head
writing logits).

The line also carries the single 896x896 linear at T = 1 (`config1`, a
latency: its weights stay in the L2 cache), the full 8-node tree
verification step on the 24-layer Qwen2.5-0.5B shape at a 1024-row cache
(`decoder`), the device-resident windows on that decoder (`window`), and the
CPU oracle on bounded samples of these workloads (`cpu_baseline`).

Prints one JSON line (rank 0). `value` is the algorithmic bytes of the step
(weights, activation codes and scales, linear outputs, quantisation traffic,
argmax pairs, compaction moves) divided by the step time, in
GB/s, at T = 8.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# Figures of the linear kernel taken by rocprofv3 on this bench's own command
# (profiles/w4a8_linear_llama8b_T8*.md), stored with the hash of the kernel
# source they were taken on: HBM bytes per linear launch of the T = 8 step
# from the FETCH_SIZE and WRITE_SIZE counter passes (each scaled by a plain
# 256 MiB device copy), and the kernel trace's mean duration per launch.
LINEAR_PROFILE = {"source_sha256": "2c3ddf8187a92a1296ebea7d5ce4c03aaa74ae7822172efec00270e8eae6d924",
                  "T": 8, "workload": "llama3-8b", "bytes_per_launch": 33625599,
                  "rocprof_mean_us": 7.961, "summary": "profiles/w4a8_linear_llama8b_T8.md"}


def linear_profile(T, workload):
    """The stored rocprofv3 figures, or None when the kernel source has
    changed since they were taken (or the workload differs)."""
    import hashlib
    src = os.path.join(ROOT, "speculative_verification_amd", "csrc", "linear.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    ok = h == LINEAR_PROFILE["source_sha256"] and T == LINEAR_PROFILE["T"] and workload == LINEAR_PROFILE["workload"]
    return LINEAR_PROFILE if ok else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads():
    """Host CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def graph_us(torch, fn, n, reps=5):
    """Median time of a graph of fn's launches divided by n (fn enqueues on
    the current stream); fn runs once eagerly first."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    del g
    return float(np.median(ts)) / n
METRIC = "W4A8 verify GB/s & % HBM peak at T=1..8; T=8/T=1 cost ratio; µs/verify"

MODELS = {
    "llama3-8b": dict(hidden=4096, layers=32, qkv=4096 + 2 * 1024, inter=14336, vocab=128256,
                      kv_heads=8, head_dim=128, copies=1, distinct=4),
    "qwen2.5-0.5b": dict(hidden=896, layers=24, qkv=896 + 2 * 128, inter=4864, vocab=151936,
                         kv_heads=2, head_dim=64, copies=4, distinct=4),
}


def layer_linears(m):
    return [("qkv", m["qkv"], m["hidden"]), ("o", m["hidden"], m["hidden"]),
            ("gate_up", 2 * m["inter"], m["hidden"]), ("down", m["hidden"], m["inter"])]


def weight_bytes(N, K):
    return N * K // 2 + N * (K // 32) * 2


def linear_bytes(T, N, K):
    """Algorithmic bytes of one W4A8 linear launch."""
    return weight_bytes(N, K) + T * K + 4 * T + 4 * T * N


def argmax_linear_bytes(T, N, K, chunks):
    """Algorithmic bytes of the fused lm_head + argmax launch: weights,
    activation codes and scales, and one (value, index) pair per token and
    workgroup (the logits are not written)."""
    return weight_bytes(N, K) + T * K + 4 * T + 8 * T * chunks


def quant_bytes(T, K):
    return 4 * T * K + T * K + 4 * T


def timing_events(torch):
    """A pair of timing events, created now (torch creates events lazily at
    their first record) so their handles can be passed to the library."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    return e0, e1


class Model:
    def __init__(self, name, torch, sv, sg, Tmax):
        m = MODELS[name]
        self.m, self.torch, self.sv = m, torch, sv
        dev = torch.device("cuda")
        self.copies = []
        host_sets = []
        t0 = time.time()
        for d in range(m["distinct"]):
            lay = {}
            for i, (nm, N, K) in enumerate(layer_linears(m)):
                wq, ws, _ = sg.linear_case(d, 1, N, K, layer=16 * d + i)
                lay[nm] = (wq, ws)
            host_sets.append(lay)
        wq, ws, _ = sg.linear_case(99, 1, m["vocab"], m["hidden"], layer=1000)
        host_lm = (wq, ws)
        self.host_sets, self.gen_s = host_sets, time.time() - t0
        def pack(a, b):  # interchange nibbles and scales -> the library's packed tile layout
            return sv.pack_weights(torch.from_numpy(a).to(dev), torch.from_numpy(b.view(np.int16)).to(dev))

        def clone(p):
            return sv.Packed(p.wp.clone(), p.sp.clone(), p.N, p.K)
        dev_sets = [{nm: pack(a, b) for nm, (a, b) in s.items()} for s in host_sets]
        for c in range(m["copies"]):
            layers = []
            for l in range(m["layers"]):
                src = dev_sets[(l + c) % m["distinct"]]
                layers.append({nm: clone(p) for nm, p in src.items()})
            lm = pack(*host_lm)
            self.copies.append((layers, lm if c == 0 else clone(lm)))
        del dev_sets
        # activations: every linear of the step has its own fp32 input rows,
        # generated once per K as [inputs][Tmax][K]
        self.inputs = {}   # K -> number of linears of the step that consume K-wide rows
        self.in_index = []  # per layer: {linear name: input index within its K}
        for l in range(m["layers"]):
            idx = {}
            for nm, _, K in layer_linears(m):
                idx[nm] = self.inputs.get(K, 0)
                self.inputs[K] = idx[nm] + 1
            self.in_index.append(idx)
        self.lm_index = self.inputs.get(m["hidden"], 0)
        self.inputs[m["hidden"]] = self.lm_index + 1
        self.host_x = {K: sg.normal_f32(sg.stream_key(5, 3 + K), n * Tmax * K).reshape(n, Tmax, K)
                       for K, n in self.inputs.items()}
        self.act_T = None
        self.y = {nm: torch.empty((Tmax * N,), dtype=torch.float32, device=dev)
                  for nm, N, _ in layer_linears(m)}
        # tree, control block and KV cache
        self.L0 = 1024
        self.cap = self.L0 + 4096
        self.kc = torch.zeros((m["layers"], m["kv_heads"], self.cap, m["head_dim"]), dtype=torch.int16, device=dev)
        self.vc = torch.zeros_like(self.kc)
        self.ws_lmarg = torch.empty(int(sv.LIB.w4a8_linear_argmax_workspace(min(Tmax, 16), m["vocab"],
                                                                            m["hidden"])),
                                    dtype=torch.uint8, device=dev)
        self.logits = None  # [T][vocab] of the prefill bucket, allocated on first use
        self.argmax = torch.empty(16, dtype=torch.int32, device=dev)
        self.path = torch.zeros(16, dtype=torch.int32, device=dev)
        self.stats = torch.zeros(3, dtype=torch.int32, device=dev)
        self.ring = torch.zeros(4096, dtype=torch.int32, device=dev)
        self.ctrl = torch.zeros(8, dtype=torch.int32, device=dev)
        self.sg = sg

    def set_tree(self, T, token_plant=None):
        torch, sg = self.torch, self.sg
        parent = sg.random_tree_parents(sg.stream_key(T, sg.TID_PARENT), T)
        token = sg.tokens(sg.stream_key(T, sg.TID_TOKEN), T, self.m["vocab"])
        if token_plant is not None:
            depth = np.zeros(T, np.int32)
            for i in range(1, T):
                depth[i] = depth[parent[i]] + 1
            c = int(np.argmax(depth))
            while c != 0:
                token[c] = token_plant[parent[c]]
                c = int(parent[c])
        self.parent = torch.from_numpy(parent).cuda()
        self.token = torch.from_numpy(token).cuda()

    def prepare_acts(self, T):
        """Device copies of the step's fp32 inputs at T tokens, [inputs][T][K]
        contiguous, and their quantised buffers."""
        torch = self.torch
        if self.act_T == T:
            return
        dev = torch.device("cuda")
        self.xa = {K: torch.from_numpy(np.ascontiguousarray(hx[:, :T])).to(dev) for K, hx in self.host_x.items()}
        self.xqa = {K: torch.empty(tuple(x.shape), dtype=torch.int8, device=dev) for K, x in self.xa.items()}
        self.xsa = {K: torch.empty(tuple(x.shape[:2]), dtype=torch.float32, device=dev) for K, x in self.xa.items()}
        self.act_T = T

    def reset_ctrl(self, T):
        self.ctrl.copy_(self.torch.tensor([self.L0, T, self.cap - 16, 0, 0, 0, 0, 0], dtype=self.torch.int32))

    def step(self, T, copy=0, events=None):
        """Enqueue one verify step: the quantisation of every input row of the
        step (one launch per K), the linears, the lm_head with acceptance from
        its argmax pairs, compaction.
        events: list to which (start, end, bytes, name) of each linear launch
        are appended (eager roofline timing only)."""
        sv, torch, m = self.sv, self.torch, self.m
        layers, lm = self.copies[copy]
        self.prepare_acts(T)
        for K, x in self.xa.items():
            n = x.shape[0]
            sv.quantize_act(x.view(n * T, K), self.xqa[K].view(n * T, K), self.xsa[K].view(n * T))

        def lin(name, w, K, N, y, i):
            xq, xs = self.xqa[K][i], self.xsa[K][i]
            if events is not None:   # kernel begin/end timestamps of this launch
                e0, e1 = timing_events(torch)
                sv.check("specv_time_next_linear", sv.LIB.specv_time_next_linear(e0.cuda_event, e1.cuda_event))
            if y is None:            # lm_head: argmax epilogue, then acceptance from its pairs
                sv.linear_argmax_accept(w, xq, xs, self.parent, self.token, self.ctrl, argmax=self.argmax[:T],
                                        path=self.path, stats=self.stats, ring=self.ring, workspace=self.ws_lmarg)
                nb = argmax_linear_bytes(T, N, K, self.lm_chunks(T))
            else:
                sv.linear(w, xq, xs, y[: T * N].view(T, N))
                nb = linear_bytes(T, N, K)
            if events is not None:
                events.append((e0, e1, nb, name))

        for l, lay in enumerate(layers):
            for nm, N, K in layer_linears(m):
                lin(nm, lay[nm], K, N, self.y[nm], self.in_index[l][nm])
        lin("lm_head", lm, m["hidden"], m["vocab"], None, self.lm_index)
        sv.kv_compact(self.kc, self.vc, self.path, self.ctrl)

    def prefill_step(self, T, copy=0, events=None):
        """The step's linears at T tokens (the prefill bucket, T up to 32):
        the quantisation of every input row, the 128 layer linears and the
        lm_head writing its logits (no tree: acceptance and the argmax
        epilogue take at most 16 nodes)."""
        sv, torch, m = self.sv, self.torch, self.m
        layers, lm = self.copies[copy]
        self.prepare_acts(T)
        if self.logits is None or self.logits.shape[0] < T:
            self.logits = torch.empty((T, m["vocab"]), dtype=torch.float32, device="cuda")
        for K, x in self.xa.items():
            n = x.shape[0]
            sv.quantize_act(x.view(n * T, K), self.xqa[K].view(n * T, K), self.xsa[K].view(n * T))

        def lin(name, w, K, N, y, i):
            xq, xs = self.xqa[K][i], self.xsa[K][i]
            if events is not None:
                e0, e1 = timing_events(torch)
                sv.check("specv_time_next_linear", sv.LIB.specv_time_next_linear(e0.cuda_event, e1.cuda_event))
            sv.linear(w, xq, xs, y)
            if events is not None:
                events.append((e0, e1, linear_bytes(T, N, K), name))

        for l, lay in enumerate(layers):
            for nm, N, K in layer_linears(m):
                lin(nm, lay[nm], K, N, self.y[nm][: T * N].view(T, N), self.in_index[l][nm])
        lin("lm_head", lm, m["hidden"], m["vocab"], self.logits[:T], self.lm_index)

    def prefill_bytes(self, T):
        m = self.m
        b = sum(m["layers"] * (linear_bytes(T, N, K) + quant_bytes(T, K)) for _, N, K in layer_linears(m))
        return b + linear_bytes(T, m["vocab"], m["hidden"]) + quant_bytes(T, m["hidden"])

    def lm_chunks(self, T):
        """(value, index) pairs per token of the fused lm_head: one per workgroup."""
        m = self.m
        return int(self.sv.LIB.w4a8_linear_argmax_workspace(T, m["vocab"], m["hidden"])) // (8 * T)

    def step_bytes(self, T, m_acc):
        m = self.m
        b = 0
        for _, N, K in layer_linears(m):
            b += m["layers"] * (linear_bytes(T, N, K) + quant_bytes(T, K))
        b += argmax_linear_bytes(T, m["vocab"], m["hidden"], self.lm_chunks(T)) + quant_bytes(T, m["hidden"])
        b += 8 * T * self.lm_chunks(T)                                  # acceptance reads the argmax pairs
        b += 2 * 2 * m_acc * m["layers"] * m["kv_heads"] * m["head_dim"] * 2  # K and V rows read + written
        return b

    def weight_bytes_total(self):
        m = self.m
        return m["layers"] * sum(weight_bytes(N, K) for _, N, K in layer_linears(m)) + \
            weight_bytes(m["vocab"], m["hidden"])


def run_T(model, T, steps, warmup, torch):
    """Graph-captured steps at T nodes: returns ms per step, accepted m,
    and whether graph replays reproduce the eager outputs bit for bit."""
    copies = len(model.copies)
    model.prepare_acts(T)
    model.set_tree(T)
    model.reset_ctrl(T)
    model.step(T)                      # eager step: find the predictions, then plant drafts
    torch.cuda.synchronize()
    model.set_tree(T, token_plant=model.argmax[:T].cpu().numpy())
    model.reset_ctrl(T)
    model.step(T)
    torch.cuda.synchronize()
    def snapshot():   # every output the replays must reproduce bit for bit
        return torch.cat([model.argmax[:T].view(torch.float32)] +
                         [model.y[nm][: T * N] for nm, N, _ in layer_linears(model.m)])
    eager_out = snapshot().clone()
    m_acc = int(model.ctrl[4].item())

    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(copies):
            model.step(T, copy=c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            model.step(T, copy=c)
        graphs.append(g)
    model.reset_ctrl(T)
    for i in range(warmup):
        graphs[i % copies].replay()
    # the eager outputs are those of copy 0 (copies differ in layer order)
    graphs[0].replay()
    torch.cuda.synchronize()
    replay_ok = snapshot().view(torch.int32).equal(eager_out.view(torch.int32))
    model.reset_ctrl(T)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % copies].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # five more timed runs of the same K replays, for the median of 5
    runs = []
    for _ in range(5):
        model.reset_ctrl(T)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            graphs[i % copies].replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / steps)
    graphs[0].replay()
    torch.cuda.synchronize()
    replay_ok = replay_ok and snapshot().view(torch.int32).equal(eager_out.view(torch.int32))
    del graphs
    return ms, m_acc, replay_ok, float(np.median(runs))


def prefill_bench(model, T, steps, torch, reps=3):
    """The prefill bucket on the same weights: graph replays of
    prefill_step at T tokens (µs, GB/s of its algorithmic bytes), and the
    mean per-launch time of each shape from kernel-attached events in eager
    steps."""
    model.prefill_step(T)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        model.prefill_step(T)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del g
    durs, names = [], []
    for r in range(reps):
        ev = []
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(200_000_000)
        model.prefill_step(T, events=ev)
        torch.cuda.synchronize()
        for a, b, nb, nm in ev:
            durs.append(a.elapsed_time(b) * 1e3)
            names.append(nm)
    by_shape = {}
    for nm in dict.fromkeys(names):
        v = [d for d, n in zip(durs, names) if n == nm]
        by_shape[nm] = round(float(np.mean(v)), 2)
    nb = model.prefill_bytes(T)
    out = {"workload": f"the same {model.m['layers']}-layer set at T={T} tokens (the dense 32-token bucket; down, "
                       f"K = 14336, streams its activation operands through LDS): quantisation + 128 layer "
                       f"linears + lm_head writing logits, HIP-graph replay",
           "T": T, "us": round(us, 2), "GB/s": round(nb / us / 1e3, 1),
           "pct_hbm_peak": round(100 * nb / us / 1e3 / HBM_PEAK_GBS, 2), "bytes": nb, "by_shape_us": by_shape}
    print(f"[bench] prefill: {out}", file=sys.stderr, flush=True)
    return out


def roofline_linear(model, T, reps, torch):
    """Live per-launch timing of the W4A8 linear kernel: each launch of an
    eager step records a pair of HIP events at its kernel's begin and end
    (hipExtLaunchKernel on the stream the kernel runs on). A spin kernel
    first holds the GPU so the host has enqueued every launch before they
    execute back to back."""
    durs, byts, names = [], [], []
    model.reset_ctrl(T)
    for r in range(reps):
        ev = []
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(200_000_000)
        model.step(T, copy=r % len(model.copies), events=ev)
        torch.cuda.synchronize()
        for a, b, nb, nm in ev:
            durs.append(a.elapsed_time(b) * 1e-3)
            byts.append(nb)
            names.append(nm)
    durs, byts = np.array(durs), np.array(byts, dtype=np.float64)
    by_shape = {}
    for nm in dict.fromkeys(names):
        sel = np.array([n == nm for n in names])
        us = float(durs[sel].mean() * 1e6)
        by_shape[nm] = {"us": round(us, 2), "GB/s": round(float(byts[sel].mean()) / us / 1e3, 1)}
    avg_s, avg_b = float(durs.mean()), float(byts.mean())
    return avg_b / avg_s / 1e9, avg_s, avg_b, len(durs) // reps, by_shape


def ceilings(model, T, torch, sv):
    """Rates of plain streaming reads (specv_stream_read: no arithmetic) on
    the same device, as ceilings for the step: one read of all the step's
    weight bytes; an empty launch per graph node; and a dependent chain of
    129 reads, one per linear launch of the step, of the same byte counts
    from distinct regions (cold), in graph replays; and per linear shape, a
    chain of that shape's reads alone (its 32 layer regions, or the lm_head
    region), in us per launch beside the shape's weight bytes."""
    m = model.m
    sizes = []
    for _ in range(m["layers"]):
        sizes += [weight_bytes(N, K) for _, N, K in layer_linears(m)]
    sizes.append(weight_bytes(m["vocab"], m["hidden"]))
    offs, tot = [], 0
    for b in sizes:
        offs.append(tot)
        tot += (b + 4095) // 4096 * 4096
    buf = torch.ones(tot // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    base, sp = buf.data_ptr(), sink.data_ptr()

    def graph_chain(fn, n):   # fn takes the capture stream's handle
        return graph_us(torch, lambda: fn(torch.cuda.current_stream().cuda_stream), n)

    def read(ptr, nb, grid, st):
        sv.check("specv_stream_read", sv.LIB.specv_stream_read(ptr, nb, sp, grid, st))

    empty = graph_chain(lambda st: [read(base, 0, 512, st) for _ in range(200)], 200)
    whole = min(graph_chain(lambda st: read(base, tot, g, st), 1) for g in (512, 1024, 2048))
    chain = graph_chain(lambda st: [read(base + o, b, 512, st) for o, b in zip(offs, sizes)], 1)
    names = [nm for nm, _, _ in layer_linears(m)]
    per_shape = {}
    for si, nm in enumerate(names + ["lm_head"]):
        idx = list(range(si, len(sizes) - 1, len(names))) if nm != "lm_head" else [len(sizes) - 1]
        us = graph_chain(lambda st: [read(base + offs[i], sizes[i], 512, st) for i in idx], len(idx))
        per_shape[nm] = {"us": round(us, 2), "weight_bytes": sizes[idx[0]],
                         "GB/s": round(sizes[idx[0]] / us / 1e3, 1)}
    del buf
    return {"read_all_weights_GBs": round(tot / whole / 1e3, 1), "empty_launch_us": round(empty, 3),
            "read_chain_us": round(chain, 2), "read_chain_GBs": round(sum(sizes) / chain / 1e3, 1),
            "read_per_shape": per_shape,
            "note": "plain streaming reads with no arithmetic (specv_stream_read), graph replays, cold: one read "
                    "of the step's weight bytes; an empty launch; a dependent chain of 129 reads with the byte "
                    "counts of the step's linear launches; per shape, a chain of that shape's reads (us per launch)"}


def cpu_baseline(model, T, dec=None, seconds=(6.0, 6.0)):
    """The oracle, as it stands, on bounded samples of the same workloads, on
    this host:
    - the 8B linear set (`value`): quantize + W4A8 linear over the generated
      layer sets (qkv, o, gate_up, down) at T tokens, one linear after
      another, first on one host thread for at least seconds[0], then with
      each linear's output rows split over every host thread this process
      may use (the C oracle releases the interpreter lock; rows are
      independent, so results are identical) for at least seconds[1];
    - the single 896x896 linear at T = 1 (quantize + linear, one thread);
    - the 0.5B linear set at T: its seven matrices and the lm_head, once, on
      every thread;
    - the 0.5B decoder (`dec`: model arrays, configuration, cache, L0): one
      8-node tree step and the 8 sequential single-token steps of a chain,
      each on one thread (the oracle's forward is not threaded)."""
    import oracle
    sg = model.sg
    lins = [(s, nm, N, K) for s in model.host_sets for nm, N, K in layer_linears(model.m)]
    threads = host_threads()

    def run(nthreads, min_s):
        t0 = time.perf_counter()
        nbytes, n = 0, 0
        while n == 0 or time.perf_counter() - t0 < min_s:
            lay, nm, N, K = lins[n % len(lins)]
            x = sg.normal_f32(sg.stream_key(5, 3 + K), T * K).reshape(T, K)
            xq, xs = oracle.quantize_act(x)
            if nthreads == 1:
                oracle.w4a8_linear(lay[nm][0], lay[nm][1], xq, xs)
            else:
                oracle.w4a8_linear_threads(lay[nm][0], lay[nm][1], xq, xs, nthreads)
            nbytes += linear_bytes(T, N, K) + quant_bytes(T, K)
            n += 1
        return nbytes, n, time.perf_counter() - t0

    b1, n1, t1 = run(1, seconds[0])
    bt, nt, tt = run(threads, seconds[1])
    out = {"value": round(bt / tt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "single_thread_value": round(b1 / t1 / 1e9, 4), "cpu_model": cpu_model(),
           "sample": f"quantize + W4A8 linear over the {model.m['hidden']}-hidden layer sets (qkv, o, gate_up, "
                     f"down) at T={T}, one linear after another: {n1} linears ({b1/1e6:.1f} MB algorithmic) in "
                     f"{t1:.2f} s on one thread, then {nt} linears ({bt/1e6:.1f} MB) in {tt:.2f} s with output "
                     f"rows split over {threads} threads, on {platform.machine()} ({os.cpu_count()} host cpus "
                     f"visible, {threads} usable)"}

    # the single-linear configuration: 896 x 896 at T = 1
    wq, ws, x = sg.linear_case(0, 1, 896, 896)
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        xq, xs = oracle.quantize_act(x)
        oracle.w4a8_linear(wq, ws, xq, xs)
        ts.append(time.perf_counter() - t0)
    out["config1_us"] = round(float(np.median(ts)) * 1e6, 1)

    # the 0.5B linear set at T, every matrix once, on every thread
    m5 = MODELS["qwen2.5-0.5b"]
    shapes = layer_linears(m5) + [("lm_head", m5["vocab"], m5["hidden"])]
    gen = [(sg.linear_case(0, T, N, K, layer=i), N, K) for i, (nm, N, K) in enumerate(shapes)]
    nb = sum(linear_bytes(T, N, K) + quant_bytes(T, K) for _, N, K in gen)
    t0 = time.perf_counter()
    for (wq, ws, x), N, K in gen:
        xq, xs = oracle.quantize_act(x)
        oracle.w4a8_linear_threads(wq, ws, xq, xs, threads)
    dt = time.perf_counter() - t0
    out["small_set"] = {"us": round(dt * 1e6, 1), "GB/s": round(nb / dt / 1e9, 4), "threads": threads,
                        "sample": f"quantize + W4A8 linear of the 0.5B set (qkv, o, gate_up, down, lm_head) at "
                                  f"T={T}, each matrix once"}
    del gen

    if dec is not None:
        arrays, cfg, kc, vc, L0 = dec
        c, sn = oracle.rope_table(cfg["max_pos"], cfg["head_dim"], 1e6)
        om = oracle.Model(dict(arrays, rope_cos=c, rope_sin=sn), cfg)
        parent, token = decoder_tree(sg, cfg, 8)
        t0 = time.perf_counter()
        r = oracle.tree_step(om, kc.copy(), vc.copy(), L0, parent, token)
        t_tree = time.perf_counter() - t0
        ks, vs = kc.copy(), vc.copy()
        t0 = time.perf_counter()
        for d in range(8):
            oracle.forward(om, ks, vs, L0 + d, np.array([-1], np.int32), np.array([token[min(d, 7)]], np.int32))
        t_seq = time.perf_counter() - t0
        out["config3"] = {"tree8_s": round(t_tree, 3), "sequential8_s": round(t_seq, 3), "threads": 1,
                          "accepted": int(r["m"]),
                          "sample": f"24-layer qwen2.5-0.5b-shaped decoder at L={L0}: one 8-node tree step "
                                    "(forward, argmax, acceptance, compaction), then 8 single-token forwards of "
                                    "a chain"}
    return out


def config1_bench(torch, sv, sg, reps=200):
    """One W4A8 linear, K = N = 896, T = 1, seed 0 (the single-linear
    configuration). Its 451,584 weight bytes stay in the L2 cache, so this is
    a latency: us per launch in a graph of `reps` launches, the kernel's own
    duration from kernel-attached events (median of 20 back-to-back
    launches), and quantisation + linear as a pair per graph node pair."""
    T, N, K = 1, 896, 896
    wq, ws, x = sg.linear_case(0, T, N, K)
    dev = torch.device("cuda")
    w = sv.pack_weights(torch.from_numpy(wq).to(dev), torch.from_numpy(ws.view(np.int16)).to(dev))
    xd = torch.from_numpy(x).to(dev)
    xq, xs = sv.quantize_act(xd)
    y = torch.empty((T, N), dtype=torch.float32, device=dev)
    lin_us = graph_us(torch, lambda: [sv.linear(w, xq, xs, y) for _ in range(reps)], reps)
    pair_us = graph_us(torch, lambda: [(sv.quantize_act(xd, xq, xs), sv.linear(w, xq, xs, y))
                                       for _ in range(reps)], reps)
    # kernel-attached events on 21 launches enqueued behind a spin kernel, so
    # they run back to back (as in a step), not each after an idle gap
    evs = []
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)
    for _ in range(21):
        e0, e1 = timing_events(torch)
        sv.check("specv_time_next_linear", sv.LIB.specv_time_next_linear(e0.cuda_event, e1.cuda_event))
        sv.linear(w, xq, xs, y)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    kern = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs[1:]]))
    wb = weight_bytes(N, K)
    return {"workload": "W4A8 linear 896x896, T=1, int4 g32 fp16 scales U(0.005,0.02), N(0,1) activations, "
                        "seed 0 (L2-resident: a latency)",
            "us_per_launch": round(lin_us, 3), "kernel_us": round(kern, 3),
            "quant_plus_linear_us": round(pair_us, 3), "weight_bytes": wb,
            "kernel_GBs": round(wb / kern / 1e3, 1)}


def decoder_tree(sg, cfg, N):
    """The configuration's tree: random topological parents and random draft
    tokens in [0, V), seed 0."""
    parent = sg.random_tree_parents(sg.stream_key(0, sg.TID_PARENT), N)
    token = sg.tokens(sg.stream_key(0, sg.TID_TOKEN), N, cfg["vocab"])
    return parent, token


def decoder_bench(torch, sv, sg, dm, cfg, L0, reps=20):
    """Full tree verification on the 24-layer Qwen2.5-0.5B shape over a
    1024-row fp16 KV cache: one 8-node step (tree-masked forward, the
    lm_head reduced to each node's argmax in its epilogue, acceptance,
    compaction), and a single-token step (a root-only tree) for comparison.
    Graph replays of (control-block reset + step): every replay verifies the
    same tree from the same committed state."""
    out = {}
    for N in (8, 1):
        parent, token = decoder_tree(sg, cfg, N)
        p = torch.from_numpy(parent).cuda()
        t = torch.from_numpy(token).cuda()
        c0 = sv.new_ctrl(L0, N, dm.c.kv_capacity - 16, root_token=int(token[0]))
        ctrl = c0.clone()
        stats = torch.zeros(3, dtype=torch.int32, device="cuda")

        def step():
            torch.mul(c0, 1, out=ctrl)      # reset by a kernel, not a memset or copy node
            dm.tree_step(ctrl, p, t, N, stats=stats, want_logits=False)
        us = graph_us(torch, lambda: [step() for _ in range(reps)], reps)
        out[str(N)] = {"us": round(us, 2), "accepted": int(ctrl[4].item())}
        print(f"[bench] decoder step N={N}: {out[str(N)]}", file=sys.stderr, flush=True)
    return {"workload": f"qwen2.5-0.5b-shaped 24-layer decoder, tree verification at L={L0} (fp16 KV), random "
                        "topological tree with random drafts, seed 0: forward + fused argmax + acceptance + "
                        "KV compaction, HIP-graph replay",
            "tree8_us": out["8"]["us"], "single_token_us": out["1"]["us"],
            "tree8_over_single": round(out["8"]["us"] / out["1"]["us"], 4), "by_N": out}


def window_bench(torch, sv, sg, dm, widths, L0, W=16, max_windows=400):
    """Device-resident windows on the Qwen2.5-0.5B shape: W-step windows of
    draft -> tree verify -> accept -> compact, each ending in a pinned
    readback of the control block and W statistics records. The context
    starts from 1024 committed rows and grows until the device sets done at
    4096. The drafter copies the width-1 greedy stream with per-node
    acceptance 0.6. Each window is timed with events on the stream; only
    windows whose W steps all ran (none after done) are counted."""
    cfg = sg.QWEN05
    ctx, root = 4096, 9
    stats = torch.zeros((W, 3), dtype=torch.int32, device="cuda")
    ring = torch.zeros(8192, dtype=torch.int32, device="cuda")
    rb = torch.zeros(32 + 12 * W, dtype=torch.uint8, pin_memory=True)
    draws = torch.from_numpy(sg.draft_draws(5, 256).view(np.int32)).cuda()
    ref = torch.zeros(ctx + 64, dtype=torch.int32, device="cuda")
    out = {}
    for width in [1] + [w for w in widths if w != 1]:
        ctrl = sv.new_ctrl(L0, width, ctx, root_token=root)
        kw = {} if width == 1 else dict(reference=ref, draws=draws, threshold=int(0.6 * 2 ** 32))
        dm.window(ctrl, stats, width, W, ring=ring, readback=rb, **kw)       # capture + warm
        torch.cuda.synchronize()
        ctrl.copy_(sv.new_ctrl(L0, width, ctx, root_token=root))
        ring.zero_()
        t_us, steps, tokens = 0.0, 0, 0
        for _ in range(max_windows):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dm.window(ctrl, stats, width, W, ring=ring, readback=rb, **kw)
            e1.record()
            e1.synchronize()
            st = rb[32:].numpy().view(np.int32).reshape(W, 3)
            if (st[:, 0] < 0).any():
                break
            t_us += e0.elapsed_time(e1) * 1e3
            steps += W
            tokens += int(st[:, 0].sum()) + W
        if width == 1:   # the greedy stream drives the drafter at every other width
            n = int(rb[:4].numpy().view(np.int32)[0]) - L0
            ref[L0] = root
            ref[L0 + 1:L0 + 1 + n] = ring[:n]
        out[str(width)] = {"us_per_step": round(t_us / max(steps, 1), 2),
                           "tokens_per_step": round(tokens / max(steps, 1), 3),
                           "tokens_per_s": round(tokens / (t_us * 1e-6), 1) if t_us else None,
                           "windows": steps // W}
        print(f"[bench] window width={width}: {out[str(width)]}", file=sys.stderr, flush=True)
    t1 = out["1"]["us_per_step"]
    for v in out.values():
        v["step_cost_vs_width1"] = round(v["us_per_step"] / t1, 3)
    cm = cm_window_bench(torch, sv, dm, ref, widths, L0, ctx, root, cfg["vocab"], W, max_windows)
    return {"workload": f"qwen2.5-0.5b-shaped decoder, {W}-step windows from 1024 to 4096 context, "
                        f"synthetic drafter at acceptance 0.6, pinned readback of {32 + 12 * W} B per window",
            "W": W, "by_width": out, "context_mixing": cm}


def cm_window_bench(torch, sv, dm, ref, widths, L0, ctx, root, vocab, W, max_windows, echo=512):
    """Windows drafted by the context-mixing drafter from the token history
    in the ring, on a synthetic history: 1024 committed tokens of a seeded
    random page in which the root and the next `echo` tokens of the greedy
    reply appear once, as a passage the reply repeats; after the passage the
    history no longer predicts the reply. Fixed widths first, then the width
    controller (its load-time costs are the fixed-width step costs, its window
    size calibrated at load from windows of 1, 2 and 4 steps), two windows in
    flight."""
    from speculative_verification_amd.controller import (WidthController, WindowBuffers, calibrate_window,
                                                         run_controlled)
    page = np.random.default_rng(5).integers(0, vocab, size=L0).astype(np.int32)
    page[199] = root
    page[200:200 + echo] = ref[L0 + 1:L0 + 1 + echo].cpu().numpy()
    hist = torch.from_numpy(np.concatenate([page, [root]]).astype(np.int32)).cuda()
    ring = torch.zeros(8192, dtype=torch.int32, device="cuda")
    stats = torch.zeros((W, 3), dtype=torch.int32, device="cuda")
    rb = torch.zeros(32 + 12 * W, dtype=torch.uint8, pin_memory=True)

    def reset(c=None):
        ring.zero_()
        ring[:L0 + 1] = hist
        v = sv.new_ctrl(L0, 1, ctx, root_token=root)
        v[7] = L0 + 1   # ring_head: the ring holds the whole stream
        if c is None:
            return v
        c.copy_(v)
        return c

    out = {}
    for width in [1] + [w for w in widths if w != 1]:
        ctrl = reset()
        dm.window_cm(ctrl, stats, width, W, ring, readback=rb)      # capture + warm
        torch.cuda.synchronize()
        ctrl = reset()
        t_us, steps, tokens = 0.0, 0, 0
        for _ in range(max_windows):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dm.window_cm(ctrl, stats, width, W, ring, readback=rb)
            e1.record()
            e1.synchronize()
            st = rb[32:].numpy().view(np.int32).reshape(W, 3)
            if (st[:, 0] < 0).any():
                break
            t_us += e0.elapsed_time(e1) * 1e3
            steps += W
            tokens += int(st[:, 0].sum()) + W
        out[str(width)] = {"us_per_step": round(t_us / max(steps, 1), 2),
                           "tokens_per_step": round(tokens / max(steps, 1), 3),
                           "tokens_per_s": round(tokens / (t_us * 1e-6), 1) if t_us else None,
                           "windows": steps // W}
        print(f"[bench] cm window width={width}: {out[str(width)]}", file=sys.stderr, flush=True)
    costs = {int(w): v["us_per_step"] for w, v in out.items()}
    # window size at load: short decodes with windows of 1, 2 and 4 steps
    bufs = WindowBuffers(4, ring.device)
    W_cal, us_by_W = calibrate_window(dm, reset, lambda: WidthController(costs), ring, sizes=(1, 2, 4),
                                      steps=16, bufs=bufs)
    print(f"[bench] cm window size {W_cal}: us per token {us_by_W}", file=sys.stderr, flush=True)
    ctl = WidthController(costs)
    first = ctl.width
    ctrl = reset()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    log = run_controlled(dm, ctrl, ring, ctl, W_cal, 10 ** 6, bufs=bufs)
    e1.record()
    torch.cuda.synchronize()
    tokens = int(ctrl[0].item()) - L0
    us = e0.elapsed_time(e1) * 1e3
    hist_w = {}
    for w, _, _ in log:
        hist_w[str(w)] = hist_w.get(str(w), 0) + 1
    ctl_out = {"first_width": first, "window_size": W_cal,
               "window_size_us_per_token": {str(k): round(v, 2) for k, v in us_by_W.items()},
               "windows_by_width": hist_w, "tokens": tokens,
               "tokens_per_s": round(tokens / (us * 1e-6), 1),
               "note": "window size chosen at load (smallest of 1, 2, 4 steps within 10 % of the fastest time "
                       "per token on a 16-step decode); wall time from the first enqueue to the last "
                       "completion, host decisions included"}
    print(f"[bench] cm controller: {ctl_out}", file=sys.stderr, flush=True)
    return {"workload": f"context-mixing drafter on a 1024-token synthetic page echoing {echo} tokens of the "
                        f"reply; {W}-step windows to the 4096 context",
            "by_width": out, "controller": ctl_out}


def linear_set(name, Ts, steps, warmup, reps, torch, sv, sg):
    """The same verify step on another shape set (the 0.5B linear set): the
    T sweep and the linear kernel's live per-launch roofline at the largest T,
    in a compact form for the JSON line."""
    model = Model(name, torch, sv, sg, max(Ts))
    per_T = {}
    for T in Ts:
        ms, m_acc, ok, med5 = run_T(model, T, steps, warmup, torch)
        nb = model.step_bytes(T, m_acc)
        per_T[str(T)] = {"us": round(ms * 1e3, 2), "us_median5": round(med5 * 1e3, 2),
                         "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                         "graph_replay_exact": ok}
        print(f"[bench] {name} T={T}: {per_T[str(T)]}", file=sys.stderr, flush=True)
    Tr = max(Ts)
    ach, avg_s, _, nlaunch, by_shape = roofline_linear(model, Tr, reps, torch)
    m = MODELS[name]
    out = {"workload": (f"{name}-shaped verify step: {m['layers']} x (qkv, o, gate_up, down) + lm_head W4A8 g32 "
                        f"with fused argmax, tree accept + KV compaction, HIP-graph replay; "
                        f"{len(model.copies)} copies of the weights in rotation (cold)"),
           "weight_bytes": model.weight_bytes_total(), "per_T": per_T,
           "t8_over_t1": round(per_T["8"]["us"] / per_T["1"]["us"], 4) if "8" in per_T and "1" in per_T else None,
           "linear_roofline": {"T": Tr, "achieved": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4),
                               "avg_launch_us": round(avg_s * 1e6, 3), "launches_per_step": nlaunch,
                               "by_shape": by_shape}}
    del model
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=8)
    ap.add_argument("--workload", choices=sorted(MODELS), default="llama3-8b")
    ap.add_argument("--sweep", default="1,2,4,8", help="T values timed besides --T")
    ap.add_argument("--roofline-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window-widths", default="1,2,4,8,16",
                    help="tree widths of the speculation-window measurement (empty: skip)")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false",
                    help="skip the plain streaming-read ceilings")
    ap.add_argument("--small-set", default="qwen2.5-0.5b",
                    help="second shape set whose verify step is timed at T = 1, 2, 4, 8 (empty: skip)")
    ap.add_argument("--prefill-T", type=int, default=32,
                    help="token count of the prefill-bucket measurement on the same weights (0: skip)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.prefill_T > 32:
        ap.error("--prefill-T takes at most 32 tokens (the largest bucket)")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the verification step of one request runs on one device).", file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_verification_amd as sv
    import synthgen as sg
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    Ts = sorted({args.T, *[int(t) for t in args.sweep.split(",") if t]})
    model = Model(args.workload, torch, sv, sg, max(Ts + [args.prefill_T]))
    print(f"[bench] {args.workload}: weights {model.weight_bytes_total()/1e9:.3f} GB x {len(model.copies)} "
          f"copies, generated in {model.gen_s:.1f} s", file=sys.stderr, flush=True)

    per_T = {}
    for T in Ts:
        ms, m_acc, ok, med5 = run_T(model, T, args.steps if T == args.T else max(5, args.steps // 2),
                                    args.warmup, torch)
        nb = model.step_bytes(T, m_acc)
        per_T[T] = {"ms": ms, "GB/s": nb / (ms * 1e-3) / 1e9, "accepted": m_acc, "graph_replay_exact": ok,
                    "bytes": nb, "ms_median5": med5}
        print(f"[bench] T={T}: {ms*1e3:.1f} us/step, {per_T[T]['GB/s']:.0f} GB/s, m={m_acc}, "
              f"replay exact={ok}", file=sys.stderr, flush=True)

    ach, avg_s, avg_b, nlaunch, by_shape = roofline_linear(model, args.T, args.roofline_reps, torch)
    prefill = prefill_bench(model, args.prefill_T, max(5, args.steps // 2), torch) if args.prefill_T > 16 else None
    small = None
    if args.small_set and args.small_set != args.workload:
        small = linear_set(args.small_set, [1, 2, 4, 8], max(5, args.steps // 2), args.warmup,
                           args.roofline_reps, torch, sv, sg)
    ceil = ceilings(model, args.T, torch, sv) if args.ceilings else None
    if ceil:
        ceil["step_pct_of_read_all"] = round(100 * per_T[args.T]["GB/s"] / ceil["read_all_weights_GBs"], 1)
        ceil["step_over_read_chain"] = round(per_T[args.T]["ms"] * 1e3 / ceil["read_chain_us"], 3)
        print(f"[bench] ceilings: {ceil}", file=sys.stderr, flush=True)
    config1 = config1_bench(torch, sv, sg)
    print(f"[bench] config1: {config1}", file=sys.stderr, flush=True)
    # the 24-layer 0.5B decoder: the tree verification step, then the windows
    cfg5 = sg.QWEN05
    L0, cap5 = 1024, 4096 + 32
    arrays5 = sg.model_case(3, cfg5)
    kc5, vc5 = sg.kv_prefix(41, cfg5, L0, cap5)
    dm5 = sv.DeviceModel(arrays5, cfg5, cap5, kc5, vc5)
    decoder = decoder_bench(torch, sv, sg, dm5, cfg5, L0)
    widths = [int(w) for w in args.window_widths.split(",") if w]
    window = window_bench(torch, sv, sg, dm5, widths, L0) if widths else None
    del dm5
    torch.cuda.empty_cache()
    prof = linear_profile(args.T, args.workload)
    main_T = per_T[args.T]
    out = {
        "metric": METRIC,
        "value": round(main_T["GB/s"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_T["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8->int32,fp32",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.workload}-shaped verify step: {MODELS[args.workload]['layers']} x (qkv, o, "
                         f"gate_up, down) + lm_head W4A8 g32 with fused argmax, tree accept + KV compaction, "
                         f"T={args.T} tree nodes, HIP-graph replay"),
            "T": args.T,
            "weight_bytes": model.weight_bytes_total(),
            "step_bytes": main_T["bytes"],
        },
        "pct_hbm_peak": round(100 * main_T["GB/s"] / HBM_PEAK_GBS, 2),
        "us_per_verify": round(main_T["ms"] * 1e3, 2),
        "t8_over_t1": round(per_T[8]["ms"] / per_T[1]["ms"], 4) if 8 in per_T and 1 in per_T else None,
        "per_T": {str(T): {"us": round(v["ms"] * 1e3, 2), "us_median5": round(v["ms_median5"] * 1e3, 2),
                           "GB/s": round(v["GB/s"], 1),
                           "pct_hbm_peak": round(100 * v["GB/s"] / HBM_PEAK_GBS, 2),
                           "accepted": v["accepted"], "graph_replay_exact": v["graph_replay_exact"]}
                  for T, v in per_T.items()},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4),
                     "frac_basis": "live: kernel-attached HIP events (hipExtLaunchKernel begin/end on the launch's "
                                   "stream) around every linear launch of one eager step, mean over the launches",
                     "traffic": prof["bytes_per_launch"] if prof else None,
                     "frac_rocprof": (round(avg_b / (prof["rocprof_mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if prof else None),
                     "profile_source": (f"stored, not of this run: rocprofv3 kernel traces (mean "
                                        f"{prof['rocprof_mean_us']} us per launch over two runs of this command on "
                                        f"two devices) and FETCH_SIZE + WRITE_SIZE "
                                        f"counter passes of this command on linear.hip sha256 "
                                        f"{prof['source_sha256'][:16]}, {prof['summary']}") if prof else
                                       "none: linear.hip changed since the stored rocprofv3 figures were taken",
                     "kernel": f"w4a8_linear_stream_kernel<{args.T},P,*,false,false> (P = 7 for down, 4 otherwise; "
                               f"the lm_head runs the argmax specialisation)",
                     "lm_head_chunks": model.lm_chunks(args.T),
                     "avg_launch_us": round(avg_s * 1e6, 3),
                     "avg_launch_bytes": round(avg_b), "launches_per_step": nlaunch,
                     "by_shape": by_shape},
        "ceilings": ceil,
        "prefill": prefill,
        "small_set": small,
        "config1": config1,
        "decoder": decoder,
        "window": window,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(model, args.T,
                                                                        dec=(arrays5, cfg5, kc5, vc5, L0)),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""The width controller driving context-mixing windows on the device, two
windows in flight (GPU-Resident Speculative Decoding for In-Browser LLM
Inference with WebGPU, Feedback Control of Speculation Width). Whatever
widths it picks, tree verification is exact, so the emitted stream must equal
the oracle's greedy stream; the load-time cost measurement must give a
positive cost per width, and windows of the size calibrated at load time
must emit the same greedy stream."""
import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

pytestmark = pytest.mark.gpu
L0, CAP, ROOT = 30, 400, 5


def case(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_verification_amd as m
    return m


def setup(sv, seed=11):
    cfg = sg.TINY
    arrays = sg.model_case(7, cfg)
    c, s = oracle.rope_table(cfg["max_pos"], cfg["head_dim"], 1e6)
    arrays = dict(arrays, rope_cos=c, rope_sin=s)
    om = oracle.Model(arrays, cfg)
    kc, vc = sg.kv_prefix(seed, cfg, L0, CAP)
    ctrl = dict(committed_len=L0, n_nodes=1, ctx_len=10 ** 6, done=0, accept_len=0, root_token=ROOT, step=0,
                ring_head=0)
    _, greedy = oracle.window(om, kc.copy(), vc.copy(), ctrl, 1, 200, np.zeros(1, np.int32),
                              np.zeros((1, 16), np.uint32), 0)
    rng = np.random.default_rng(17)
    hist = rng.integers(100, 200, size=L0).tolist()
    hist[6] = ROOT
    hist[7:L0] = greedy[:L0 - 7]          # the reply echoes an earlier passage
    return cfg, arrays, kc, vc, hist + [ROOT], greedy


def fresh(sv, cfg, arrays, kc, vc, hist, ctx_len):
    dm = sv.DeviceModel(arrays, cfg, CAP, kc, vc)
    ctrl = torch.tensor([L0, 1, ctx_len, 0, 0, ROOT, 0, L0 + 1], dtype=torch.int32, device="cuda")
    ring = torch.zeros(1024, dtype=torch.int32, device="cuda")
    ring[:L0 + 1] = torch.tensor(hist, dtype=torch.int32)
    return dm, ctrl, ring


def test_controlled_windows_emit_the_greedy_stream(sv):
    from speculative_verification_amd.controller import WidthController, run_controlled
    cfg, arrays, kc, vc, hist, greedy = setup(sv)
    dm, ctrl, ring = fresh(sv, cfg, arrays, kc, vc, hist, L0 + 150)
    ctl = WidthController({1: 1000.0, 2: 1020.0, 4: 1080.0, 8: 1150.0, 16: 1700.0})
    case(f"controlled windows, first width {ctl.width}")
    log = run_controlled(dm, ctrl, ring, ctl, 4, 40)
    torch.cuda.synchronize()
    c = ctrl.cpu().tolist()
    n_emit = c[0] - L0                      # committed rows beyond the prefix = emitted tokens
    assert n_emit > 0 and c[7] == c[0] + 1
    assert ring.cpu().numpy()[L0 + 1:L0 + 1 + n_emit].tolist() == greedy[:n_emit]
    steps = [r for _, st, _ in log for r in st.tolist() if r[0] >= 0]
    assert sum(m + 1 for m, _, _ in steps) == n_emit
    assert sum(m for m, _, _ in steps) > 0  # the echoed passage was accepted
    widths = {w for w, _, _ in log}
    assert widths <= set(ctl.widths)


def test_measure_costs(sv):
    from speculative_verification_amd.controller import measure_costs
    cfg, arrays, kc, vc, hist, _ = setup(sv)
    case("load-time step costs")

    def run_window(width, W):
        dm, ctrl, ring = fresh(sv, cfg, arrays, kc, vc, hist, CAP - 20)
        stats = torch.zeros((W, 3), dtype=torch.int32, device="cuda")
        dm.window_cm(ctrl, stats, width, W, ring)       # builds the graph
        dm, ctrl, ring = fresh(sv, cfg, arrays, kc, vc, hist, CAP - 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dm.window_cm(ctrl, stats, width, W, ring)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    costs = measure_costs(run_window, (1, 2, 4, 8, 16), W=4, reps=1)
    assert set(costs) == {1, 2, 4, 8, 16} and all(v > 0 for v in costs.values())


def test_calibrated_window_emits_the_greedy_stream(sv):
    """Load-time window size: short decodes from the same state with windows
    of 1, 2 and 4 steps; the chosen size is within 10 % of the fastest time
    per token, and a controlled decode at that size emits the oracle's
    greedy stream."""
    from speculative_verification_amd.controller import (WidthController, WindowBuffers, calibrate_window,
                                                         run_controlled)
    cfg, arrays, kc, vc, hist, greedy = setup(sv)
    dm, ctrl0, ring = fresh(sv, cfg, arrays, kc, vc, hist, L0 + 150)
    init = ctrl0.clone()
    hist_t = torch.tensor(hist, dtype=torch.int32, device="cuda")

    def reset(c=None):
        ring.zero_()
        ring[:L0 + 1] = hist_t
        if c is None:
            return init.clone()
        c.copy_(init)
        return c

    costs = {1: 1000.0, 2: 1020.0, 4: 1080.0, 8: 1150.0, 16: 1700.0}
    bufs = WindowBuffers(4, "cuda")
    W, us = calibrate_window(dm, reset, lambda: WidthController(costs), ring, steps=16, bufs=bufs)
    case(f"calibrated window size {W}: {us}")
    assert set(us) == {1, 2, 4} and all(v > 0 for v in us.values())
    assert W in us and us[W] <= 1.1 * min(us.values())
    assert all(us[w] > 1.1 * min(us.values()) for w in us if w < W)
    ctrl = reset()
    log = run_controlled(dm, ctrl, ring, WidthController(costs), W, 400, bufs=bufs)
    torch.cuda.synchronize()
    c = ctrl.cpu().tolist()
    n_emit = c[0] - L0
    assert n_emit > 0 and c[3] == 1         # ran to the context limit
    assert ring.cpu().numpy()[L0 + 1:L0 + 1 + n_emit].tolist() == greedy[:n_emit]
    assert all(len(st) == W for _, st, _ in log)

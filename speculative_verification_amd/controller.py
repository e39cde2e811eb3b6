"""Width and window controller of the speculation loop (GPU-Resident
Speculative Decoding for In-Browser LLM Inference with WebGPU, Feedback
Control of Speculation Width). Host policy between windows; every step of a
window runs on the device (spec_window_run_cm).

The policy, as this module implements it:

- Costs. T(N) is the device time of one step at tree width N, measured at
  load time for every candidate width and refined online: with two windows
  in flight, the interval between the completions of two consecutive
  windows is the cost of the later one, and it enters the cost of its width
  through an exponential moving average.
- Acceptance statistics. Each step reports its accepted draft count m and
  the drafter's best match length l. The controller keeps, per (l, width),
  an exponential moving average of m, and per l an acceptance rate: a chain
  of depth D = min(width - 1, 8) that accepted m < D drafts shows m accepted
  nodes and one rejection, one that accepted all D shows D accepted nodes
  and no rejection (it was cut by the depth, not rejected). The rate is
  (S + 2a) / (S + F + 2), with S and F the accepted and rejected counts,
  each decayed by (1 - ema) per window, and two pseudo-observations at the
  prior rate a = `prior_accept`.
- Decision. For the next window it estimates the expected tokens of each
  candidate width, 1 + the mean over the recent steps' match lengths of the
  estimated m at that (l, width), and takes the width with the most expected
  tokens per microsecond (ties go to the narrower width).
- Estimates. The moving average of m is used while it is fresh (updated in
  the last `stale` windows). Otherwise, and for a pair never observed, m is
  estimated as a chain whose nodes are accepted independently at l's rate:
  sum_{d=1}^{D} rate^d. With no observation at all the rate is the prior,
  and the first width is the best under it.
- Break-even. Speculating at width N beats plain decoding exactly when its
  expected tokens exceed T(N) / T(1); under the prior, when
  (1 - a^(D+1)) / (1 - a) > T(N) / T(1). The drafter and the fixed costs of
  a step are inside the measured T(N), because they run on the device as
  part of the step.
- Probing. After `spacing` consecutive windows of plain decoding the
  controller probes the best width under the prior for one window. The
  spacing spends at most `probe_budget` of the time on probes:
  ceil((T(Np) / T(1) - 1) / probe_budget) windows, so a device on which wide
  steps are expensive probes rarely.
- Window size. At load time a short decode is timed with windows of 1, 2
  and 4 steps; the smallest whose time per token is within 10 % of the
  fastest is kept.
"""
from __future__ import annotations

import math
from collections import deque

MAX_DEPTH = 8  # the drafter extends a candidate by at most 8 tokens


def prior_drafts(width: int, a: float) -> float:
    """Expected accepted drafts of a chain of depth min(width - 1, 8) whose
    nodes are accepted independently with probability a."""
    return sum(a ** d for d in range(1, min(width - 1, MAX_DEPTH) + 1))


def window_size(us_per_token: dict) -> int:
    """The smallest window (steps per submission) whose time per token is
    within 10 % of the fastest."""
    best = min(us_per_token.values())
    return min(w for w, t in us_per_token.items() if t <= 1.1 * best)


class WidthController:
    def __init__(self, costs_us: dict, ema: float = 0.25, probe_budget: float = 0.05, prior_accept: float = 0.5,
                 recent: int = 32, stale: int = 16):
        if 1 not in costs_us or any(c <= 0 for c in costs_us.values()):
            raise ValueError("costs must include width 1 and be positive")
        self.widths = sorted(costs_us)
        self.cost = {w: float(c) for w, c in costs_us.items()}
        self.ema, self.a = float(ema), float(prior_accept)
        self.acc: dict = {}        # (l, width) -> (EMA of m, window of its last update)
        self.succ = [0.0] * 9      # per l: decayed accepted-node and rejection counts
        self.fail = [0.0] * 9
        self.recent = deque(maxlen=recent)
        self.plain = 0
        self.windows = 0
        self.stale = stale
        wide = [w for w in self.widths if w > 1]
        self.probe = max(wide, key=lambda w: (self._prior_tokens(w) / self.cost[w], -w)) if wide else None
        self.spacing = (max(1, math.ceil((self.cost[self.probe] / self.cost[1] - 1.0) / probe_budget))
                        if self.probe else None)
        self.width = self._best(lambda w: self._prior_tokens(w))

    def _prior_tokens(self, width: int) -> float:
        return 1.0 + prior_drafts(width, self.a)

    def rate(self, l: int) -> float:
        return (self.succ[l] + 2.0 * self.a) / (self.succ[l] + self.fail[l] + 2.0)

    def _est(self, l: int, width: int) -> float:
        v = self.acc.get((l, width))
        if v is not None and self.windows - v[1] <= self.stale:
            return v[0]
        return prior_drafts(width, self.rate(l))

    def expected_tokens(self, width: int) -> float:
        if not self.recent:
            return self._prior_tokens(width)
        return 1.0 + sum(self._est(l, width) for l in self.recent) / len(self.recent)

    def _best(self, tokens) -> int:
        return max(self.widths, key=lambda w: (tokens(w) / self.cost[w], -w))

    def update(self, stats, width: int, window_us: float | None = None) -> None:
        """Fold one window's step records (m, best match, nodes), run at
        `width`, and, if given, the window's measured device time."""
        self.windows += 1
        self.succ = [v * (1.0 - self.ema) for v in self.succ]
        self.fail = [v * (1.0 - self.ema) for v in self.fail]
        depth = min(width - 1, MAX_DEPTH)
        ran = 0
        for m, l, _ in stats:
            if m < 0:
                continue  # a step after done did nothing
            ran += 1
            l = int(l)
            key = (l, width)
            old = self.acc.get(key)
            self.acc[key] = (float(m) if old is None else old[0] + self.ema * (m - old[0]), self.windows)
            if depth > 0:
                self.succ[l] += m
                self.fail[l] += 1.0 if m < depth else 0.0
            self.recent.append(l)
        if window_us is not None and ran == len(stats) and ran > 0:
            sample = window_us / ran
            self.cost[width] = self.cost[width] + self.ema * (sample - self.cost[width])

    def next(self) -> int:
        """The width of the next window to enqueue."""
        best = self._best(self.expected_tokens)
        if best == 1 and self.probe is not None:
            self.plain += 1
            if self.plain >= self.spacing:
                self.plain = 0
                best = self.probe
        else:
            self.plain = 0
        self.width = best
        return best


def measure_costs(run_window, widths, W: int = 8, reps: int = 2) -> dict:
    """Load-time step costs: `run_window(width, W)` runs one window and
    returns its device time in microseconds; the best of `reps` windows."""
    return {w: min(run_window(w, W) for _ in range(reps)) / W for w in widths}


class WindowBuffers:
    """The readback and statistics buffers of two windows in flight, for
    windows of up to W_max steps. Reusing one set keeps the buffers, and so
    the cached window graphs, the same from one run to the next."""

    def __init__(self, W_max: int, device):
        import torch
        self.W_max = W_max
        self.rbs = [torch.zeros(32 + 12 * W_max, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.stats = [torch.zeros((W_max, 3), dtype=torch.int32, device=device) for _ in range(2)]


def run_controlled(dm, ctrl, ring, ctl: WidthController, W: int, max_windows: int, params=None,
                   bufs: WindowBuffers | None = None):
    """Context-mixing windows of W steps with the width chosen by `ctl`, two
    windows in flight: while window k+1 runs, the host reads window k's
    readback, folds its statistics and the interval between the two
    completions into the controller, and enqueues window k+2. Stops after
    the window in which the device set done. Returns, per window, (width,
    step records, device microseconds or None for the first)."""
    import numpy as np
    import torch

    bufs = bufs if bufs is not None else WindowBuffers(W, ring.device)
    if W > bufs.W_max:
        raise ValueError("window longer than its buffers")
    rbs, stats = bufs.rbs, bufs.stats
    events, widths, log = [], [], []

    def enqueue(k, width):
        dm.window_cm(ctrl, stats[k % 2], width, W, ring, params, readback=rbs[k % 2])
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        events.append(e)
        widths.append(width)

    enqueue(0, ctl.width)
    if max_windows > 1:
        enqueue(1, ctl.width)
    for k in range(max_windows):
        events[k].synchronize()
        rb = rbs[k % 2].numpy()[: 32 + 12 * W].copy()
        c = rb[:32].view(np.int32)
        st = rb[32:].view(np.int32).reshape(W, 3)
        us = events[k - 1].elapsed_time(events[k]) * 1e3 if k > 0 else None
        ctl.update(st.tolist(), widths[k], us)
        log.append((widths[k], st, us))
        if c[3]:  # done: the window already in flight is all no-ops
            if k + 1 < len(events):
                events[k + 1].synchronize()
            break
        if k + 2 < max_windows:
            enqueue(k + 2, ctl.next())
    return log


def calibrate_window(dm, reset, make_controller, ring, sizes=(1, 2, 4), steps: int = 16, params=None,
                     bufs: WindowBuffers | None = None):
    """The window size, chosen at load time: a short decode of `steps` steps
    from the same state is timed with windows of each size (two windows in
    flight, widths chosen by a fresh controller from make_controller()), and
    the smallest size whose time per emitted token is within 10 % of the
    fastest is kept (window_size). reset(ctrl=None) restores the decode
    state, ring included, into ctrl (a fresh control block when None) and
    returns it. Each size runs once untimed first, so graph captures stay
    out of the timing. Returns (size, {size: us per token})."""
    import torch

    bufs = bufs if bufs is not None else WindowBuffers(max(sizes), ring.device)
    ctrl = reset()
    us = {}
    for timed in (False, True):
        for W in sizes:
            reset(ctrl)
            L0 = int(ctrl[0].item())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run_controlled(dm, ctrl, ring, make_controller(), W, max(1, steps // W), params, bufs)
            e1.record()
            torch.cuda.synchronize()
            if timed:
                tokens = int(ctrl[0].item()) - L0
                us[W] = e0.elapsed_time(e1) * 1e3 / max(tokens, 1)
    return window_size(us), us

"""GPU context-mixing drafter (GPU-Resident Speculative Decoding for In-Browser
LLM Inference with WebGPU, Draft-Free Drafting From Web Context) against the
oracle: the tree of cm_draft on random and repetitive streams (one to several
thousand tokens, so the scan spans many workgroups and a ragged last one), and
the speculation window drafted by it (spec_window_run_cm) on the tiny decoder
and on a two-layer decoder with Qwen2.5-0.5B's attention geometry, compared
bit for bit with the oracle's window: control block, statistics, ring, and
both KV caches. All values are integers, so equality is exact."""
import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

pytestmark = pytest.mark.gpu
FIELDS = ("committed_len", "n_nodes", "ctx_len", "done", "accept_len", "root_token", "step", "ring_head")


def case(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_verification_amd as m
    return m


def stream_case(seed, n, vocab, periodic=False):
    rng = np.random.default_rng(seed)
    if periodic:
        per = rng.integers(0, vocab, size=int(rng.integers(3, 40)))
        s = np.resize(per, n)
        flips = rng.random(n) < 0.05   # an occasional deviation
        s[flips] = rng.integers(0, vocab, size=int(flips.sum()))
        return s.astype(np.int32)
    return rng.integers(0, vocab, size=n).astype(np.int32)


PARAMS = [(8, 16, 8, oracle.CM_WEIGHT), (3, 32, 5, [0, 5, 9, 2, 7, 1, 1, 1, 1]), (1, 1, 1, [0] + [1] * 8),
          (8, 7, 8, [0, 1, 1, 1, 1, 1, 1, 1, 1]), (5, 24, 3, [0, 3, 1, 4, 1, 5, 9, 2, 6])]


@pytest.mark.parametrize("n,vocab,periodic", [(1, 5, False), (2, 2, False), (40, 3, False), (255, 4, False),
                                              (256, 4, True), (257, 50, True), (1000, 6, False),
                                              (4097, 151936, True), (5000, 3, False), (9000, 30, True)])
def test_cm_draft_parity(sv, n, vocab, periodic):
    s = stream_case(n * 7 + vocab, n, vocab, periodic)
    st = torch.from_numpy(s).cuda()
    for pi, (mo, c, d, w) in enumerate(PARAMS):
        for width in (1, 2, 5, 8, 16):
            case(f"cm_draft n={n} vocab={vocab} periodic={periodic} params={pi} width={width}")
            p = sv.cm_params(mo, c, d, w)
            parent, token, out = sv.cm_draft(st, width, p)
            torch.cuda.synchronize()
            ep, et, en, ebm = oracle.cm_draft(s, width, mo, c, d, w)
            nn, bm = out.cpu().tolist()
            assert (nn, bm) == (en, ebm)
            assert parent.cpu().numpy()[:nn].tolist() == ep.tolist()
            assert token.cpu().numpy()[:nn].tolist() == et.tolist()


# ------------------------------------------------------------------ window, tiny decoder

L0, CAP, ROOT = 30, 400, 5


# Qwen2.5-0.5B's attention geometry (14 query heads over 2 KV heads, head
# dim 64, hidden 896) in two layers: the grouped attention with and without
# the head split, under the drafter's trees.
G7 = dict(n_layers=2, hidden=896, n_heads=14, n_kv_heads=2, head_dim=64, inter=1024, vocab=1000,
          eps=1e-6, max_pos=640)
_MODELS = {}


def model_cached(name="tiny"):
    if name not in _MODELS:
        cfg, seed = {"tiny": (sg.TINY, 7), "g7": (G7, 17)}[name]
        arrays = sg.model_case(seed, cfg)
        c, s = oracle.rope_table(cfg["max_pos"], cfg["head_dim"], 1e6)
        arrays = dict(arrays, rope_cos=c, rope_sin=s)
        _MODELS[name] = (cfg, arrays, oracle.Model(arrays, cfg))
    return _MODELS[name]


def tiny_cached():
    return model_cached("tiny")


def greedy_future(om, cfg, seed, n):
    """The oracle's greedy continuation after the root (width-1 steps)."""
    kc, vc = sg.kv_prefix(seed, cfg, L0, CAP)
    ctrl = dict(committed_len=L0, n_nodes=1, ctx_len=10 ** 6, done=0, accept_len=0, root_token=ROOT, step=0,
                ring_head=0)
    _, emit = oracle.window(om, kc, vc, ctrl, 1, n, np.zeros(1, np.int32), np.zeros((1, 16), np.uint32), 0)
    return emit


def history(kind, future):
    """Committed tokens of rows 0..L0-1, then the root. 'echo' places the root
    and the model's own greedy continuation earlier in the history, as a
    passage the reply repeats; 'random' has no such echo."""
    rng = np.random.default_rng(17)
    h = rng.integers(100, 200, size=L0).tolist()
    if kind == "echo":
        h[6] = ROOT
        h[7:L0] = future[:L0 - 7]
    return h + [ROOT]


def run_cm_pair(sv, width, windows, kind, ctx_len=CAP - 16, params=None, ring_cap=1024, model="tiny"):
    cfg, arrays, om = model_cached(model)
    seed = 11
    hist = history(kind, greedy_future(om, cfg, seed, 40))
    kc0, vc0 = sg.kv_prefix(seed, cfg, L0, CAP)
    kc, vc = kc0.copy(), vc0.copy()
    oc = dict(committed_len=L0, n_nodes=width, ctx_len=ctx_len, done=0, accept_len=0, root_token=ROOT, step=0,
              ring_head=L0 + 1)
    dm = sv.DeviceModel(arrays, cfg, CAP, kc0, vc0)
    ctrl = torch.tensor([oc[f] for f in FIELDS], dtype=torch.int32, device="cuda")
    stats = torch.full((64, 3), 7777, dtype=torch.int32, device="cuda")
    ring = torch.zeros(ring_cap, dtype=torch.int32, device="cuda")
    ring[:L0 + 1] = torch.tensor(hist, dtype=torch.int32)
    mo, c, d, w = params or (8, 16, 8, oracle.CM_WEIGHT)
    p = sv.cm_params(mo, c, d, w)
    o_hist = list(hist)
    all_stats = []
    for wi, W in enumerate(windows):
        o_stats, _ = oracle.window_cm(om, kc, vc, oc, width, W, o_hist, mo, c, d, w)
        rb = torch.zeros(32 + 12 * W, dtype=torch.uint8, pin_memory=True)
        dm.window_cm(ctrl, stats, width, W, ring, p, readback=rb)
        torch.cuda.synchronize()
        where = f"window {wi} width {width} {kind}"
        g_ctrl = ctrl.cpu().numpy()
        g_stats = stats.cpu().numpy()[:W]
        assert rb.numpy()[:32].tobytes() == g_ctrl.tobytes() and rb.numpy()[32:].tobytes() == g_stats.tobytes()
        assert [int(x) for x in g_ctrl] == [oc[f] for f in FIELDS], where
        assert [tuple(int(v) for v in r) for r in g_stats] == [tuple(s) for s in o_stats], where
        assert ring.cpu().numpy()[:len(o_hist)].tolist() == o_hist, where
        assert np.array_equal(dm.k_cache.cpu().numpy().view(np.uint16), kc), where
        assert np.array_equal(dm.v_cache.cpu().numpy().view(np.uint16), vc), where
        all_stats += o_stats
    return all_stats, o_hist


@pytest.mark.parametrize("width", [1, 2, 4, 8, 16])
def test_cm_window_echo(sv, width):
    case(f"cm window width={width}, history echoes the reply")
    stats, _ = run_cm_pair(sv, width, (16, 16), "echo")
    if width > 1:
        assert sum(m for m, _, _ in stats) > 0     # the echoed passage is accepted


@pytest.mark.parametrize("width", [4, 16])
def test_cm_window_random_history(sv, width):
    case(f"cm window width={width}, random history")
    run_cm_pair(sv, width, (16,), "random", params=(3, 32, 5, [0, 5, 9, 2, 7, 1, 1, 1, 1]))


@pytest.mark.parametrize("width", [2, 4, 8])
def test_cm_window_qwen_attention_geometry(sv, width):
    """The same windows on a decoder with Qwen2.5-0.5B's attention geometry:
    trees of 2 and 4 nodes split each KV group's heads over two workgroups,
    8-node trees do not."""
    case(f"cm window width={width}, 14 heads over 2 KV heads, hidden 896")
    stats, _ = run_cm_pair(sv, width, (16, 8), "echo", model="g7")
    assert sum(m for m, _, _ in stats) > 0


def test_cm_window_reaches_context_limit(sv):
    case("cm window width=8, context limit inside the window")
    stats, _ = run_cm_pair(sv, 8, (16, 8), "echo", ctx_len=L0 + 20)
    assert stats[-1][0] == -1


def test_cm_window_inconsistent_ring_drafts_root_only(sv):
    """A ring that does not hold the stream (ring_head != committed_len + 1):
    every step drafts the root alone, as documented."""
    case("cm window with an inconsistent ring")
    cfg, arrays, om = tiny_cached()
    kc0, vc0 = sg.kv_prefix(11, cfg, L0, CAP)
    dm = sv.DeviceModel(arrays, cfg, CAP, kc0, vc0)
    ctrl = torch.tensor([L0, 8, CAP - 16, 0, 0, ROOT, 0, 3], dtype=torch.int32, device="cuda")
    stats = torch.zeros((16, 3), dtype=torch.int32, device="cuda")
    ring = torch.zeros(1024, dtype=torch.int32, device="cuda")
    dm.window_cm(ctrl, stats, 8, 8, ring)
    torch.cuda.synchronize()
    assert stats.cpu().numpy()[:8].tolist() == [[0, 0, 1]] * 8
    fut = greedy_future(om, cfg, 11, 8)
    assert ring.cpu().numpy()[3:11].tolist() == fut

"""Pins of the oracle's forward pass, exp, norm, rotary table, attention,
drafter and window against facts that do not come from the oracle: closed
forms, library routines, exact arithmetic with an error bound, and the
central invariant that a tree step reproduces sequential single-token steps
(GPU-Resident Speculative Decoding for In-Browser LLM Inference with WebGPU,
Implementation and GPU-Resident Speculation Loop)."""
import math
import os

import numpy as np
import pytest

import synthgen as sg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(text: str) -> float:
    text = text.strip()
    return float.fromhex(text) if "0x" in text else float(text)


def _golden_lines(name: str):
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            yield [part.strip() for part in line.split("|")]


# ------------------------------------------------------------------ exp, silu, norm, rope

def test_det_exp_special_values(orc):
    assert orc.det_exp(0.0) == np.float32(1.0)
    assert orc.det_exp(-0.0) == np.float32(1.0)
    assert orc.det_exp(88.5) == np.inf
    assert orc.det_exp(-87.5) == np.float32(0.0)
    assert np.isfinite(orc.det_exp(88.0)) and orc.det_exp(-87.0) > 0


def test_det_exp_accuracy_and_monotonicity(orc):
    """Within 4 ulp of exp over [-87, 88] (relative to the double result),
    and nondecreasing along a dense sorted sample."""
    xs = np.sort(np.concatenate([np.linspace(-87, 88, 20001), sg.uniform_f32(sg.stream_key(1, 60), 20000, -87, 88),
                                 np.linspace(-1, 1, 4001)]).astype(np.float32))
    ys = np.array([orc.det_exp(float(x)) for x in xs], np.float32)
    ref = np.exp(xs.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err_ulp = np.abs(ys.astype(np.float64) - ref) / ulp
    assert err_ulp.max() <= 4.0, err_ulp.max()
    assert np.all(np.diff(ys) >= 0)


def test_silu_closed_forms(orc):
    assert orc.silu(0.0) == np.float32(0.0)
    assert orc.silu(100.0) == np.float32(100.0)             # exp(-100) -> +0, 1 + 0 = 1
    v = orc.silu(-100.0)                                     # exp(100) = inf -> -100/inf = -0
    assert v == 0 and math.copysign(1.0, float(v)) < 0
    for g in (-3.5, -0.25, 0.75, 2.0, 6.0):
        ref = g / (1 + math.exp(-g))
        assert abs(float(orc.silu(g)) - ref) <= 8 * abs(ref) * 2 ** -24


def test_rmsnorm_bound_and_closed_form(orc):
    """Relative error within a few ulp of the exact x/sqrt(mean x^2 + eps)*w;
    a constant vector of ones normalises to 1/sqrt(1 + eps) exactly rounded."""
    x = sg.normal_f32(sg.stream_key(2, 61), 896) * np.float32(3)
    w = sg.uniform_f32(sg.stream_key(2, 62), 896, 0.9, 1.1)
    y = orc.rmsnorm(x, w)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt(np.mean(x64 * x64) + np.float64(np.float32(1e-6))) * w.astype(np.float64)
    assert np.max(np.abs(y - ref) / np.abs(ref)) <= 12 * 2 ** -24
    ones = np.ones(64, np.float32)
    yo = orc.rmsnorm(ones, ones)
    rs = np.float32(np.float32(1.0) / np.float32(np.sqrt(np.float32(1.0) + np.float32(1e-6))))
    assert np.all(yo == rs)


def _rmsnorm_cases():
    return [tuple(np.array([_num(a) for a in part.split(",")], np.float32) for part in parts)
            for parts in _golden_lines("rmsnorm_worked.txt")]


@pytest.mark.parametrize("x,w,want", _rmsnorm_cases())
def test_rmsnorm_worked_example(orc, x, w, want):
    """Hand-worked bits (tests/golden/rmsnorm_worked.txt): with |x| = 3072,
    (x * rs) rounds to +-1, so the stated order (x * rs) * w returns +-w
    exactly, where x * (rs * w) would not."""
    y = orc.rmsnorm(x, w)
    assert y.tobytes() == want.tobytes(), [float(v).hex() for v in y]


def test_rope_table_matches_library(orc):
    c, s = orc.rope_table(300, 64, 1e6)
    p = np.arange(300, dtype=np.float64)[:, None]
    inv = np.power(1e6, -2.0 * np.arange(32) / 64)[None, :]
    assert np.array_equal(c, np.cos(p * inv).astype(np.float32))
    assert np.array_equal(s, np.sin(p * inv).astype(np.float32))
    assert np.all(c[0] == 1) and np.all(s[0] == 0)


# ------------------------------------------------------------------ attention

def _f16(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def test_attention_single_row_returns_v(orc):
    hd = 64
    k = _f16(sg.normal_f32(sg.stream_key(3, 63), 5 * hd).reshape(5, hd))
    v = _f16(sg.normal_f32(sg.stream_key(3, 64), 5 * hd).reshape(5, hd))
    q = sg.normal_f32(sg.stream_key(3, 65), hd)
    out = orc.attention(q, k, v, [3])
    assert np.array_equal(out, v[3].view(np.float16).astype(np.float32))


@pytest.mark.parametrize("length", [1, 7, 256, 257, 600])
def test_attention_uniform_scores_is_exact_mean(orc, length):
    """q = 0 makes every score 0, every weight E(0) = 1 and every chunk weight
    1; with small integer values all sums are exact, so the output is the mean
    rounded once."""
    hd = 16
    cap = 700
    k = _f16(sg.normal_f32(sg.stream_key(4, 66), cap * hd).reshape(cap, hd))
    vals = (sg.u32(sg.stream_key(4, 67), cap * hd) % np.uint32(21)).astype(np.int64).reshape(cap, hd) - 10
    v = _f16(vals)
    rows = np.arange(length)[::-1].copy()
    out = orc.attention(np.zeros(hd, np.float32), k, v, rows)
    want = np.array([np.float32(np.float32(vals[rows, d].sum()) / np.float32(length)) for d in range(hd)])
    assert np.array_equal(out, want)


def _attention_cases():
    def plane(n, items):
        a = np.zeros((n, 64), np.float16)
        for item in items.split():
            rows, dim, val = item.split(":")
            lo, _, hi = rows.partition("..")
            a[int(lo): int(hi or lo) + 1, int(dim)] = np.float16(_num(val))
        return a

    out = []
    for name, n, vnz, knz, qtext, want in _golden_lines("attention_chunks_worked.txt"):
        n = int(n)
        v = plane(n, vnz)
        k = plane(n, "" if knz == "-" else knz)
        q = np.ones(64, np.float32)
        if qtext != "ones":
            q[:] = 0
            for item in qtext.split():
                d, val = item.split(":")
                q[int(d)] = np.float32(_num(val))
        d, val = want.split(":")
        out.append(pytest.param(q, k, v, int(d), np.float32(_num(val)), id=name))
    return out


@pytest.mark.parametrize("q,k,v,dim,want", _attention_cases())
def test_attention_chunking_worked_example(orc, q, k, v, dim, want):
    """Hand-worked bits (tests/golden/attention_chunks_worked.txt) whose value
    depends on the chunk size (256 logical positions), on R16 inside a chunk,
    on R16 across chunks and on R16 in the score: 128- or 512-position
    chunks, or a sequential sum at any of these places, give other bits."""
    n = v.shape[0]
    out = orc.attention(q, k.view(np.uint16), v.view(np.uint16), np.arange(n, dtype=np.int32))
    assert out[dim].tobytes() == want.tobytes(), float(out[dim]).hex()
    others = np.delete(out, dim)
    assert np.all(others == 0)


def test_attention_close_to_softmax(orc):
    hd, cap = 64, 1100
    k = _f16(sg.normal_f32(sg.stream_key(5, 68), cap * hd).reshape(cap, hd))
    v = _f16(sg.normal_f32(sg.stream_key(5, 69), cap * hd).reshape(cap, hd))
    q = sg.normal_f32(sg.stream_key(5, 70), hd) * np.float32(2)
    rows = np.arange(1030)
    out = orc.attention(q, k, v, rows)
    K = k.view(np.float16).astype(np.float64)[rows]
    V = v.view(np.float16).astype(np.float64)[rows]
    s = K @ q.astype(np.float64) / np.sqrt(hd)
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ V
    assert np.max(np.abs(out - ref)) <= 1e-5 * max(1.0, np.abs(V).max())


# ------------------------------------------------------------------ forward invariants

@pytest.fixture(scope="module")
def tiny(orc):
    arr = sg.model_case(7, sg.TINY)
    c, s = orc.rope_table(sg.TINY["max_pos"], sg.TINY["head_dim"], 1e6)
    arr["rope_cos"], arr["rope_sin"] = c, s
    return orc.Model(arr, sg.TINY)


def _tree(seed, n):
    return sg.random_tree_parents(sg.stream_key(seed, sg.TID_PARENT), n)


@pytest.mark.parametrize("seed,N,L", [(1, 8, 300), (2, 6, 40), (3, 16, 511), (4, 1, 256)])
def test_tree_step_equals_sequential_steps(orc, tiny, seed, N, L):
    """For every node of a random tree, its logits and K/V rows equal those of
    depth+1 single-token steps along the root-to-node path."""
    cfg = sg.TINY
    cap = L + N + 4
    kc0, vc0 = sg.kv_prefix(seed, cfg, L, cap)
    parent = _tree(seed, N)
    token = sg.tokens(sg.stream_key(seed, sg.TID_TOKEN), N, cfg["vocab"])
    kc, vc = kc0.copy(), vc0.copy()
    logits = orc.forward(tiny, kc, vc, L, parent, token)
    for i in range(N):
        chain = [i]
        while chain[-1] != 0:
            chain.append(int(parent[chain[-1]]))
        chain.reverse()
        ks, vs = kc0.copy(), vc0.copy()
        for d, node in enumerate(chain):
            lg = orc.forward(tiny, ks, vs, L + d, np.array([-1], np.int32), np.array([token[node]], np.int32))
        assert lg[0].tobytes() == logits[i].tobytes(), f"node {i}"
        assert np.array_equal(ks[:, :, L + len(chain) - 1], kc[:, :, L + i])
        assert np.array_equal(vs[:, :, L + len(chain) - 1], vc[:, :, L + i])


def test_tree_step_commits_the_greedy_path(orc, tiny):
    """Drafts planted along a chain equal to the greedy continuation are all
    accepted; the committed cache equals the sequential one."""
    cfg = sg.TINY
    L, N = 50, 6
    kc0, vc0 = sg.kv_prefix(9, cfg, L, L + 16)
    # greedy continuation by sequential steps
    ks, vs = kc0.copy(), vc0.copy()
    toks = [17]
    for d in range(N):
        lg = orc.forward(tiny, ks, vs, L + d, np.array([-1], np.int32), np.array([toks[-1]], np.int32))
        toks.append(int(np.argmax(lg[0])))
    parent = np.array([-1, 0, 1, 2, 3, 4], np.int32)
    token = np.array(toks[:N], np.int32)
    kc, vc = kc0.copy(), vc0.copy()
    r = orc.tree_step(tiny, kc, vc, L, parent, token)
    assert r["m"] == N - 1 and r["bonus"] == toks[N] and r["L"] == L + N
    assert np.array_equal(kc[:, :, :L + N], ks[:, :, :L + N]) and np.array_equal(vc[:, :, :L + N], vs[:, :, :L + N])


# ------------------------------------------------------------------ drafter and window

@pytest.mark.parametrize("width", [1, 2, 4, 8, 16])
def test_draft_tree_shape(orc, width):
    greedy = np.arange(1000, dtype=np.int32) * 3 % 300
    draws = np.zeros(16, np.uint32)
    parent, token, bm = orc.draft_tree(width, 10, 123, greedy, draws, 2 ** 32 - 1, 300)
    D = min(width - 1, 8)
    assert bm == D and parent[0] == -1 and token[0] == 123
    assert list(parent[1:D + 1]) == list(range(D))
    assert list(parent[D + 1:]) == [(e - D - 1) % max(D, 1) for e in range(D + 1, width)]
    assert list(token[1:D + 1]) == [int(greedy[10 + k]) for k in range(1, D + 1)]   # draw 0 < threshold
    _, token0, _ = orc.draft_tree(width, 10, 123, greedy, draws, 0, 300)              # never copies
    assert all(int(token0[k]) != int(greedy[10 + k]) for k in range(1, D + 1))


@pytest.mark.parametrize("width", [2, 4, 8, 16])
def test_window_reproduces_greedy_stream(orc, tiny, width):
    """A window whose drafter copies the greedy stream emits exactly that
    stream; with random acceptance it still emits the same tokens."""
    cfg = sg.TINY
    L0, W = 30, 6
    kc0, vc0 = sg.kv_prefix(11, cfg, L0, 200)
    kc, vc = kc0.copy(), vc0.copy()
    ctrl = dict(committed_len=L0, n_nodes=1, ctx_len=190, done=0, accept_len=0, root_token=5, step=0, ring_head=0)
    _, g_emit = orc.window(tiny, kc, vc, ctrl, 1, 60, np.zeros(1, np.int32), sg.draft_draws(1, 4), 0)
    greedy = np.zeros(L0 + 1 + len(g_emit), np.int32)
    greedy[L0] = 5
    greedy[L0 + 1:] = g_emit
    for thr in (2 ** 32 - 1, int(0.6 * 2 ** 32)):
        kc, vc = kc0.copy(), vc0.copy()
        ctrl = dict(committed_len=L0, n_nodes=width, ctx_len=190, done=0, accept_len=0, root_token=5, step=0,
                    ring_head=0)
        stats, emit = orc.window(tiny, kc, vc, ctrl, width, W, greedy, sg.draft_draws(3, 64), thr)
        assert emit == list(greedy[L0 + 1:L0 + 1 + len(emit)])
        if thr == 2 ** 32 - 1:
            assert all(m == min(width - 1, 8) for m, _, _ in stats)


# ------------------------------------------------------------------ structure pin (float64 route)

def _deq(w, s):
    """Dequantise by the packing's word-level statement: eight codes per
    little-endian u32, code j at bits 4j, stored 0..15 meaning -8..7."""
    rows, kh = w.shape
    words = w.view(np.uint32).reshape(rows, kh // 4).astype(np.int64)
    codes = np.empty((rows, kh * 2), np.float64)
    for j in range(8):
        codes[:, j::8] = ((words >> (4 * j)) & 15) - 8
    return codes * np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)


def _np_forward_one(arr, cfg, kc, vc, L, tok):
    """One greedy step in float64 with the textbook formulas of a
    Qwen2.5-style decoder (absmax int8 activation quantisation emulated)."""
    H, nh, nkv, hd = cfg["hidden"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]

    def qlin(x, w, s):
        a = np.abs(x).max()
        xq = np.round(x * (127 / a))
        return (a / 127) * (_deq(w, s) @ xq)

    def norm(x, w):
        return x / np.sqrt(np.mean(x * x) + cfg["eps"]) * w

    def rope(x, p):
        half = hd // 2
        z = x[:half] + 1j * x[half:]
        ang = p * np.power(1e6, -2.0 * np.arange(half) / hd)
        z = z * np.exp(1j * ang)
        return np.concatenate([z.real, z.imag])

    h = _deq(arr["wlm"][tok:tok + 1], arr["slm"][tok:tok + 1])[0]
    for l in range(cfg["n_layers"]):
        r = norm(h, arr["norm_attn"][l])
        q = qlin(r, arr["wq"][l], arr["sq"][l]).reshape(nh, hd)
        k = qlin(r, arr["wk"][l], arr["sk"][l]).reshape(nkv, hd)
        v = qlin(r, arr["wv"][l], arr["sv"][l]).reshape(nkv, hd)
        q = np.array([rope(qq, L) for qq in q])
        k = np.array([rope(kk, L) for kk in k])
        att = np.empty((nh, hd))
        for hh in range(nh):
            g = hh // (nh // nkv)
            K = np.vstack([kc[l, g, :L].view(np.float16).astype(np.float64), k[g].astype(np.float16).astype(np.float64)])
            V = np.vstack([vc[l, g, :L].view(np.float16).astype(np.float64), v[g].astype(np.float16).astype(np.float64)])
            sc = K @ q[hh] / np.sqrt(hd)
            p = np.exp(sc - sc.max())
            att[hh] = (p / p.sum()) @ V
        h = h + qlin(att.reshape(-1), arr["wo"][l], arr["so"][l])
        r = norm(h, arr["norm_mlp"][l])
        gg = qlin(r, arr["wg"][l], arr["sg"][l])
        uu = qlin(r, arr["wu"][l], arr["su"][l])
        h = h + qlin(gg / (1 + np.exp(-gg)) * uu, arr["wd"][l], arr["sd"][l])
    return qlin(norm(h, arr["norm_final"]), arr["wlm"], arr["slm"])


def test_forward_structure_matches_float64_textbook(orc, tiny):
    """The oracle's single-token step agrees with a float64 implementation of
    the standard decoder equations (different code, different precision) to
    within the int8/fp16 rounding the method adds."""
    cfg = sg.TINY
    arr = tiny.arrays
    for L, tok in ((0, 3), (40, 17), (300, 250)):
        kc, vc = sg.kv_prefix(21, cfg, L, L + 4)
        ref = _np_forward_one(arr, cfg, kc, vc, L, tok)
        got = orc.forward(tiny, kc.copy(), vc.copy(), L, np.array([-1], np.int32), np.array([tok], np.int32))[0]
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err < 2e-2, (L, err)
        assert np.corrcoef(got, ref)[0, 1] > 0.999


def test_layer0_kv_rows_exact(orc, tiny):
    """The K/V rows a step writes in layer 0 are the fp16 (round-to-nearest,
    numpy's conversion) of v = W4A8_v(RMSNorm(embedding)) and of k rotated
    by the pinned table, built here from separately pinned parts: the exact
    embedding dequantisation, RMSNorm, quantisation and the linear."""
    cfg, arr = sg.TINY, tiny.arrays
    L, tok = 37, 123
    kc, vc = sg.kv_prefix(5, cfg, L, L + 2)
    orc.forward(tiny, kc, vc, L, np.array([-1], np.int32), np.array([tok], np.int32))
    h = _deq(arr["wlm"][tok:tok + 1], arr["slm"][tok:tok + 1])[0].astype(np.float32)   # exact in fp32
    r = orc.rmsnorm(h, arr["norm_attn"][0])
    xq, xs = orc.quantize_act(r[None, :])
    k = orc.w4a8_linear(arr["wk"][0], arr["sk"][0], xq, xs)[0]
    v = orc.w4a8_linear(arr["wv"][0], arr["sv"][0], xq, xs)[0]
    hd, half = cfg["head_dim"], cfg["head_dim"] // 2
    cos, sin = arr["rope_cos"][L], arr["rope_sin"][L]
    for g in range(cfg["n_kv_heads"]):
        kk = k[g * hd:(g + 1) * hd]
        a, b = kk[:half], kk[half:]
        rot = np.concatenate([a * cos - b * sin, b * cos + a * sin]).astype(np.float32)
        assert np.array_equal(kc[0, g, L], rot.astype(np.float16).view(np.uint16))
        assert np.array_equal(vc[0, g, L], v[g * hd:(g + 1) * hd].astype(np.float16).view(np.uint16))

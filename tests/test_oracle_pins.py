"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against one of: values worked by hand from the
pages' statement of the method (tests/golden), closed forms, exact rational
arithmetic with an error bound, brute force on tiny inputs by a different
route, or a library routine for a special case. None of them retypes the
oracle's own loop.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synthgen as sg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = Fraction(1, 2 ** 24)  # unit roundoff of binary32


# ------------------------------------------------------------------ fp16

def test_f16_widening_exhaustive(orc):
    """Every fp16 bit pattern widens to the value numpy's float16 gives."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_narrowing_matches_library(orc):
    """fp32 -> fp16 rounding to nearest-even agrees with numpy on random bit
    patterns concentrated on the fp16 range, and on every tie."""
    key = sg.stream_key(11, 1)
    raw = sg.u32(key, 40000)
    # exponents spread over the fp16 normal/subnormal/overflow range
    e = (raw >> np.uint32(24)) % np.uint32(48) + np.uint32(127 - 28)
    pats = (raw & np.uint32(0x807FFFFF)) | (e << np.uint32(23))
    # exact ties: low 13 bits = 0x1000
    ties = (pats & np.uint32(0xFFFFE000)) | np.uint32(0x1000)
    xs = np.concatenate([pats, ties]).view(np.float32)
    xs = np.concatenate([xs, np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -25,
                                        2.0 ** -24 * 1.5, np.inf, -np.inf], np.float32)])
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ R16

def _golden_r16():
    cases = []
    for line in open(os.path.join(GOLDEN, "r16_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, n, entries, expect = [s.strip() for s in line.split("|")]
        v = np.zeros(int(n), np.float32)
        for e in entries.split(","):
            i, x = e.split(":")
            v[int(i)] = np.float32(float(x))
        cases.append((name, v, np.float32(float(expect))))
    return cases


@pytest.mark.parametrize("name,v,expect", _golden_r16(), ids=lambda c: c if isinstance(c, str) else "")
def test_r16_worked_examples(orc, name, v, expect):
    got = orc.r16(v)
    assert got.tobytes() == expect.tobytes(), (name, got, expect)


def test_r16_exact_on_small_integers(orc):
    """Integers whose partial sums stay below 2^24 are summed exactly in any
    order, so R16 must return the exact sum."""
    rng_key = sg.stream_key(3, 2)
    for n in (0, 1, 5, 16, 17, 31, 100, 1000):
        v = (sg.u32(rng_key, n) % np.uint32(2001)).astype(np.int64) - 1000
        assert float(orc.r16(v.astype(np.float32))) == float(v.sum())


def test_r16_error_bound_vs_exact(orc):
    """|R16(v) - sum(v)| <= (ceil(n/16) + 4) * u * sum|v| (first order), the
    bound of a sum whose deepest term passes ceil(n/16)-1 slot additions and
    4 tree levels."""
    key = sg.stream_key(4, 2)
    for n in (7, 28, 128, 152, 448):
        v = sg.normal_f32(key, n) * np.float32(3.0)
        exact = sum(Fraction(float(x)) for x in v)
        got = Fraction(float(orc.r16(v)))
        bound = (math.ceil(n / 16) + 4) * U * sum(abs(Fraction(float(x))) for x in v) * Fraction(1001, 1000)
        assert abs(got - exact) <= bound


def test_r16_order_is_observable(orc):
    """Sequential and adjacent-pairwise summation give different bits from
    R16 on random data, so a test of the order can fail."""
    v = sg.normal_f32(sg.stream_key(5, 2), 448)
    seq = np.float32(0)
    for x in v:
        seq = np.float32(seq + x)
    assert orc.r16(v).tobytes() != seq.tobytes() or orc.r16(v[::-1].copy()).tobytes() != seq.tobytes()


# ------------------------------------------------------------------ quantisation

def _golden_quant():
    out = []
    for line in open(os.path.join(GOLDEN, "quant_ties.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        xs, codes, scale = [s.strip() for s in line.split("|")]
        out.append((np.array([_num(a) for a in xs.split(",")], np.float32),
                    np.array([int(c) for c in codes.split(",")], np.int8), np.float32(_num(scale))))
    return out


def _num(text: str) -> float:
    """A decimal or hex float ("0x1p-130"), as written in the golden files."""
    text = text.strip()
    return float.fromhex(text) if "0x" in text else float(text)


@pytest.mark.parametrize("x,codes,scale", _golden_quant())
def test_quant_worked_examples(orc, x, codes, scale):
    xq, xs = orc.quantize_act(x[None, :])
    assert np.array_equal(xq[0], codes)
    assert xs[0].tobytes() == scale.tobytes()


def test_quant_one_hot_closed_form(orc):
    """x = c * e_k: one code of +-127 at k, zeros elsewhere, scale |c|/127."""
    for c, k in ((3.7, 0), (-0.001, 5), (1e30, 31), (-2.0 ** -130, 17)):
        x = np.zeros((1, 32), np.float32)
        x[0, k] = np.float32(c)
        xq, xs = orc.quantize_act(x)
        want = np.zeros(32, np.int8)
        want[k] = 127 if c > 0 else -127
        assert np.array_equal(xq[0], want)
        assert xs[0] == np.float32(np.float32(abs(c)) / np.float32(127.0))


def test_quant_invariants(orc):
    """max|code| = 127 and |x - s*code| <= s*(1/2 + 2^-14) + a*2^-23, checked
    in exact arithmetic, on N(0,1) rows of the linear-set shapes."""
    x = sg.normal_f32(sg.stream_key(6, 3), 8 * 896).reshape(8, 896)
    x[3] *= np.float32(1e-3)
    xq, xs = orc.quantize_act(x)
    for t in range(8):
        assert np.abs(xq[t].astype(np.int32)).max() == 127
        a = Fraction(float(np.abs(x[t]).max()))
        s = Fraction(float(xs[t]))
        bound = s * (Fraction(1, 2) + Fraction(1, 2 ** 14)) + a * Fraction(1, 2 ** 23)
        for k in range(0, 896, 7):
            assert abs(Fraction(float(x[t, k])) - s * int(xq[t, k])) <= bound


def test_quant_codes_invariant_under_power_of_two_scaling(orc):
    """Multiplying a row by 2^e (exactly) leaves its codes unchanged, also
    when 2^e makes 127/absmax overflow: the codes are round(x * 127/absmax),
    a function of the ratios only. The scales scale by 2^e where they stay
    normal."""
    x = sg.normal_f32(sg.stream_key(6, 4), 4 * 896).reshape(4, 896)
    # magnitudes in [1/4, 3.9]: at 2^-124 every value stays normal (exact),
    # and absmax * 2^-124 < 2^-122 makes 127/absmax overflow binary32
    x[np.abs(x) < 0.25] = np.float32(0.5)
    x = np.clip(x, -3.9, 3.9).astype(np.float32)
    xq, xs = orc.quantize_act(x)
    for e in (-124, -110, -100, -60, 40, 100):
        xe = (x * np.float32(2.0 ** e)).astype(np.float32)
        assert np.array_equal((xe * np.float32(2.0 ** -e)).astype(np.float32), x)
        if e == -124:
            assert float(np.abs(xe).max()) < 127.0 / float(np.finfo(np.float32).max)
        xqe, xse = orc.quantize_act(xe)
        assert np.array_equal(xqe, xq), f"codes changed at 2^{e}"
        if float(xs.min()) * 2.0 ** e >= 2.0 ** -126:
            assert np.array_equal(xse, (xs * np.float32(2.0 ** e)).astype(np.float32))


def test_quant_tiny_subnormal_rows_near_exact(orc):
    """Rows of subnormals (bits lost against N(0,1), absmax around 1e-40):
    every code is within one of the exact rational round(x * 127/absmax),
    and equal to it where the exact value is not within 2^-10 of a tie."""
    x = (sg.normal_f32(sg.stream_key(6, 5), 2 * 300).reshape(2, 300) * np.float32(1e-40)).astype(np.float32)
    xq, xs = orc.quantize_act(x)
    for t in range(2):
        a = Fraction(float(np.abs(x[t]).max()))
        assert xs[t] == np.float32(float(a) / 127.0) or abs(Fraction(float(xs[t])) - a / 127) <= Fraction(1, 2 ** 150)
        for k in range(300):
            r = Fraction(float(x[t, k])) * 127 / a
            fl = math.floor(r)
            frac = r - fl
            want = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
            assert abs(int(xq[t, k]) - want) <= 1
            if abs(frac - Fraction(1, 2)) > Fraction(1, 2 ** 10):
                assert int(xq[t, k]) == want


# ------------------------------------------------------------------ W4A8 linear

def _codes_by_words(wq: np.ndarray) -> np.ndarray:
    """Decode the rows by the packing's own statement: eight 4-bit codes per
    little-endian 32-bit word, code j at bits 4j..4j+3, stored 0..15 meaning
    -8..7. A different route from the oracle's byte/nibble indexing."""
    N, Kh = wq.shape
    words = wq.view(np.uint32).reshape(N, Kh // 4).astype(np.int64)
    out = np.empty((N, Kh * 2), np.int64)
    for j in range(8):
        out[:, j::8] = ((words >> (4 * j)) & 15) - 8
    return out


def test_group_dots_nibble_by_int8_exhaustive(orc):
    """All 256 byte values against all 255 int8 codes: a row of one repeated
    byte b against a token of one repeated code a has group dot
    16*((b & 15) - 8)*a + 16*((b >> 4) - 8)*a."""
    wq = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    codes = np.arange(-127, 128, dtype=np.int8)
    xq = np.repeat(codes[:, None], 32, axis=1)
    d = orc.group_dots(wq, xq)  # [255][256][1]
    b = np.arange(256)
    want = 16 * (((b & 15) - 8)[None, :] + ((b >> 4) - 8)[None, :]) * codes.astype(np.int64)[:, None]
    assert np.array_equal(d[:, :, 0].astype(np.int64), want)


@pytest.mark.parametrize("T,N,K", [(1, 3, 32), (3, 5, 64), (8, 8, 96), (2, 4, 544)])
def test_group_dots_brute_force(orc, T, N, K):
    wq, _, x = sg.linear_case(21, T, N, K)
    xq = (sg.u32(sg.stream_key(21, 40), T * K) % np.uint32(255)).astype(np.int64) - 127
    xq = xq.astype(np.int8).reshape(T, K)
    d = orc.group_dots(wq, xq)
    q = _codes_by_words(wq)
    for t, n, g in itertools.product(range(T), range(N), range(K // 32)):
        assert d[t, n, g] == int(np.dot(q[n, 32 * g:32 * g + 32], xq[t, 32 * g:32 * g + 32].astype(np.int64)))


def test_linear_single_group_closed_form(orc):
    """K = 32 (one group): y = xs * (scale * d), two plain IEEE products."""
    wq, ws, x = sg.linear_case(22, 4, 16, 32)
    xq, xs = orc.quantize_act(x)
    y = orc.w4a8_linear(wq, ws, xq, xs)
    q = _codes_by_words(wq)
    s = ws.view(np.float16).astype(np.float32)
    for t in range(4):
        for n in range(16):
            d = np.float32(int(np.dot(q[n], xq[t].astype(np.int64))))
            want = np.float32(xs[t] * np.float32(s[n, 0] * d))
            assert y[t, n].tobytes() == want.tobytes()


@pytest.mark.parametrize("T,N,K", [(1, 4, 896), (2, 3, 4864), (8, 2, 4096)])
def test_linear_error_bound_vs_exact(orc, T, N, K):
    """|y - y*| <= (ceil(G/16) + 6) u xs sum|s_g d_g| with y* the exact value
    of xs * sum_g s_g d_g from exact group dots."""
    wq, ws, x = sg.linear_case(23, T, N, K)
    xq, xs = orc.quantize_act(x)
    y = orc.w4a8_linear(wq, ws, xq, xs)
    q = _codes_by_words(wq)
    s = ws.view(np.float16).astype(np.float64)
    G = K // 32
    for t in range(T):
        for n in range(N):
            terms = []
            for g in range(G):
                d = int(np.dot(q[n, 32 * g:32 * g + 32], xq[t, 32 * g:32 * g + 32].astype(np.int64)))
                terms.append(Fraction(float(s[n, g])) * d)
            exact = Fraction(float(xs[t])) * sum(terms)
            bound = (math.ceil(G / 16) + 6) * U * Fraction(float(xs[t])) * sum(abs(a) for a in terms)
            assert abs(Fraction(float(y[t, n])) - exact) <= bound * Fraction(1001, 1000)


def test_linear_rows_of_T_equal_single_token(orc):
    """The central property: row t of a T-token call equals a 1-token call on
    token t, bit for bit (the reduction never depends on T)."""
    wq, ws, x = sg.linear_case(24, 8, 40, 896)
    xq, xs = orc.quantize_act(x)
    y8 = orc.w4a8_linear(wq, ws, xq, xs)
    for t in range(8):
        y1 = orc.w4a8_linear(wq, ws, xq[t:t + 1].copy(), xs[t:t + 1].copy())
        assert y1.tobytes() == y8[t:t + 1].tobytes()


def test_linear_rows_subset_matches_full(orc):
    wq, ws, x = sg.linear_case(25, 3, 50, 128)
    xq, xs = orc.quantize_act(x)
    y = orc.w4a8_linear(wq, ws, xq, xs)
    rows = np.array([0, 7, 49, 7, 13], np.int32)
    assert orc.w4a8_linear_rows(wq, ws, xq, xs, rows).tobytes() == y[:, rows].copy().tobytes()


def test_linear_threads_equal_single_thread(orc):
    """The row-block threaded oracle (the all-cores CPU baseline) computes
    every row with the same code, so it equals the one-call result."""
    for T, N, K, th in ((8, 300, 896, 7), (1, 17, 64, 16), (3, 5, 128, 8)):
        wq, ws, x = sg.linear_case(21, T, N, K)
        xq, xs = orc.quantize_act(x)
        assert orc.w4a8_linear_threads(wq, ws, xq, xs, th).tobytes() == orc.w4a8_linear(wq, ws, xq, xs).tobytes()


def test_linear_sequential_order_differs(orc):
    """Summing the scaled group terms sequentially instead of in R16 order
    changes some output bits, so the parity tests would see a wrong order."""
    wq, ws, x = sg.linear_case(26, 1, 64, 4096)
    xq, xs = orc.quantize_act(x)
    y = orc.w4a8_linear(wq, ws, xq, xs)
    d = orc.group_dots(wq, xq)[0]
    s = ws.view(np.float16).astype(np.float32)
    differ = 0
    for n in range(64):
        acc = np.float32(0)
        for g in range(128):
            acc = np.float32(acc + np.float32(s[n, g] * np.float32(d[n, g])))
        differ += np.float32(xs[0] * acc).tobytes() != y[0, n].tobytes()
    assert differ > 0


# ------------------------------------------------------------------ argmax

def test_argmax_brute_force_and_ties(orc):
    key = sg.stream_key(30, 4)
    L = sg.normal_f32(key, 6 * 1000).reshape(6, 1000)
    L[1, 10] = L[1, 900] = np.float32(50.0)      # tie: lowest index wins
    L[2, :] = np.float32(-1.0)
    L[2, 5] = np.float32(-0.0)
    L[2, 3] = np.float32(0.0)                     # -0 == +0: index 3 wins
    L[3, :] = np.float32(7.0)                     # all equal: 0
    L[4, -1] = np.float32(np.inf)
    got = orc.argmax(L)
    for i in range(6):
        row = [float(v) for v in L[i]]
        assert got[i] == row.index(max(row))
    assert list(got[1:4]) == [10, 3, 0]


# ------------------------------------------------------------------ tree acceptance

def _brute_accept(parent, token, amax):
    """Enumerate every root-to-node path; a node is accepted when each edge on
    its path carries the parent's prediction. Deepest wins, then lowest id."""
    N = len(parent)
    best = (0, 0)  # (depth, -index)
    best_path = [0]
    for i in range(N):
        chain = [i]
        while chain[-1] != 0:
            chain.append(parent[chain[-1]])
        chain.reverse()
        ok = all(token[chain[k]] == amax[chain[k - 1]] for k in range(1, len(chain)))
        if ok and (len(chain) - 1 > best[0]):
            best, best_path = (len(chain) - 1, -i), chain
    return len(best_path) - 1, best_path, amax[best_path[-1]]


def _all_trees(n):
    for ps in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1, *ps]


def test_accept_all_small_trees(orc):
    key = sg.stream_key(31, 5)
    ctr = 0
    for n in range(1, 7):
        for parent in _all_trees(n):
            for rep in range(3):
                r = (sg.u64(key, 2 * n, start=ctr) % np.uint64(3)).astype(np.int32)
                ctr += 2 * n
                token, amax = r[:n].copy(), r[n:].copy()
                m, path, bonus = orc.tree_accept(parent, token, amax)
                bm, bpath, bbonus = _brute_accept(parent, token, amax)
                assert (m, list(path), bonus) == (bm, bpath, bbonus), (parent, token, amax)


def test_accept_chain_is_greedy_prefix(orc):
    """On a chain the accepted length is the longest prefix of drafts that
    equal the greedy predictions, and the bonus is the prediction after it."""
    for m_true in range(0, 8):
        parent = [-1] + list(range(7))
        amax = list(range(100, 108))
        token = [5] + [amax[i - 1] for i in range(1, 8)]
        if m_true < 7:
            token[m_true + 1] = 999
        m, path, bonus = orc.tree_accept(parent, token, amax)
        assert m == m_true and list(path) == list(range(m_true + 1)) and bonus == amax[m_true]


def test_accept_single_node_is_greedy_step(orc):
    m, path, bonus = orc.tree_accept([-1], [42], [17])
    assert (m, list(path), bonus) == (0, [0], 17)


def test_accept_rejects_malformed(orc):
    with pytest.raises(ValueError):
        orc.tree_accept([-1, 1], [0, 0], [0, 0])
    with pytest.raises(ValueError):
        orc.tree_accept([0, 0], [0, 0], [0, 0])


# ------------------------------------------------------------------ compaction

def test_kv_compact_equals_gather(orc):
    """In-place moves in increasing j give the same cache as gathering every
    destination row from an untouched copy (sources never precede their
    destination), on random accepted paths of random trees."""
    key = sg.stream_key(32, 7)
    layers, heads, cap, hd, L = 3, 2, 40, 16, 20
    for trial in range(30):
        cache = sg.u32(key, layers * heads * cap * hd).astype(np.uint16).reshape(layers, heads, cap, hd)
        key = sg.stream_key(32, 100 + trial)
        n = 2 + trial % 15
        parent = sg.random_tree_parents(key, n)
        # choose the deepest node and its chain as the path
        depth = [0] * n
        for i in range(1, n):
            depth[i] = depth[parent[i]] + 1
        w = int(np.argmax(depth))
        path = [w]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path = np.array(path[::-1], np.int32)
        m = len(path) - 1
        before = cache.copy()
        orc.kv_compact(cache, L, path, m)
        want = before.copy()
        for j in range(1, m + 1):
            want[:, :, L + j] = before[:, :, L + path[j]]
        assert np.array_equal(cache, want)


def test_kv_compact_rejects_bad_path(orc):
    cache = np.zeros((1, 1, 8, 4), np.uint16)
    with pytest.raises(ValueError):
        orc.kv_compact(cache, 2, np.array([0, 0], np.int32), 1)   # path[1] < 1
    with pytest.raises(ValueError):
        orc.kv_compact(cache, 6, np.array([0, 3], np.int32), 1)   # row past capacity

"""Pins of the oracle's context-mixing drafter (GPU-Resident Speculative
Decoding for In-Browser LLM Inference with WebGPU, Draft-Free Drafting From
Web Context), against things other than itself: a hand-worked example, a
brute force that builds the trie as a dictionary of token prefixes, the
structural invariants of the tree, and special cases whose result is known."""
import os
import random

import numpy as np
import pytest

import oracle

W8 = [0, 1, 2, 4, 8, 16, 32, 64, 128]


def golden():
    d = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "cm_draft_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        d[k] = [int(x) for x in v]
    return d


def test_worked_example():
    g = golden()
    parent, token, n, bm = oracle.cm_draft(g["stream"], g["width"][0], g["max_order"][0], g["candidates"][0],
                                           g["depth"][0], g["weight"])
    assert parent.tolist() == g["parent"] and token.tolist() == g["token"]
    assert n == g["nodes"][0] and bm == g["best_match"][0]


def brute(s, width, max_order, cands, depth, weight):
    """The drafter's definition, written with prefix tuples."""
    n = len(s)
    lens = {}
    for p in range(n - 1):
        l = 0
        for i in range(min(max_order, p + 1)):
            if s[p - i] != s[n - 1 - i]:
                break
            l = i + 1
        if l >= 1:
            lens[p] = l
    chosen = sorted(lens, key=lambda p: (lens[p], p), reverse=True)[:cands]
    weight_of, first = {}, {}
    for k, p in enumerate(chosen):
        cont = tuple(s[p + 1: min(p + depth, n - 1) + 1])
        for d in range(len(cont)):
            pre = cont[: d + 1]
            weight_of[pre] = weight_of.get(pre, 0) + weight[lens[p]]
            first.setdefault(pre, (k, d))
    keep = sorted(weight_of, key=lambda pre: (-weight_of[pre], len(pre), first[pre]))[: width - 1]
    rank = {pre: r for r, pre in enumerate(keep)}
    order = sorted(keep, key=lambda pre: (len(pre), rank[pre]))
    idx = {(): 0}
    parent, token = [-1], [s[-1]]
    for pre in order:
        idx[pre] = len(parent)
        parent.append(idx[pre[:-1]])
        token.append(pre[-1])
    return parent, token, len(parent), (lens[chosen[0]] if chosen else 0)


@pytest.mark.parametrize("seed", range(60))
def test_against_brute_force(seed):
    rng = random.Random(seed)
    vocab = rng.choice([2, 3, 4, 6])
    n = rng.randint(1, 60)
    s = [rng.randrange(vocab) for _ in range(n)]
    width = rng.randint(1, 16)
    max_order, cands, depth = rng.randint(1, 8), rng.randint(1, 32), rng.randint(1, 8)
    weight = [0] + [rng.randint(1, 50) for _ in range(8)]
    got = oracle.cm_draft(s, width, max_order, cands, depth, weight)
    exp = brute(s, width, max_order, cands, depth, weight)
    assert got[0].tolist() == exp[0] and got[1].tolist() == exp[1] and got[2:] == exp[2:], (s, width)


@pytest.mark.parametrize("seed", range(20))
def test_tree_invariants(seed):
    """Topological and prefix-closed, siblings distinct, and every node's path
    from the root follows an earlier occurrence of the root in the stream."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, 5, size=int(rng.integers(50, 400))).tolist()
    width = int(rng.integers(2, 17))
    parent, token, n, bm = oracle.cm_draft(s, width)
    assert n == len(parent) <= width and parent[0] == -1 and token[0] == s[-1]
    assert all(0 <= parent[i] < i for i in range(1, n))
    kids = {}
    for i in range(1, n):
        assert token[i] not in kids.setdefault(int(parent[i]), set())
        kids[int(parent[i])].add(int(token[i]))
    text = " " + " ".join(map(str, s)) + " "
    for i in range(1, n):
        path, j = [], i
        while j >= 0:
            path.append(int(token[j]))
            j = int(parent[j])
        assert (" " + " ".join(map(str, path[::-1])) + " ") in text
    assert 1 <= bm <= 8


def test_special_cases():
    # a single token: no history, the root alone
    assert oracle.cm_draft([7], 8)[2:] == (1, 0)
    # no earlier occurrence of the root
    p, t, n, bm = oracle.cm_draft([1, 2, 3, 4, 5], 8)
    assert (n, bm) == (1, 0) and t.tolist() == [5]
    # width 1 keeps the root only, but still reports the match
    assert oracle.cm_draft([1, 2, 1, 2], 1)[2:] == (1, 2)
    # a constant stream: the best candidates continue with the same token, so
    # the tree is a chain of it (one continuation per depth)
    p, t, n, bm = oracle.cm_draft([3] * 30, 6, depth=8)
    assert p.tolist() == [-1, 0, 1, 2, 3, 4] and t.tolist() == [3] * 6 and bm == 8
    # a periodic stream: the heaviest chain is the true continuation
    period = [4, 1, 5, 9, 2, 6]
    s = period * 6 + period[:3]
    p, t, n, bm = oracle.cm_draft(s, 9, depth=8)
    chain = [t[i] for i in range(1, n) if p[i] == i - 1 or (i == 1 and p[i] == 0)]
    nxt = (period * 3)[3:3 + len(chain)]
    assert chain == nxt and bm == 8


def test_rejects_bad_arguments():
    lib = oracle.lib()
    s = np.zeros(4, np.int32)
    par = np.zeros(16, np.int32)
    tok = np.zeros(16, np.int32)
    bm = np.zeros(1, np.int32)
    good = np.array(W8, np.uint32)
    zero_w = np.array([0, 0, 1, 1, 1, 1, 1, 1, 1], np.uint32)
    args = lambda n, mo, c, d, w, width: lib.orc_cm_draft(s.ctypes.data, n, mo, c, d, w.ctypes.data, width,
                                                          par.ctypes.data, tok.ctypes.data, bm.ctypes.data)
    assert args(4, 8, 16, 8, good, 8) == 4   # [0 0 0 0]: the root and a chain of three
    assert args(0, 8, 16, 8, good, 8) == -1
    assert args(4, 9, 16, 8, good, 8) == -1
    assert args(4, 8, 33, 8, good, 8) == -1
    assert args(4, 8, 16, 9, good, 8) == -1
    assert args(4, 8, 16, 8, good, 17) == -1
    assert args(4, 8, 16, 8, zero_w, 8) == -1

"""GPU parity of the tree-masked verification step (spec_tree_step) against
the CPU oracle, bit for bit: logits, greedy predictions, accepted path,
control state and the whole fp16 KV caches after compaction. Also the
property that a tree step reproduces single-token steps along every node's
path, on the GPU itself at full size (24-layer Qwen2.5-0.5B shape, 1024
committed rows, 8-node tree)."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_verification_amd as m
    return m


# Rows longer than 1024 values take the fused RMSNorm's LDS-row path (up to
# 4 tokens; the row kernel beyond), and an intermediate of 2176 the fused
# SiLU rows up to 2 tokens. Rows of up to 1024 values are spread over the
# workgroup below 4 tokens and taken by their waves from 4 to 8.
WIDE = dict(n_layers=2, hidden=1280, n_heads=10, n_kv_heads=2, head_dim=128, inter=2176, vocab=1000,
            eps=1e-6, max_pos=640)
# Head dim 128 with an attention row of 1024 values: the grouped attention
# (every head of a KV group in one workgroup, merge fused) over two column
# blocks; the wide configuration's 1280-value row takes the per-head kernel
# and the separate merge.
HD128 = dict(n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, inter=1024, vocab=700,
             eps=1e-6, max_pos=640)
# Groups of 7 and 8 query heads per KV head: trees of up to four nodes split
# a group's heads over two workgroups (heads 0..3 and the rest), larger
# trees keep them in one.
G7 = dict(n_layers=2, hidden=896, n_heads=14, n_kv_heads=2, head_dim=64, inter=1024, vocab=1000,
          eps=1e-6, max_pos=640)
G8 = dict(n_layers=2, hidden=512, n_heads=8, n_kv_heads=1, head_dim=128, inter=768, vocab=900,
          eps=1e-6, max_pos=640)
CFGS = {"tiny": (sg.TINY, 7), "wide": (WIDE, 11), "hd128": (HD128, 13), "g7": (G7, 17), "g8": (G8, 19)}


@functools.lru_cache(maxsize=4)
def model_pair(name):
    cfg, seed = CFGS.get(name, (sg.QWEN05, 3))
    arrays = sg.model_case(seed, cfg)
    c, s = oracle.rope_table(cfg["max_pos"], cfg["head_dim"], 1e6)
    arrays = dict(arrays, rope_cos=c, rope_sin=s)
    return cfg, arrays, oracle.Model(arrays, cfg)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def planted_tree(seed, N, L, cfg, orc_model, kc, vc):
    """Random tree; drafts along the deepest chain follow the oracle's greedy
    continuation so acceptance and compaction are exercised."""
    parent = sg.random_tree_parents(sg.stream_key(seed, sg.TID_PARENT), N)
    token = sg.tokens(sg.stream_key(seed, sg.TID_TOKEN), N, cfg["vocab"])
    if N > 1:
        depth = np.zeros(N, np.int32)
        for i in range(1, N):
            depth[i] = depth[parent[i]] + 1
        w = int(np.argmax(depth))
        chain = [w]
        while chain[-1] != 0:
            chain.append(int(parent[chain[-1]]))
        chain.reverse()
        ks, vs = kc.copy(), vc.copy()
        for d, node in enumerate(chain[:-1]):
            lg = oracle.forward(orc_model, ks, vs, L + d, np.array([-1], np.int32),
                                np.array([token[node]], np.int32))
            token[chain[d + 1]] = int(np.argmax(lg[0]))
    return parent, token


def compare_step(sv, name, seed, N, L, plant=True):
    cfg, arrays, om = model_pair(name)
    cap = L + N + 8
    kc0, vc0 = sg.kv_prefix(seed, cfg, L, cap)
    if plant:
        parent, token = planted_tree(seed, N, L, cfg, om, kc0, vc0)
    else:
        parent = sg.random_tree_parents(sg.stream_key(seed, sg.TID_PARENT), N)
        token = sg.tokens(sg.stream_key(seed, sg.TID_TOKEN), N, cfg["vocab"])
    kc, vc = kc0.copy(), vc0.copy()
    ro = oracle.tree_step(om, kc, vc, L, parent, token, want_logits=True)

    dm = sv.DeviceModel(arrays, cfg, cap, kc0, vc0)
    ctrl = sv.new_ctrl(L, N, cap - N, root_token=int(token[0]))
    stats = torch.zeros(3, dtype=torch.int32, device="cuda")
    logits, amax, path = dm.tree_step(ctrl, dev_i32(parent), dev_i32(token), N, stats=stats)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    bad = np.nonzero(lg.view(np.uint32) != ro["logits"].view(np.uint32))
    assert bad[0].size == 0, f"{bad[0].size} logits differ, first {bad[0][0]},{bad[1][0]}: " \
                             f"{lg[bad[0][0], bad[1][0]]} vs {ro['logits'][bad[0][0], bad[1][0]]}"
    assert np.array_equal(amax.cpu().numpy(), ro["amax"])
    m = ro["m"]
    assert np.array_equal(path.cpu().numpy()[: m + 1], ro["path"])
    c = ctrl.cpu().numpy()
    assert (c[0], c[4], c[5], c[6]) == (ro["L"], m, ro["bonus"], 1)
    assert np.array_equal(dm.k_cache.cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(dm.v_cache.cpu().numpy().view(np.uint16), vc)
    return m


@pytest.mark.parametrize("seed,N,L", [(1, 8, 300), (2, 6, 40), (3, 16, 511), (4, 1, 256), (5, 5, 0),
                                      (6, 3, 1), (8, 16, 600), (9, 2, 255)])
def test_tiny_tree_step_parity(sv, seed, N, L):
    case(f"tiny tree step seed={seed} N={N} L={L}")
    compare_step(sv, "tiny", seed, N, L)


@pytest.mark.parametrize("seed,N,L", [(41, 1, 100), (42, 4, 257), (43, 8, 64), (44, 16, 300)])
def test_wide_tree_step_parity(sv, seed, N, L):
    case(f"wide (hidden 1280) tree step seed={seed} N={N} L={L}")
    compare_step(sv, "wide", seed, N, L)


@pytest.mark.parametrize("seed,N,L", [(51, 1, 300), (52, 5, 256), (53, 16, 520), (54, 8, 0)])
def test_hd128_tree_step_parity(sv, seed, N, L):
    case(f"head dim 128 tree step seed={seed} N={N} L={L}")
    compare_step(sv, "hd128", seed, N, L)


@pytest.mark.parametrize("name,seed,N,L", [("g7", 61, 1, 300), ("g7", 62, 2, 520), ("g7", 63, 3, 255),
                                            ("g7", 64, 8, 0), ("g8", 65, 1, 256), ("g8", 66, 2, 511),
                                            ("g8", 67, 5, 40)])
def test_grouped_head_split_parity(sv, name, seed, N, L):
    case(f"{name} tree step seed={seed} N={N} L={L}")
    compare_step(sv, name, seed, N, L)


@pytest.mark.parametrize("name,seed,N,L", [("g7", 68, 9, 300), ("g7", 69, 16, 520), ("g8", 70, 12, 255),
                                            ("g8", 71, 16, 0)])
def test_grouped_half_workgroups_parity(sv, name, seed, N, L):
    """Trees of more than 8 nodes take the grouped attention in 512-thread
    workgroups (two sets, up to four heads each)."""
    case(f"{name} tree step seed={seed} N={N} L={L}")
    compare_step(sv, name, seed, N, L)


def test_tiny_unplanted_tree(sv):
    case("tiny tree step, random drafts")
    compare_step(sv, "tiny", 12, 8, 130, plant=False)


def test_qwen05_tree_step_parity(sv):
    """Full 8-node tree verification on the 24-layer Qwen2.5-0.5B shape over
    a 1024-row fp16 cache, against the oracle."""
    case("qwen0.5b tree step N=8 L=1024")
    m = compare_step(sv, "qwen", 21, 8, 1024)
    assert m >= 1


@pytest.mark.parametrize("name,seed,N,L", [("tiny", 31, 8, 200), ("tiny", 32, 1, 50), ("qwen", 23, 8, 1024),
                                            ("qwen", 24, 1, 1024), ("qwen", 25, 2, 1100)])
def test_tree_step_without_logits(sv, name, seed, N, L):
    """With no logits buffer the step writes no logits (the lm_head reduces
    to each node's argmax in its epilogue) and gives the oracle's
    predictions, path, control block and caches."""
    case(f"{name} tree step without logits N={N} L={L}")
    cfg, arrays, om = model_pair(name)
    cap = L + N + 8
    kc0, vc0 = sg.kv_prefix(seed, cfg, L, cap)
    parent, token = planted_tree(seed, N, L, cfg, om, kc0, vc0)
    kc, vc = kc0.copy(), vc0.copy()
    ro = oracle.tree_step(om, kc, vc, L, parent, token)
    dm = sv.DeviceModel(arrays, cfg, cap, kc0, vc0)
    ctrl = sv.new_ctrl(L, N, cap - N, root_token=int(token[0]))
    logits, amax, path = dm.tree_step(ctrl, dev_i32(parent), dev_i32(token), N, want_logits=False)
    torch.cuda.synchronize()
    assert logits is None
    assert np.array_equal(amax.cpu().numpy(), ro["amax"])
    m = ro["m"]
    assert np.array_equal(path.cpu().numpy()[: m + 1], ro["path"])
    c = ctrl.cpu().numpy()
    assert (c[0], c[4], c[5], c[6]) == (ro["L"], m, ro["bonus"], 1)
    assert np.array_equal(dm.k_cache.cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(dm.v_cache.cpu().numpy().view(np.uint16), vc)


def test_qwen05_tree_equals_sequential_on_gpu(sv):
    """On the GPU alone: each node's logits and K/V equal those of the
    single-token steps along its root path."""
    case("qwen0.5b tree vs sequential on gpu")
    cfg, arrays, _ = model_pair("qwen")
    L, N = 1024, 8
    cap = L + N + 8
    kc0, vc0 = sg.kv_prefix(22, cfg, L, cap)
    parent = sg.random_tree_parents(sg.stream_key(22, sg.TID_PARENT), N)
    token = sg.tokens(sg.stream_key(22, sg.TID_TOKEN), N, cfg["vocab"])
    dm = sv.DeviceModel(arrays, cfg, cap, kc0, vc0)
    ctrl = sv.new_ctrl(L, N, 10 ** 6)
    ctrl[3] = 0
    # forward only: compare logits of every node before acceptance moves rows
    tree_logits, _, _ = dm.tree_step(ctrl, dev_i32(parent), dev_i32(token), N)
    tree_logits = tree_logits.cpu().numpy()
    for i in range(N):
        chain = [i]
        while chain[-1] != 0:
            chain.append(int(parent[chain[-1]]))
        chain.reverse()
        ds = sv.DeviceModel(arrays, cfg, cap, kc0, vc0) if i == 0 else ds_reset(ds, kc0, vc0)
        for d, node in enumerate(chain):
            c1 = sv.new_ctrl(L + d, 1, 10 ** 6)
            lg, _, _ = ds.tree_step(c1, dev_i32([-1]), dev_i32([token[node]]), 1)
        torch.cuda.synchronize()
        assert lg.cpu().numpy()[0].tobytes() == tree_logits[i].tobytes(), f"node {i}"


def ds_reset(ds, kc0, vc0):
    ds.k_cache.copy_(torch.from_numpy(kc0.view(np.int16)))
    ds.v_cache.copy_(torch.from_numpy(vc0.view(np.int16)))
    return ds


def test_step_is_run_to_run_identical(sv):
    case("tiny step determinism")
    cfg, arrays, _ = model_pair("tiny")
    L, N, cap = 400, 16, 430
    kc0, vc0 = sg.kv_prefix(31, cfg, L, cap)
    parent = sg.random_tree_parents(sg.stream_key(31, sg.TID_PARENT), N)
    token = sg.tokens(sg.stream_key(31, sg.TID_TOKEN), N, cfg["vocab"])
    outs = []
    for _ in range(2):
        dm = sv.DeviceModel(arrays, cfg, cap, kc0, vc0)
        ctrl = sv.new_ctrl(L, N, cap - N)
        lg, _, _ = dm.tree_step(ctrl, dev_i32(parent), dev_i32(token), N)
        outs.append((lg.cpu().numpy().tobytes(), dm.k_cache.cpu().numpy().tobytes(), ctrl.cpu().numpy().tobytes()))
    assert outs[0] == outs[1]


def test_done_step_leaves_state(sv):
    case("tiny step with done set")
    cfg, arrays, _ = model_pair("tiny")
    L, N, cap = 60, 4, 80
    kc0, vc0 = sg.kv_prefix(32, cfg, L, cap)
    dm = sv.DeviceModel(arrays, cfg, cap, kc0, vc0)
    ctrl = sv.new_ctrl(L, N, cap - N)
    ctrl[3] = 1
    before = ctrl.cpu().numpy().copy()
    dm.tree_step(ctrl, dev_i32([-1, 0, 1, 1]), dev_i32([1, 2, 3, 4]), N)
    torch.cuda.synchronize()
    before[4] = 0
    assert list(ctrl.cpu().numpy()) == list(before)
    assert np.array_equal(dm.k_cache.cpu().numpy().view(np.uint16), kc0)
    assert np.array_equal(dm.v_cache.cpu().numpy().view(np.uint16), vc0)

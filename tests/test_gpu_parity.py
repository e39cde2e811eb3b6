"""GPU parity: every call of the C ABI against the CPU oracle, bit for bit.

Inputs come from synthgen with the configs' shapes and distributions: int4
codes uniform in [-8, 7], fp16 scales U(0.005, 0.02), fp32 N(0,1)
activations. Small and ragged shapes are compared element by element; the
full-size lm_head shapes are compared on sampled rows the oracle computes one
by one, plus properties that hold at any size (rows of T equal single-token
calls, run-to-run identity).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

pytestmark = pytest.mark.gpu

QWEN = {"q": (896, 896), "k": (128, 896), "v": (128, 896), "o": (896, 896),
        "gate": (4864, 896), "up": (4864, 896), "down": (896, 4864), "lm_head": (151936, 896)}
LLAMA = {"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
         "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336), "lm_head": (128256, 4096)}


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_verification_amd as m
    return m


def case(msg):
    print(f"\n[case] {msg}", flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def packed(wq: np.ndarray, ws: np.ndarray):
    """Interchange nibbles and scales as generated -> the library's packed
    tile layout (w4a8_pack_weights, on the device)."""
    import speculative_verification_amd as m
    return m.pack_weights(to_dev(wq), to_dev(ws))


@functools.lru_cache(maxsize=2)
def _weights(seed, N, K, layer):
    wq, ws, _ = sg.linear_case(seed, 1, N, K, layer=layer)
    return wq, ws, packed(wq, ws)


def gpu_quant_linear(sv, wq, ws, x, w=None):
    xq, xs = sv.quantize_act(to_dev(x))
    y = sv.linear(packed(wq, ws) if w is None else w, xq, xs)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy(), y.cpu().numpy()


def assert_bits(a: np.ndarray, b: np.ndarray, what: str):
    if a.tobytes() != b.tobytes():
        a32, b32 = a.view(np.uint32).ravel(), b.view(np.uint32).ravel()
        bad = np.nonzero(a32 != b32)[0]
        i = bad[0]
        rel = np.max(np.abs(a.ravel()[bad] - b.ravel()[bad]) / np.maximum(np.abs(b.ravel()[bad]), 1e-30))
        raise AssertionError(f"{what}: {bad.size} of {a32.size} differ; first at {i}: "
                             f"{a.ravel()[i]!r} vs {b.ravel()[i]!r}; max rel diff {rel:.3g}")


# ------------------------------------------------------------------ quantisation

@pytest.mark.parametrize("N,K", [(1, 32), (17, 64), (300, 896), (4096, 14336), (151936, 896)])
def test_pack_layout(sv, N, K):
    """w4a8_pack_weights moves every byte where the packed tile layout puts
    it: row 16t + r, group g at chunk (t*G + g)*16 + r, zero padding rows."""
    case(f"pack N={N} K={K}")
    wq, ws, _ = sg.linear_case(3, 1, N, K)
    w = packed(wq, ws)
    rows, G = (N + 15) // 16 * 16, K // 32
    wpad = np.zeros((rows, K // 2), np.uint8)
    wpad[:N] = wq
    spad = np.zeros((rows, G), np.uint16)
    spad[:N] = ws
    want_w = wpad.reshape(rows // 16, 16, G, 16).transpose(0, 2, 1, 3).reshape(-1)
    want_s = spad.reshape(rows // 16, 16, G).transpose(0, 2, 1).reshape(-1)
    assert np.array_equal(w.wp.cpu().numpy(), want_w)
    assert np.array_equal(w.sp.cpu().numpy().view(np.uint16), want_s)


@pytest.mark.parametrize("T,K", [(1, 896), (8, 896), (3, 4864), (16, 4096), (8, 14336), (2, 33), (5, 1),
                                 (64, 96), (3, 16388), (4, 1024), (2, 2048)])
def test_quantize_parity(sv, T, K):
    case(f"quantize T={T} K={K}")
    x = sg.normal_f32(sg.stream_key(40 + T, sg.TID_X), T * K).reshape(T, K)
    if T >= 2:
        x[1] = 0.0
        x[1, ::3] = -0.0
    if T >= 3:
        x[2] *= np.float32(1e-39)     # subnormal inputs: 127/absmax overflows binary32
    if T >= 4:
        # absmax 2^-130 with zeros, +-absmax/2 (ties), 3/4 and -1/4 of it
        tiny = np.array([2.0 ** -130, 0.0, -2.0 ** -131, 2.0 ** -131, 1.5 * 2.0 ** -131, -2.0 ** -132], np.float32)
        x[3] = np.resize(tiny, K)
    xq_o, xs_o = oracle.quantize_act(x)
    xq, xs = sv.quantize_act(to_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert_bits(xs.cpu().numpy(), xs_o, "xs")


def test_quantize_misaligned_rows(sv):
    """Rows that start off a 16-byte boundary take the scalar kernel."""
    case("quantize misaligned x")
    T, K = 4, 896
    x = sg.normal_f32(sg.stream_key(45, sg.TID_X), T * K + 1)
    xq_o, xs_o = oracle.quantize_act(x[1:].reshape(T, K).copy())
    xd = to_dev(x)[1:].view(T, K)
    assert xd.data_ptr() % 16 != 0
    xq, xs = sv.quantize_act(xd)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert_bits(xs.cpu().numpy(), xs_o, "xs")


# ------------------------------------------------------------------ linear, small and ragged

@pytest.mark.parametrize("T,N,K", [(1, 16, 32), (3, 17, 64), (5, 33, 96), (7, 40, 544), (8, 100, 896),
                                   (16, 50, 4864), (4, 1, 4096), (2, 15, 14336), (9, 31, 512),
                                   (12, 64, 1024), (6, 48, 160), (16, 130, 14336),
                                   # 3 and 5 pipeline stages (3 and 5 iterations per tile), and 7
                                   # iterations (padded to two blocks of 4)
                                   (4, 70, 1280), (16, 33, 1536), (3, 40, 2560), (5, 45, 3200),
                                   # K split in 2 (>= 256 row groups) and unsplit (>= 1024)
                                   (3, 16400, 96), (8, 16385, 544), (5, 65601, 64), (16, 65600, 160),
                                   # several 16-row tiles per workgroup, ragged rows and groups
                                   (8, 4100, 4864), (16, 4097, 8192), (1, 4111, 96), (2, 8211, 1056),
                                   # the 32-token bucket (17..32 tokens): dense products with 1, 2, 3
                                   # (padded to 4), 8 (ragged groups), 9 (padded to 10) and 10
                                   # iterations per tile, more tiles than workgroups; 11..28
                                   # iterations with the activations streamed through LDS (11 and
                                   # 16 padded to 16, 19 with ragged groups and 28 padded to 28,
                                   # one and two tiles per workgroup); past 28 iterations the
                                   # block-diagonal form
                                   (20, 33, 896), (32, 100, 544), (25, 4100, 96), (17, 16, 32),
                                   (18, 50, 1536), (31, 300, 4352), (30, 77, 5120), (32, 4117, 4064),
                                   (24, 70, 5152), (29, 8211, 2048), (32, 17, 4096),
                                   (19, 300, 8192), (27, 33, 9248), (32, 40, 14336), (17, 4100, 12288),
                                   (21, 20, 14368), (1, 900, 4864), (6, 4090, 4864), (8, 33, 4864)])
def test_linear_parity_ragged(sv, T, N, K):
    case(f"linear ragged T={T} N={N} K={K}")
    wq, ws, x = sg.linear_case(50 + T, T, N, K)
    xq_o, xs_o = oracle.quantize_act(x)
    y_o = oracle.w4a8_linear(wq, ws, xq_o, xs_o)
    xq, xs, y = gpu_quant_linear(sv, wq, ws, x)
    assert np.array_equal(xq, xq_o)
    assert_bits(y, y_o, f"y T={T} N={N} K={K}")


def test_linear_config1(sv):
    """Single linear K = N = 896, T = 1, seed 0."""
    case("linear config1 896x896 T=1 seed 0")
    wq, ws, x = sg.linear_case(0, 1, 896, 896)
    xq_o, xs_o = oracle.quantize_act(x)
    y_o = oracle.w4a8_linear(wq, ws, xq_o, xs_o)
    _, _, y = gpu_quant_linear(sv, wq, ws, x)
    assert_bits(y, y_o, "config1")


def _sample_rows(N, seed, n=96):
    r = (sg.u32(sg.stream_key(seed, 77), n) % np.uint32(N)).astype(np.int32)
    return np.unique(np.concatenate([r, [0, 1, 15, 16, N // 2, N - 17, N - 16, N - 1]]).astype(np.int32))


@pytest.mark.parametrize("T", [1, 2, 4, 8])
@pytest.mark.parametrize("name", list(QWEN))
def test_linear_qwen_shapes(sv, name, T):
    N, K = QWEN[name]
    for seed in ((0, 1, 2, 3) if T == 8 else (0,)):
        case(f"linear qwen {name} N={N} K={K} T={T} seed={seed}")
        wq, ws, w = _weights(seed, N, K, list(QWEN).index(name))
        _, _, x = sg.linear_case(seed, T, 1, K, layer=list(QWEN).index(name))
        xq_o, xs_o = oracle.quantize_act(x)
        _, _, y = gpu_quant_linear(sv, wq, ws, x, w)
        if N * K <= 896 * 4864:
            assert_bits(y, oracle.w4a8_linear(wq, ws, xq_o, xs_o), f"{name} T={T} seed={seed}")
        else:
            rows = _sample_rows(N, seed)
            assert_bits(y[:, rows].copy(), oracle.w4a8_linear_rows(wq, ws, xq_o, xs_o, rows),
                        f"{name} T={T} seed={seed} sampled")


@pytest.mark.parametrize("T", [1, 2, 4, 8, 17, 32])
@pytest.mark.parametrize("name", list(LLAMA))
def test_linear_llama_shapes_sampled(sv, name, T):
    N, K = LLAMA[name]
    seed = 0
    case(f"linear llama {name} N={N} K={K} T={T}")
    wq, ws, w = _weights(seed, N, K, 100 + list(LLAMA).index(name))
    _, _, x = sg.linear_case(seed, T, 1, K, layer=100 + list(LLAMA).index(name))
    xq_o, xs_o = oracle.quantize_act(x)
    _, _, y = gpu_quant_linear(sv, wq, ws, x, w)
    rows = _sample_rows(N, seed, n=48)
    assert_bits(y[:, rows].copy(), oracle.w4a8_linear_rows(wq, ws, xq_o, xs_o, rows), f"{name} T={T}")


def test_linear_rows_of_T_equal_single_token(sv):
    """Property at full size: row t of a T-token call equals a 1-token call
    on token t, for every T bucket, on the 8B-shaped q projection."""
    N, K = LLAMA["q"]
    wq, ws, x = sg.linear_case(7, 16, N, K)
    w = packed(wq, ws)
    xq, xs = sv.quantize_act(to_dev(x))
    singles = [sv.linear(w, xq[t:t + 1].contiguous(), xs[t:t + 1].contiguous()) for t in range(16)]
    single = torch.cat(singles, 0).cpu().numpy()
    for T in range(1, 17):
        case(f"rows-of-T T={T}")
        yT = sv.linear(w, xq[:T].contiguous(), xs[:T].contiguous()).cpu().numpy()
        assert_bits(yT, single[:T].copy(), f"T={T} vs single-token")


def test_linear_run_to_run_identical(sv):
    case("determinism lm_head qwen T=8")
    N, K = QWEN["lm_head"]
    wq, ws, x = sg.linear_case(8, 8, N, K)
    w = packed(wq, ws)
    xq, xs = sv.quantize_act(to_dev(x))
    a = sv.linear(w, xq, xs).cpu().numpy()
    b = sv.linear(w, xq, xs).cpu().numpy()
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("T,N,K", [(16, 16400, 10240), (16, 4096, 14336), (8, 4096, 14336), (8, 28672, 4096),
                                   (8, 6144, 4096), (32, 4096, 14336), (24, 9728, 4864), (32, 28672, 4096),
                                   (17, 5000, 896), (32, 8211, 10240), (26, 4097, 14336)])
def test_linear_layouts_sampled(sv, T, N, K):
    """Activations kept in LDS across a workgroup's tiles, and reloaded with
    every tile when T x K does not fit (T = 16 at K = 14336 or 10240, and
    the 32-token bucket at K = 4864 and 14336), on sampled rows."""
    case(f"linear layout T={T} N={N} K={K}")
    wq, ws, x = sg.linear_case(11, T, N, K)
    xq_o, xs_o = oracle.quantize_act(x)
    _, _, y = gpu_quant_linear(sv, wq, ws, x)
    rows = _sample_rows(N, 11, n=40)
    assert_bits(y[:, rows].copy(), oracle.w4a8_linear_rows(wq, ws, xq_o, xs_o, rows), f"T={T} N={N} K={K}")


@pytest.mark.parametrize("T,N,K", [(1, 48, 1 << 20), (8, 48, 1 << 20), (2, (1 << 24) - 16, 32),
                                   (32, 48, 1 << 20), (32, (1 << 24) - 16, 32)])
def test_linear_maximum_sizes(sv, T, N, K):
    """The ABI's limits: K = 2^20 (the reloading layout, 2048 iterations per
    wave), every row against the oracle; N = 2^24 - 16 rows (a million
    tiles over the grid; at 32 tokens the dense kernel's workgroups walk
    about 4096 tiles each), on sampled rows and the last tile's rows."""
    case(f"linear maximum sizes T={T} N={N} K={K}")
    wq, ws, x = sg.linear_case(13, T, N, K)
    xq_o, xs_o = oracle.quantize_act(x)
    _, _, y = gpu_quant_linear(sv, wq, ws, x)
    if N <= 64:
        assert_bits(y, oracle.w4a8_linear(wq, ws, xq_o, xs_o), f"T={T} N={N} K={K}")
    else:
        rows = np.concatenate([_sample_rows(N, 13, n=64), np.arange(N - 16, N, dtype=np.int32)])
        assert_bits(y[:, rows].copy(), oracle.w4a8_linear_rows(wq, ws, xq_o, xs_o, rows), f"T={T} N={N} K={K}")


@pytest.mark.parametrize("T,N,K", [(16, 4096, 14336), (16, 16400, 10240), (8, 128256, 896), (32, 8000, 4096)])
def test_linear_repeated_and_interleaved_calls(sv, T, N, K):
    """Calls of other shapes in between leave a shape's result unchanged."""
    case(f"repeated calls T={T} N={N} K={K}")
    wq, ws, x = sg.linear_case(10, T, N, K)
    w = packed(wq, ws)
    xq, xs = sv.quantize_act(to_dev(x))
    first = sv.linear(w, xq, xs).cpu().numpy()
    for T2 in (1, 5, 16, 27):
        T2 = min(T2, T)
        sv.linear(w.rows(N // 32 * 16), xq[:T2].contiguous(),
                  xs[:T2].contiguous())
        again = sv.linear(w, xq, xs).cpu().numpy()
        assert again.tobytes() == first.tobytes()
    rows = _sample_rows(N, 10, n=32)
    xq_o, xs_o = oracle.quantize_act(x)
    assert_bits(first[:, rows].copy(), oracle.w4a8_linear_rows(wq, ws, xq_o, xs_o, rows), "repeat sampled")


def test_linear_32_bucket_rows_equal_single_token(sv):
    """Tokens 17..32 run in the 32-token kernel: every row still equals the
    1-token call on its token (8B-shaped q projection)."""
    N, K = LLAMA["q"]
    wq, ws, x = sg.linear_case(12, 32, N, K)
    w = packed(wq, ws)
    xq, xs = sv.quantize_act(to_dev(x))
    single = torch.cat([sv.linear(w, xq[t:t + 1].contiguous(), xs[t:t + 1].contiguous())
                        for t in range(32)], 0).cpu().numpy()
    for T in (17, 20, 31, 32):
        case(f"32-token bucket T={T}")
        yT = sv.linear(w, xq[:T].contiguous(), xs[:T].contiguous()).cpu().numpy()
        assert_bits(yT, single[:T].copy(), f"T={T} vs single-token")


# ------------------------------------------------------------------ per-block activation scales

@pytest.mark.parametrize("T,K", [(1, 32), (3, 896), (8, 4096), (16, 14336), (32, 4864), (5, 96)])
def test_quantize_blocks_parity(sv, T, K):
    case(f"quantize blocks T={T} K={K}")
    x = sg.normal_f32(sg.stream_key(60 + T, sg.TID_X), T * K).reshape(T, K)
    x[0, :32] = 0.0                                  # an all-zero block
    if K >= 96:
        x[-1, 64:96] *= np.float32(1e-30)            # a block of tiny values
        x[0, 32:64] *= np.float32(1e-39)             # subnormals: 127/absmax overflows binary32
    xq, xs = sv.quantize_act_blocks(to_dev(x))
    torch.cuda.synchronize()
    xq_o, xs_o = oracle.quantize_act_blocks(x)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert_bits(xs.cpu().numpy(), xs_o, "xs blocks")


@pytest.mark.parametrize("T,N,K", [(1, 16, 32), (3, 17, 64), (8, 100, 896), (16, 50, 4864), (2, 15, 14336),
                                   (7, 4111, 96), (12, 64, 1024), (32, 40, 544), (20, 33, 896),
                                   (16, 130, 14336), (32, 50, 4864)])
def test_linear_blocks_parity(sv, T, N, K):
    case(f"linear blocks T={T} N={N} K={K}")
    wq, ws, x = sg.linear_case(80 + T, T, N, K)
    xq, xs = sv.quantize_act_blocks(to_dev(x))
    y = sv.linear_blocks(packed(wq, ws), xq, xs)
    torch.cuda.synchronize()
    xq_o, xs_o = oracle.quantize_act_blocks(x)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert_bits(y.cpu().numpy(), oracle.w4a8_linear_blocks(wq, ws, xq_o, xs_o), f"blocks T={T} N={N} K={K}")


@pytest.mark.parametrize("T", [1, 8, 16, 32])
@pytest.mark.parametrize("name", ["q", "gate", "down", "lm_head"])
def test_linear_blocks_llama_sampled(sv, name, T):
    N, K = LLAMA[name]
    case(f"linear blocks llama {name} N={N} K={K} T={T}")
    wq, ws, w = _weights(0, N, K, 100 + list(LLAMA).index(name))
    _, _, x = sg.linear_case(0, T, 1, K, layer=200 + list(LLAMA).index(name))
    xq, xs = sv.quantize_act_blocks(to_dev(x))
    y = sv.linear_blocks(w, xq, xs).cpu().numpy()
    xq_o, xs_o = oracle.quantize_act_blocks(x)
    rows = _sample_rows(N, 3, n=32)
    assert_bits(y[:, rows].copy(), oracle.w4a8_linear_blocks(wq[rows], ws[rows], xq_o, xs_o), f"{name} T={T}")


@pytest.mark.parametrize("T", [4, 20])
def test_linear_degenerate_values(sv, T):
    """All-zero token, negative and subnormal fp16 scales, tiny activations
    with subnormal outputs, and an empty matrix (at 20 tokens: the dense
    32-token kernel, whose scaled products are one fma each)."""
    case(f"linear degenerate values T={T}")
    N, K = 37, 288
    wq, ws, x = sg.linear_case(9, T, N, K)
    x[0] = 0.0
    x[2] *= np.float32(1e-36)
    ws = ws.copy()
    ws[::3] ^= np.uint16(0x8000)                 # negative scales
    ws[5] = np.uint16(1)                          # smallest subnormal fp16
    ws[6, :2] = np.uint16(0)                      # zero scales
    xq_o, xs_o = oracle.quantize_act(x)
    y_o = oracle.w4a8_linear(wq, ws, xq_o, xs_o)
    _, _, y = gpu_quant_linear(sv, wq, ws, x)
    assert_bits(y, y_o, "degenerate")
    no_rows = sv.Packed(torch.zeros(16, dtype=torch.uint8, device="cuda"),
                        torch.zeros(1, dtype=torch.int16, device="cuda"), 0, 32)
    empty = sv.linear(no_rows, torch.zeros((1, 32), dtype=torch.int8, device="cuda"), torch.ones(1, device="cuda"))
    assert empty.shape == (1, 0)


@pytest.mark.parametrize("T", [1, 4, 7])
def test_linear_nonfinite_scales(sv, T):
    """Below 8 tokens infinite and NaN fp16 scales give the IEEE products of
    the plain definition: inf * d, inf * 0 = NaN, inf + -inf = NaN (from 8
    tokens the scaled products are one fma each, which needs finite
    scales)."""
    case(f"linear non-finite scales T={T}")
    N, K = 40, 544
    wq, ws, x = sg.linear_case(14, T, N, K)
    ws = ws.copy()
    ws[0, 3] = np.uint16(0x7C00)                 # +inf
    ws[1, 0] = np.uint16(0xFC00)                 # -inf
    ws[2, 7] = np.uint16(0x7E00)                 # NaN
    ws[5, 1] = np.uint16(0x7C00)
    ws[5, 9] = np.uint16(0xFC00)                 # +inf and -inf in one row
    ws[33, 16] = np.uint16(0x7C00)               # a later tile, slot 0 of iteration 1
    x[0, :32] = 0.0                              # token 0's group 0 dots are 0: -inf * 0 = NaN
    xq_o, xs_o = oracle.quantize_act(x)
    y_o = oracle.w4a8_linear(wq, ws, xq_o, xs_o)
    _, _, y = gpu_quant_linear(sv, wq, ws, x)
    nan_o, nan_g = np.isnan(y_o), np.isnan(y)
    assert np.array_equal(nan_g, nan_o), f"NaN positions differ: {np.argwhere(nan_g != nan_o)[:4]}"
    assert nan_o.any() and np.isinf(y_o).any()
    assert_bits(np.where(nan_g, 0, y).astype(np.float32), np.where(nan_o, 0, y_o).astype(np.float32), "non-NaN outputs")


# ------------------------------------------------------------------ argmax + acceptance + compaction

def _plant_tree(seed, n, amax_o, V, accept_path):
    """Random topological tree; drafts along a chosen chain equal the parent's
    prediction, the rest are random, so the accepted depth is controlled."""
    key = sg.stream_key(seed, sg.TID_PARENT)
    parent = sg.random_tree_parents(key, n)
    token = sg.tokens(sg.stream_key(seed, sg.TID_TOKEN), n, V)
    if accept_path and n > 1:
        depth = np.zeros(n, np.int32)
        for i in range(1, n):
            depth[i] = depth[parent[i]] + 1
        w = int(np.argmax(depth))
        chain = [w]
        while chain[-1] != 0:
            chain.append(int(parent[chain[-1]]))
        for c in chain[:-1]:
            token[c] = amax_o[parent[c]]
    return parent, token


@pytest.mark.parametrize("V", [151936, 128256, 1000, 1])
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_argmax_accept_compact_parity(sv, V, n):
    for seed, plant in ((n * 7 + V % 97, True), (n * 11 + 1, False)):
        case(f"argmax/accept/compact V={V} n={n} seed={seed} planted={plant}")
        logits = sg.normal_f32(sg.stream_key(seed, sg.TID_LOGITS), n * V).reshape(n, V)
        if V > 10:
            logits[0, V // 3] = logits[0, V // 2] = np.float32(9.0)     # tie: lowest index
            if n > 1:
                logits[1, :] = np.float32(-1.0)
                logits[1, 7] = np.float32(-0.0)
                logits[1, 5] = np.float32(0.0)                           # -0 == +0: index 5
        amax_o = oracle.argmax(logits)
        parent, token = _plant_tree(seed, n, amax_o, V, plant)
        m_o, path_o, bonus_o = oracle.tree_accept(parent, token, amax_o)

        L0, ctx = 1024, 1040
        layers, heads, cap, hd = 24, 2, 1040, 64
        kv = sg.u32(sg.stream_key(seed, sg.TID_KV), 2 * layers * heads * cap * hd).astype(np.uint16)
        kv = kv.reshape(2, layers, heads, cap, hd)
        ctrl = sv.new_ctrl(committed_len=L0, n_nodes=n, ctx_len=ctx, root_token=int(token[0]))
        stats = torch.full((3,), 77, dtype=torch.int32, device="cuda")
        ring = torch.full((5,), -1, dtype=torch.int32, device="cuda")
        ctrl[7] = 3  # ring_head
        amax, path = sv.tree_argmax_accept(to_dev(logits), to_dev(parent), to_dev(token), ctrl,
                                           stats=stats, ring=ring)
        kc, vc = to_dev(kv[0]), to_dev(kv[1])
        sv.kv_compact(kc, vc, path, ctrl)
        torch.cuda.synchronize()

        assert np.array_equal(amax.cpu().numpy(), amax_o)
        assert np.array_equal(path.cpu().numpy()[: m_o + 1], path_o)
        c = ctrl.cpu().numpy()
        L1 = L0 + m_o + 1
        assert list(c) == [L1, n, ctx, int(L1 + n > ctx), m_o, bonus_o, 1, 3 + m_o + 1]
        assert list(stats.cpu().numpy()) == [m_o, 77, n]
        emitted = [int(token[p]) for p in path_o[1:]] + [bonus_o]
        ring_o = [-1] * 5
        for i, tkn in enumerate(emitted):
            ring_o[(3 + i) % 5] = tkn
        assert list(ring.cpu().numpy()) == ring_o
        for i, t in enumerate((kc, vc)):
            ref = kv[i].copy()
            oracle.kv_compact(ref, L0, path_o, m_o)
            got = t.cpu().numpy().view(np.uint16)
            assert np.array_equal(got[:, :, :L1], ref[:, :, :L1])


def test_done_step_is_noop(sv):
    """With done set on entry, acceptance writes only accept_len = 0 and a
    no-op statistics record, and compaction then moves nothing."""
    case("done flag no-op")
    n, V = 8, 4096
    logits = sg.normal_f32(sg.stream_key(3, sg.TID_LOGITS), n * V).reshape(n, V)
    parent = sg.random_tree_parents(sg.stream_key(3, sg.TID_PARENT), n)
    token = sg.tokens(sg.stream_key(3, sg.TID_TOKEN), n, V)
    ctrl = sv.new_ctrl(100, n, 200)
    ctrl[3] = 1
    ctrl[4] = 5
    before = ctrl.cpu().numpy().copy()
    kc = torch.arange(2 * 2 * 200 * 8, dtype=torch.int16, device="cuda").reshape(2, 2, 200, 8)
    vc = kc.clone() + 1
    k0, v0 = kc.clone(), vc.clone()
    stats = torch.zeros(3, dtype=torch.int32, device="cuda")
    _, path = sv.tree_argmax_accept(to_dev(logits), to_dev(parent), to_dev(token), ctrl, stats=stats)
    sv.kv_compact(kc, vc, path, ctrl)
    torch.cuda.synchronize()
    after = ctrl.cpu().numpy()
    before[4] = 0
    assert list(after) == list(before)
    assert list(stats.cpu().numpy()) == [-1, 0, n]
    assert torch.equal(kc, k0) and torch.equal(vc, v0)


def test_context_limit_sets_done(sv):
    case("ctx limit sets done")
    n, V = 4, 64
    logits = np.zeros((n, V), np.float32)
    logits[:, 3] = 1.0
    parent = np.array([-1, 0, 1, 2], np.int32)
    token = np.array([9, 3, 3, 3], np.int32)       # every draft accepted: m = 3
    ctrl = sv.new_ctrl(10, n, 10 + 4 + n - 1)      # after commit: 14 + 4 > 17
    sv.tree_argmax_accept(to_dev(logits), to_dev(parent), to_dev(token), ctrl)
    torch.cuda.synchronize()
    c = ctrl.cpu().numpy()
    assert (c[0], c[3], c[4]) == (14, 1, 3)

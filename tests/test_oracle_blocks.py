"""Pins of the oracle's per-block activation mode (GPU-Resident Speculative
Decoding for In-Browser LLM Inference with WebGPU, Small-Batch Verification
Kernels: activations quantised to 8-bit integers per block of 32 values):
quantisation invariants, bit equality with the per-token mode where the two
must agree (every block's scale the same power of two), an exact-rational
error bound, T-invariance, and that the stated order of the two scale
multiplications is observable."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthgen as sg


def test_quantize_blocks_invariants():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(5, 256)).astype(np.float32) * rng.uniform(0.01, 100, size=(5, 1)).astype(np.float32)
    x[2, 64:96] = 0.0                                  # an all-zero block
    xq, xs = oracle.quantize_act_blocks(x)
    assert xs.shape == (5, 8)
    for t in range(5):
        for g in range(8):
            blk, q, s = x[t, 32 * g:32 * g + 32], xq[t, 32 * g:32 * g + 32], xs[t, g]
            if not blk.any():
                assert s == 0 and not q.any()
                continue
            assert np.abs(q).max() == 127 and s == np.float32(np.abs(blk).max()) / np.float32(127)
            err = np.abs(blk.astype(np.float64) - float(s) * q.astype(np.float64))
            assert err.max() <= float(s) / 2 * (1 + 1e-5)
    # blocks are independent: one block changed, the others' codes stay
    y = x.copy()
    y[1, 32:64] *= 3
    yq, ys = oracle.quantize_act_blocks(y)
    keep = np.ones(256, bool)
    keep[32:64] = False
    assert np.array_equal(yq[1, keep], xq[1, keep]) and np.array_equal(np.delete(ys[1], 1), np.delete(xs[1], 1))


def test_quantize_blocks_equals_per_token_on_one_block():
    x = np.random.default_rng(2).normal(size=(3, 32)).astype(np.float32)
    q1, s1 = oracle.quantize_act_blocks(x)
    q2, s2 = oracle.quantize_act(x)
    assert np.array_equal(q1, q2) and np.array_equal(s1[:, 0], s2)


@pytest.mark.parametrize("K", [32, 96, 4096])
def test_linear_blocks_equals_per_token_at_equal_power_of_two_scales(K):
    """Every block's absmax is 127 * 2^e, so every block scale is exactly 2^e.
    Scaling by a power of two commutes with rounding, so the per-block sum
    equals 2^e times R16 of the unscaled products, which is the per-token
    result bit for bit."""
    T, N = 3, 40
    wq, ws, x = sg.linear_case(8, T, N, K)
    x = np.clip(x, -100, 100)
    for t in range(T):
        e = [-3, 0, 5][t]
        x[t, ::32] = np.float32(127 * 2.0 ** e)      # the largest value of each block
        x[t] = np.where(np.arange(K) % 32 == 0, x[t], np.clip(x[t], -127 * 2.0 ** e, 127 * 2.0 ** e))
    xqb, xsb = oracle.quantize_act_blocks(x)
    xqt, xst = oracle.quantize_act(x)
    assert np.array_equal(xqb, xqt)
    assert np.array_equal(xsb, np.repeat(xst[:, None], K // 32, axis=1))
    yb = oracle.w4a8_linear_blocks(wq, ws, xqb, xsb)
    yt = oracle.w4a8_linear(wq, ws, xqt, xst)
    assert yb.tobytes() == yt.tobytes()


def test_linear_blocks_error_bound():
    """Against the exact rational value: two roundings per product and the
    fixed-order sum's depth bound the error."""
    T, N, K = 2, 12, 1024
    wq, ws, x = sg.linear_case(9, T, N, K)
    xq, xs = oracle.quantize_act_blocks(x)
    y = oracle.w4a8_linear_blocks(wq, ws, xq, xs)
    d = oracle.group_dots(wq, xq)                     # exact integers [T][N][G]
    G = K // 32
    u = 2.0 ** -24
    depth = 2 + (G + 15) // 16 + 4
    gam = depth * u / (1 - depth * u)
    for t in range(T):
        for n in range(N):
            terms = [Fraction(oracle.f16_to_f32(int(ws[n, g]))) * Fraction(float(xs[t, g])) * int(d[t, n, g])
                     for g in range(G)]
            exact = sum(terms)
            mag = sum(abs(v) for v in terms)
            assert abs(Fraction(float(y[t, n])) - exact) <= Fraction(gam) * mag


def test_linear_blocks_t_invariance():
    wq, ws, x = sg.linear_case(10, 8, 50, 896)
    xq, xs = oracle.quantize_act_blocks(x)
    y8 = oracle.w4a8_linear_blocks(wq, ws, xq, xs)
    for t in range(8):
        y1 = oracle.w4a8_linear_blocks(wq, ws, xq[t:t + 1], xs[t:t + 1])
        assert y1.tobytes() == y8[t:t + 1].tobytes()


def test_scale_order_is_observable():
    """fl(fl(w * a) * d) and fl(w * fl(a * d)) differ for some inputs, so the
    stated order is a real choice that the kernel must follow."""
    rng = np.random.default_rng(3)
    w = rng.uniform(0.005, 0.02, 20000).astype(np.float16).astype(np.float32)
    a = rng.uniform(1e-3, 1e-1, 20000).astype(np.float32)
    d = rng.integers(-30000, 30000, 20000).astype(np.float32)
    first = (w * a) * d
    other = w * (a * d)
    assert (first != other).any()

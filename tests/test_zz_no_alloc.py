"""The no-allocation entry point (w4a8_linear_argmax_T_noalloc) against the
workspace entry point it varies (w4a8_linear_argmax_T), through the C ABI:
the same predictions and output bits on two calls in a row, the second with
a smaller input, so the static scratch keeps the first call's pairs when the
second starts. Collected last (the file name), so that it also runs after
every other GPU test in one process."""
import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"\n[case] {msg}", flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_verification_amd as m
    return m


def _inputs(sv, seed, T, N, K):
    wq, ws, x = sg.linear_case(seed, T, N, K)
    xq, xs = oracle.quantize_act(x)
    return sv.pack_weights(to_dev(wq), to_dev(ws)), to_dev(xq), to_dev(xs)


@pytest.mark.parametrize("first,second", [((16, 151936, 896), (8, 4096, 4096)),
                                          ((8, 128256, 4096), (1, 896, 896)),
                                          ((5, 16385, 128), (3, 17, 64))])
def test_noalloc_equals_workspace_entry(sv, first, second):
    for i, (T, N, K) in enumerate((first, second)):
        case(f"noalloc call {i}: T={T} N={N} K={K}")
        w, xq, xs = _inputs(sv, 300 + 7 * i + T, T, N, K)
        y_ref = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        a_ref = sv.linear_argmax(w, xq, xs, y=y_ref)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        a = torch.full((T,), -1, dtype=torch.int32, device="cuda")
        sv.linear_argmax_noalloc(w, xq, xs, a, y=y)
        a2 = torch.full((T,), -1, dtype=torch.int32, device="cuda")
        sv.linear_argmax_noalloc(w, xq, xs, a2)          # outputs not written
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), a_ref.cpu().numpy())
        assert np.array_equal(a2.cpu().numpy(), a_ref.cpu().numpy())
        assert y.cpu().numpy().tobytes() == y_ref.cpu().numpy().tobytes()

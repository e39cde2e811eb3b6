"""The C ABI on the host: every declared symbol is exported, struct layouts
match their documented sizes, and invalid arguments return the documented
negative status before anything is enqueued (these calls never reach the
HIP runtime, so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specv.h")

OK, E_INVAL, E_SHAPE, E_ALIGN, E_HIP, E_WORKSPACE = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    from speculative_verification_amd._lib import LIB
    return LIB


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"w4a8_quantize_act", "w4a8_linear_T", "tree_argmax_accept", "kv_compact"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    from speculative_verification_amd._lib import SIGNATURES
    assert set(SIGNATURES) == set(names)


def test_struct_sizes(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "specv.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(specv_ctrl), sizeof(specv_step_stats),'
                   ' offsetof(specv_ctrl, ring_head), sizeof(specv_model), offsetof(specv_model, w_qkv),'
                   ' sizeof(specv_drafter), offsetof(specv_drafter, draws), offsetof(specv_drafter, accept_threshold));'
                   ' return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    import ctypes
    from speculative_verification_amd._lib import SpecvDrafter, SpecvModel
    assert out == ["32", "12", "28", str(ctypes.sizeof(SpecvModel)), str(SpecvModel.w_qkv.offset),
                   "32", str(SpecvDrafter.draws.offset), str(SpecvDrafter.accept_threshold.offset)]


def test_status_strings(lib):
    for s in (OK, E_INVAL, E_SHAPE, E_ALIGN, E_HIP, E_WORKSPACE, 99):
        assert lib.specv_status_string(s)


A = 0x10000  # a fake, 64 KiB-aligned address: validation never dereferences it


def test_linear_rejects_bad_arguments(lib):
    for f, args in ((lib.w4a8_linear_T, lambda *a: a + (A, 1 << 30, None)),
                    (lib.w4a8_linear_blocks_T, lambda *a: a + (None,))):
        assert f(*args(A, A, A, A, A, 1, 16, 33)) == E_SHAPE        # K not a multiple of 32
        assert f(*args(A, A, A, A, A, 0, 16, 64)) == E_SHAPE        # T < 1
        assert f(*args(A, A, A, A, A, 33, 16, 64)) == E_SHAPE       # T > 32
        assert f(*args(A, A, A, A, A, 1, -1, 64)) == E_SHAPE
        assert f(*args(A, A, A, A, A, 1, 1 << 22, 1024)) == E_SHAPE  # weights >= 2 GiB
        assert f(*args(None, A, A, A, A, 1, 16, 64)) == E_INVAL
        assert f(*args(A, A, A, A, None, 1, 16, 64)) == E_INVAL
        assert f(*args(A + 8, A, A, A, A, 1, 16, 64)) == E_ALIGN     # wq not 16-byte aligned
        assert f(*args(A, A, A + 4, A, A, 1, 16, 64)) == E_ALIGN     # xq not 16-byte aligned
        assert f(*args(A, A + 1, A, A, A, 1, 16, 64)) == E_ALIGN
        assert f(*args(None, None, None, None, None, 1, 0, 64)) == OK  # N == 0: nothing to do
        assert f(*args(None, None, None, None, None, 32, 0, 64)) == OK
    # no layout needs a workspace
    for T, N, K in ((8, 4096, 4096), (16, 4096, 14336), (32, 28672, 4096), (1, 16, 64)):
        assert lib.w4a8_linear_workspace(T, N, K) == 0


def test_pack_sizes_and_bad_arguments(lib):
    # rows padded to whole 16-row tiles; 16 bytes and one fp16 scale per row and group
    for N, K in ((1, 32), (16, 64), (17, 896), (151936, 896), (128256, 4096), (4096, 14336)):
        rows = (N + 15) // 16 * 16
        assert lib.w4a8_packed_weight_bytes(N, K) == rows * K // 2
        assert lib.w4a8_packed_scale_bytes(N, K) == rows * (K // 32) * 2
    for N, K in ((0, 64), (16, 48), (16, 0), (1 << 22, 1024), (-1, 64)):
        assert lib.w4a8_packed_weight_bytes(N, K) == 0 and lib.w4a8_packed_scale_bytes(N, K) == 0
    f = lib.w4a8_pack_weights
    assert f(A, A, 16, 48, A, A, None) == E_SHAPE
    assert f(A, A, 0, 64, A, A, None) == E_SHAPE
    assert f(A, A, 1 << 22, 1024, A, A, None) == E_SHAPE         # packed weights >= 2 GiB
    assert f(None, A, 16, 64, A, A, None) == E_INVAL
    assert f(A, A, 16, 64, A, None, None) == E_INVAL
    assert f(A + 8, A, 16, 64, A, A, None) == E_ALIGN
    assert f(A, A, 16, 64, A + 8, A, None) == E_ALIGN
    assert f(A, A + 1, 16, 64, A, A, None) == E_ALIGN


def test_quantize_blocks_rejects_bad_arguments(lib):
    f = lib.w4a8_quantize_act_blocks
    assert f(A, 2, 48, A, A, None) == E_SHAPE                     # K not a multiple of 32
    assert f(A, -1, 64, A, A, None) == E_SHAPE
    assert f(A, 1 << 20, 1 << 12, A, A, None) == E_SHAPE          # T*K >= 2^31
    assert f(None, 2, 64, A, A, None) == E_INVAL
    assert f(A, 2, 64, A, None, None) == E_INVAL
    assert f(A + 4, 2, 64, A, A, None) == E_ALIGN                 # x not 16-byte aligned
    assert f(A, 2, 64, A + 2, A, None) == E_ALIGN
    assert f(None, 0, 64, None, None, None) == OK


def test_time_next_linear_arguments(lib):
    assert lib.specv_time_next_linear(A, None) == E_INVAL
    assert lib.specv_time_next_linear(None, A) == E_INVAL
    assert lib.specv_time_next_linear(None, None) == OK


def test_stream_read_arguments(lib):
    f = lib.specv_stream_read
    assert f(A, 1 << 20, A, 0, None) == E_INVAL            # grid < 1
    assert f(A, 1 << 20, A, 65537, None) == E_INVAL
    assert f(A, 24, A, 512, None) == E_INVAL                # not a multiple of 16
    assert f(None, 32, A, 512, None) == E_INVAL
    assert f(A, 32, None, 512, None) == E_INVAL
    assert f(A + 8, 32, A, 512, None) == E_ALIGN
    assert f(A, 32, A + 2, 512, None) == E_ALIGN


def test_quantize_rejects_bad_arguments(lib):
    f = lib.w4a8_quantize_act
    assert f(A, 0, 64, A, A, None) == OK                      # T == 0: nothing to do
    assert f(A, 1, 0, A, A, None) == E_SHAPE
    assert f(A, (1 << 20) + 1, 64, A, A, None) == E_SHAPE
    assert f(None, 1, 64, A, A, None) == E_INVAL
    assert f(A + 2, 1, 64, A, A, None) == E_ALIGN


def test_accept_rejects_bad_arguments(lib):
    f = lib.tree_argmax_accept
    need = lib.tree_argmax_accept_workspace(151936, 8)
    assert need == 8 * 38 * 8
    assert f(A, 151936, 17, A, A, A, A, A, None, None, 0, A, need, None) == E_SHAPE
    assert f(A, 0, 8, A, A, A, A, A, None, None, 0, A, need, None) == E_SHAPE
    assert f(A, 151936, 8, None, A, A, A, A, None, None, 0, A, need, None) == E_INVAL
    assert f(A, 151936, 8, A, A, A, A, A, None, A, 0, A, need, None) == E_INVAL   # ring without capacity
    assert f(A, 151936, 8, A, A, A, A, A, None, None, 0, A, need - 1, None) == E_WORKSPACE
    assert f(A, 151936, 8, A, A, A, A, A, None, None, 0, None, need, None) == E_WORKSPACE
    assert f(A + 4, 151936, 8, A, A, A, A, A, None, None, 0, A, need, None) == E_ALIGN


def test_compact_rejects_bad_arguments(lib):
    f = lib.kv_compact
    assert f(A, A, 24, 2, 1040, 12, A, A, None) == E_SHAPE    # head_dim not a multiple of 8
    assert f(A, A, 0, 2, 1040, 64, A, A, None) == E_SHAPE
    assert f(A, None, 24, 2, 1040, 64, A, A, None) == E_INVAL
    assert f(A + 8, A, 24, 2, 1040, 64, A, A, None) == E_ALIGN


def test_rope_table_matches_oracle(lib, orc):
    """The library's host rotary table and the oracle's are written
    separately; both evaluate the angle in double with libm, so they agree
    bit for bit."""
    import numpy as np
    c = np.empty((700, 32), np.float32)
    s_ = np.empty((700, 32), np.float32)
    assert lib.specv_rope_table(c.ctypes.data, s_.ctypes.data, 700, 64, 1e6) == OK
    oc, os_ = orc.rope_table(700, 64, 1e6)
    assert np.array_equal(c, oc) and np.array_equal(s_, os_)
    assert lib.specv_rope_table(c.ctypes.data, s_.ctypes.data, 700, 63, 1e6) == E_SHAPE


def test_step_rejects_bad_model(lib):
    from speculative_verification_amd._lib import SpecvModel
    import ctypes
    m = SpecvModel()
    assert lib.spec_step_workspace(ctypes.addressof(m), 8) == 0          # all sizes zero
    assert lib.spec_tree_step(ctypes.addressof(m), A, A, A, 8, A, A, A, None, None, 0, A, 1 << 30, None) == E_SHAPE
    assert lib.spec_tree_step(None, A, A, A, 8, A, A, A, None, None, 0, A, 1 << 30, None) == E_INVAL


def fake_model(**over):
    """A specv_model of the tiny shape whose pointers are fake, aligned
    addresses: enough for host validation, never dereferenced."""
    from speculative_verification_amd._lib import SpecvModel
    m = SpecvModel()
    cfg = dict(n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, inter=96, vocab=300, max_pos=640)
    cfg.update(over)
    for k, v in cfg.items():
        setattr(m, k, v)
    m.eps, m.kv_capacity = 1e-6, 600
    for k, _ in SpecvModel._fields_[10:]:
        setattr(m, k, A)
    return m


def test_model_needs_rotary_rows_for_every_position(lib):
    """Every position a step can reach (below kv_capacity) has a rotary table
    row: a model whose max_pos is below its capacity is rejected."""
    ok, short = fake_model(max_pos=600), fake_model(max_pos=599)
    assert lib.spec_step_workspace(ctypes.addressof(ok), 8) > 0
    assert lib.spec_step_workspace(ctypes.addressof(short), 8) == 0


def test_window_rejects_bad_arguments(lib):
    from speculative_verification_amd._lib import SpecvDrafter
    m = fake_model()
    mp = ctypes.addressof(m)
    need = lib.spec_window_workspace(mp, 8)
    assert need == lib.spec_step_workspace(mp, 8) > 0
    d = SpecvDrafter(A, 100, 4, A, 1 << 31, 0)
    dp = ctypes.byref(d)
    f = lib.spec_window_run
    assert f(mp, A, A, None, 0, dp, 0, 4, A, need, None, None) == E_SHAPE        # width < 1
    assert f(mp, A, A, None, 0, dp, 17, 4, A, need, None, None) == E_SHAPE       # width > 16
    assert f(mp, A, A, None, 0, dp, 8, -1, A, need, None, None) == E_SHAPE       # W < 0
    assert f(mp, A, A, None, 0, dp, 8, 4097, A, need, None, None) == E_SHAPE
    assert f(mp, None, A, None, 0, dp, 8, 4, A, need, None, None) == E_INVAL     # no ctrl
    assert f(mp, A, None, None, 0, dp, 8, 4, A, need, None, None) == E_INVAL     # no stats
    assert f(mp, A, A, A, 0, dp, 8, 4, A, need, None, None) == E_INVAL           # ring without capacity
    assert f(mp, A, A, None, 0, None, 8, 4, A, need, None, None) == E_INVAL      # drafter needed
    bad = SpecvDrafter(A, 0, 4, A, 0, 0)
    assert f(mp, A, A, None, 0, ctypes.byref(bad), 8, 4, A, need, None, None) == E_INVAL
    bad = SpecvDrafter(A, 10, 0, A, 0, 0)
    assert f(mp, A, A, None, 0, ctypes.byref(bad), 8, 4, A, need, None, None) == E_INVAL
    assert f(mp, A + 2, A, None, 0, dp, 8, 4, A, need, None, None) == E_ALIGN
    assert f(mp, A, A, None, 0, dp, 8, 4, A, need - 1, None, None) == E_WORKSPACE
    assert f(mp, A, A, None, 0, dp, 8, 4, None, need, None, None) == E_WORKSPACE
    assert f(mp, A, A, None, 0, dp, 8, 4, A + 16, need, None, None) == E_ALIGN
    assert f(mp, A, A, None, 0, dp, 8, 0, A, need, None, None) == OK             # W == 0: nothing to do
    assert f(mp, A, A, None, 0, None, 1, 0, A, lib.spec_window_workspace(mp, 1), None, None) == OK
    assert f(None, A, A, None, 0, dp, 8, 4, A, need, None, None) == E_INVAL
    m1 = fake_model(vocab=1)
    assert f(ctypes.addressof(m1), A, A, None, 0, dp, 8, 4, A, need, None, None) == E_SHAPE
    assert f(ctypes.addressof(m1), A, A, None, 0, None, 1, 0, A, need, None, None) == OK
    m2 = fake_model(head_dim=15)
    assert f(ctypes.addressof(m2), A, A, None, 0, dp, 8, 4, A, need, None, None) == E_SHAPE


def test_linear_argmax_rejects_bad_arguments(lib):
    f = lib.w4a8_linear_argmax_T
    need = lib.w4a8_linear_argmax_workspace(8, 151936, 896)
    # one (value, row) pair per token per workgroup: one workgroup per 16-row
    # tile, capped near two per CU
    chunks = need // (8 * 8)
    assert need == 8 * chunks * 8 and 32 <= chunks <= 151936 // 16
    assert lib.w4a8_linear_argmax_workspace(8, 896, 896) == 8 * 56 * 8   # 56 tiles: 56 workgroups
    assert lib.w4a8_linear_argmax_workspace(16, 4096, 14336) == 16 * 256 * 8   # reloading layout: 256 tiles
    assert lib.w4a8_linear_argmax_workspace(17, 4096, 4096) == 0     # argmax only up to 16 tokens
    assert f(A, A, A, A, None, A, 17, 4096, 4096, A, 1 << 20, None) == E_SHAPE
    assert f(A, A, A, A, None, A, 8, 0, 896, A, need, None) == E_SHAPE   # no rows
    assert f(A, A, A, A, None, A, 0, 896, 896, A, need, None) == E_SHAPE
    assert f(A, A, A, A, None, None, 8, 151936, 896, A, need, None) == E_INVAL
    assert f(None, A, A, A, None, A, 8, 151936, 896, A, need, None) == E_INVAL
    assert f(A, A, A, A, None, A, 8, 151936, 896, A, need - 1, None) == E_WORKSPACE
    assert f(A, A, A, A, None, A, 8, 151936, 896, None, need, None) == E_WORKSPACE
    assert f(A, A, A, A, A + 2, A, 8, 151936, 896, A, need, None) == E_ALIGN
    assert f(A, A, A, A, None, A + 2, 8, 151936, 896, A, need, None) == E_ALIGN
    assert f(A + 8, A, A, A, None, A, 8, 151936, 896, A, need, None) == E_ALIGN


def test_linear_argmax_noalloc_rejects_bad_arguments(lib):
    """The no-allocation variant validates like w4a8_linear_argmax_T, with no
    workspace arguments (no GPU is touched on these paths)."""
    f = lib.w4a8_linear_argmax_T_noalloc
    assert f(A, A, A, A, None, A, 17, 4096, 4096, None) == E_SHAPE      # argmax only up to 16 tokens
    assert f(A, A, A, A, None, A, 0, 896, 896, None) == E_SHAPE
    assert f(A, A, A, A, None, A, 8, 0, 896, None) == E_SHAPE
    assert f(A, A, A, A, None, A, 8, 896, 100, None) == E_SHAPE        # K not a multiple of 32
    assert f(A, A, A, A, None, None, 8, 151936, 896, None) == E_INVAL  # no argmax output
    assert f(None, A, A, A, None, A, 8, 151936, 896, None) == E_INVAL
    assert f(A, A, A, A, A + 2, A, 8, 151936, 896, None) == E_ALIGN
    assert f(A, A, A, A, None, A + 2, 8, 151936, 896, None) == E_ALIGN
    assert f(A + 8, A, A, A, None, A, 8, 151936, 896, None) == E_ALIGN


def test_linear_argmax_accept_rejects_bad_arguments(lib):
    """The lm_head + acceptance entry validates like w4a8_linear_argmax_T and
    tree_accept together (no GPU is touched on these paths)."""
    f = lib.w4a8_linear_argmax_accept_T
    need = lib.w4a8_linear_argmax_workspace(8, 151936, 896)
    ok = (A, A, A, A, 8, 151936, 896, A, A, A, A, A, None, None, 0, A, need, None)

    def call(**kw):
        names = ("wq", "ws", "xq", "xs", "T", "N", "K", "parent", "token", "argmax", "path", "ctrl", "stats",
                 "ring", "ring_cap", "ws_ptr", "ws_bytes", "stream")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    assert call(T=17, N=4096, K=4096) == E_SHAPE      # acceptance takes at most 16 nodes
    assert call(T=0) == E_SHAPE
    assert call(N=0) == E_SHAPE
    assert call(K=100) == E_SHAPE
    assert call(wq=None) == E_INVAL
    assert call(parent=None) == E_INVAL
    assert call(path=None) == E_INVAL
    assert call(ctrl=None) == E_INVAL
    assert call(ring=A, ring_cap=0) == E_INVAL       # ring without capacity
    assert call(ws_bytes=need - 1) == E_WORKSPACE
    assert call(ws_ptr=None) == E_WORKSPACE
    assert call(wq=A + 8) == E_ALIGN
    assert call(argmax=A + 2) == E_ALIGN
    assert call(ws_ptr=A + 4) == E_ALIGN


def test_tree_accept_rejects_bad_arguments(lib):
    f = lib.tree_accept
    assert f(A, 0, A, A, A, A, None, None, 0, None) == E_SHAPE
    assert f(A, 17, A, A, A, A, None, None, 0, None) == E_SHAPE
    assert f(None, 8, A, A, A, A, None, None, 0, None) == E_INVAL
    assert f(A, 8, A, A, A, None, None, None, 0, None) == E_INVAL
    assert f(A, 8, A, A, A, A, None, A, 0, None) == E_INVAL       # ring without capacity
    assert f(A + 2, 8, A, A, A, A, None, None, 0, None) == E_ALIGN


def test_cm_params_layout(tmp_path):
    src = tmp_path / "cm.c"
    src.write_text('#include "specv.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu\\n", sizeof(specv_cm_params), offsetof(specv_cm_params, weight));'
                   ' return 0;}\n')
    exe = tmp_path / "cm"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    from speculative_verification_amd._lib import SpecvCmParams
    assert out == ["48", "12"] == [str(ctypes.sizeof(SpecvCmParams)), str(SpecvCmParams.weight.offset)]


def test_cm_draft_rejects_bad_arguments(lib):
    from speculative_verification_amd._lib import cm_params
    p = cm_params()
    pp = ctypes.byref(p)
    need = lib.cm_draft_workspace(4097, pp)
    assert need == 17 * 16 * 4                     # 17 scan workgroups of 256 positions, 16 keys each
    assert lib.cm_draft_workspace(0, pp) == 0
    for bad in (cm_params(max_order=0), cm_params(max_order=9), cm_params(candidates=33), cm_params(depth=0),
                cm_params(depth=9), cm_params(weight=(0, 0, 1, 1, 1, 1, 1, 1, 1)),
                cm_params(weight=(0, 1, 1, 1, 1, 1, 1, 1, (1 << 24) + 1))):
        assert lib.cm_draft_workspace(100, ctypes.byref(bad)) == 0
        assert lib.cm_draft(A, 100, ctypes.byref(bad), 8, A, A, A, A, 1 << 20, None) == E_INVAL
    f = lib.cm_draft
    assert f(A, 0, pp, 8, A, A, A, A, need, None) == E_SHAPE
    assert f(A, 4097, pp, 0, A, A, A, A, need, None) == E_SHAPE
    assert f(A, 4097, pp, 17, A, A, A, A, need, None) == E_SHAPE
    assert f(None, 4097, pp, 8, A, A, A, A, need, None) == E_INVAL
    assert f(A, 4097, None, 8, A, A, A, A, need, None) == E_INVAL
    assert f(A, 4097, pp, 8, None, A, A, A, need, None) == E_INVAL
    assert f(A, 4097, pp, 8, A, A, None, A, need, None) == E_INVAL
    assert f(A + 2, 4097, pp, 8, A, A, A, A, need, None) == E_ALIGN
    assert f(A, 4097, pp, 8, A, A, A, A, need - 1, None) == E_WORKSPACE
    assert f(A, 4097, pp, 8, A, A, A, None, need, None) == E_WORKSPACE


def test_cm_window_rejects_bad_arguments(lib):
    from speculative_verification_amd._lib import cm_params
    m = fake_model()
    mp = ctypes.addressof(m)
    p = cm_params()
    pp = ctypes.byref(p)
    need = lib.spec_window_cm_workspace(mp, 8, 1024, pp)
    assert need == lib.spec_step_workspace(mp, 8) + 4 * 16 * 4
    assert lib.spec_window_cm_workspace(mp, 8, 0, pp) == 0
    assert lib.spec_window_cm_workspace(mp, 17, 1024, pp) == 0
    f = lib.spec_window_run_cm
    assert f(mp, A, A, A, 1024, pp, 0, 4, A, need, None, None) == E_SHAPE
    assert f(mp, A, A, A, 1024, pp, 8, 4097, A, need, None, None) == E_SHAPE
    assert f(mp, A, A, None, 1024, pp, 8, 4, A, need, None, None) == E_INVAL     # the ring is the history
    assert f(mp, A, A, A, 0, pp, 8, 4, A, need, None, None) == E_INVAL
    assert f(mp, A, A, A, 1024, None, 8, 4, A, need, None, None) == E_INVAL
    assert f(mp, A, A, A, 1024, ctypes.byref(cm_params(depth=9)), 8, 4, A, need, None, None) == E_INVAL
    assert f(mp, None, A, A, 1024, pp, 8, 4, A, need, None, None) == E_INVAL
    assert f(mp, A, A, A + 2, 1024, pp, 8, 4, A, need, None, None) == E_ALIGN
    assert f(mp, A, A, A, 1024, pp, 8, 4, A, need - 1, None, None) == E_WORKSPACE
    assert f(mp, A, A, A, 1024, pp, 8, 4, A + 16, need, None, None) == E_ALIGN
    assert f(mp, A, A, A, 1024, pp, 8, 0, A, need, None, None) == OK

"""C ABI on the host: the library loads, exports every declared symbol, the
host planner matches the oracle bit for bit, and bad arguments are rejected
before anything is launched.  No GPU needed."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import window_attention_amd as wa
from oracle import plan as oplan

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "winattn.h")


def _declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s+(win_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = wa.load_library()
    names = _declared_functions()
    assert set(names) >= {"win_plan", "win_permute", "win_transition", "win_attn_fwd", "win_strerror",
                          "win_build_info"}
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {wa.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_status_strings_and_build_info():
    lib = wa.load_library()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.win_strerror(code).decode() != "unknown status"
    assert lib.win_strerror(-99).decode() == "unknown status"
    assert "gfx950" in wa.build_info()


def _host_plan(T, H, W, nt, nh, nw, method):
    p = wa.plan(T, H, W, nt, nh, nw, method)
    return p


def _compare(T, H, W, nt, nh, nw, method):
    o = oplan.plan(T, H, W, nt, nh, nw, method)
    p = _host_plan(T, H, W, nt, nh, nw, method)
    assert (p.wt, p.wh, p.ww) == (o.wt, o.wh, o.ww)
    assert p.num_windows == o.num_windows and p.max_seqlen == o.max_seqlen and p.num_tokens == T * H * W
    assert p.segs == (len(oplan.axis_segments(T, o.wt, method)), len(oplan.axis_segments(H, o.wh, method)),
                      len(oplan.axis_segments(W, o.ww, method)))
    assert np.array_equal(p.perm.numpy(), np.asarray(o.perm, dtype=np.int32))
    assert np.array_equal(p.inv.numpy(), np.asarray(o.inv, dtype=np.int32))
    assert np.array_equal(p.cu_seqlens.numpy(), np.asarray(o.cu_seqlens, dtype=np.int32))
    assert np.array_equal(p.boxes.numpy(), np.asarray(o.boxes, dtype=np.int32).reshape(-1, 6))


_NS = (1, 2, 3, 5, 9, 17, 33, 65, 129)


@pytest.mark.parametrize("grid", [(1, 3, 4), (2, 5, 7), (3, 6, 6), (5, 9, 16), (6, 11, 5), (7, 4, 13), (31, 3, 2)])
@pytest.mark.parametrize("method", [0, 1])
def test_host_planner_matches_oracle_sweep(grid, method):
    for nt, nh, nw in itertools.product((1, 2, 3, 4, 31), _NS, _NS):
        _compare(*grid, nt, nh, nw, method)


@pytest.mark.parametrize("cfg", [(5, 9, 16, 2, 3, 3), (4, 45, 80, 4, 3, 3), (21, 45, 80, 4, 3, 3),
                                 (21, 68, 120, 4, 3, 3), (9, 9, 64, 2, 3, 5), (3, 3, 192, 1, 2, 7),
                                 (40, 17, 23, 3, 2, 2)])
@pytest.mark.parametrize("method", [0, 1])
def test_host_planner_matches_oracle_workload_grids(cfg, method):
    _compare(*cfg, method)


@pytest.mark.slow
@pytest.mark.parametrize("method", [0, 1])
def test_host_planner_matches_oracle_long_grid(method):
    _compare(31, 90, 160, 4, 3, 3, method)


def _status(*args):
    lib = wa.load_library()
    info = wa._PlanInfo()
    return lib.win_plan(*args[:7], ctypes.byref(info), None, None, None, None, args[7], None)


def test_plan_rejects_bad_geometry():
    assert _status(0, 4, 4, 1, 1, 1, 0, 0) == -1
    assert _status(4, 4, -4, 1, 1, 1, 0, 0) == -1
    assert _status(4, 4, 4, 1, 0, 1, 0, 0) == -1
    assert _status(4, 4, 4, 1, 1, 1, 2, 0) == -1          # unknown method
    assert _status(4, 4, 4, 1, 1, 1, 0, 2) == -1          # on_device must be 0/1
    assert _status(2048, 1024, 1024, 1, 1, 1, 0, 0) == -3  # L = 2^31
    lib = wa.load_library()
    assert lib.win_plan(4, 4, 4, 1, 1, 1, 0, None, None, None, None, None, 0, None) == -1  # info required
    assert _status(4, 4, 4, 1, 1, 1, 0, 0) == 0


def test_plan_size_query_only():
    lib = wa.load_library()
    info = wa._PlanInfo()
    assert lib.win_plan(21, 45, 80, 4, 3, 3, 1, ctypes.byref(info), None, None, None, None, 0, None) == 0
    assert (info.wt, info.wh, info.ww, info.num_windows, info.max_seqlen, info.num_tokens) == \
        (6, 15, 27, 64, 2430, 75600)


def test_device_entry_points_validate_before_launch():
    lib = wa.load_library()
    A = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first
    B = ctypes.c_void_p(0x20000)
    M = ctypes.c_void_p(0x10008)   # misaligned
    I = ctypes.c_void_p(0x30000)
    # permute
    assert lib.win_permute(None, B, I, 10, 1, 64, 0, 0, None) == -1
    assert lib.win_permute(A, B, None, 10, 1, 64, 0, 0, None) == -1
    assert lib.win_permute(A, B, I, 10, 1, 64, 9, 0, None) == -2     # dtype
    assert lib.win_permute(M, B, I, 10, 1, 64, 0, 0, None) == -2     # alignment
    assert lib.win_permute(A, B, I, 10, 1, 3, 0, 0, None) == -2      # row not a multiple of 16 bytes
    assert lib.win_permute(A, A, I, 10, 1, 64, 0, 0, None) == -1     # in place
    assert lib.win_permute(A, B, I, 10, 1, 64, 0, 7, None) == -1     # mode
    assert lib.win_permute(A, B, I, 1 << 31, 1, 64, 0, 0, None) == -3
    assert lib.win_permute(A, B, I, -1, 1, 64, 0, 0, None) == -1
    assert lib.win_permute(A, B, I, 10, 0, 64, 0, 0, None) == -1
    assert lib.win_permute(A, B, I, 0, 1, 64, 0, 0, None) == 0       # empty: nothing to do
    assert lib.win_permute(None, None, None, 0, 1, 64, 0, 0, None) == 0
    # transition
    assert lib.win_transition(A, B, None, I, 10, 1, 64, 0, None) == -1
    assert lib.win_transition(A, B, I, None, 10, 1, 64, 0, None) == -1
    assert lib.win_transition(A, A, I, I, 10, 1, 64, 0, None) == -1
    # attention
    f = ctypes.c_float
    C = ctypes.c_void_p(0x40000)
    O = ctypes.c_void_p(0x1000000)
    assert lib.win_attn_fwd(None, A, B, O, None, I, 1, 8, 8, 1, 1, 128, f(0.1), None) == -1
    assert lib.win_attn_fwd(A, A, A, O, None, None, 1, 8, 8, 1, 1, 128, f(0.1), None) == -1
    assert lib.win_attn_fwd(A, A, A, O, None, I, 1, 8, 8, 1, 1, 96, f(0.1), None) == -2   # head_dim
    assert lib.win_attn_fwd(A, A, A, O, None, I, 1, 8, 8, 1, 1, 128, f(-0.1), None) == -1  # scale
    assert lib.win_attn_fwd(A, A, A, O, None, I, 1, 8, 8, 1, 1, 128, f(float("inf")), None) == -1
    # 0 selects the default scale; the call still fails on the head_dim
    assert lib.win_attn_fwd(A, A, A, O, None, I, 1, 8, 8, 1, 1, 96, f(0.0), None) == -2
    assert lib.win_attn_fwd(A, A, A, O, None, I, 1, 8, 8, 1, 1, 128, f(float("nan")), None) == -1
    assert lib.win_attn_fwd(M, A, A, O, None, I, 1, 8, 8, 1, 1, 128, f(0.1), None) == -2
    assert lib.win_attn_fwd(A, B, C, A, None, I, 1, 8, 8, 1, 1, 128, f(0.1), None) == -1  # o aliases q
    assert lib.win_attn_fwd(A, B, C, O, None, I, 1, 9, 8, 1, 1, 128, f(0.1), None) == -1  # max_seqlen > L
    assert lib.win_attn_fwd(A, B, C, O, None, I, -1, 8, 8, 1, 1, 128, f(0.1), None) == -1
    assert lib.win_attn_fwd(A, B, C, O, None, I, 1, 8, 1 << 31, 1, 1, 128, f(0.1), None) == -3
    assert lib.win_attn_fwd(A, B, C, O, None, I, 0, 0, 8, 1, 1, 128, f(0.1), None) == 0   # no windows
    # 64 rows of heads * head_dim bf16 must span less than 2^31 bytes (32-bit tile offsets)
    Q2, K2, V2, O2 = (ctypes.c_void_p(i << 40) for i in (1, 2, 3, 4))
    assert lib.win_attn_fwd(Q2, K2, V2, O2, None, I, 1, 8, 8, 1, 1 << 17, 128, f(0.1), None) == -3
    assert lib.win_attn_fwd(Q2, K2, V2, O2, None, I, 0, 8, 8, 1, (1 << 17) - 1, 128, f(0.1), None) == 0
    # byte counts are bounded before they are formed: batch * L < 2^38
    assert lib.win_attn_fwd(Q2, K2, V2, O2, None, I, 1, 8, (1 << 31) - 1, 1 << 8, 1, 128, f(0.1), None) == -3
    # text: batch * text_len < 2^38, and per-window text outputs below 2^40 elements
    T1, T2, T3, T4, P = (ctypes.c_void_p(i << 40) for i in (5, 6, 7, 8, 9))
    targs = lambda N, B, T: (Q2, K2, V2, O2, None, I, N, 8, 8, B, 1, 128, f(0.1), T1, T2, T3, T, T4, P, None)  # noqa
    assert lib.win_attn_fwd_text(*targs(1, 1 << 14, 1 << 24)) == -3
    assert lib.win_attn_fwd_text(*targs(1, 1, 1 << 25)) == -3
    assert lib.win_attn_fwd_text(*targs(1 << 13, 1, 1 << 20)) == -3
    # permutes and the rotated gather: row_elems < 2^33, and batch * L rows of at most 2^62 bytes
    assert lib.win_permute(A, B, I, 10, 1, 1 << 33, 0, 0, None) == -3
    assert lib.win_permute(Q2, K2, I, 1 << 30, 1, 1 << 32, 0, 0, None) == -3
    assert lib.win_transition(Q2, K2, I, I, 1 << 30, 1, 1 << 32, 0, None) == -3
    assert lib.win_permute_rope(Q2, K2, I, None, I, A, 3, 15, 27, 1 << 30, 1, 1 << 26, 128, 6, None) == -3


@pytest.mark.parametrize("grid", [(1, 1, 20000), (3, 1, 15000), (2, 20000, 1)])
def test_plan_rejects_zero_rescaled_extent(grid):
    """rh or rw rounds to 0 (1x20000 gives H * scale = 0.42): WIN_EINVAL for
    the size query and the host and device fills, nothing written."""
    lib = wa.load_library()
    info = wa._PlanInfo()
    assert lib.win_plan(*grid, 1, 1, 1, 0, ctypes.byref(info), None, None, None, None, 0, None) == -1
    L = grid[0] * grid[1] * grid[2]
    perm = np.full(L, -7, dtype=np.int32)
    assert lib.win_plan(*grid, 1, 1, 1, 1, ctypes.byref(info), perm.ctypes.data, None, None, None, 0, None) == -1
    assert np.all(perm == -7)
    # device fill: rejected before anything is enqueued (the pointer is never touched)
    assert lib.win_plan(*grid, 1, 1, 1, 0, ctypes.byref(info), ctypes.c_void_p(0x10000), None, None, None, 1,
                        None) == -1


def test_noalloc_text_attention_refuses_work_past_its_scratch():
    """win_attn_fwd_text_noalloc checks the size of its per-window text
    outputs against the static scratch before anything else touches the
    device (fake pointers: never dereferenced)."""
    lib = wa.load_library()
    f = ctypes.c_float
    Q, K, V, O, I, TQ, TK, TV, TO = (ctypes.c_void_p(i << 32) for i in range(1, 10))
    args = lambda N, T, B=1, H=24: (Q, K, V, O, None, I, N, 8, 8, B, H, 128, f(0.0), TQ, TK, TV, T, TO, None)  # noqa
    for N, T, B, H in ((8, 683, 1, 24), (64, 86, 1, 24), (1 << 30, 1 << 30, 1 << 30, 1 << 30)):
        assert lib.win_attn_fwd_text_noalloc(*args(N, T, B, H)) == -5
    assert "scratch" in lib.win_strerror(-5).decode()

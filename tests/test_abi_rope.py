"""Host side of window-local RoPE (CPU only): win_plan_local's host fill and
win_rope_table against the oracle, and argument errors."""
import ctypes
import math

import numpy as np
import torch
import pytest

import window_attention_amd as wa
from oracle import plan as oplan
from oracle import rope as orope
from tests import oracle_pins as pins

GRIDS = [(1, 3, 4, 1, 26, 35), (5, 9, 16, 2, 3, 3), (5, 9, 16, 2, 6, 6), (3, 10, 12, 2, 2, 2), (21, 45, 80, 4, 3, 3),
         (7, 4, 13, 3, 2, 5)]


def _lib_positions(p_oracle, text_len):
    p = wa.plan(p_oracle.T, p_oracle.H, p_oracle.W, *p_oracle.counts_, p_oracle.method)
    loc = wa.local_positions(p).numpy()
    return [(int(a) + text_len, int(b), int(c)) for a, b, c in loc]


class _OPlan:
    """Oracle plan remembering its window counts."""
    def __new__(cls, *args):
        p = oplan.plan(*args)
        p.counts_ = args[3:6]
        return p


def test_worked_positions():
    class Shim:
        REGULAR, SHIFTED = oplan.REGULAR, oplan.SHIFTED

        @staticmethod
        def plan(*a):
            return _OPlan(*a)
    pins.check_rope_positions(_lib_positions, Shim)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("method", [oplan.REGULAR, oplan.SHIFTED])
def test_local_positions_match_oracle(grid, method):
    o = _OPlan(*grid, method)
    assert _lib_positions(o, 7) == [tuple(x) for x in orope.window_local_positions(o, 7)]


@pytest.mark.parametrize("rope_dim,text_len,base", [(12, 5, 10000.0), (128, 0, 10000.0), (60, 77, 500.0)])
def test_rope_table_matches_oracle_angles(rope_dim, text_len, base):
    p = wa.plan(21, 45, 80, 4, 3, 3, wa.REGULAR)
    t = wa.rope_table(p, text_len, rope_dim, base).numpy().reshape(-1, rope_dim // 3 // 2, 2)
    d = rope_dim // 3
    rows = [text_len + x for x in range(p.wt)] + list(range(p.wh)) + list(range(p.ww))
    assert t.shape[0] == len(rows)
    for r, pos in enumerate(rows):
        for i in range(d // 2):
            ang = pos * base ** (-2.0 * i / d)
            for k, v in enumerate((math.cos(ang), math.sin(ang))):
                assert abs(float(t[r, i, k]) - v) <= 2.0 ** -24 * max(abs(v), 2.0 ** -126) * 1.0001 + 1e-45


def test_table_rotates_as_the_oracle():
    """A rotation assembled from the table's fp32 entries matches the fp64
    oracle rotation to float precision (the table feeds the kernel)."""
    p = wa.plan(1, 3, 4, 1, 26, 35, wa.REGULAR)
    t = wa.rope_table(p, 5, 12).numpy().reshape(-1, 2, 2)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(14)
    pos = (5 + 0, 1, 1)
    y = np.array(x)
    rows = (pos[0] - 5, p.wt + pos[1], p.wt + p.wh + pos[2])
    for axis in range(3):
        for i in range(2):
            c, s = t[rows[axis], i]
            a = axis * 4 + 2 * i
            y[a], y[a + 1] = x[a] * c - x[a + 1] * s, x[a] * s + x[a + 1] * c
    assert np.allclose(y, orope.rotate(x, pos, 12), rtol=0, atol=1e-6)


def test_errors():
    lib = wa.load_library()
    buf = np.zeros(4096, dtype=np.float32)
    assert lib.win_rope_table(6, 15, 27, 0, 128, 10000.0, buf.ctypes.data) == 0
    assert lib.win_rope_table(6, 15, 27, 0, 64, 10000.0, buf.ctypes.data) == -2      # 64 / 3 = 21 is odd
    assert lib.win_rope_table(0, 15, 27, 0, 128, 10000.0, buf.ctypes.data) == -1
    assert lib.win_rope_table(6, 15, 27, -1, 128, 10000.0, buf.ctypes.data) == -1
    assert lib.win_rope_table(6, 15, 27, 0, 128, 1.0, buf.ctypes.data) == -1
    assert lib.win_rope_table(6, 15, 27, 0, 128, float("inf"), buf.ctypes.data) == -1
    assert lib.win_rope_table(6, 15, 27, 0, 128, 10000.0, None) == -1
    loc = np.zeros(3 * 720, dtype=np.int32)
    assert lib.win_plan_local(5, 9, 16, 2, 3, 3, 0, loc.ctypes.data, 0, None) == 0
    assert lib.win_plan_local(5, 9, 16, 2, 3, 3, 0, None, 0, None) == -1
    assert lib.win_plan_local(5, 9, 16, 2, 3, 3, 7, loc.ctypes.data, 0, None) == -1
    assert lib.win_plan_local(5, 9, 16, 2, 3, 3, 0, loc.ctypes.data, 2, None) == -1
    A, B, I = (ctypes.c_void_p(x) for x in (0x10000, 0x1000000, 0x2000000))
    f = lib.win_permute_rope
    # every call below is rejected by host validation before anything is launched
    assert f(A, B, I, None, I, I, 6, 15, 27, 8, 1, 1, 96, 96, None) == -2             # head_dim
    assert f(A, B, I, None, I, I, 6, 15, 27, 8, 1, 1, 64, 64, None) == -2             # rope_dim / 3 odd
    assert f(A, B, I, None, I, I, 6, 15, 27, 8, 1, 1, 64, 128, None) == -2            # rope_dim > head_dim
    assert f(A, A, I, None, I, I, 6, 15, 27, 8, 1, 1, 128, 126, None) == -1           # in place
    assert f(None, B, I, None, I, I, 6, 15, 27, 8, 1, 1, 128, 126, None) == -1
    assert f(A, B, I, None, None, I, 6, 15, 27, 8, 1, 1, 128, 126, None) == -1        # local missing
    assert f(A, B, I, None, I, ctypes.c_void_p(0x2000004), 6, 15, 27, 8, 1, 1, 128, 126, None) == -2  # table alignment
    assert f(None, None, None, None, None, None, 6, 15, 27, 0, 1, 1, 128, 126, None) == 0  # empty


@pytest.mark.parametrize("what", ["idx", "perm_dst", "local", "table", "rope_dim"])
def test_binding_rejects_tables_of_another_size(what):
    """The binding checks every table against the source before calling the
    library, whose kernel reads them through raw pointers: an index table,
    local table or rotation table of another grid, layout or rope_dim is
    refused (checked first, so host tensors show it without a GPU)."""
    p = wa.plan(5, 9, 16, 2, 3, 3, wa.SHIFTED)
    L = p.num_tokens
    src = torch.zeros((1, L, 2, 128), dtype=torch.bfloat16)
    idx, perm_dst = torch.zeros(L, dtype=torch.int32), torch.zeros(L, dtype=torch.int32)
    local = torch.zeros(3 * L, dtype=torch.int32)
    rope_dim = 126
    table = torch.zeros((p.wt + p.wh + p.ww) * (rope_dim // 3), dtype=torch.float32)
    if what == "idx":
        idx = idx[:-1]
    elif what == "perm_dst":
        perm_dst = torch.zeros(L + 1, dtype=torch.int32)
    elif what == "local":
        local = local[:-3]
    elif what == "table":
        table = torch.zeros(table.numel() - 2, dtype=torch.float32)
    else:
        rope_dim = 120  # a table made for 126 channels
    with pytest.raises(wa.WinAttnError) as e:
        wa._permute_rope(src, idx, perm_dst, local, table, p, rope_dim, None)
    assert "must be a device tensor" not in str(e.value)

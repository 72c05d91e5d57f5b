"""win_pack (host library) against the packing oracle and its pins (CPU
only: win_pack is host integer work)."""
import ctypes

import numpy as np
import pytest

import window_attention_amd as wa
from oracle import pack as opack
from oracle import plan as oplan
from tests import oracle_pins as pins


def _lib_pack(perms, cus, align):
    lib = wa.load_library()
    R = len(perms)
    toks = (ctypes.c_int64 * R)(*[len(p) for p in perms])
    nwin = (ctypes.c_int32 * R)(*[len(c) - 1 for c in cus])
    P = np.ascontiguousarray(np.concatenate([np.asarray(p, dtype=np.int32) for p in perms]))
    C = np.ascontiguousarray(np.concatenate([np.asarray(c, dtype=np.int32) for c in cus]))
    offsets = (ctypes.c_int64 * (R + 1))()
    perm_out = np.full(sum(len(p) + align for p in perms), -7, dtype=np.int32)
    cu_out = np.full(sum(len(c) for c in cus) + 1, -7, dtype=np.int32)
    mx = ctypes.c_int32(-7)
    st = lib.win_pack(R, toks, nwin, P.ctypes.data, C.ctypes.data, align, offsets, perm_out.ctypes.data,
                      cu_out.ctypes.data, ctypes.byref(mx))
    assert st == 0, st
    total = offsets[R]
    assert np.all(perm_out[total:] == -7)   # nothing written past the packed rows
    return list(offsets), perm_out[:total].tolist(), cu_out.tolist(), mx.value


def test_page_worked_example():
    pins.check_pack_worked_example(_lib_pack)


_REQUESTS = [
    [(4, 45, 80, 4, 3, 3, oplan.REGULAR)],
    [(5, 9, 16, 2, 3, 3, oplan.SHIFTED), (3, 10, 12, 2, 2, 2, oplan.REGULAR)],
    [(1, 3, 4, 1, 26, 35, oplan.SHIFTED), (5, 9, 16, 2, 6, 6, oplan.REGULAR), (2, 5, 7, 1, 2, 3, oplan.SHIFTED),
     (21, 45, 80, 4, 3, 3, oplan.SHIFTED)],
]


@pytest.mark.parametrize("reqs", _REQUESTS)
@pytest.mark.parametrize("align", [1, 7, 64, 4096])
def test_matches_oracle_bit_exact(reqs, align):
    plans = [oplan.plan(*r) for r in reqs]
    perms, cus = [list(p.perm) for p in plans], [list(p.cu_seqlens) for p in plans]
    got = _lib_pack(perms, cus, align)
    want = opack.pack_plans(perms, cus, align)
    assert got == (want.offsets, want.perm, want.cu_seqlens, want.max_seqlen)
    pins.check_pack_invariants(_lib_pack, perms, cus, align)


def test_binding_matches_oracle():
    reqs = _REQUESTS[1]
    plans = [wa.plan(*r) for r in reqs]
    k = wa.pack(plans, 64)
    o = [oplan.plan(*r) for r in reqs]
    want = opack.pack_plans([list(p.perm) for p in o], [list(p.cu_seqlens) for p in o], 64)
    assert k.offsets == want.offsets and k.perm.tolist() == want.perm and k.cu_seqlens.tolist() == want.cu_seqlens
    assert k.max_seqlen == want.max_seqlen and k.num_windows == len(want.cu_seqlens) - 1


def test_errors_write_nothing():
    lib = wa.load_library()
    i64, i32 = ctypes.c_int64, ctypes.c_int32

    def call(toks, nwin, perm, cu, align, with_perm=True):
        R = len(toks)
        T = (i64 * R)(*toks)
        N = (i32 * R)(*nwin)
        P = np.asarray(perm, dtype=np.int32)
        C = np.asarray(cu, dtype=np.int32)
        off = (i64 * (R + 1))(*([-5] * (R + 1)))
        po = np.full(64, -5, dtype=np.int32)
        co = np.full(16, -5, dtype=np.int32)
        mx = i32(-5)
        st = lib.win_pack(R, T, N, P.ctypes.data if with_perm else None, C.ctypes.data, align, off,
                          po.ctypes.data if with_perm else None, co.ctypes.data, ctypes.byref(mx))
        if st != 0:
            assert list(off) == [-5] * (R + 1) and np.all(po == -5) and np.all(co == -5) and mx.value == -5
        return st

    assert call([4], [2], [0, 1, 2, 3], [0, 2, 4], 4) == 0
    assert call([4], [2], [0, 1, 2, 3], [0, 2, 4], 0) == -1          # align
    assert call([4], [2], [0, 1, 2, 3], [1, 2, 4], 4) == -1          # cu[0] != 0
    assert call([4], [2], [0, 1, 2, 3], [0, 2, 5], 4) == -1          # cu[N] != L
    assert call([4], [2], [0, 1, 2, 3], [0, 3, 4], 4) == 0
    assert call([4], [2], [0, 1, 2, 3], [0, 3, 2], 4) == -1          # decreasing
    assert call([4], [2], [0, 1, 2, 4], [0, 2, 4], 4) == -1          # perm entry out of range
    assert call([4], [2], [0, 1, 2, 4], [0, 2, 4], 4, with_perm=False) == 0   # perm not asked for
    assert call([0], [1], [], [0, 0], 4) == -1                        # empty request
    assert call([1 << 31], [1], [0], [0, 0], 4, with_perm=False) == -3
    assert lib.win_pack(0, None, None, None, None, 4, None, None, None, None) == -1

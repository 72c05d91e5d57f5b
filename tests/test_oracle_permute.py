"""Oracle permutes against their pins (CPU only)."""
import numpy as np
import pytest

from oracle import permute as operm
from oracle import plan as oplan
from tests import oracle_pins as pins


@pytest.mark.parametrize("cfg", [(1, 3, 4, 1, 26, 35), (5, 9, 16, 2, 6, 6), (3, 5, 7, 2, 17, 9)])
def test_gather_scatter_transition_identities(cfg):
    T, H, W = cfg[:3]
    L = T * H * W
    r = oplan.plan(*cfg, oplan.REGULAR)
    s = oplan.plan(*cfg, oplan.SHIFTED)
    x = np.random.default_rng(0).integers(0, 2 ** 16, size=(2, L, 3), dtype=np.uint16)
    for p in (r, s):
        g = operm.gather(x, p.perm)
        # explicit loop definition of the gather
        for j in range(L):
            assert np.array_equal(g[:, j], x[:, p.perm[j]])
        assert np.array_equal(operm.scatter(g, p.perm), x)
    xr, xs = operm.gather(x, r.perm), operm.gather(x, s.perm)
    assert np.array_equal(operm.transition(xr, r.perm, s.perm), xs)
    assert np.array_equal(operm.transition(xs, s.perm, r.perm), xr)
    # the one-pass composed index used by a fused transition
    assert np.array_equal(xr[:, np.asarray(r.inv)[np.asarray(s.perm)]], xs)


def test_transition_index_worked_example():
    g = pins.load_golden("transition_worked_example.json")
    T, H, W = g["grid"]
    nt, nh, nw = g["num_windows_param"]
    r = oplan.plan(T, H, W, nt, nh, nw, oplan.REGULAR)
    s = oplan.plan(T, H, W, nt, nh, nw, oplan.SHIFTED)
    L = T * H * W
    x = np.arange(L, dtype=np.int64)[None, :]
    xr, xs = operm.gather(x, r.perm), operm.gather(x, s.perm)
    # positions in layout A at which each layout-B row is found
    pos_r = np.empty(L, dtype=np.int64)
    pos_r[np.asarray(r.perm)] = np.arange(L)
    pos_s = np.empty(L, dtype=np.int64)
    pos_s[np.asarray(s.perm)] = np.arange(L)
    idx_rs = pos_r[operm.transition(xr, r.perm, s.perm)[0]]
    idx_sr = pos_s[operm.transition(xs, s.perm, r.perm)[0]]
    assert idx_rs.tolist() == g["regular_to_shifted"]
    assert idx_sr.tolist() == g["shifted_to_regular"]

"""Oracle planner against its pins (CPU only)."""
import itertools

import pytest

from oracle import plan as oplan
from tests import oracle_pins as pins


def test_worked_examples():
    pins.check_worked_examples(oplan)


def test_size_invariance_across_resolutions():
    pins.check_size_invariance(oplan)


def test_temporal_cap():
    pins.check_temporal_cap(oplan)


def test_exact_scales_and_round_half_even():
    pins.check_exact_scales(oplan)


@pytest.mark.parametrize("n", range(1, 41))
def test_axis_segment_geometry(n):
    for w in range(1, 45):
        pins.check_shift_geometry(oplan, n, w)


# window-count parameters chosen so that the rescaled sizes of small grids
# land on every window extent from 1 up to the whole axis
_NS = (1, 2, 3, 5, 9, 17, 33, 65, 129)
_GRIDS = [(1, 3, 4), (2, 5, 7), (3, 6, 6), (4, 2, 9), (5, 9, 16), (6, 11, 5), (7, 4, 13), (31, 3, 2)]


@pytest.mark.parametrize("grid", _GRIDS)
@pytest.mark.parametrize("method", [oplan.REGULAR, oplan.SHIFTED])
def test_plan_invariants_sweep(grid, method):
    T, H, W = grid
    for nt, nh, nw in itertools.product((1, 2, 3, 4, 8, 31), _NS, _NS):
        p = oplan.plan(T, H, W, nt, nh, nw, method)
        pins.check_plan_invariants(oplan, p, T, H, W, nt, nh, nw, method)


@pytest.mark.parametrize("cfg", [(5, 9, 16, 2, 3, 3), (4, 45, 80, 4, 3, 3), (21, 45, 80, 4, 3, 3)])
@pytest.mark.parametrize("method", [oplan.REGULAR, oplan.SHIFTED])
def test_plan_invariants_workload_grids(cfg, method):
    p = oplan.plan(*cfg, method)
    pins.check_plan_invariants(oplan, p, *cfg, method)


def test_shifted_differs_from_regular():
    # a layout genuinely different from the regular one whenever some axis has
    # a window of at least 2 that does not cover it
    for T, H, W in _GRIDS:
        for nt, nh, nw in itertools.product((1, 2, 3), _NS, _NS):
            r = oplan.plan(T, H, W, nt, nh, nw, oplan.REGULAR)
            s = oplan.plan(T, H, W, nt, nh, nw, oplan.SHIFTED)
            split = any(2 <= w < n for w, n in ((r.wt, T), (r.wh, H), (r.ww, W)))
            assert (r.boxes != s.boxes) == split


@pytest.mark.parametrize("bad", [(0, 4, 4, 1, 1, 1), (4, -1, 4, 1, 1, 1), (4, 4, 4, 0, 1, 1), (4, 4, 4, 1, 1, -2)])
def test_rejects_non_positive(bad):
    with pytest.raises(ValueError):
        oplan.plan(*bad, oplan.REGULAR)


def test_rejects_unknown_method():
    with pytest.raises(ValueError):
        oplan.plan(2, 3, 4, 1, 1, 1, 7)


@pytest.mark.parametrize("grid", [(1, 1, 20000), (3, 1, 15000), (2, 20000, 1)])
def test_zero_rescaled_extent_is_rejected(grid):
    """A rescaled extent of zero (1x20000: H * sqrt(3600 / 20000) = 0.42
    rounds to 0) gives no window size: the planner refuses the grid."""
    with pytest.raises(ValueError):
        oplan.window_size(*grid, 1, 1, 1)

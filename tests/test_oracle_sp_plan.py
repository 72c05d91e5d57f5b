"""Oracle tables of window-aligned sequence parallelism (LPT assignment and
Plan A redistribution), against their pins, with the exchange simulated on
fake ranks (CPU only)."""
import pytest

from oracle import plan as oplan
from oracle import sp_plan as sp
from tests import oracle_pins as pins


def _lpt(sizes, ranks):
    return sp.lpt_assign(sizes, ranks)


def _plan_a(z_src, z_dst):
    a = sp.plan_a(z_src, z_dst)
    return a.counts, a.send_rows, a.recv_pos, a.exchange_required


def _sizes(p):
    cu = list(p.cu_seqlens)
    return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def test_lpt_worked_examples():
    pins.check_lpt_worked_examples(_lpt)


def test_plan_a_worked_example():
    pins.check_plan_a_worked_example(_plan_a)


GRIDS = [(1, 3, 4, 1, 26, 35), (5, 9, 16, 2, 6, 6), (21, 45, 80, 4, 3, 3), (3, 10, 12, 2, 2, 2)]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("ranks", [1, 2, 3, 8])
def test_lpt_invariants(grid, ranks):
    for m in (oplan.REGULAR, oplan.SHIFTED):
        pins.check_lpt_invariants(_lpt, _sizes(oplan.plan(*grid, m)), ranks)


@pytest.mark.parametrize("grid", GRIDS[:2] + GRIDS[3:])
@pytest.mark.parametrize("ranks", [1, 2, 3, 5])
def test_plan_a_exchange_on_fake_ranks(grid, ranks):
    pr, ps = oplan.plan(*grid, oplan.REGULAR), oplan.plan(*grid, oplan.SHIFTED)
    zr = sp.rank_tokens(pr.perm, pr.cu_seqlens, _lpt(_sizes(pr), ranks)[1])
    zs = sp.rank_tokens(ps.perm, ps.cu_seqlens, _lpt(_sizes(ps), ranks)[1])
    for a, b in ((zr, zs), (zs, zr), (zr, zr)):
        pins.check_plan_a_invariants(_plan_a, a, b)
    # same layout, same assignment: nothing crosses ranks
    assert not sp.plan_a(zr, zr).exchange_required
    # and simulate_exchange delivers exactly the destination holdings
    assert sp.simulate_exchange(zr, sp.plan_a(zr, zs)) == zs


def test_one_rank_is_the_local_transition():
    """With one rank Plan A is the local permutation: the send table of the
    single rank is the transition index inv_A[perm_B]."""
    pr, ps = oplan.plan(21, 45, 80, 4, 3, 3, oplan.REGULAR), oplan.plan(21, 45, 80, 4, 3, 3, oplan.SHIFTED)
    za = sp.rank_tokens(pr.perm, pr.cu_seqlens, [list(range(pr.num_windows))])
    zb = sp.rank_tokens(ps.perm, ps.cu_seqlens, [list(range(ps.num_windows))])
    a = sp.plan_a(za, zb)
    L = len(pr.perm)
    assert a.counts == [[L]] and not a.exchange_required
    assert a.send_rows[0] == [pr.inv[c] for c in ps.perm]
    assert a.recv_pos[0] == list(range(L))

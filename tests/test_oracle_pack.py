"""Oracle packing of several requests into one varlen call, against its pins
(CPU only)."""
import pytest

from oracle import pack as opack
from oracle import plan as oplan
from tests import oracle_pins as pins


def _oracle(perms, cus, align):
    p = opack.pack_plans(perms, cus, align)
    return p.offsets, p.perm, p.cu_seqlens, p.max_seqlen


def test_page_worked_example():
    pins.check_pack_worked_example(_oracle)


_REQUESTS = [
    [(4, 45, 80, 4, 3, 3, oplan.REGULAR)],
    [(5, 9, 16, 2, 3, 3, oplan.SHIFTED), (3, 10, 12, 2, 2, 2, oplan.REGULAR)],
    [(1, 3, 4, 1, 26, 35, oplan.SHIFTED), (5, 9, 16, 2, 6, 6, oplan.REGULAR), (2, 5, 7, 1, 2, 3, oplan.SHIFTED)],
]


@pytest.mark.parametrize("reqs", _REQUESTS)
@pytest.mark.parametrize("align", [1, 7, 64, 4096])
def test_pack_invariants(reqs, align):
    plans = [oplan.plan(*r) for r in reqs]
    pins.check_pack_invariants(_oracle, [list(p.perm) for p in plans], [list(p.cu_seqlens) for p in plans], align)


def test_pack_of_one_request_with_aligned_rows_is_the_plan_plus_an_empty_tail():
    p = oplan.plan(4, 45, 80, 4, 3, 3, oplan.REGULAR)
    k = opack.pack_plans([list(p.perm)], [list(p.cu_seqlens)], 64)   # 14400 rows = 225 * 64
    assert k.perm == list(p.perm) and k.cu_seqlens == list(p.cu_seqlens) + [14400] and k.offsets == [0, 14400]

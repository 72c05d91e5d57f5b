"""win_lpt and win_plan_a (host library) against the oracle and its pins,
the exchange simulated on fake ranks (CPU only)."""
import ctypes

import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import plan as oplan
from oracle import sp_plan as osp
from tests import oracle_pins as pins


def _lib_lpt(sizes, ranks):
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    a = wa.lpt(cu, ranks)
    lists = [a.windows_of(r) for r in range(ranks)]
    return a.owner.tolist(), lists, a.rank_tokens.tolist()


def _lib_plan_a_from_holdings(z_src, z_dst):
    """Plan A of two holdings given as lists of canonical ids: each rank's
    holding is made one window of its own layout."""
    P = len(z_src)
    L = sum(len(z) for z in z_src)

    def layout(z):
        perm = torch.tensor([c for zz in z for c in zz], dtype=torch.int32)
        cu = torch.tensor(np.concatenate([[0], np.cumsum([len(zz) for zz in z])]), dtype=torch.int32)
        p = wa.Plan(1, 1, L, 0, 1, 1, 1, (1, 1, P), P, 0, L, perm, None, cu, None)
        a = wa.Assignment(P, torch.arange(P, dtype=torch.int32), torch.arange(P, dtype=torch.int32),
                          torch.arange(P + 1, dtype=torch.int32), None)
        return p, a
    (ps, as_), (pd, ad) = layout(z_src), layout(z_dst)
    r = wa.plan_a(ps, as_, pd, ad)
    send, recv, k = [], [], 0
    for z in z_src:
        send.append(r.send_rows[k:k + len(z)].tolist())
        k += len(z)
    k = 0
    for z in z_dst:
        recv.append(r.recv_pos[k:k + len(z)].tolist())
        k += len(z)
    return r.counts.tolist(), send, recv, r.exchange_required


def test_lpt_worked_examples():
    pins.check_lpt_worked_examples(_lib_lpt)


def test_plan_a_worked_example():
    pins.check_plan_a_worked_example(_lib_plan_a_from_holdings)


GRIDS = [(1, 3, 4, 1, 26, 35), (5, 9, 16, 2, 6, 6), (21, 45, 80, 4, 3, 3), (3, 10, 12, 2, 2, 2)]


def _sizes(p):
    cu = list(p.cu_seqlens)
    return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("ranks", [1, 2, 3, 8, 64])
def test_lpt_matches_oracle(grid, ranks):
    for m in (oplan.REGULAR, oplan.SHIFTED):
        sizes = _sizes(oplan.plan(*grid, m))
        assert _lib_lpt(sizes, ranks) == tuple(osp.lpt_assign(sizes, ranks))
        pins.check_lpt_invariants(_lib_lpt, sizes, ranks)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("ranks", [1, 2, 5, 8])
def test_plan_a_matches_oracle_and_exchanges(grid, ranks):
    lp = {m: wa.plan(*grid, m) for m in (wa.REGULAR, wa.SHIFTED)}
    la = {m: wa.lpt(lp[m], ranks) for m in lp}
    op = {m: oplan.plan(*grid, m) for m in (oplan.REGULAR, oplan.SHIFTED)}
    z = {m: osp.rank_tokens(op[m].perm, op[m].cu_seqlens, osp.lpt_assign(_sizes(op[m]), ranks)[1]) for m in op}
    for a, b in ((wa.REGULAR, wa.SHIFTED), (wa.SHIFTED, wa.REGULAR), (wa.REGULAR, wa.REGULAR)):
        got = wa.plan_a(lp[a], la[a], lp[b], la[b])
        want = osp.plan_a(z[a], z[b])
        assert got.counts.tolist() == want.counts and got.exchange_required == want.exchange_required
        assert got.send_rows.tolist() == [i for s in want.send_rows for i in s]
        assert got.recv_pos.tolist() == [i for s in want.recv_pos for i in s]
        if grid[0] * grid[1] * grid[2] <= 2000:
            pins.check_plan_a_invariants(_lib_plan_a_from_holdings, z[a], z[b])


def test_one_rank_send_table_is_the_transition_index():
    pr, ps = wa.plan(21, 45, 80, 4, 3, 3, wa.REGULAR), wa.plan(21, 45, 80, 4, 3, 3, wa.SHIFTED)
    r = wa.plan_a(pr, wa.lpt(pr, 1), ps, wa.lpt(ps, 1))
    assert torch.equal(r.send_rows, pr.inv[ps.perm.long()]) and not r.exchange_required
    assert torch.equal(r.recv_pos, torch.arange(pr.num_tokens, dtype=torch.int32))


def test_errors():
    lib = wa.load_library()
    cu = np.array([0, 2, 5], dtype=np.int32)
    out = [np.zeros(4, dtype=np.int32) for _ in range(3)]
    toks = np.zeros(4, dtype=np.int64)
    assert lib.win_lpt(2, cu.ctypes.data, 2, *(o.ctypes.data for o in out), toks.ctypes.data) == 0
    assert lib.win_lpt(2, cu.ctypes.data, 0, *(o.ctypes.data for o in out), toks.ctypes.data) == -1
    bad = np.array([0, 3, 2], dtype=np.int32)
    assert lib.win_lpt(2, bad.ctypes.data, 2, *(o.ctypes.data for o in out), toks.ctypes.data) == -1
    assert lib.win_lpt(2, None, 2, *(o.ctypes.data for o in out), toks.ctypes.data) == -1
    # plan_a: a perm that is not a permutation, an assignment that is not a partition
    p = wa.plan(1, 3, 4, 1, 26, 35, wa.REGULAR)
    a = wa.lpt(p, 2)
    broken = wa.Plan(**{**p.__dict__, "perm": torch.zeros(12, dtype=torch.int32)})
    with pytest.raises(wa.WinAttnError):
        wa.plan_a(broken, a, p, a)
    a2 = wa.Assignment(2, a.owner, torch.zeros_like(a.order), a.rank_offsets, a.rank_tokens)
    with pytest.raises(wa.WinAttnError):
        wa.plan_a(p, a2, p, a)

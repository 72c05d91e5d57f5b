"""Plan A redistribution driven through the library's permute kernels (GPU).

Page "Window-Aligned Sequence Parallelism (SeedVR2)", sections "Planner" and
"Plan A redistribution": P ranks, each holding the rows of its LPT-assigned
windows, re-shard the hidden state at a layout boundary with one
variable-split all-to-all.  Here the P ranks are slices of one GPU's memory:
  * rank r's send buffer is win_permute(GATHER, send_rows of r) of its
    holding (rows grouped by destination, each group in destination-local
    order);
  * the all-to-all is plain slicing: destination d concatenates, in source
    order, the counts[r][d] rows each rank r sends it (the collective a real
    run would make over RCCL; no arithmetic of the method);
  * destination d places what it received with win_permute(SCATTER,
    recv_pos of d).
Each destination's result must be, bit for bit, the rows the oracle's
simulated exchange delivers, which are the rows of its windows in the
destination layout.  With one rank the send table is the transition index,
and the send buffer equals win_transition."""
import numpy as np
import pytest
import torch

import window_attention_amd as wa
from oracle import plan as oplan
from oracle import sp_plan as osp
from tests.gpu_helpers import say
from window_attention_amd.inputs import normal

pytestmark = pytest.mark.gpu
DEV = "cuda"
# (T, H, W, nt, nh, nw): the 21x45x80 video grid, a ragged small grid
GRIDS = [(21, 45, 80, 4, 3, 3), (5, 9, 16, 2, 6, 6)]
HEADS, D = 2, 64  # 256-byte rows: the kernels' row handling, not attention


def _dev_i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _sizes(op):
    cu = op.cu_seqlens
    return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def _holding_rows(p, lists, r):
    """Window-order positions of rank r's rows: its windows in listed order."""
    cu = p.cu_seqlens.cpu().tolist()
    return [j for w in lists[r] for j in range(cu[w], cu[w + 1])]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("ranks", [1, 2, 3, 8])
@pytest.mark.parametrize("direction", [(wa.REGULAR, wa.SHIFTED), (wa.SHIFTED, wa.REGULAR)])
def test_plan_a_exchange_on_device(grid, ranks, direction):
    a, b = direction
    say(f"plan A exchange grid={grid} ranks={ranks} {a}->{b}")
    pa, pb = (wa.plan(*grid, m, device=DEV) for m in (a, b))
    L = pa.num_tokens
    x = normal((1, L, HEADS, D), 4242, device=DEV)  # canonical hidden state
    xa = wa.gather(x, pa.perm)                        # layout A, window order
    asg_a, asg_b = wa.lpt(pa, ranks), wa.lpt(pb, ranks)
    lists_a = [asg_a.windows_of(r) for r in range(ranks)]
    red = wa.plan_a(pa, asg_a, pb, asg_b)
    counts = red.counts.tolist()

    # the oracle's tables and exchange, on canonical ids
    op = {m: oplan.plan(*grid, m) for m in (a, b)}
    z_a = osp.rank_tokens(op[a].perm, op[a].cu_seqlens, osp.lpt_assign(_sizes(op[a]), ranks)[1])
    z_b = osp.rank_tokens(op[b].perm, op[b].cu_seqlens, osp.lpt_assign(_sizes(op[b]), ranks)[1])
    want_tables = osp.plan_a(z_a, z_b)
    delivered = osp.simulate_exchange(z_a, want_tables)
    assert delivered == z_b

    # each rank's holding (set-up of the fake ranks' memory, not part of the
    # exchange): the rows of its windows of layout A, in listed order
    holdings = [xa[:, _dev_i32(_holding_rows(pa, lists_a, r)).long()].contiguous() if len(lists_a[r]) else None
                for r in range(ranks)]
    send, off = [], 0
    for r in range(ranks):
        n_r = sum(counts[r])
        rows = red.send_rows[off:off + n_r]
        off += n_r
        send.append(wa.gather(holdings[r], rows.to(DEV)) if n_r else None)
    # all-to-all: destination d receives counts[r][d] rows of every rank r, in source order
    off = 0
    for d in range(ranks):
        parts = []
        for r in range(ranks):
            start = sum(counts[r][:d])
            if counts[r][d]:
                parts.append(send[r][:, start:start + counts[r][d]])
        n_d = sum(counts[r][d] for r in range(ranks))
        pos = red.recv_pos[off:off + n_d]
        off += n_d
        if n_d == 0:
            assert not z_b[d]
            continue
        got = wa.scatter(torch.cat(parts, dim=1).contiguous(), pos.to(DEV))
        want = x[:, torch.as_tensor(np.asarray(delivered[d], dtype=np.int64), device=DEV)]
        assert torch.equal(got, want), (grid, ranks, d)
    if ranks == 1:
        assert torch.equal(send[0], wa.transition(xa, pa.inv, pb.perm))
        assert not red.exchange_required

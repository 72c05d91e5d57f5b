"""Oracle of the single-GPU tables of window-aligned sequence parallelism (test
infrastructure only; see ``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)", sections
"Planner" (the deterministic LPT assignment) and "Plan A redistribution" (the
count matrix, split sizes, destination-local packing, one argsort at the
receiver, and the globally computed exchange flag).

Only tables are computed here.  The exchange itself (an all-to-all between
ranks) is simulated by ``simulate_exchange`` with plain lists standing for the
ranks' buffers, so the tables can be checked end to end on one CPU.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence


def lpt_assign(sizes: Sequence[int], ranks: int):
    """Section "Planner": windows taken by (-tokens, window id); each goes to
    the rank with the smallest (assigned tokens, rank id); each rank then
    lists its windows in ascending window id.  Returns (owner of each window,
    window list of each rank, tokens of each rank)."""
    assert ranks > 0
    order = sorted(range(len(sizes)), key=lambda w: (-sizes[w], w))
    load = [0] * ranks
    owner = [-1] * len(sizes)
    for w in order:
        r = min(range(ranks), key=lambda x: (load[x], x))
        owner[w] = r
        load[r] += sizes[w]
    lists = [[w for w in range(len(sizes)) if owner[w] == r] for r in range(ranks)]
    return owner, lists, load


def rank_tokens(perm: Sequence[int], cu: Sequence[int], lists: Sequence[Sequence[int]]) -> List[List[int]]:
    """Canonical token ids held by each rank, in the rank's local order: its
    windows in its listed order, tokens row-major inside each window (the
    plan's window order)."""
    return [[perm[j] for w in ws for j in range(cu[w], cu[w + 1])] for ws in lists]


@dataclass
class PlanA:
    counts: List[List[int]]        # C[r][d]: rows rank d needs from rank r
    send_rows: List[List[int]]     # per source rank: its local rows to send, grouped by destination,
                                   # each group in destination-local order
    recv_pos: List[List[int]]      # per destination rank: destination-local position of each received
                                   # row, received rows concatenated in source-rank order
    exchange_required: bool        # some row changes rank (same value on every rank)

    def input_split_sizes(self, r):
        return list(self.counts[r])

    def output_split_sizes(self, r):
        return [row[r] for row in self.counts]


def plan_a(z_src: Sequence[Sequence[int]], z_dst: Sequence[Sequence[int]]) -> PlanA:
    """Section "Plan A redistribution" for source holdings z_src[r] and
    destination holdings z_dst[d] (canonical ids in local order)."""
    P = len(z_src)
    assert len(z_dst) == P
    src_of = {}
    for r, z in enumerate(z_src):
        for i, c in enumerate(z):
            src_of[c] = (r, i)
    counts = [[0] * P for _ in range(P)]
    groups = [[[] for _ in range(P)] for _ in range(P)]   # groups[r][d]: (dest position, source local row)
    for d, z in enumerate(z_dst):
        for pos, c in enumerate(z):
            r, i = src_of[c]
            counts[r][d] += 1
            groups[r][d].append((pos, i))
    send_rows, recv_parts = [], [[] for _ in range(P)]
    for r in range(P):
        rows = []
        for d in range(P):
            seg = sorted(groups[r][d])            # destination-local order
            rows.extend(i for _, i in seg)
            recv_parts[d].append([pos for pos, _ in seg])
        send_rows.append(rows)
    recv_pos = [[p for part in recv_parts[d] for p in part] for d in range(P)]
    exchange = any(counts[r][d] for r in range(P) for d in range(P) if r != d)
    return PlanA(counts, send_rows, recv_pos, exchange)


def simulate_exchange(x_src: Sequence[Sequence[object]], a: PlanA) -> List[List[object]]:
    """The all-to-all the tables drive, with lists for buffers: rank r sends
    its rows send_rows[r] split by counts[r]; rank d concatenates what it
    receives in source order and puts each row at its destination position
    (one argsort of recv_pos)."""
    P = len(x_src)
    outbox = []
    for r in range(P):
        rows = [x_src[r][i] for i in a.send_rows[r]]
        segs, k = [], 0
        for d in range(P):
            segs.append(rows[k:k + a.counts[r][d]])
            k += a.counts[r][d]
        outbox.append(segs)
    out = []
    for d in range(P):
        received = [row for r in range(P) for row in outbox[r][d]]
        order = sorted(range(len(received)), key=lambda t: a.recv_pos[d][t])   # the receiver's one argsort
        out.append([received[t] for t in order])
    return out

"""Oracle of multi-request packing (test infrastructure only; see ``oracle/__init__``).

Source: page "vLLM-Omni diffusion runtime" (blog post), section 4.2 on packing
several requests into one forward.  What it fixes:

* the requests' rows are laid out back to back, each followed by an alignment
  tail that pads it to a whole number of alignment units;
* the cumulative boundaries keep, for every request, its real document(s) and
  its tail as separate segments; a tail of length zero still contributes its
  (repeated) boundary, so the layout does not change shape when no padding is
  needed;
* ``max_seqlen`` is the length of the longest document, not of the packed
  sequence;
* segments are independent documents;
* the index that places a row in the packed tensor gets the request's row
  offset added, while positional coordinates stay request-local.

Applied to window attention, a request's documents are its windows (its plan's
``cu_seqlens``), and its rows are placed by its plan's ``perm`` shifted by the
request's offset.  Two readings where the page is silent (listed in the design
notes):

* The tail rows are padding: the packed gather maps each of them to itself.
* ``max_seqlen`` covers every segment of the packed call, tails included (a
  tail is shorter than the alignment unit, so this differs from the longest
  document only when the alignment exceeds every window).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence


@dataclass
class Packed:
    offsets: List[int]      # row offset of each request; offsets[R] = total rows
    perm: List[int]         # packed gather table (window order -> packed canonical row)
    cu_seqlens: List[int]   # packed segment boundaries
    max_seqlen: int


def tail_rows(n: int, align: int) -> int:
    """Rows that pad ``n`` up to a multiple of ``align``."""
    return (align - n % align) % align


def pack_plans(perms: Sequence[Sequence[int]], cus: Sequence[Sequence[int]], align: int) -> Packed:
    """Pack request r's plan (``perms[r]``, ``cus[r]``) after the requests
    before it, each request followed by its alignment tail."""
    assert align > 0 and len(perms) == len(cus) and len(perms) > 0
    offsets = [0]
    perm: List[int] = []
    cu = [0]
    longest = 0
    for p, c in zip(perms, cus):
        n = len(p)
        o = offsets[-1]
        assert c[0] == 0 and c[-1] == n
        # the request's windows: its own boundaries moved by its row offset
        for a, b in zip(c[:-1], c[1:]):
            cu.append(o + b)
            longest = max(longest, b - a)
        # its rows: the physical index gets the row offset added
        perm.extend(o + x for x in p)
        # its alignment tail: one more segment, empty when no padding is needed
        t = tail_rows(n, align)
        perm.extend(range(o + n, o + n + t))
        cu.append(o + n + t)
        longest = max(longest, t)
        offsets.append(o + n + t)
    return Packed(offsets, perm, cu, longest)

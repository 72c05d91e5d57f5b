"""Oracle window planner (test infrastructure only; see ``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)", section
"Window layouts" (the size formulas block, the regular and shifted methods, the
enumeration order and the canonical id) and the "Consequences that matter"
list under it.

Readings where the page is silent (each is listed in the design notes):

* Odd window, "half a window" shift: the moved cut of regular cut ``k*w`` is the
  slice index obtained by truncating ``(k - 1/2) * w`` toward zero, then
  clipped to ``[0, n]``.  For ``k >= 1`` that is ``floor((2k-1) w / 2)``.
* A window that already covers its axis (``w >= n``) is not shifted on that
  axis: the axis keeps the single segment ``[0, n)``.
* ``round`` is Python's round-half-to-even of the IEEE double product, with
  ``scale`` rounded to double first.
* Empty segments produced by clipping are dropped; segments continue until the
  clipped start reaches ``n``.

Everything here is Python integers except the three double operations of the
size formula, so results are exact and reproducible.

Parity unpinned by the pages: the page prints no window table, so the first
two readings above (the cut of an odd window, no shift on a covered axis) are
fixed only by the hand-derived worked examples written under them and by the
invariants the page states; every other part of the plan is pinned by those
invariants, exact-scale grids and the windowing-arange twin.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Tuple

REGULAR = 0
SHIFTED = 1

# Area of the 720p reference post-patch grid (45 x 80 tokens) and the temporal
# cap; both come from the size formula block of section "Window layouts".
REFERENCE_AREA = 45 * 80
MAX_TEMPORAL_WINDOW = 30


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def window_size(T: int, H: int, W: int, nt: int, nh: int, nw: int) -> Tuple[int, int, int]:
    """Window extent ``(wt, wh, ww)`` of the 720p-normalised formula.

    Section "Window layouts", size formula block: scale is the square root of
    the reference area over ``H*W``; the spatial sizes are the ceilings of the
    rounded, rescaled extents over the window counts; the temporal size is the
    ceiling of ``min(T, 30)`` over ``nt``.
    """
    for name, v in (("T", T), ("H", H), ("W", W), ("nt", nt), ("nh", nh), ("nw", nw)):
        if not isinstance(v, int) or v <= 0:
            raise ValueError(f"{name} must be a positive int, got {v!r}")
    scale = math.sqrt(REFERENCE_AREA / (H * W))
    rh = round(H * scale)
    rw = round(W * scale)
    if rh <= 0 or rw <= 0:
        raise ValueError(f"rescaled extent is zero (rh={rh}, rw={rw})")
    wh = _ceil_div(rh, nh)
    ww = _ceil_div(rw, nw)
    wt = _ceil_div(min(T, MAX_TEMPORAL_WINDOW), nt)
    return wt, wh, ww


def regular_segments(n: int, w: int) -> List[Tuple[int, int]]:
    """Regular tiling of one axis: ``[k*w, min((k+1)*w, n))`` for every k that
    starts inside the axis (section "Window layouts", regular method)."""
    return [(k * w, min((k + 1) * w, n)) for k in range(_ceil_div(n, w))]


def _half_shifted_cut(k: int, w: int) -> int:
    """Regular cut ``k*w`` moved back by half a window, as a slice index:
    ``(k - 1/2) * w`` truncated toward zero (exact integer arithmetic)."""
    twice = (2 * k - 1) * w
    return twice // 2 if twice >= 0 else -((-twice) // 2)


def shifted_segments(n: int, w: int) -> List[Tuple[int, int]]:
    """Shifted tiling of one axis (section "Window layouts", shifted method):
    every cut moves by half a window and the windows are clipped to the axis
    with ``max(., 0)`` / ``min(., n)``; nothing wraps around.  An axis that one
    window already covers keeps its single segment."""
    if w >= n:
        return [(0, n)]
    segs = []
    k = 0
    while True:
        lo = max(_half_shifted_cut(k, w), 0)
        if lo >= n:
            break
        hi = min(_half_shifted_cut(k + 1, w), n)
        if hi > lo:
            segs.append((lo, hi))
        k += 1
    return segs


def axis_segments(n: int, w: int, method: int) -> List[Tuple[int, int]]:
    if method == REGULAR:
        return regular_segments(n, w)
    if method == SHIFTED:
        return shifted_segments(n, w)
    raise ValueError(f"unknown method {method!r}")


@dataclass
class Plan:
    """Integer tables of one window layout.

    ``boxes[i] = (t0, t1, h0, h1, w0, w1)`` is window i; ``perm[j]`` is the
    canonical id of the token at window-order position j; ``inv`` is the
    inverse permutation; ``cu_seqlens`` are the prefix sums of window sizes.
    """
    T: int
    H: int
    W: int
    method: int
    wt: int
    wh: int
    ww: int
    boxes: List[Tuple[int, int, int, int, int, int]] = field(default_factory=list)
    perm: List[int] = field(default_factory=list)
    inv: List[int] = field(default_factory=list)
    cu_seqlens: List[int] = field(default_factory=list)

    @property
    def num_windows(self) -> int:
        return len(self.boxes)

    @property
    def max_seqlen(self) -> int:
        return max((self.cu_seqlens[i + 1] - self.cu_seqlens[i] for i in range(self.num_windows)), default=0)


def plan(T: int, H: int, W: int, nt: int, nh: int, nw: int, method: int) -> Plan:
    """Window layout tables for a ``(T, H, W)`` token grid.

    Section "Window layouts": windows are enumerated w outermost, then h, then
    t innermost; tokens inside a window are row-major in ``(t, h, w)``; the
    canonical id of token ``(t, h, w)`` is ``(t*H + h)*W + w``.
    """
    wt, wh, ww = window_size(T, H, W, nt, nh, nw)
    st = axis_segments(T, wt, method)
    sh = axis_segments(H, wh, method)
    sw = axis_segments(W, ww, method)
    p = Plan(T, H, W, method, wt, wh, ww)
    p.cu_seqlens.append(0)
    for (w0, w1) in sw:
        for (h0, h1) in sh:
            for (t0, t1) in st:
                p.boxes.append((t0, t1, h0, h1, w0, w1))
                for t in range(t0, t1):
                    for h in range(h0, h1):
                        for w in range(w0, w1):
                            p.perm.append((t * H + h) * W + w)
                p.cu_seqlens.append(len(p.perm))
    p.inv = [0] * len(p.perm)
    for j, c in enumerate(p.perm):
        p.inv[c] = j
    return p

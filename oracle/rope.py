"""Oracle of window-local 3D rotary position embedding (test infrastructure
only; see ``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)", section
"Reference quirks reproduced on purpose": RoPE positions are window-local, a
video token at window-local ``(dt, dh, dw)`` uses axial indices
``(text_len + dt, dh, dw)`` and every window restarts at 0; the rotary span is
``3 * (rope_dim // 3)`` channels and the channels after it pass through.  The
diffusion-runtime post (section 4.2) adds that positional coordinates stay
request-local while physical row indices move; the position of a row here is
computed from its window's box, never from its row index.

Readings where the pages are silent (listed in the design notes):

* Axial layout: the rotated span is three consecutive blocks of
  ``d = rope_dim // 3`` channels, for the t, h and w indices in that order.
* Rotation inside a block: rotary position embedding as defined by Su et al.
  (RoFormer, 2021): channels ``(2i, 2i+1)`` of the block form a plane rotated
  by the angle ``position * base**(-2i/d)``, ``i = 0 .. d/2 - 1``, with
  ``base = 10000``.
* RoPE rotates queries and keys; values are not rotated.

Everything is fp64 on the exact values of the bf16 inputs.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

DEFAULT_BASE = 10000.0


def rotary_span(rope_dim: int) -> int:
    return 3 * (rope_dim // 3)


def window_local_positions(plan, text_len: int) -> List[Tuple[int, int, int]]:
    """Axial indices of every row of the plan's window order: the token's
    coordinate minus its window's first coordinate on each axis, with
    ``text_len`` added on the t axis."""
    H, W = plan.H, plan.W
    out = []
    for i, (t0, t1, h0, h1, w0, w1) in enumerate(plan.boxes):
        for j in range(plan.cu_seqlens[i], plan.cu_seqlens[i + 1]):
            c = plan.perm[j]
            t, rem = divmod(c, H * W)
            h, w = divmod(rem, W)
            assert t0 <= t < t1 and h0 <= h < h1 and w0 <= w < w1
            out.append((text_len + t - t0, h - h0, w - w0))
    return out


def rotate(x: np.ndarray, pos: Sequence[int], rope_dim: int, base: float = DEFAULT_BASE) -> np.ndarray:
    """Rotate the last axis (head_dim >= rope_dim channels) of ``x`` (fp64) for
    one token at axial indices ``pos = (pt, ph, pw)``."""
    d = rope_dim // 3
    assert d % 2 == 0, "each axis block holds whole channel pairs"
    y = np.array(x, dtype=np.float64, copy=True)
    for axis in range(3):
        p = pos[axis]
        for i in range(d // 2):
            ang = p * base ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            a = axis * d + 2 * i
            x0, x1 = x[..., a], x[..., a + 1]
            y[..., a] = x0 * c - x1 * s
            y[..., a + 1] = x0 * s + x1 * c
    return y


def rope_rows(x: np.ndarray, positions: Sequence[Tuple[int, int, int]], rope_dim: int,
              base: float = DEFAULT_BASE) -> np.ndarray:
    """``x`` is [B, L, heads, head_dim] in window order (fp64); row j is
    rotated for ``positions[j]``, every head alike."""
    y = np.empty_like(x, dtype=np.float64)
    for j, pos in enumerate(positions):
        y[:, j] = rotate(x[:, j], pos, rope_dim, base)
    return y

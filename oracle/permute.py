"""Oracle row permutes (test infrastructure only; see ``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)".  Section
"SeedVR2 integration" gives the entry distribution (canonical rows into window
order) and the final reconstruction (back to canonical order); section
"Motivation" and "Plan A redistribution" give the layout transition, which on
one device is a local permutation of rows.

Arrays are ``[B, L, ...]``: the permutation acts on axis 1, the same plan for
every batch element.  All three are exact copies of whole rows, so any dtype
(including raw bf16 bit patterns as uint16) works.
"""
from __future__ import annotations

import numpy as np


def gather(x_canonical: np.ndarray, perm) -> np.ndarray:
    """Canonical order -> window order: row ``j`` of the result is canonical
    row ``perm[j]``."""
    perm = np.asarray(perm, dtype=np.int64)
    return x_canonical[:, perm]


def scatter(x_window: np.ndarray, perm) -> np.ndarray:
    """Window order -> canonical order: canonical row ``perm[j]`` receives
    window-order row ``j``."""
    perm = np.asarray(perm, dtype=np.int64)
    out = np.empty_like(x_window)
    out[:, perm] = x_window
    return out


def transition(x_layout_a: np.ndarray, perm_a, perm_b) -> np.ndarray:
    """Layout A -> layout B by its definition: back to canonical order under
    A's permutation, then into B's window order."""
    return gather(scatter(x_layout_a, perm_a), perm_b)

"""Oracle window attention in fp64 (test infrastructure only; see
``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)", section
"Motivation" (each layer attends only inside each 3D window, never globally)
and section "SeedVR2 integration" (one packed variable-length attention call
over segments delimited by ``cu_seqlens``).  The page leaves the softmax scale
and causality open; the reading used is the scaled-dot-product default,
``1/sqrt(D)``, non-causal, no dropout, video tokens only.

Per window ``i`` (rows ``cu[i]:cu[i+1]``) and head ``h``::

    S = Q_i K_i^T * scale
    P = exp(S - rowmax(S)) / rowsum(exp(S - rowmax(S)))
    O_i = P V_i,     LSE_i = rowmax(S) + log(rowsum(exp(S - rowmax(S))))

``masked_full_attention`` is the brute-force twin: attention over all tokens at
once, in canonical order, with a mask that only admits pairs in the same
window.  Window attention is exactly that masked attention, reordered.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (given as uint16/int16): a bf16 is
    the upper half of an IEEE float32."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of one window and one head.

    ``q``, ``k``: ``[n, D]``; ``v``: ``[n, Dv]``, fp64.  Returns ``(O, LSE)``
    with ``O`` ``[n, Dv]`` and ``LSE`` ``[n]`` (natural log).
    """
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ v) / z
    return o, (m + np.log(z))[:, 0]


def window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens, scale: float | None = None):
    """Attention restricted to each window of a window-ordered sequence.

    ``q``, ``k``, ``v``: ``[B, L, Hh, D]`` fp64, rows already in window order;
    ``cu_seqlens``: ``N+1`` prefix sums (zero-length windows allowed).  Returns
    ``(O [B, L, Hh, D], LSE [B, Hh, L])``; rows not covered by any window stay
    zero in ``O`` and ``-inf`` in ``LSE``.
    """
    B, L, Hh, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, L, Hh, v.shape[3]), dtype=np.float64)
    lse = np.full((B, Hh, L), -np.inf, dtype=np.float64)
    cu = [int(c) for c in cu_seqlens]
    for b in range(B):
        for i in range(len(cu) - 1):
            a, e = cu[i], cu[i + 1]
            if e <= a:
                continue
            for h in range(Hh):
                oh, lh = head_attention(q[b, a:e, h], k[b, a:e, h], v[b, a:e, h], scale)
                o[b, a:e, h] = oh
                lse[b, h, a:e] = lh
    return o, lse


def masked_full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window_of_token, scale: float | None = None):
    """Brute force: full attention over all ``L`` tokens of ``[B, L, Hh, D]``
    inputs in any token order, where token ``a`` may attend to token ``c`` only
    if ``window_of_token[a] == window_of_token[c]``.  Returns ``(O, LSE)`` as
    ``window_attention`` does.  Costs ``O(L^2)``: tiny grids only."""
    B, L, Hh, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    win = np.asarray(window_of_token)
    allowed = win[:, None] == win[None, :]
    o = np.empty((B, L, Hh, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hh, L), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            s = (q[b, :, h] @ k[b, :, h].T) * scale
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            o[b, :, h] = (e @ v[b, :, h]) / z
            lse[b, h] = (m + np.log(z))[:, 0]
    return o, lse


def attention_flops(cu_seqlens, batch: int, heads: int, head_dim: int) -> int:
    """Useful multiply-add work of window attention, counted as 2 flops per
    multiply-add for ``Q K^T`` and for ``P V``: ``4 n^2 D`` per window, head
    and batch element."""
    cu = [int(c) for c in cu_seqlens]
    return sum(4 * (cu[i + 1] - cu[i]) ** 2 * head_dim for i in range(len(cu) - 1)) * heads * batch

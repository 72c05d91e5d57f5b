"""Oracle of text-augmented window attention (test infrastructure only; see
``oracle/__init__``).

Source: page "Window-Aligned Sequence Parallelism (SeedVR2)":

* section "SeedVR2 integration": window attention is a packed variable-length
  call over ``[video window, replicated text]`` segments, i.e. every window's
  segment is its video rows followed by the text rows, and attention runs over
  the whole segment;
* section "Text stream": text is replicated and stays identical; each
  layer's attention produces one text output per window, and the text passed
  on is the sum of the per-window text outputs divided by the global window
  count of the layout -- neither a token-weighted mean nor a mean of rank
  means.

Readings where the page is silent (listed in the design notes):

* Video rows of a window attend to the window's video keys and to the text
  keys; text rows attend, once per window, to that window's video keys and to
  the text keys (the segment is one document).
* Every segment of the call counts as a window in the division, zero-length
  segments included (their text output is attention over the text alone).

fp64 throughout; the per-segment attention is ``oracle.attention.head_attention``
over the concatenated rows.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import head_attention


def text_window_attention(q, k, v, cu, tq, tk, tv, scale=None):
    """``q, k, v``: fp64 [B, L, heads, D] in window order; ``cu``: the
    segments; ``tq, tk, tv``: fp64 [B, T, heads, D] text rows.  Returns
    (video outputs [B, L, heads, D], text output [B, T, heads, D], per-window
    text outputs [B, N, T, heads, D])."""
    B, L, Hh, D = q.shape
    T = tq.shape[1]
    s = 1.0 / math.sqrt(D) if scale is None else scale
    N = len(cu) - 1
    o = np.zeros((B, L, Hh, D))
    per = np.zeros((B, N, T, Hh, D))
    for b in range(B):
        for i in range(N):
            a, e = cu[i], cu[i + 1]
            n = e - a
            for h in range(Hh):
                qs = np.concatenate([q[b, a:e, h], tq[b, :, h]])
                ks = np.concatenate([k[b, a:e, h], tk[b, :, h]])
                vs = np.concatenate([v[b, a:e, h], tv[b, :, h]])
                if len(qs) == 0:
                    continue
                os_, _ = head_attention(qs, ks, vs, s)
                o[b, a:e, h] = os_[:n]
                per[b, i, :, h] = os_[n:]
    text = per.sum(axis=1) / N if N else np.zeros((B, T, Hh, D))
    return o, text, per

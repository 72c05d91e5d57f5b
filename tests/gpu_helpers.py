"""Shared helpers of the GPU parity tests: layout chains, oracle calls on
host copies of device data, and the error measures."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import window_attention_amd as wa
from oracle import attention as oatt
from window_attention_amd.inputs import bf16_bits

# tolerance of bf16-in / fp32-accumulate attention against the fp64 oracle
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# LSE bound per query row.  The kernel's scores are fp32 sums of exact bf16
# products and its normaliser is the fp32 sum of fp32 probabilities, so its
# LSE error is at the fp32 level; the bound is deliberately looser:
#  * 2^-9 for a normaliser summed from bf16-rounded probabilities;
#  * 2^-9 * scale * sum_d |q_d k_d| for a score computed from operands
#    rounded once more to bf16 (a log-sum-exp moves by at most the largest
#    such change over the keys) -- the kernel rounds none, and a kernel that
#    folded the softmax scale into a bf16 Q would fail it on peaked rows;
#  * 5e-4 for exp2 / log and the fp32 accumulations.
LSE_SLACK = 5e-4


def lse_bound(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Per-row LSE tolerance for one window and head: q, k are [n, D]."""
    worst = (np.abs(q) @ np.abs(k).T).max(axis=1)
    return 2.0 ** -9 + 2.0 ** -9 * scale * worst + LSE_SLACK


def lse_bound_windows(q, k, cu, scale=None):
    """lse_bound for [B, L, Hh, D] window-ordered inputs, as [B, Hh, L]."""
    B, L, Hh, D = q.shape
    s = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.full((B, Hh, L), np.inf)
    for b in range(B):
        for i in range(len(cu) - 1):
            a, e = int(cu[i]), int(cu[i + 1])
            for h in range(Hh):
                if e > a:
                    out[b, h, a:e] = lse_bound(q[b, a:e, h], k[b, a:e, h], s)
    return out


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(x: torch.Tensor) -> np.ndarray:
    if x.dtype == torch.bfloat16:
        return oatt.bf16_bits_to_float64(bf16_bits(x))
    return x.detach().cpu().double().numpy()


def method_of(letter: str) -> int:
    return wa.REGULAR if letter == "R" else wa.SHIFTED


def check_window_head(q, k, v, o, lse, cu_host, b, i, h, scale=None):
    """Oracle attention of (batch b, window i, head h) on host copies of the
    device inputs; returns (max_abs, mean_abs, lse_max_abs, rows)."""
    a, e = int(cu_host[i]), int(cu_host[i + 1])
    if e <= a:
        return 0.0, 0.0, 0.0, 0
    D = q.shape[3]
    s = 1.0 / math.sqrt(D) if scale is None else scale
    qh, kh, vh = (to_f64(x[b, a:e, h]) for x in (q, k, v))
    ref, ref_lse = oatt.head_attention(qh, kh, vh, s)
    got = to_f64(o[b, a:e, h])
    err = np.abs(got - ref)
    lerr = 0.0
    if lse is not None:
        # error as a fraction of the per-row bound (<= 1 passes)
        bound = lse_bound(qh, kh, s)
        lerr = float(np.max(np.abs(lse[b, h, a:e].double().cpu().numpy() - ref_lse) / bound))
    return float(err.max()), float(err.mean()), lerr, e - a


def assert_close_full(o, lse, ref_o, ref_lse, lse_tol=None):
    """Element-wise comparison of all outputs; lse_tol is the per-row LSE
    bound (lse_bound_windows) when lse is checked."""
    got = to_f64(o)
    err = np.abs(got - ref_o)
    assert err.max() <= MAX_ABS, f"max abs err {err.max()}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean()}"
    if lse is not None:
        le = np.abs(lse.double().cpu().numpy() - ref_lse)
        assert np.all(le <= lse_tol), f"lse err {le.max()} (worst ratio to bound {(le / lse_tol).max():.3f})"
    return float(err.max()), float(err.mean())

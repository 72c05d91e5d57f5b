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
# LSE bound per query row, from the kernel's arithmetic (no bf16 rounding
# touches the LSE: the bf16 probabilities only feed the P V product).
# LSE = log sum_k exp(x_k) with x_k = scale * s_k moves by at most
# max_k |dx_k| (its gradient is the softmax row), so the bound is:
#  * scores: s_k is an fp32 sum of D exact bf16 products, at most D
#    roundings of 2^-23 relative to sum_d |q_d k_d| (truncation covered);
#    c = scale * log2(e) and the caller's scale are fp32, 2^-22 relative
#    to |x_k| in all; the fma c * s - ref rounds once, relative to a result
#    of at most ~2^5 for any key that contributes (2^-18);
#  * normaliser: fp32 exp2 per probability (2^-21 relative), row sums of
#    positive terms added in chains of at most 32 + tiles + 2 roundings, and
#    one exp2 factor (2^-21) and one product (2^-24) per reference move, at
#    most one move per 64-key tile; a relative error e of the sum is e in
#    the log;
#  * the final fp32 combination ref * ln 2 + log(sum): 2^-21 relative to
#    the magnitudes involved, at most max_k |x_k| + log(n) + 8 * ln 2
#    (probabilities stay below 2^8 against the reference).
KEY_TILE = 64


def lse_bound(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Per-row LSE tolerance for one segment and head: q [n, D] queries,
    k [m, D] the keys they attend to (fp64 copies of the bf16 inputs)."""
    D = q.shape[1]
    m = k.shape[0]
    s_abs = np.abs(q @ k.T) * scale
    score = (D * 2.0 ** -23 * scale * (np.abs(q) @ np.abs(k).T) + 2.0 ** -22 * s_abs).max(axis=1) + 2.0 ** -18
    tiles = math.ceil(m / KEY_TILE) + 1  # text keys start on a tile of their own
    norm = 2.0 ** -21 + (32 + tiles + 2) * 2.0 ** -24 + tiles * (2.0 ** -21 + 2.0 ** -24)
    final = 2.0 ** -21 * (s_abs.max(axis=1) + math.log(max(m, 1)) + 8 * math.log(2.0))
    return score + norm + final


def output_bound(q: np.ndarray, k: np.ndarray, o_ref: np.ndarray, pv_abs: np.ndarray, scale: float) -> np.ndarray:
    """Per-element bound on |O_gpu - O| for one segment and head, from the
    kernel's arithmetic, for values of any magnitude: q [n, D], k [m, D],
    o_ref [n, Dv] the exact output and pv_abs [n, Dv] = sum_k p_k |v_k| (the
    oracle applied to |V|).
      * P V takes bf16 roundings of the fp32 probabilities: 2^-8 relative
        each, so 2^-8 * sum_k p_k |v_k|;
      * the fp32 probabilities themselves: the score terms of lse_bound
        (relative error of each p_k), the normaliser's chain of adds and
        reference moves (relative error of the row sum, hence of O);
      * the fp32 P V accumulation over m keys, n_tiles deferred rescales
        (an exp2 factor and a product each) and the final 1 / l product:
        m * 2^-24 + tiles * 2^-20 + 2^-22 relative to sum_k p_k |v_k|;
      * the bf16 rounding of the output: 2^-8 relative to the computed value.
    """
    D = q.shape[1]
    m = k.shape[0]
    s_abs = np.abs(q @ k.T) * scale
    score = (D * 2.0 ** -23 * scale * (np.abs(q) @ np.abs(k).T) + 2.0 ** -22 * s_abs).max(axis=1) + 2.0 ** -18
    tiles = math.ceil(m / KEY_TILE) + 1
    norm = 2.0 ** -21 + (32 + tiles + 2) * 2.0 ** -24 + tiles * (2.0 ** -21 + 2.0 ** -24)
    acc = m * 2.0 ** -24 + tiles * 2.0 ** -20 + 2.0 ** -22
    rel = 2.0 ** -8 + np.expm1(score)[:, None] + norm + acc
    return 2.0 ** -8 * np.abs(o_ref) + (1 + 2.0 ** -8) * rel * pv_abs


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
